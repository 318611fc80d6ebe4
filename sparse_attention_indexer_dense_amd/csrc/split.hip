// split.hip - kernels for few query rows over long key ranges (decode shape).
//
// A decode step of the PIVOT paper (Method, decode groups formed by the MTP
// drafts of one step) scores only g new rows per request against a long
// cache, so there are too few rows to fill the GPU with one workgroup per row.
// The key axis is split instead:
//   split_score_kernel  - a workgroup owns (batch item, row, span of key
//                         positions); each wave streams its own contiguous
//                         part of the span in 32-key tiles through a private
//                         pair of LDS buffers filled by global->LDS DMA (the
//                         DMA of tile t+1 overlaps the MFMAs on tile t), runs
//                         the MFMA score tile and the ReLU/weight/head-sum
//                         epilogue, and stores one fp32 score per position;
//   split_select_kernel - one workgroup per score row finds the exact top-sel
//                         (ties to the lower index) in three passes: a
//                         level-1 histogram; per-wave counts of the sure
//                         entries plus the boundary bin gathered into LDS and
//                         resolved there; one ordered emission in ascending
//                         index order at per-wave offsets.
// Only the score vectors of the few decode rows are stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "kernels.h"

namespace dsaidx {

// Row r of a split pass: its query/weights, key source and causal limit.
struct SplitRow {
    const uint16_t *q;
    const float *w;
    const int32_t *list;  // kRefine: the group's candidate list
    int npos;             // positions to consider
    int lim;              // last eligible key index
};

__device__ __forceinline__ SplitRow split_row(const SplitScoreParams &p, int H, int D, int bi, int64_t r)
{
    SplitRow s;
    const int64_t off = p.L - p.q_len;
    if (p.mode == kProxy) {
        const int64_t grow = (int64_t)bi * p.G + r;
        const int64_t r1 = ((r + 1) * p.g < p.q_len) ? (r + 1) * p.g : p.q_len;
        s.q = p.Q + grow * H * D;
        s.w = p.W + grow * H;
        s.list = nullptr;
        s.lim = (int)(off + r1 - 1);
        s.npos = s.lim + 1;
    } else {
        const int64_t row = (int64_t)bi * p.q_len + r;
        s.q = p.Q + row * H * D;
        s.w = p.W + row * H;
        s.lim = (int)(off + r);
        if (p.mode == kDense) {
            s.list = nullptr;
            s.npos = s.lim + 1;
        } else {
            const int64_t m = r / p.g;
            const int64_t r1 = ((m + 1) * p.g < p.q_len) ? (m + 1) * p.g : p.q_len;
            const int64_t t_last = off + r1 - 1;
            s.list = p.cand + ((int64_t)bi * p.G + m) * p.c;
            s.npos = (int)((p.c < t_last + 1) ? p.c : t_last + 1);
        }
    }
    return s;
}

// ------------------------------------------------------------------ scoring
// s_waitcnt with only the vector-memory counter constrained to <= n (gfx9
// encoding: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Each wave streams its span of positions through a private ring of kRing
// LDS tiles of 32 keys; tile t+kRing-1 is in flight while tile t is scored.
// Every tile costs exactly DMA_PER_TILE DMA instructions (lanes without a key
// fetch row 0 into a slot that is never read) and exactly one score store, so
// the number of vector-memory operations issued after tile t's DMA is known
// and the wait for it is exact.
constexpr int kRing = 4;

template <int H, int D, bool LIST>
__global__ __launch_bounds__(kSplitWaves * kWave) void split_score_kernel(SplitScoreParams p)
{
    using S = Shape<H, D>;
    constexpr int MB = S::MB, KS = S::KS, ROWB = S::ROWB, CHUNKS = S::CHUNKS;
    constexpr int TILE_BYTES = 32 * ROWB;
    constexpr int DMA_PER_TILE = TILE_BYTES / 1024;
    constexpr int RPI = kWave / CHUNKS;  // key rows per DMA instruction
    __shared__ __align__(1024) unsigned char ring[kSplitWaves][kRing][TILE_BYTES];
    __shared__ int32_t lst[kSplitWaves][LIST ? kSplitSpanMax : 1];

    const int bi = blockIdx.z;
    const int64_t r = blockIdx.y;
    const int wave = uniform(threadIdx.x / kWave);  // wave-uniform (SGPR)
    const int lane = threadIdx.x % kWave;
    const int half = lane >> 5;
    const int col = lane & 31;
    const SplitRow sr = split_row(p, H, D, bi, r);
    const int span = (int)(p.chunk / kSplitWaves);
    const int w0 = (int)(blockIdx.x * p.chunk) + wave * span;
    if (w0 >= sr.npos)
        return;
    const int w1 = (w0 + span < sr.npos) ? w0 + span : sr.npos;
    const int ntile = (w1 - w0 + 31) / 32;
    const uint16_t *Kb = p.K + (int64_t)bi * p.L * D;
    float *out = p.scores + ((int64_t)bi * p.nrows + r) * p.rowlen;
    int32_t *wl = lst[wave];

    if (LIST) {
        for (int x = lane; x < w1 - w0; x += kWave)
            wl[x] = sr.list[w0 + x];
        __builtin_amdgcn_wave_barrier();
    }

    // DMA of tile t into ring slot t % kRing: lane l of instruction i fetches
    // the chunk that the XOR swizzle puts in slot l of the i-th KiB
    auto issue = [&](int t) {
        unsigned char *dst = ring[wave][t % kRing];
#pragma unroll
        for (int i = 0; i < DMA_PER_TILE; ++i) {
            const int n = i * RPI + lane / CHUNKS;
            const int pos = w0 + t * 32 + n;
            const int c = (lane % CHUNKS) ^ (n & (CHUNKS - 1));
            int key = 0;
            if (t < ntile && pos < w1) {
                key = LIST ? wl[pos - w0] : pos;
                key = (key >= 0 && key < p.L) ? key : 0;
            }
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(Kb + (int64_t)key * D + c * 8),
                (__attribute__((address_space(3))) void *)(dst + i * 1024), 16, 0, 0);
        }
    };

    bf16x8 qa[MB][KS];
    float wv[MB][16];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int head = mb * 32 + col;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (head < H)
                v = *reinterpret_cast<const u32x4 *>(sr.q + (int64_t)head * D + (half * KS + ks) * 8);
            qa[mb][ks] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int hr = mb * 32 + 8 * (rr / 4) + 4 * half + (rr % 4);
            wv[mb][rr] = hr < H ? sr.w[hr] : 0.f;
        }
    }
    uint32_t koff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        koff[ks] = (uint32_t)(col * ROWB + (((half * KS + ks) ^ (col & (CHUNKS - 1))) * 16));

    auto tile = [&](int t) {
        const unsigned char *src = ring[wave][t % kRing];
        f32x16 acc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            acc[mb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(src + koff[ks]));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], kf, acc[mb], 0, 0, 0);
        }
        float part[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            part[mb] = 0.f;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr)
                part[mb] = fmaf(wv[mb][rr], relu(acc[mb][rr]), part[mb]);
        }
        float s = part[0];
#pragma unroll
        for (int mb = 1; mb < MB; ++mb)
            s += part[mb];
        const float total = half_wave_sum(s) + 0.0f;
        // one store instruction per tile: lane 0 always holds a position of
        // the tile; positions whose key is beyond the row's limit get a score
        // too, which the selection ignores
        const int pos = w0 + t * 32 + col;
        if (lane < 32 && pos < w1)
            out[pos] = total;
    };

    // operands loaded, then the ring primed with kRing - 1 tiles
    __builtin_amdgcn_s_waitcnt(0);
    for (int t = 0; t < kRing - 1; ++t)
        issue(t);
    for (int t = 0; t < ntile; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        if (t == 0)
            wait_vmcnt<(kRing - 2) * DMA_PER_TILE>();
        else if (t == 1)
            wait_vmcnt<(kRing - 2) * DMA_PER_TILE + 1>();
        else if (t == 2)
            wait_vmcnt<(kRing - 2) * DMA_PER_TILE + 2>();
        else
            wait_vmcnt<(kRing - 2) * DMA_PER_TILE + 3>();
        __builtin_amdgcn_sched_barrier(0);
        issue(t + kRing - 1);
        tile(t);
    }
    // no DMA may still be writing this workgroup's LDS when it exits
    __builtin_amdgcn_s_waitcnt(0);
}

// ---------------------------------------------------------------- selection
constexpr int kSelWaves = kSelectThreads / kWave;
constexpr int kBoundaryCap = 4096;  // boundary-bin entries resolved in LDS
constexpr int kQuadsPerLane = 8;    // float4 loads in flight per lane and pass

struct SelRow {
    const float *sc;
    const int32_t *list;
    int npos, lim;
};

// Row selection bins: level 1 = top 14 bits of the score key (sign, exponent,
// five mantissa bits), then 9 + 9 bits inside the boundary bin.
constexpr int kSelBins1 = 16384;
constexpr int kSelBins2 = 512;

struct SelScratch {
    uint32_t h1[kSelBins1];
    uint32_t hs[kBins2];
    uint32_t bkey[kBoundaryCap];
    int32_t bpos[kBoundaryCap];
    int wgt[kSelWaves];  // per wave: sure entries (bin above the cut bin)
    int wbd[kSelWaves];  // per wave: selected boundary entries
    int woff[kSelWaves];
    int nb;
    int bc[8];
};

__device__ __forceinline__ bool sel_valid(const SelRow &s, int pos)
{
    return pos < s.npos && (s.list == nullptr || s.list[pos] <= s.lim);
}

// The row's positions split into kSelWaves contiguous segments; a wave walks
// its segment in steps of 256 positions (one float4 per lane), kQuadsPerLane
// steps per batch with all their loads issued first.
struct Segment {
    int b, e;
};

__device__ __forceinline__ Segment wave_segment(int npos, int wave)
{
    const int per = (((npos + kSelWaves - 1) / kSelWaves) + 255) / 256 * 256;
    Segment g;
    g.b = wave * per;
    g.e = (g.b + per < npos) ? g.b + per : npos;
    if (g.b > npos)
        g.b = npos;
    return g;
}

template <typename F>
__device__ __forceinline__ void segment_pass(const SelRow &s, Segment g, F &&f)
{
    const int lane = threadIdx.x % kWave;
    for (int base = g.b; base < g.e; base += kQuadsPerLane * 256) {
        float v[kQuadsPerLane][4];
#pragma unroll
        for (int u = 0; u < kQuadsPerLane; ++u) {
            const int p0 = base + u * 256 + lane * 4;
#pragma unroll
            for (int x = 0; x < 4; ++x)
                v[u][x] = (p0 + x < g.e) ? s.sc[p0 + x] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kQuadsPerLane; ++u) {
            const int p0 = base + u * 256 + lane * 4;
            if (base + u * 256 < g.e)
                f(v[u], p0);
        }
    }
}

__device__ __forceinline__ int wave_exclusive_sum(int v, int &total)
{
    const int lane = threadIdx.x % kWave;
    int x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o, kWave);
        if (lane >= o)
            x += y;
    }
    total = __shfl(x, kWave - 1, kWave);
    return x - v;
}

// Exclusive prefix count of `flag` over the block in thread order (fallback path).
__device__ __forceinline__ int block_prefix(bool flag, int *wtot, int &total)
{
    const int wave = uniform(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const uint64_t m = ballot(flag);
    if (lane == 0)
        wtot[wave] = __popcll(m);
    __syncthreads();
    int off = 0, tot = 0;
    for (int w = 0; w < kSelWaves; ++w) {
        const int v = wtot[w];
        off += (w < wave) ? v : 0;
        tot += v;
    }
    __syncthreads();
    total = tot;
    return off + prefix_count(m);
}

__device__ __forceinline__ void block_clear(uint32_t *h, int n)
{
    for (int i = threadIdx.x; i < n; i += blockDim.x)
        h[i] = 0u;
}

// Largest bin with suffix count >= target, found by wave 0 and broadcast.
template <int NB>
__device__ __forceinline__ void block_find_bin(const uint32_t *h, int target, SelScratch &sm, int &x, int &above)
{
    if (threadIdx.x < kWave) {
        int bx, ab;
        find_bin<NB>(h, target, bx, ab);
        if (threadIdx.x == 0) {
            sm.bc[0] = bx;
            sm.bc[1] = ab;
        }
    }
    __syncthreads();
    x = sm.bc[0];
    above = sm.bc[1];
    __syncthreads();
}

// Fallback cut over the whole row (used when the boundary bin does not fit
// in LDS): levels 2 and 3 by passes over the row; ties by index order.
__device__ Cut block_cut(const SelRow &s, SelScratch &sm, int count, int sel)
{
    Cut c;
    c.keq = 0u;
    c.req = 0;
    if (count <= sel) {
        c.kgt = -1;
        return c;
    }
    block_clear(sm.h1, kBins1);
    __syncthreads();
    for (int pos = threadIdx.x; pos < s.npos; pos += blockDim.x)
        if (sel_valid(s, pos))
            atomicAdd(&sm.h1[bin1(score_key(s.sc[pos]))], 1u);
    __syncthreads();
    int b1, above;
    block_find_bin<kBins1>(sm.h1, sel, sm, b1, above);
    const int r1 = sel - above;
    const int hb1 = (int)sm.h1[b1];
    if (r1 == hb1) {
        c.kgt = (int64_t)b1 * (1ll << 21) - 1;
        return c;
    }
    block_clear(sm.hs, kBins2);
    __syncthreads();
    for (int pos = threadIdx.x; pos < s.npos; pos += blockDim.x) {
        if (!sel_valid(s, pos))
            continue;
        const uint32_t key = score_key(s.sc[pos]);
        if ((int)(key >> 21) == b1)
            atomicAdd(&sm.hs[(key >> 10) & (kBins2 - 1)], 1u);
    }
    __syncthreads();
    int b2, a2;
    block_find_bin<kBins2>(sm.hs, r1, sm, b2, a2);
    const int r2 = r1 - a2;
    const int hb2 = (int)sm.hs[b2];
    const uint32_t pre = ((uint32_t)b1 << 11) | (uint32_t)b2;
    __syncthreads();
    if (r2 == hb2) {
        c.kgt = (int64_t)pre * 1024 - 1;
        return c;
    }
    block_clear(sm.hs, kBins3);
    __syncthreads();
    for (int pos = threadIdx.x; pos < s.npos; pos += blockDim.x) {
        if (!sel_valid(s, pos))
            continue;
        const uint32_t key = score_key(s.sc[pos]);
        if ((key >> 10) == pre)
            atomicAdd(&sm.hs[key & (kBins3 - 1)], 1u);
    }
    __syncthreads();
    int b3, a3;
    block_find_bin<kBins3>(sm.hs, r2, sm, b3, a3);
    const uint32_t kstar = (pre << 10) | (uint32_t)b3;
    c.kgt = (int64_t)kstar;
    c.keq = kstar;
    c.req = r2 - a3;
    return c;
}

__device__ void block_emit_fallback(const SelRow &s, SelScratch &sm, const Cut &c, int sel, int32_t *oidx,
                                    float *osc, int fan, int64_t fstride)
{
    int emitted = 0, eqseen = 0;
    for (int base = 0; base < s.npos; base += blockDim.x) {
        const int pos = base + threadIdx.x;
        const bool v = sel_valid(s, pos);
        float score = 0.f;
        uint32_t key = 0u;
        if (v) {
            score = s.sc[pos];
            key = score_key(score);
        }
        const bool eq = v && c.req > 0 && key == c.keq;
        int eqtot;
        const int er = eqseen + block_prefix(eq, sm.wgt, eqtot);
        const bool in = v && ((int64_t)key > c.kgt || (eq && er < c.req));
        int intot;
        const int opos = emitted + block_prefix(in, sm.wgt, intot);
        if (in && opos < sel) {
            const int32_t idx = s.list ? s.list[pos] : pos;
            for (int f = 0; f < fan; ++f) {
                oidx[f * fstride + opos] = idx;
                if (osc)
                    osc[f * fstride + opos] = score;
            }
        }
        emitted += intot;
        eqseen += eqtot;
    }
    for (int x = emitted + threadIdx.x; x < sel; x += blockDim.x) {
        for (int f = 0; f < fan; ++f) {
            oidx[f * fstride + x] = -1;
            if (osc)
                osc[f * fstride + x] = -__builtin_inff();
        }
    }
}

// Top-`sel` of the row (level-1 histogram already in sm.h1, `count` valid
// positions): collect the boundary bin into LDS, resolve it there, then emit.
// h1 must be rebuilt by the caller before another call (the fallback reuses it).
__device__ void select_row(const SelRow &s, SelScratch &sm, int count, int sel, int32_t *oidx, float *osc,
                           int fan, int64_t fstride)
{
    const int wave = uniform(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const Segment seg = wave_segment(s.npos, wave);
    // cut bin and how many of its entries are taken
    int b1 = 0, above = 0;
    if (count > sel)
        block_find_bin<kSelBins1>(sm.h1, sel, sm, b1, above);
    const bool all = count <= sel;
    const int r1 = all ? 0 : sel - above;
    const int hb1 = all ? 0 : (int)sm.h1[b1];
    __syncthreads();
    if (!all && hb1 > kBoundaryCap) {
        const Cut c = block_cut(s, sm, count, sel);
        block_emit_fallback(s, sm, c, sel, oidx, osc, fan, fstride);
        return;
    }
    const bool whole = all || r1 == hb1;  // every entry of the cut bin is taken

    // pass 1: per-wave counts of sure entries; boundary entries into LDS
    if (threadIdx.x == 0)
        sm.nb = 0;
    __syncthreads();
    int sure = 0;
    segment_pass(s, seg, [&](const float (&v)[4], int p0) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int pos = p0 + x;
            bool bnd = false;
            uint32_t key = 0u;
            if (pos < seg.e && sel_valid(s, pos)) {
                key = score_key(v[x]);
                const int bn = (int)(key >> 18);
                if (all || bn > b1 || (whole && bn == b1))
                    ++sure;
                else
                    bnd = bn == b1;
            }
            const uint64_t m = ballot(bnd);
            if (m) {
                int base = 0;
                if (lane == 0)
                    base = atomicAdd(&sm.nb, __popcll(m));
                base = __shfl(base, 0, kWave);
                if (bnd) {
                    const int slot = base + prefix_count(m);
                    sm.bkey[slot] = key;
                    sm.bpos[slot] = pos;
                }
            }
        }
    });
    sure = wave_sum(sure);
    if (lane == 0) {
        sm.wgt[wave] = sure;
        sm.wbd[wave] = 0;
    }
    __syncthreads();

    // resolve the boundary: the r1 best of its nb entries by (key desc, pos asc)
    uint32_t kcut = 0xFFFFFFFFu;  // boundary entries with key > kcut are in
    uint32_t keq = 0u;            // ... and those with key == keq and pos <= pcut
    int pcut = -1;
    if (!whole) {
        const int nb = sm.nb;
        block_clear(sm.hs, kSelBins2);
        __syncthreads();
        for (int i = threadIdx.x; i < nb; i += blockDim.x)
            atomicAdd(&sm.hs[(sm.bkey[i] >> 9) & (kSelBins2 - 1)], 1u);
        __syncthreads();
        int b2, a2;
        block_find_bin<kSelBins2>(sm.hs, r1, sm, b2, a2);
        const int r2 = r1 - a2;
        const uint32_t pre = ((uint32_t)b1 << 9) | (uint32_t)b2;
        block_clear(sm.hs, kSelBins2);
        __syncthreads();
        for (int i = threadIdx.x; i < nb; i += blockDim.x)
            if ((sm.bkey[i] >> 9) == pre)
                atomicAdd(&sm.hs[sm.bkey[i] & (kSelBins2 - 1)], 1u);
        __syncthreads();
        int b3, a3;
        block_find_bin<kSelBins2>(sm.hs, r2, sm, b3, a3);
        const int r3 = r2 - a3;
        keq = (pre << 9) | (uint32_t)b3;
        kcut = keq;
        const int m3 = (int)sm.hs[b3];
        __syncthreads();
        if (r3 >= m3) {
            pcut = 0x7FFFFFFF;
        } else {
            // the r3 lowest positions among the m3 entries equal to keq: the
            // entry with exactly r3 - 1 lower equal positions is the last one in
            if (threadIdx.x == 0)
                sm.bc[4] = -1;
            __syncthreads();
            for (int i = threadIdx.x; i < nb; i += blockDim.x) {
                if (sm.bkey[i] != keq)
                    continue;
                int lower = 0;
                for (int j2 = 0; j2 < nb; ++j2)
                    lower += (sm.bkey[j2] == keq && sm.bpos[j2] < sm.bpos[i]) ? 1 : 0;
                if (lower == r3 - 1)
                    sm.bc[4] = sm.bpos[i];
            }
            __syncthreads();
            pcut = sm.bc[4];
        }
        // selected boundary entries per wave segment (segment = pos / per)
        const int per = (((s.npos + kSelWaves - 1) / kSelWaves) + 255) / 256 * 256;
        for (int i = threadIdx.x; i < nb; i += blockDim.x) {
            const uint32_t key = sm.bkey[i];
            if (key > kcut || (key == keq && sm.bpos[i] <= pcut))
                atomicAdd(&sm.wbd[sm.bpos[i] / per], 1);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        int o = 0;
        for (int w = 0; w < kSelWaves; ++w) {
            sm.woff[w] = o;
            o += sm.wgt[w] + sm.wbd[w];
        }
        sm.bc[5] = o;
    }
    __syncthreads();
    const int emitted_total = sm.bc[5];

    // pass 2: ordered emission of this wave's segment
    int run = sm.woff[wave];
    segment_pass(s, seg, [&](const float (&v)[4], int p0) {
        bool in[4];
        int n = 0;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int pos = p0 + x;
            in[x] = false;
            if (pos < seg.e && sel_valid(s, pos)) {
                const uint32_t key = score_key(v[x]);
                const int bn = (int)(key >> 18);
                if (all || bn > b1 || (whole && bn == b1))
                    in[x] = true;
                else if (bn == b1)
                    in[x] = key > kcut || (key == keq && pos <= pcut);
            }
            n += in[x] ? 1 : 0;
        }
        int tot;
        int o = run + wave_exclusive_sum(n, tot);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            if (in[x]) {
                if (o < sel) {
                    const int pos = p0 + x;
                    const int32_t idx = s.list ? s.list[pos] : pos;
                    for (int f = 0; f < fan; ++f) {
                        oidx[f * fstride + o] = idx;
                        if (osc)
                            osc[f * fstride + o] = v[x];
                    }
                }
                ++o;
            }
        }
        run += tot;
    });
    for (int x = emitted_total + threadIdx.x; x < sel; x += blockDim.x) {
        for (int f = 0; f < fan; ++f) {
            oidx[f * fstride + x] = -1;
            if (osc)
                osc[f * fstride + x] = -__builtin_inff();
        }
    }
    __syncthreads();
}

// pass 0: level-1 histogram of the valid positions; returns their count
__device__ int row_histogram(const SelRow &s, SelScratch &sm)
{
    const int wave = uniform(threadIdx.x / kWave);  // wave-uniform (SGPR)
    block_clear(sm.h1, kSelBins1);
    __syncthreads();
    const Segment seg = wave_segment(s.npos, wave);
    int cnt = 0;
    segment_pass(s, seg, [&](const float (&v)[4], int p0) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int pos = p0 + x;
            if (pos < seg.e && sel_valid(s, pos)) {
                atomicAdd(&sm.h1[score_key(v[x]) >> 18], 1u);
                ++cnt;
            }
        }
    });
    cnt = wave_sum(cnt);
    if (threadIdx.x % kWave == 0)
        sm.wgt[wave] = cnt;
    __syncthreads();
    int count = 0;
    for (int w = 0; w < kSelWaves; ++w)
        count += sm.wgt[w];
    __syncthreads();
    return count;
}

__global__ __launch_bounds__(kSelectThreads) void split_select_kernel(SplitSelectParams p)
{
    __shared__ SelScratch sm;
    const int bi = blockIdx.y;
    const int64_t r = blockIdx.x;
    const int64_t off = p.L - p.q_len;

    SelRow s;
    s.sc = p.scores + ((int64_t)bi * p.nrows + r) * p.rowlen;
    int32_t *o1, *o2 = nullptr;
    float *s1, *s2 = nullptr;
    int fan1 = 1, fan2 = 0;
    if (p.mode == kProxy) {
        const int64_t r0 = r * p.g;
        const int64_t r1 = (r0 + p.g < p.q_len) ? r0 + p.g : p.q_len;
        s.list = nullptr;
        s.lim = (int)(off + r1 - 1);
        s.npos = s.lim + 1;
        const int64_t mrow = (int64_t)bi * p.q_len + r0;
        const int64_t grow = (int64_t)bi * p.G + r;
        if (p.o1_members) {
            o1 = p.o1_idx + mrow * p.sel;
            s1 = p.o1_score ? p.o1_score + mrow * p.sel : nullptr;
            fan1 = (int)(r1 - r0);
        } else {
            o1 = p.o1_idx + grow * p.sel;
            s1 = p.o1_score ? p.o1_score + grow * p.sel : nullptr;
        }
        if (p.sel2 > 0) {
            o2 = p.o2_idx + mrow * p.sel2;
            s2 = p.o2_score ? p.o2_score + mrow * p.sel2 : nullptr;
            fan2 = (int)(r1 - r0);
        }
    } else {
        const int64_t row = (int64_t)bi * p.q_len + r;
        s.lim = (int)(off + r);
        if (p.mode == kDense) {
            s.list = nullptr;
            s.npos = s.lim + 1;
        } else {
            const int64_t m = r / p.g;
            const int64_t r1 = ((m + 1) * p.g < p.q_len) ? (m + 1) * p.g : p.q_len;
            const int64_t t_last = off + r1 - 1;
            s.list = p.cand + ((int64_t)bi * p.G + m) * p.c;
            s.npos = (int)((p.c < t_last + 1) ? p.c : t_last + 1);
        }
        o1 = p.o1_idx + row * p.sel;
        s1 = p.o1_score ? p.o1_score + row * p.sel : nullptr;
    }

    const int count = row_histogram(s, sm);
    select_row(s, sm, count, p.sel, o1, s1, fan1, p.sel);
    if (p.sel2 > 0) {
        row_histogram(s, sm);
        select_row(s, sm, count, p.sel2, o2, s2, fan2, p.sel2);
    }
}

// ------------------------------------------------------------- launchers
template <int H, int D>
static hipError_t launch_split_score_t(const SplitScoreParams &prm, dim3 grid, hipStream_t stream)
{
    if (prm.mode == kRefine)
        hipLaunchKernelGGL((split_score_kernel<H, D, true>), grid, dim3(kSplitWaves * kWave), 0, stream, prm);
    else
        hipLaunchKernelGGL((split_score_kernel<H, D, false>), grid, dim3(kSplitWaves * kWave), 0, stream, prm);
    return hipGetLastError();
}

hipError_t launch_split_score(int H, int D, const SplitScoreParams &prm, dim3 grid, hipStream_t stream)
{
    if (prm.chunk % (32 * kSplitWaves) != 0 || prm.chunk / kSplitWaves > kSplitSpanMax)
        return hipErrorInvalidValue;
    if (H == 64 && D == 128)
        return launch_split_score_t<64, 128>(prm, grid, stream);
    if (H == 4 && D == 32)
        return launch_split_score_t<4, 32>(prm, grid, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_split_select(const SplitSelectParams &prm, hipStream_t stream)
{
    hipLaunchKernelGGL(split_select_kernel, dim3((unsigned)prm.nrows, (unsigned)prm.B),
                       dim3(kSelectThreads), 0, stream, prm);
    return hipGetLastError();
}

}  // namespace dsaidx
