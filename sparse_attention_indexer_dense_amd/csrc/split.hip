// split.hip - kernels for few query rows over long key ranges (decode shape).
//
// A decode step of the PIVOT paper (Method, decode groups formed by the MTP
// drafts of one step) scores only g new rows per request against a long
// cache, so there are too few rows to fill the GPU with one workgroup per row.
// The key axis is split instead:
//   split_score_kernel  - workgroups own (batch item, row, key chunk); every
//                         wave stages 32 keys at a time through its own LDS
//                         tile with coalesced 16-byte loads (or gathers the
//                         candidate rows, for Refine), computes the 64-head
//                         score tile with bf16 MFMA and the ReLU/weight/head-sum
//                         epilogue, and stores one fp32 score per position;
//   split_select_kernel - one workgroup per score row runs the exact
//                         three-level radix cut (ties to the lower index) and
//                         writes the selection in ascending index order.
// Only per-row score vectors of the few decode rows are stored.
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
    int64_t npos;         // positions to consider
    int64_t lim;          // last eligible key index
};

template <int H, int D>
__device__ __forceinline__ SplitRow split_row(const SplitScoreParams &p, int bi, int64_t r)
{
    SplitRow s;
    const int64_t off = p.L - p.q_len;
    if (p.mode == kProxy) {
        const int64_t grow = (int64_t)bi * p.G + r;
        const int64_t r1 = ((r + 1) * p.g < p.q_len) ? (r + 1) * p.g : p.q_len;
        s.q = p.Q + grow * H * D;
        s.w = p.W + grow * H;
        s.list = nullptr;
        s.lim = off + r1 - 1;
        s.npos = s.lim + 1;
    } else {
        const int64_t row = (int64_t)bi * p.q_len + r;
        s.q = p.Q + row * H * D;
        s.w = p.W + row * H;
        s.lim = off + r;
        if (p.mode == kDense) {
            s.list = nullptr;
            s.npos = s.lim + 1;
        } else {
            const int64_t m = r / p.g;
            const int64_t r1 = ((m + 1) * p.g < p.q_len) ? (m + 1) * p.g : p.q_len;
            const int64_t t_last = off + r1 - 1;
            s.list = p.cand + ((int64_t)bi * p.G + m) * p.c;
            s.npos = (p.c < t_last + 1) ? p.c : t_last + 1;
        }
    }
    return s;
}

template <int H, int D>
__global__ __launch_bounds__(kSplitWaves * kWave) void split_score_kernel(SplitScoreParams p)
{
    using S = Shape<H, D>;
    constexpr int MB = S::MB, KS = S::KS, ROWS = S::ROWS, CHUNKS = S::CHUNKS;
    constexpr int TILE_CHUNKS = 32 * CHUNKS;
    constexpr int LPL = (TILE_CHUNKS + kWave - 1) / kWave;  // 16-byte loads per lane per tile
    __shared__ __align__(16) unsigned char tiles[kSplitWaves][32 * ROWS];

    const int bi = blockIdx.z;
    const int64_t r = blockIdx.y;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int half = lane >> 5;
    const int col = lane & 31;
    const SplitRow sr = split_row<H, D>(p, bi, r);
    const int64_t p0 = (int64_t)blockIdx.x * p.chunk;
    if (p0 >= sr.npos)
        return;
    const int64_t p1 = (p0 + p.chunk < sr.npos) ? p0 + p.chunk : sr.npos;
    const uint16_t *Kb = p.K + (int64_t)bi * p.L * D;
    float *out = p.scores + ((int64_t)bi * p.nrows + r) * p.rowlen;
    unsigned char *tile = tiles[wave];

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

    for (int64_t pt = p0 + wave * 32; pt < p1; pt += kSplitWaves * 32) {
        // stage 32 key rows: consecutive lanes read consecutive 16-byte chunks
        u32x4 regs[LPL];
#pragma unroll
        for (int i = 0; i < LPL; ++i) {
            const int c = lane + i * kWave;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (c < TILE_CHUNKS) {
                const int kk = c / CHUNKS, part = c % CHUNKS;
                const int64_t pos = pt + kk;
                if (pos < p1) {
                    const int64_t key = sr.list ? (int64_t)sr.list[pos] : pos;
                    if (key >= 0 && key < p.L)
                        v = *reinterpret_cast<const u32x4 *>(Kb + key * D + part * 8);
                }
            }
            regs[i] = v;
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < LPL; ++i) {
            const int c = lane + i * kWave;
            if (c < TILE_CHUNKS) {
                const int kk = c / CHUNKS, part = c % CHUNKS;
                *reinterpret_cast<u32x4 *>(tile + kk * ROWS + part * 16) = regs[i];
            }
        }
        __builtin_amdgcn_wave_barrier();

        f32x16 acc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            acc[mb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 kv = *reinterpret_cast<const u32x4 *>(tile + col * ROWS + (half * KS + ks) * 16);
            bf16x8 kb = __builtin_bit_cast(bf16x8, kv);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], kb, acc[mb], 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
        float part = 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr)
                part = fmaf(wv[mb][rr], relu(acc[mb][rr]), part);
        const float total = half_wave_sum(part) + 0.0f;
        const int64_t pos = pt + col;
        if (lane < 32 && pos < p1) {
            const int64_t key = sr.list ? (int64_t)sr.list[pos] : pos;
            if (key <= sr.lim)
                out[pos] = total;
        }
    }
}

// ------------------------------------------------------------- selection
constexpr int kSelWaves = kSelectThreads / kWave;

struct SelRow {
    const float *sc;
    const int32_t *list;
    int64_t npos, lim;
};

struct BlockScratch {
    uint32_t h1[kBins1];
    uint32_t hs[kBins2];
    int wtot[kSelWaves];
    int bc[4];
};

__device__ __forceinline__ bool sel_valid(const SelRow &s, int64_t pos)
{
    return pos < s.npos && (s.list == nullptr || (int64_t)s.list[pos] <= s.lim);
}

// Exclusive prefix count of `flag` over the block in thread order, and the total.
__device__ __forceinline__ int block_prefix(bool flag, int *wtot, int &total)
{
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
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

// Cut for the top-`sel` of the valid positions (count of them = count);
// sm.h1 holds the level-1 histogram (kept), sm.hs is scratch.
__device__ Cut block_cut(const SelRow &s, BlockScratch &sm, int count, int sel)
{
    Cut c;
    c.keq = 0u;
    c.req = 0;
    if (count <= sel) {
        c.kgt = -1;
        return c;
    }
    if (threadIdx.x < kWave) {
        int x, above;
        find_bin<kBins1>(sm.h1, sel, x, above);
        if (threadIdx.x == 0) {
            sm.bc[0] = x;
            sm.bc[1] = sel - above;
        }
    }
    __syncthreads();
    const int b1 = sm.bc[0], r1 = sm.bc[1];
    const int hb1 = (int)sm.h1[b1];
    __syncthreads();
    if (r1 == hb1) {
        c.kgt = (int64_t)b1 * (1ll << 21) - 1;
        return c;
    }
    block_clear(sm.hs, kBins2);
    __syncthreads();
    for (int64_t pos = threadIdx.x; pos < s.npos; pos += blockDim.x) {
        if (!sel_valid(s, pos))
            continue;
        const uint32_t key = score_key(s.sc[pos]);
        if ((int)(key >> 21) == b1)
            atomicAdd(&sm.hs[(key >> 10) & (kBins2 - 1)], 1u);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
        int x, above;
        find_bin<kBins2>(sm.hs, r1, x, above);
        if (threadIdx.x == 0) {
            sm.bc[2] = x;
            sm.bc[3] = r1 - above;
        }
    }
    __syncthreads();
    const int b2 = sm.bc[2], r2 = sm.bc[3];
    const int hb2 = (int)sm.hs[b2];
    const uint32_t pre = ((uint32_t)b1 << 11) | (uint32_t)b2;
    __syncthreads();
    if (r2 == hb2) {
        c.kgt = (int64_t)pre * 1024 - 1;
        return c;
    }
    block_clear(sm.hs, kBins3);
    __syncthreads();
    for (int64_t pos = threadIdx.x; pos < s.npos; pos += blockDim.x) {
        if (!sel_valid(s, pos))
            continue;
        const uint32_t key = score_key(s.sc[pos]);
        if ((key >> 10) == pre)
            atomicAdd(&sm.hs[key & (kBins3 - 1)], 1u);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
        int x, above;
        find_bin<kBins3>(sm.hs, r2, x, above);
        if (threadIdx.x == 0) {
            sm.bc[0] = x;
            sm.bc[1] = r2 - above;
        }
    }
    __syncthreads();
    const uint32_t kstar = (pre << 10) | (uint32_t)sm.bc[0];
    c.kgt = (int64_t)kstar;
    c.keq = kstar;
    c.req = sm.bc[1];
    __syncthreads();
    return c;
}

__device__ void block_emit(const SelRow &s, BlockScratch &sm, const Cut &c, int sel,
                           int32_t *oidx, float *osc, int fan, int64_t fstride)
{
    int emitted = 0, eqseen = 0;
    for (int64_t base = 0; base < s.npos; base += blockDim.x) {
        const int64_t pos = base + threadIdx.x;
        const bool v = sel_valid(s, pos);
        float score = 0.f;
        uint32_t key = 0u;
        if (v) {
            score = s.sc[pos];
            key = score_key(score);
        }
        const bool eq = v && c.req > 0 && key == c.keq;
        int eqtot;
        const int er = eqseen + block_prefix(eq, sm.wtot, eqtot);
        const bool in = v && ((int64_t)key > c.kgt || (eq && er < c.req));
        int intot;
        const int opos = emitted + block_prefix(in, sm.wtot, intot);
        if (in && opos < sel) {
            const int32_t idx = s.list ? s.list[pos] : (int32_t)pos;
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

__global__ __launch_bounds__(kSelectThreads) void split_select_kernel(SplitSelectParams p)
{
    __shared__ BlockScratch sm;
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
        s.lim = off + r1 - 1;
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
        s.lim = off + r;
        if (p.mode == kDense) {
            s.list = nullptr;
            s.npos = s.lim + 1;
        } else {
            const int64_t m = r / p.g;
            const int64_t r1 = ((m + 1) * p.g < p.q_len) ? (m + 1) * p.g : p.q_len;
            const int64_t t_last = off + r1 - 1;
            s.list = p.cand + ((int64_t)bi * p.G + m) * p.c;
            s.npos = (p.c < t_last + 1) ? p.c : t_last + 1;
        }
        o1 = p.o1_idx + row * p.sel;
        s1 = p.o1_score ? p.o1_score + row * p.sel : nullptr;
    }

    block_clear(sm.h1, kBins1);
    __syncthreads();
    int cnt = 0;
    for (int64_t pos = threadIdx.x; pos < s.npos; pos += blockDim.x) {
        if (!sel_valid(s, pos))
            continue;
        atomicAdd(&sm.h1[bin1(score_key(s.sc[pos]))], 1u);
        ++cnt;
    }
    cnt = wave_sum(cnt);
    if (threadIdx.x % kWave == 0)
        sm.wtot[threadIdx.x / kWave] = cnt;
    __syncthreads();
    int count = 0;
    for (int w = 0; w < kSelWaves; ++w)
        count += sm.wtot[w];
    __syncthreads();

    const Cut c1 = block_cut(s, sm, count, p.sel);
    block_emit(s, sm, c1, p.sel, o1, s1, fan1, p.sel);
    if (p.sel2 > 0) {
        const Cut c2 = block_cut(s, sm, count, p.sel2);
        block_emit(s, sm, c2, p.sel2, o2, s2, fan2, p.sel2);
    }
}

// ------------------------------------------------------------- launchers
template <int H, int D>
static hipError_t launch_split_score_t(const SplitScoreParams &prm, dim3 grid, hipStream_t stream)
{
    hipLaunchKernelGGL((split_score_kernel<H, D>), grid, dim3(kSplitWaves * kWave), 0, stream, prm);
    return hipGetLastError();
}

hipError_t launch_split_score(int H, int D, const SplitScoreParams &prm, dim3 grid, hipStream_t stream)
{
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
