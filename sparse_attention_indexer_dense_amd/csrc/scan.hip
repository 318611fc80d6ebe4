// scan.hip - fused score + select kernels for many query rows (prefill shape),
// and the group-proxy pooling kernel.
//
// One workgroup owns NW rows (one per wave) that share a stream of key tiles.
// Per 64-key stage, the keys are staged in LDS once for all NW rows. Each wave
// computes, for its row and 32 keys at a time, the 64-head score tile
// S[j][s] = q_j . k_s with bf16 MFMA 32x32x16 (fp32 accumulate), then the
// epilogue I(s) = sum_j w_j * max(0, S[j][s]) in registers (Eq. (1) of the
// PIVOT paper, arXiv 2607.24593, as described in its observation-O3
// paragraph), the causal mask, and a threshold filter: a key is kept only if
// its score beats a running threshold below which it provably cannot reach
// the row's top-sel. Kept (score, index) pairs go, in index order, to a
// per-row buffer in the workspace; a per-row LDS histogram of kept scores
// raises the threshold as keys stream by. After the last tile, an exact
// three-level radix cut over the buffer yields the top-sel set (ties to the
// lower index), written in ascending index order. The L x L score matrix is
// never written.
//
// Modes:
//   kDense  - rows are query rows; keys 0..pos(row)            (dense indexer)
//   kProxy  - rows are group proxies; keys 0..t_last(group)     (PIVOT scan:
//             top-c candidates and/or the top-k shared by the members, Reuse)
//   kRefine - rows are the members of one group; keys are the group's
//             candidate list, causal per member                (PIVOT Refine)
#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "kernels.h"

namespace dsaidx {

constexpr int kStage = 64;  // keys per LDS stage (two 32-key MFMA N-tiles)

// ----------------------------------------------------------- per-row select
struct RowState {
    float theta_exact;  // exact floor set by a compaction (-inf before)
    float theta;        // admission threshold: keep a key only if score > theta
    int b;              // level-1 bin of the current floor
    int count_ge;       // kept entries in level-1 bins >= b
    int nbuf;           // entries in the buffer (dead ones included)
};

struct Level1 {
    int b1, r1, h1;
    bool all;
};

// Level-1 part of the cut for the top-`sel` of the live entries.
__device__ __forceinline__ Level1 level1(const uint32_t *h, const RowState &st, int sel)
{
    Level1 a;
    if (st.count_ge <= sel) {
        a.b1 = st.b;
        a.r1 = 0;
        a.h1 = 0;
        a.all = true;
        return a;
    }
    int x, above;
    find_bin<kBins1>(h, sel, x, above);
    a.b1 = x;
    a.r1 = sel - above;
    a.h1 = uniform((int)h[x]);
    a.all = false;
    return a;
}

// Finish a cut with levels 2 and 3 (passes over the buffer); h is scratch.
__device__ Cut finish_cut(const Entry *buf, int nbuf, uint32_t *h, const Level1 &a)
{
    Cut c;
    const int lane = lane_id();
    if (a.all || a.r1 == a.h1) {
        c.kgt = (int64_t)a.b1 * (1ll << 21) - 1;
        c.keq = 0u;
        c.req = 0;
        return c;
    }
    clear_hist<kBins2>(h);
    for (int i = lane; i < nbuf; i += kWave) {
        uint32_t key = score_key(buf[i].score);
        if ((int)(key >> 21) == a.b1)
            atomicAdd(&h[(key >> 10) & (kBins2 - 1)], 1u);
    }
    int b2, a2;
    find_bin<kBins2>(h, a.r1, b2, a2);
    int r2 = a.r1 - a2;
    int h2 = uniform((int)h[b2]);
    uint32_t pre = ((uint32_t)a.b1 << 11) | (uint32_t)b2;
    if (r2 == h2) {
        c.kgt = (int64_t)pre * 1024 - 1;
        c.keq = 0u;
        c.req = 0;
        return c;
    }
    clear_hist<kBins3>(h);
    for (int i = lane; i < nbuf; i += kWave) {
        uint32_t key = score_key(buf[i].score);
        if ((key >> 10) == pre)
            atomicAdd(&h[key & (kBins3 - 1)], 1u);
    }
    int b3, a3;
    find_bin<kBins3>(h, r2, b3, a3);
    uint32_t kstar = (pre << 10) | (uint32_t)b3;
    c.kgt = (int64_t)kstar;
    c.keq = kstar;
    c.req = r2 - a3;
    return c;
}

// Write the entries of the cut, in buffer (= ascending index) order, to
// `fan` output rows spaced `fstride` apart; pad each row to `sel` with -1/-inf.
__device__ void emit(const Entry *buf, int nbuf, const Cut &c, int sel,
                     int32_t *oidx, float *osc, int fan, int64_t fstride)
{
    const int lane = lane_id();
    int emitted = 0, eqseen = 0;
    for (int base = 0; base < nbuf; base += kWave) {
        int i = base + lane;
        bool v = i < nbuf;
        Entry e;
        e.score = 0.f;
        e.idx = -1;
        if (v)
            e = buf[i];
        uint32_t key = score_key(e.score);
        bool eq = v && c.req > 0 && key == c.keq;
        uint64_t meq = ballot(eq);
        int er = eqseen + prefix_count(meq);
        bool in = v && ((int64_t)key > c.kgt || (eq && er < c.req));
        uint64_t min_ = ballot(in);
        int pos = emitted + prefix_count(min_);
        if (in && pos < sel) {
            for (int f = 0; f < fan; ++f) {
                oidx[f * fstride + pos] = e.idx;
                if (osc)
                    osc[f * fstride + pos] = e.score;
            }
        }
        emitted += __popcll(min_);
        eqseen += __popcll(meq);
    }
    for (int x = emitted + lane; x < sel; x += kWave) {
        for (int f = 0; f < fan; ++f) {
            oidx[f * fstride + x] = -1;
            if (osc)
                osc[f * fstride + x] = -__builtin_inff();
        }
    }
}

// Keep only the top-`sel` entries of the buffer (stable, in place) and rebuild
// the level-1 histogram from them. Used when a buffer is about to overflow.
__device__ void compact(Entry *buf, uint32_t *h, RowState &st, int sel)
{
    const int lane = lane_id();
    __threadfence_block();
    Level1 a = level1(h, st, sel);
    Cut c = finish_cut(buf, st.nbuf, h, a);
    int kept = 0, eqseen = 0;
    for (int base = 0; base < st.nbuf; base += kWave) {
        int i = base + lane;
        bool v = i < st.nbuf;
        Entry e;
        e.score = 0.f;
        e.idx = -1;
        if (v)
            e = buf[i];
        uint32_t key = score_key(e.score);
        bool eq = v && c.req > 0 && key == c.keq;
        uint64_t meq = ballot(eq);
        int er = eqseen + prefix_count(meq);
        bool in = v && ((int64_t)key > c.kgt || (eq && er < c.req));
        uint64_t min_ = ballot(in);
        int pos = kept + prefix_count(min_);
        if (in)
            buf[pos] = e;  // pos <= i: never overwrites an entry not yet read
        kept += __popcll(min_);
        eqseen += __popcll(meq);
    }
    __threadfence_block();
    clear_hist<kBins1>(h);
    for (int i = lane; i < kept; i += kWave)
        atomicAdd(&h[bin1(score_key(buf[i].score))], 1u);
    st.nbuf = kept;
    st.count_ge = kept;
    st.b = a.b1;
    if (c.req > 0)
        st.theta_exact = key_score(c.keq);
    else
        st.theta_exact = (c.kgt + 1 < (4ll << 21)) ? -__builtin_inff() : key_score((uint32_t)(c.kgt + 1));
    st.theta = fmaxf(st.theta_exact, bin1_floor(st.b));
}

// ------------------------------------------------------------- block plans
struct WaveRow {
    bool valid;
    const uint16_t *q;
    const float *w;
    int64_t lim;  // last eligible key index
    int32_t *o1;
    float *s1;
    int fan1;
    int32_t *o2;
    float *s2;
    int fan2;
};

struct BlockKeys {
    const uint16_t *Kb;   // keys of this batch item
    const int32_t *list;  // candidate list (kRefine) or nullptr (prefix)
    int64_t nkeys;        // list length, or number of prefix keys
};

template <int H, int D, int NW, int MODE>
__device__ __forceinline__ void plan_block(const ScanParams &p, int64_t j, int wave,
                                           WaveRow &wr, BlockKeys &bk)
{
    const int bi = (int)(j % p.B);
    const int64_t jj = j / p.B;
    const int64_t off = p.L - p.q_len;  // position of query row 0
    wr.o2 = nullptr;
    wr.s2 = nullptr;
    wr.fan2 = 0;
    if (MODE == kDense) {
        const int64_t rb = p.nblk_per_batch - 1 - jj;
        const int64_t r = rb * NW + wave;
        const int64_t rlast = (rb * NW + NW < p.q_len ? rb * NW + NW : p.q_len) - 1;
        wr.valid = r < p.q_len;
        const int64_t row = (int64_t)bi * p.q_len + r;
        wr.q = p.Q + row * H * D;
        wr.w = p.W + row * H;
        wr.lim = off + r;
        wr.o1 = p.o1_idx + row * p.sel;
        wr.s1 = p.o1_score ? p.o1_score + row * p.sel : nullptr;
        wr.fan1 = 1;
        bk.Kb = p.K + (int64_t)bi * p.L * D;
        bk.list = nullptr;
        bk.nkeys = off + rlast + 1;
    } else if (MODE == kProxy) {
        const int64_t rb = p.nblk_per_batch - 1 - jj;
        const int64_t m = rb * NW + wave;
        const int64_t mlast = (rb * NW + NW < p.G ? rb * NW + NW : p.G) - 1;
        wr.valid = m < p.G;
        const int64_t grow = (int64_t)bi * p.G + m;
        const int64_t r0 = m * p.g;
        const int64_t r1 = (r0 + p.g < p.q_len) ? r0 + p.g : p.q_len;
        wr.q = p.Q + grow * H * D;
        wr.w = p.W + grow * H;
        wr.lim = off + r1 - 1;
        const int64_t r1last = ((mlast + 1) * p.g < p.q_len) ? (mlast + 1) * p.g : p.q_len;
        bk.nkeys = off + r1last;
        // output 1: candidate rows [B][G][sel] or the member rows
        if (p.o1_members) {
            const int64_t row = (int64_t)bi * p.q_len + r0;
            wr.o1 = p.o1_idx + row * p.sel;
            wr.s1 = p.o1_score ? p.o1_score + row * p.sel : nullptr;
            wr.fan1 = (int)(r1 - r0);
        } else {
            wr.o1 = p.o1_idx + grow * p.sel;
            wr.s1 = p.o1_score ? p.o1_score + grow * p.sel : nullptr;
            wr.fan1 = 1;
        }
        if (p.sel2 > 0) {
            const int64_t row = (int64_t)bi * p.q_len + r0;
            wr.o2 = p.o2_idx + row * p.sel2;
            wr.s2 = p.o2_score ? p.o2_score + row * p.sel2 : nullptr;
            wr.fan2 = (int)(r1 - r0);
        }
        bk.Kb = p.K + (int64_t)bi * p.L * D;
        bk.list = nullptr;
    } else {  // kRefine
        const int64_t m = p.G - 1 - jj / p.member_chunks;
        const int chunk = (int)(jj % p.member_chunks);
        const int64_t r0 = m * p.g;
        const int64_t r1 = (r0 + p.g < p.q_len) ? r0 + p.g : p.q_len;
        const int64_t r = r0 + (int64_t)chunk * NW + wave;
        wr.valid = r < r1;
        const int64_t row = (int64_t)bi * p.q_len + r;
        wr.q = p.Q + row * H * D;
        wr.w = p.W + row * H;
        wr.lim = off + r;
        wr.o1 = p.o1_idx + row * p.sel;
        wr.s1 = p.o1_score ? p.o1_score + row * p.sel : nullptr;
        wr.fan1 = 1;
        const int64_t t_last = off + r1 - 1;
        bk.Kb = p.K + (int64_t)bi * p.L * D;
        bk.list = p.cand + ((int64_t)bi * p.G + m) * p.c;
        bk.nkeys = (p.c < t_last + 1) ? p.c : t_last + 1;
    }
}

// ------------------------------------------------------------------ kernel
template <int H, int D, int NW, int MODE>
__global__ __launch_bounds__(NW * kWave) void scan_select_kernel(ScanParams p)
{
    using S = Shape<H, D>;
    constexpr int MB = S::MB, KS = S::KS, ROWS = S::ROWS, CHUNKS = S::CHUNKS;
    constexpr int NT = NW * kWave;
    constexpr int STAGE_CHUNKS = kStage * CHUNKS;
    constexpr int LPT = (STAGE_CHUNKS + NT - 1) / NT;  // 16-byte loads per thread per stage
    constexpr int STAGE_BYTES = kStage * ROWS;

    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *kst = smem;
    uint32_t *hist_all = reinterpret_cast<uint32_t *>(smem + 2 * STAGE_BYTES);

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int half = lane >> 5;
    const int col = lane & 31;
    uint32_t *h = hist_all + wave * kBins1;
    Entry *buf = p.slots + ((int64_t)blockIdx.x * NW + wave) * p.cap;

    for (int64_t it = 0;; ++it) {
        const int64_t j = it * gridDim.x + ((it & 1) ? (gridDim.x - 1 - blockIdx.x) : blockIdx.x);
        if (j >= p.nblocks)
            break;
        WaveRow wr;
        BlockKeys bk;
        plan_block<H, D, NW, MODE>(p, j, wave, wr, bk);

        // this wave's query row as MFMA A fragments, weights per accumulator row
        bf16x8 qa[MB][KS];
        float wv[MB][16];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int head = mb * 32 + col;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (wr.valid && head < H)
                    v = *reinterpret_cast<const u32x4 *>(wr.q + (int64_t)head * D + (half * KS + ks) * 8);
                qa[mb][ks] = __builtin_bit_cast(bf16x8, v);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int hr = mb * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                wv[mb][r] = (wr.valid && hr < H) ? wr.w[hr] : 0.f;
            }
        }

        RowState st;
        st.theta_exact = -__builtin_inff();
        st.theta = -__builtin_inff();
        st.b = 0;
        st.count_ge = 0;
        st.nbuf = 0;
        if (wr.valid)
            clear_hist<kBins1>(h);

        const int64_t nkeys = bk.nkeys;
        const int64_t ntiles = (nkeys + kStage - 1) / kStage;
        u32x4 regs[LPT];

        auto load_stage = [&](int64_t t) {
#pragma unroll
            for (int i = 0; i < LPT; ++i) {
                const int c = tid + i * NT;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (c < STAGE_CHUNKS) {
                    const int kk = c / CHUNKS, part = c % CHUNKS;
                    const int64_t pp = t * kStage + kk;
                    if (pp < nkeys) {
                        const int64_t key = bk.list ? (int64_t)bk.list[pp] : pp;
                        if (key >= 0 && key < p.L)
                            v = *reinterpret_cast<const u32x4 *>(bk.Kb + key * D + part * 8);
                    }
                }
                regs[i] = v;
            }
        };
        auto store_stage = [&](int s) {
#pragma unroll
            for (int i = 0; i < LPT; ++i) {
                const int c = tid + i * NT;
                if (c < STAGE_CHUNKS) {
                    const int kk = c / CHUNKS, part = c % CHUNKS;
                    *reinterpret_cast<u32x4 *>(kst + s * STAGE_BYTES + kk * ROWS + part * 16) = regs[i];
                }
            }
        };

        if (ntiles > 0) {
            load_stage(0);
            store_stage(0);
        }
        __syncthreads();

        for (int64_t t = 0; t < ntiles; ++t) {
            const int s = (int)(t & 1);
            if (t + 1 < ntiles)
                load_stage(t + 1);
            if (wr.valid) {
#pragma unroll
                for (int nt = 0; nt < kStage / 32; ++nt) {
                    const int64_t p0 = t * kStage + nt * 32;
                    if (p0 >= nkeys)
                        break;
                    const int64_t first = bk.list ? (int64_t)bk.list[p0] : p0;
                    if (first > wr.lim)
                        break;
                    f32x16 acc[MB];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[mb] = f32x16{};
                    const unsigned char *kb_base = kst + s * STAGE_BYTES + (nt * 32 + col) * ROWS;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        u32x4 kv = *reinterpret_cast<const u32x4 *>(kb_base + (half * KS + ks) * 16);
                        bf16x8 kb = __builtin_bit_cast(bf16x8, kv);
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], kb, acc[mb], 0, 0, 0);
                    }
                    // epilogue: ReLU, head weights, head sum (Eq. (1))
                    float part = 0.f;
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            part = fmaf(wv[mb][r], fmaxf(acc[mb][r], 0.f), part);
                    const float total = half_wave_sum(part) + 0.0f;

                    // causal mask and threshold filter (lanes 0..31 own the 32 keys)
                    const int64_t pidx = p0 + col;
                    bool ok = false;
                    int64_t key = -1;
                    if (lane < 32 && pidx < nkeys) {
                        key = bk.list ? (int64_t)bk.list[pidx] : pidx;
                        ok = key <= wr.lim;
                    }
                    const bool adm = ok && total > st.theta;
                    const uint64_t m = ballot(adm);
                    if (m) {
                        const int cnt = __popcll(m);
                        if (adm) {
                            const int pos = st.nbuf + prefix_count(m);
                            Entry e;
                            e.score = total;
                            e.idx = (int32_t)key;
                            buf[pos] = e;
                            atomicAdd(&h[bin1(score_key(total))], 1u);
                        }
                        st.nbuf += cnt;
                        st.count_ge += cnt;
                        int bb = st.b, cg = st.count_ge;
                        while (bb < kBins1 - 1) {
                            const int hb = (int)h[bb];
                            if (cg - hb < p.sel)
                                break;
                            cg -= hb;
                            ++bb;
                        }
                        st.b = uniform(bb);
                        st.count_ge = uniform(cg);
                        st.theta = fmaxf(st.theta_exact, bin1_floor(st.b));
                        if (st.nbuf > p.cap - kWave)
                            compact(buf, h, st, p.sel);
                    }
                }
            }
            if (t + 1 < ntiles)
                store_stage(s ^ 1);
            __syncthreads();
        }

        if (wr.valid) {
            __threadfence_block();
            Level1 a1 = level1(h, st, p.sel);
            Level1 a2 = a1;
            if (p.sel2 > 0)
                a2 = level1(h, st, p.sel2);
            Cut c1 = finish_cut(buf, st.nbuf, h, a1);
            emit(buf, st.nbuf, c1, p.sel, wr.o1, wr.s1, wr.fan1, p.sel);
            if (p.sel2 > 0) {
                Cut c2 = finish_cut(buf, st.nbuf, h, a2);
                emit(buf, st.nbuf, c2, p.sel2, wr.o2, wr.s2, wr.fan2, p.sel2);
            }
        }
    }
}

// -------------------------------------------------------------- pooling
// Proxy of group m (PIVOT, experimental setup: mean pooling per head): the
// members' queries summed in row order in fp32, divided by the member count
// (IEEE division), rounded to bf16 nearest-even; weights likewise in fp32.
template <int H, int D>
__global__ __launch_bounds__(256) void pool_kernel(PoolParams p)
{
    const int64_t grp = blockIdx.x;
    const int bi = (int)(grp / p.G);
    const int64_t m = grp % p.G;
    const int64_t r0 = m * p.g;
    const int64_t r1 = (r0 + p.g < p.q_len) ? r0 + p.g : p.q_len;
    const float n = (float)(r1 - r0);
    const uint16_t *Qb = p.Q + ((int64_t)bi * p.q_len) * H * D;
    const float *Wb = p.W + ((int64_t)bi * p.q_len) * H;
    for (int x = threadIdx.x * 8; x < H * D; x += blockDim.x * 8) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int64_t r = r0; r < r1; ++r) {
            u32x4 v = *reinterpret_cast<const u32x4 *>(Qb + r * H * D + x);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += __uint_as_float(v[e] << 16);
                acc[2 * e + 1] += __uint_as_float(v[e] & 0xFFFF0000u);
            }
        }
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t lo = __bfloat16_as_ushort(__float2bfloat16(__fdiv_rn(acc[2 * e], n)));
            uint32_t hi = __bfloat16_as_ushort(__float2bfloat16(__fdiv_rn(acc[2 * e + 1], n)));
            o[e] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4 *>(p.Qp + grp * H * D + x) = o;
    }
    for (int jh = threadIdx.x; jh < H; jh += blockDim.x) {
        float acc = 0.f;
        for (int64_t r = r0; r < r1; ++r)
            acc += Wb[r * H + jh];
        p.Wp[grp * H + jh] = __fdiv_rn(acc, n);
    }
}

// ------------------------------------------------------------- launchers
template <int H, int D, int NW, int MODE>
static hipError_t launch_scan(const ScanParams &prm, int grid, hipStream_t stream)
{
    constexpr size_t lds = 2 * kStage * Shape<H, D>::ROWS + (size_t)NW * kBins1 * 4;
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&scan_select_kernel<H, D, NW, MODE>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
        attr = true;
    }
    hipLaunchKernelGGL((scan_select_kernel<H, D, NW, MODE>), dim3(grid), dim3(NW * kWave), lds, stream, prm);
    return hipGetLastError();
}

template <int H, int D>
static hipError_t launch_pool_t(const PoolParams &prm, hipStream_t stream)
{
    hipLaunchKernelGGL((pool_kernel<H, D>), dim3((unsigned)(prm.B * prm.G)), dim3(256), 0, stream, prm);
    return hipGetLastError();
}

size_t scan_lds_bytes(int H, int D, int NW)
{
    int rows = 2 * D + 16;
    (void)H;
    return 2 * (size_t)kStage * rows + (size_t)NW * kBins1 * 4;
}

hipError_t launch_scan_select(int H, int D, int NW, int mode, const ScanParams &prm, int grid,
                              hipStream_t stream)
{
#define DSAIDX_SCAN_CASE(HH, DD, NN, MM)                                   \
    if (H == HH && D == DD && NW == NN && mode == MM)                      \
        return launch_scan<HH, DD, NN, MM>(prm, grid, stream);
    DSAIDX_SCAN_CASE(64, 128, 8, kDense)
    DSAIDX_SCAN_CASE(64, 128, 8, kProxy)
    DSAIDX_SCAN_CASE(64, 128, 4, kRefine)
    DSAIDX_SCAN_CASE(64, 128, 8, kRefine)
    DSAIDX_SCAN_CASE(4, 32, 8, kDense)
    DSAIDX_SCAN_CASE(4, 32, 8, kProxy)
    DSAIDX_SCAN_CASE(4, 32, 4, kRefine)
    DSAIDX_SCAN_CASE(4, 32, 8, kRefine)
#undef DSAIDX_SCAN_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_pool(int H, int D, const PoolParams &prm, hipStream_t stream)
{
    if (H == 64 && D == 128)
        return launch_pool_t<64, 128>(prm, stream);
    if (H == 4 && D == 32)
        return launch_pool_t<4, 32>(prm, stream);
    return hipErrorInvalidValue;
}

}  // namespace dsaidx
