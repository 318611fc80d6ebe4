// split.hip - kernels for few query rows over long key ranges (decode shape).
//
// A decode step of the PIVOT paper (Method, decode groups formed by the MTP
// drafts of one step) scores only g new rows per request against a long
// cache, so there are too few rows to fill the GPU with one workgroup per row.
// The key axis is split instead:
//   split_score_kernel  - workgroups per (batch item, row), one round of
//                         workgroups for all rows; the row's waves take its
//                         32-key tiles in turn (a Refine wave: a contiguous
//                         span of its group's candidate list), loaded straight into
//                         registers as MFMA B fragments (several tiles in
//                         flight while one is scored), runs the MFMA score
//                         tile and the ReLU/weight/head-sum epilogue, and
//                         stores one fp32 score per position (a Refine
//                         wave scores two member rows of one group on each
//                         gathered tile when g is even);
//   split_select_kernel - one workgroup per score row finds the exact top-sel
//                         (ties to the lower index): a row that fits in LDS
//                         is staged whole; a longer one is first reduced to
//                         the scores above a threshold taken from a sample,
//                         with an exact pass over the row as the fallback;
//                         an exact radix cut and one ordered emission in
//                         ascending index order follow.
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
    const uint16_t *Kb;   // keys of the request
    const int32_t *list;  // kRefine: the group's candidate list
    int L;                // keys of the request
    int npos;             // positions to consider (0: no such row)
    int lim;              // last eligible key index
};

// Score row r of request bi in a split pass: a dense row (r < the request's
// dense rows), a group proxy (group m0 + r), or a Refine member row (row
// r_g + r, where rows [0, r_g) belong to guarded groups). Rows beyond the
// request's count get npos = 0.
__device__ __forceinline__ SplitRow split_row(const SplitScoreParams &p, int H, int D, int bi, int64_t r)
{
    SplitRow s;
    const Req rq = request_of(p.req, bi, p.L, p.q_len, p.g, p.m0);
    const int64_t off = rq.L - rq.q_len;
    s.list = nullptr;
    s.npos = 0;
    s.lim = -1;
    s.q = p.Q;
    s.w = p.W;
    s.Kb = p.K + rq.key_off * D;
    s.L = (int)rq.L;
    if (p.mode == kProxy) {
        const int64_t m = rq.m0 + r;
        if (m >= rq.G)
            return s;
        const int64_t grow = rq.g_off + m;
        const int64_t r1 = ((m + 1) * p.g < rq.q_len) ? (m + 1) * p.g : rq.q_len;
        s.q = p.Q + grow * H * D;
        s.w = p.W + grow * H;
        s.lim = (int)(off + r1 - 1);
        if (p.glim) {  // chunk summaries complete at the group's last position
            s.lim = p.glim[grow];
            s.Kb = p.K + (int64_t)bi * p.krows * D;
            s.L = (int)p.krows;
        }
        s.npos = s.lim + 1;
    } else if (p.mode == kDense) {
        if (r >= dense_rows(rq, p.g, p.guard_rows))
            return s;
        const int64_t row = rq.q_off + r;
        s.q = p.Q + row * H * D;
        s.w = p.W + row * H;
        s.lim = (int)(off + r);
        s.npos = s.lim + 1;
    } else {
        const int64_t rr = dense_rows(rq, p.g, 1) + r;  // rows past the guarded groups
        if (rr >= rq.q_len)
            return s;
        const int64_t row = rq.q_off + rr;
        s.q = p.Q + row * H * D;
        s.w = p.W + row * H;
        s.lim = (int)(off + rr);
        const int64_t m = rr / p.g;
        const int64_t r1 = ((m + 1) * p.g < rq.q_len) ? (m + 1) * p.g : rq.q_len;
        const int64_t t_last = off + r1 - 1;
        s.list = p.cand + (rq.g_off + m) * p.c;
        s.npos = p.cand_n ? p.cand_n[rq.g_off + m] : (int)((p.c < t_last + 1) ? p.c : t_last + 1);
    }
    return s;
}

// ------------------------------------------------------------------ scoring
// Key rows are read once and used by one row's MFMAs only, so they go straight
// from global memory into registers as B fragments, with no LDS staging. K-step
// ks of a fragment holds the 16-byte chunk 2*ks + half of its row (half = lane
// / 32): the 32 rows of a tile are then read 32 contiguous bytes per row per
// load instruction, and the query fragments use the same chunk order, so
// every dot product sums the same terms. A ring of kSplitDepth tiles keeps
// the loads of the next tiles in flight while one tile is scored; the loads
// are plain vector loads, whose completion the compiler tracks exactly.
constexpr int kSplitDepth = 4;

template <int H, int D, bool LIST, int MR>
__global__ __launch_bounds__(kSplitWaves * kWave) void split_score_kernel(SplitScoreParams p)
{
    using S = Shape<H, D>;
    constexpr int MB = S::MB, KS = S::KS;
    constexpr int P = MR == 1 ? kSplitDepth : kSplitDepth / 2;  // two rows: twice the work per tile
    static_assert(MR == 1 || (MR == 2 && LIST), "rows share a wave only over one candidate list");
    __shared__ int32_t lst[kSplitWaves][LIST ? kSplitSpanMax : 1];

    const int bi = blockIdx.z;
    const int64_t r = p.row0 + (int64_t)blockIdx.y * MR;
    const int wave = uniform(threadIdx.x / kWave);  // wave-uniform (SGPR)
    const int lane = threadIdx.x % kWave;
    const int half = lane >> 5;
    const int col = lane & 31;
    const SplitRow sr = split_row(p, H, D, bi, r);
    // Tiles of a row without a list are dealt to the row's waves in turn
    // (wave wr of nwr takes tiles wr, wr + nwr, ...), so that the row's waves
    // read neighbouring key rows at any moment; with a list, each wave takes
    // a contiguous span (its part of the list is staged in LDS).
    const int nwr = (int)gridDim.x * kSplitWaves;
    const int wr = (int)blockIdx.x * kSplitWaves + wave;
    const int ntr = (sr.npos + 31) / 32;  // tiles of the row
    const int span = (int)(p.chunk / kSplitWaves);
    const int w0 = LIST ? (int)(blockIdx.x * p.chunk) + wave * span : 0;
    const int w1 = LIST ? ((w0 + span < sr.npos) ? w0 + span : sr.npos) : sr.npos;
    const int ntile = LIST ? (w1 - w0 + 31) / 32 : (wr < ntr ? (ntr - wr + nwr - 1) / nwr : 0);
    if (LIST ? w0 >= sr.npos : ntile == 0)
        return;
    // position of lane col in the wave's tile t
    auto tile_pos = [&](int t) { return (LIST ? w0 + t * 32 : (t * nwr + wr) * 32) + col; };
    const uint16_t *Kb = sr.Kb;
    float *out = p.scores + ((int64_t)bi * p.nrows + r) * p.rowlen;  // row r + m at out + m * rowlen
    int32_t *wl = lst[wave];

    // With MR = 2 the wave also scores row r + 1, the next member of the same
    // group (rows are paired only when g is even, so a pair never straddles
    // two groups): both rows use every gathered key tile. A second row past
    // the request's end scores row r's query and stores nothing.
    const uint16_t *qrow[MR];
    const float *wrow[MR];
    bool live[MR];
    qrow[0] = sr.q;
    wrow[0] = sr.w;
    live[0] = true;
#pragma unroll
    for (int m = 1; m < MR; ++m) {
        const SplitRow s2 = split_row(p, H, D, bi, r + m);
        live[m] = s2.npos > 0;
        qrow[m] = live[m] ? s2.q : sr.q;
        wrow[m] = live[m] ? s2.w : sr.w;
    }

    if (LIST) {
        for (int x = lane; x < w1 - w0; x += kWave)
            wl[x] = sr.list[w0 + x];
        __builtin_amdgcn_wave_barrier();
    }

    // the query rows as MFMA A fragments (chunk order as above) and the
    // weights per accumulator row
    bf16x8 qa[MR][MB][KS];
    float wv[MR][MB][16];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int head = mb * 32 + col;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (head < H)
                    v = *reinterpret_cast<const u32x4 *>(qrow[m] + (int64_t)head * D + (2 * ks + half) * 8);
                qa[m][mb][ks] = __builtin_bit_cast(bf16x8, v);
            }
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int hr = mb * 32 + 8 * (rr / 4) + 4 * half + (rr % 4);
                wv[m][mb][rr] = hr < H ? wrow[m][hr] : 0.f;
            }
        }
    }

    // B fragments of tile t: key row tile_pos(t) (through the list for
    // Refine); a lane without a key (past the row, the span or the list's
    // valid entries, or beyond the ring's last tile) reads row 0, whose score
    // is never stored
    bf16x8 kq[P][KS];
    auto load_tile = [&](int t, bf16x8 (&kf)[KS]) {
        const int pos = tile_pos(t);
        const bool ok = t < ntile && pos < w1;
        int key = pos;
        if (LIST)
            key = wl[ok ? pos - w0 : 0];
        key = (ok && key >= 0 && key < sr.L) ? key : 0;
        const uint16_t *src = Kb + (int64_t)key * D + half * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(src + ks * 16));
    };
    auto mfma_tile = [&](const bf16x8 (&kf)[KS], f32x16 (&acc)[MR][MB]) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[m][mb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[m][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[m][mb][ks], kf[ks], acc[m][mb], 0, 0, 0);
    };
    // epilogue of tile t and its store: positions whose key is beyond the
    // row's limit get a score too, which the selection ignores. With two
    // rows one lane swap leaves row r's totals in lanes 0-31 and row r+1's
    // in lanes 32-63 (the same additions as for one row).
    auto finish = [&](int t, const f32x16 (&acc)[MR][MB]) {
        float srow[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            float part[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                part[mb] = 0.f;
#pragma unroll
                for (int rr = 0; rr < 16; ++rr)
                    part[mb] = fmaf(wv[m][mb][rr], relu(acc[m][mb][rr]), part[mb]);
            }
            srow[m] = part[0];
#pragma unroll
            for (int mb = 1; mb < MB; ++mb)
                srow[m] += part[mb];
        }
        const int pos = tile_pos(t);
        if constexpr (MR == 1) {
            const float total = half_wave_sum(srow[0]) + 0.0f;
            if (lane < 32 && pos < w1)
                out[pos] = total;
        } else {
            const float total = half_wave_sum2(srow[0], srow[MR - 1]) + 0.0f;
            if (pos < w1 && live[half])
                out[(int64_t)half * p.rowlen + pos] = total;
        }
    };

    // ring slots are compile-time: P tiles per trip; the MFMAs of tile t run
    // next to the epilogue of tile t - 1
#pragma unroll
    for (int u = 0; u < P - 1; ++u)
        load_tile(u, kq[u]);
    f32x16 a0[MR][MB], a1[MR][MB];
    for (int t0 = 0; t0 < ntile; t0 += P) {
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const int t = t0 + u;
            if (t >= ntile)
                break;
            load_tile(t + P - 1, kq[(u + P - 1) % P]);
            if (t == 0) {
                mfma_tile(kq[u], a0);
            } else {
                if (t & 1) {
                    mfma_tile(kq[u], a1);
                    finish(t - 1, a0);
                } else {
                    mfma_tile(kq[u], a0);
                    finish(t - 1, a1);
                }
#pragma unroll
                for (int q = 0; q < KS * MB * MR; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                }
            }
        }
    }
    if (ntile > 0) {
        if ((ntile - 1) & 1)
            finish(ntile - 1, a1);
        else
            finish(ntile - 1, a0);
    }
}

// ---------------------------------------------------------------- selection
// One workgroup per score row. The valid positions of a row always form a
// prefix [0, n): position p <= lim for keys 0..lim, and candidate lists are
// ascending, so their causal entries come first.
//
// A row that fits in LDS is copied there whole. A longer row is reduced first:
// the floor of the histogram bin that holds an order statistic of a strided
// sample is a lower bound theta that, with high probability, at least `sel`
// scores of the row reach; the scores
// >= theta are packed into LDS in index order (one read of the row, held in
// registers between counting and packing). The exact top-`sel` lies among
// them whenever there are at least `sel`; when there are fewer, or more than
// LDS holds, the selection runs exactly on the row in global memory instead.
// On the LDS entries, an exact radix cut (digits taken relative to the
// smallest key, so that close scores still spread over the bins) and one
// ordered pass write the selection, ties going to the lower index.
constexpr int kSelWaves = kSelectThreads / kWave;
constexpr int kCandCap = 12288;   // scores held in LDS
constexpr int kSampleMax = 8192;  // strided sample of a long row
constexpr int kRegSteps = 16;     // float4 steps per lane held in registers
constexpr int kStageSteps = 4;    // the same when staging a whole row
constexpr int kBoundaryCap = 1024;  // boundary-bin entries ranked directly

struct SelShared {
    __attribute__((aligned(16))) float cs[kCandCap];
    int32_t cp[kCandCap];
    uint32_t h[kBins1];
    uint32_t bkey[kBoundaryCap];
    int32_t bpos[kBoundaryCap];
    int nbnd;
    int wt[kSelWaves];
    uint32_t wlo[kSelWaves], whi[kSelWaves];
    int bc[5];
};

struct SelRow {
    const float *sc;
    const int32_t *list;
    int npos, lim;
};

struct SelOut {
    int sel;
    int32_t *idx;
    float *score;
    int fan;  // rows the selection is written to, sel entries apart
};

// Per-wave totals gathered over the block: the exclusive prefix of t in wave
// order, its total, and the key range. t, lo and hi are wave-uniform.
struct WaveTotals {
    int off, total;
    uint32_t lo, hi;
};

__device__ __forceinline__ WaveTotals wave_totals(int t, uint32_t lo, uint32_t hi, SelShared &sm)
{
    const int wave = uniform(threadIdx.x / kWave);
    if (lane_id() == 0) {
        sm.wt[wave] = t;
        sm.wlo[wave] = lo;
        sm.whi[wave] = hi;
    }
    lds_sync();
    WaveTotals r{0, 0, 0xFFFFFFFFu, 0u};
    for (int w = 0; w < kSelWaves; ++w) {
        const int x = sm.wt[w];
        r.off += (w < wave) ? x : 0;
        r.total += x;
        r.lo = min(r.lo, sm.wlo[w]);
        r.hi = max(r.hi, sm.whi[w]);
    }
    lds_sync();
    return r;
}

// Largest bin with suffix count >= target (wave 0 finds it, all threads get it).
__device__ __forceinline__ void block_find_bin(const uint32_t *h, int target, SelShared &sm, int &x, int &above)
{
    if (threadIdx.x < kWave) {
        int bx, ab;
        find_bin<kBins1>(h, target, bx, ab);
        if (threadIdx.x == 0) {
            sm.bc[0] = bx;
            sm.bc[1] = ab;
        }
    }
    lds_sync();
    x = sm.bc[0];
    above = sm.bc[1];
}

// Exact cut of the best `sel` of m keys key_at(0..m-1), each in [base, hi],
// where entry order is index order. Level 1 counts 2048 bins of the top bits
// of u = key - base (so that close keys still spread over the bins). When
// the bin holding the sel-th key has at most kBoundaryCap entries, they are
// gathered and ranked exactly (key descending, then entry order); otherwise
// two more radix levels narrow it down to one key, whose equal entries are
// then taken in index order when the selection is written.
template <typename KeyAt>
__device__ __forceinline__ Cut block_radix_cut(int m, int sel, uint32_t base, uint32_t hi, KeyAt key_at, SelShared &sm)
{
    Cut c;
    c.keq = 0u;
    c.req = 0;
    if (m <= sel) {
        c.kgt = (int64_t)base - 1;
        return c;
    }
    const int lane = lane_id();
    const uint32_t span = hi - base;
    const int nb = span ? 32 - __builtin_clz(span) : 0;
    const int s1 = nb > 11 ? nb - 11 : 0;
    const int s2 = s1 > 11 ? s1 - 11 : 0;

    // level 1
    for (int i = threadIdx.x; i < kBins1; i += kSelectThreads)
        sm.h[i] = 0u;
    if (threadIdx.x == 0)
        sm.nbnd = 0;
    lds_sync();
    for (int i = threadIdx.x; i < m; i += kSelectThreads)
        atomicAdd(&sm.h[(key_at(i) - base) >> s1], 1u);
    lds_sync();
    int b1, a1;
    block_find_bin(sm.h, sel, sm, b1, a1);
    const int r1 = sel - a1;
    const int cnt1 = (int)sm.h[b1];
    if (r1 == cnt1) {  // the whole bin is in
        c.kgt = (int64_t)base + ((int64_t)b1 << s1) - 1;
        lds_sync();
        return c;
    }
    if (s1 == 0) {  // a bin is one key
        c.keq = base + (uint32_t)b1;
        c.kgt = (int64_t)c.keq;
        c.req = r1;
        lds_sync();
        return c;
    }
    if (cnt1 <= kBoundaryCap) {
        // gather the boundary bin (wave-aggregated slots), then rank it
        const int S = (m + kSelectThreads - 1) / kSelectThreads * kWave;  // per-wave span of entries
        const int wave = uniform(threadIdx.x / kWave);
        const int e0 = wave * S;
        const int e1 = (e0 + S < m) ? e0 + S : m;
        for (int i0 = e0; i0 < e1; i0 += kWave) {
            const int i = i0 + lane;
            const uint32_t k = i < e1 ? key_at(i) : 0u;
            const bool hit = i < e1 && (int)((k - base) >> s1) == b1;
            const uint64_t bm = ballot(hit);
            if (bm) {
                int slot0 = 0;
                if (lane == 0)
                    slot0 = atomicAdd(&sm.nbnd, __popcll(bm));
                slot0 = __builtin_amdgcn_readlane(slot0, 0);
                if (hit) {
                    const int sl = slot0 + prefix_count(bm);
                    sm.bkey[sl] = k;
                    sm.bpos[sl] = i;
                }
            }
        }
        lds_sync();
        // entry e has rank (#keys above) + (#equal keys earlier); the one of
        // rank r1 - 1 fixes the cut
        for (int e = threadIdx.x; e < cnt1; e += kSelectThreads) {
            const uint32_t ke = sm.bkey[e];
            const int pe = sm.bpos[e];
            int above = 0, before = 0, equal = 0;
            for (int f = 0; f < cnt1; ++f) {
                const uint32_t kf = sm.bkey[f];
                above += kf > ke ? 1 : 0;
                equal += kf == ke ? 1 : 0;
                before += (kf == ke && sm.bpos[f] < pe) ? 1 : 0;
            }
            if (above + before == r1 - 1) {
                sm.bc[2] = (int)ke;
                sm.bc[3] = before + 1;          // equal keys taken
                sm.bc[4] = equal;
            }
        }
        lds_sync();
        const uint32_t kstar = (uint32_t)sm.bc[2];
        const int take = sm.bc[3], equal = sm.bc[4];
        lds_sync();
        if (take == equal) {
            c.kgt = (int64_t)kstar - 1;
        } else {
            c.kgt = (int64_t)kstar;
            c.keq = kstar;
            c.req = take;
        }
        return c;
    }
    // levels 2 and 3
    lds_sync();
    uint32_t pre = (uint32_t)b1;  // digits fixed so far: u >> prev == pre
    int prev = s1;
    int r = r1;
    for (int lev = 1; lev < 3; ++lev) {
        const int sh = lev == 1 ? s2 : 0;
        const uint32_t mask = (1u << (prev - sh)) - 1u;
        for (int i = threadIdx.x; i < kBins1; i += kSelectThreads)
            sm.h[i] = 0u;
        lds_sync();
        for (int i = threadIdx.x; i < m; i += kSelectThreads) {
            const uint32_t u = key_at(i) - base;
            if ((u >> prev) == pre)
                atomicAdd(&sm.h[(u >> sh) & mask], 1u);
        }
        lds_sync();
        int b, a;
        block_find_bin(sm.h, r, sm, b, a);
        const int rr = r - a;
        const int cnt = (int)sm.h[b];
        pre = (pre << (prev - sh)) | (uint32_t)b;
        lds_sync();
        if (rr == cnt) {
            c.kgt = (int64_t)base + ((int64_t)pre << sh) - 1;
            return c;
        }
        if (sh == 0) {
            c.keq = base + pre;
            c.kgt = (int64_t)c.keq;
            c.req = rr;
            return c;
        }
        r = rr;
        prev = sh;
    }
    return c;  // not reached: the last level has shift 0
}

// A lower bound for the rk-th largest of the m keys key_at(0..m-1), all in
// [base, hi]: the floor of the level-1 bin (2048 bins of the top bits of
// key - base) that holds it, so at least rk of the keys reach it. One
// histogram pass; the boundary bin is not resolved.
template <typename KeyAt>
__device__ __forceinline__ uint32_t rank_bin_floor(int m, int rk, uint32_t base, uint32_t hi, KeyAt key_at,
                                                   SelShared &sm)
{
    const uint32_t span = hi - base;
    const int nb = span ? 32 - __builtin_clz(span) : 0;
    const int s1 = nb > 11 ? nb - 11 : 0;
    for (int i = threadIdx.x; i < kBins1; i += kSelectThreads)
        sm.h[i] = 0u;
    lds_sync();
    for (int i = threadIdx.x; i < m; i += kSelectThreads)
        atomicAdd(&sm.h[(key_at(i) - base) >> s1], 1u);
    lds_sync();
    int b1, a1;
    block_find_bin(sm.h, rk, sm, b1, a1);
    return base + ((uint32_t)b1 << s1);
}

// Writes the entries of a cut over m entries in index order (entry i: score
// score_at(i), row position pos_at(i)). Wave w takes the w-th contiguous
// segment; ballots give ranks among equal keys and output slots. The
// selection is padded to sel with -1 / -inf.
template <typename ScoreAt, typename PosAt>
__device__ __forceinline__ void block_emit(int m, const Cut &c, const SelOut &o, const int32_t *list, ScoreAt score_at,
                           PosAt pos_at, SelShared &sm)
{
    const int wave = uniform(threadIdx.x / kWave), lane = lane_id();
    const int S = (m + kSelWaves * kWave - 1) / (kSelWaves * kWave) * kWave;
    const int b0 = wave * S;
    const int b1 = (b0 + S < m) ? b0 + S : m;
    int eq0 = 0;
    if (c.req > 0) {
        int ceq = 0;
        for (int i0 = b0; i0 < b1; i0 += kWave) {
            const int i = i0 + lane;
            ceq += __popcll(ballot(i < b1 && score_key(score_at(i)) == c.keq));
        }
        eq0 = wave_totals(ceq, 0u, 0u, sm).off;
    }
    int cin = 0, er = eq0;
    for (int i0 = b0; i0 < b1; i0 += kWave) {
        const int i = i0 + lane;
        const uint32_t k = i < b1 ? score_key(score_at(i)) : 0u;
        const bool v = i < b1;
        const uint64_t be = ballot(v && c.req > 0 && k == c.keq);
        const bool eq = (be >> lane) & 1u;
        const bool in = v && ((int64_t)k > c.kgt || (eq && er + prefix_count(be) < c.req));
        cin += __popcll(ballot(in));
        er += __popcll(be);
    }
    const WaveTotals t = wave_totals(cin, 0u, 0u, sm);
    int slot0 = t.off;
    er = eq0;
    for (int i0 = b0; i0 < b1; i0 += kWave) {
        const int i = i0 + lane;
        const bool v = i < b1;
        const float sc = v ? score_at(i) : 0.f;
        const uint32_t k = score_key(sc);
        const uint64_t be = ballot(v && c.req > 0 && k == c.keq);
        const bool eq = (be >> lane) & 1u;
        const bool in = v && ((int64_t)k > c.kgt || (eq && er + prefix_count(be) < c.req));
        const uint64_t bi = ballot(in);
        const int slot = slot0 + prefix_count(bi);
        if (in && slot < o.sel) {
            const int pos = pos_at(i);
            const int32_t idx = list ? list[pos] : pos;
            for (int f = 0; f < o.fan; ++f) {
                o.idx[(int64_t)f * o.sel + slot] = idx;
                if (o.score)
                    o.score[(int64_t)f * o.sel + slot] = sc;
            }
        }
        slot0 += __popcll(bi);
        er += __popcll(be);
    }
    for (int x = t.total + threadIdx.x; x < o.sel; x += kSelectThreads) {
        for (int f = 0; f < o.fan; ++f) {
            o.idx[(int64_t)f * o.sel + x] = -1;
            if (o.score)
                o.score[(int64_t)f * o.sel + x] = -__builtin_inff();
        }
    }
    lds_sync();
}

// Wave w's contiguous segment of a row of n scores, in float4 steps of 256
// positions, kRegSteps steps per batch (all loads of a batch issued at once).
struct RowSeg {
    int b0, b1, S;
};

__device__ __forceinline__ RowSeg row_segment(int n)
{
    const int wave = uniform(threadIdx.x / kWave);
    RowSeg g;
    g.S = (n + kSelWaves * 256 - 1) / (kSelWaves * 256) * 256;
    g.b0 = wave * g.S;
    g.b1 = (g.b0 + g.S < n) ? g.b0 + g.S : n;
    return g;
}

template <int NQ>
__device__ __forceinline__ void load_batch(const float *sc, int i0, int b1, float4 (&v)[NQ])
{
    const int lane = lane_id();
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int p = i0 + q * 256 + 4 * lane;
        v[q] = p < b1 ? *reinterpret_cast<const float4 *>(sc + p) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

__device__ __forceinline__ float f4(const float4 &v, int x)
{
    return x == 0 ? v.x : (x == 1 ? v.y : (x == 2 ? v.z : v.w));
}

// Lower bound theta for the top-`sel` of the n scores of a row: the floor of
// the histogram bin holding an order statistic of a sample of contiguous
// 64-score chunks spread evenly over the row, of rank chosen with slack so
// that, with high probability, at least sel scores of the row reach it.
// Whether they do is checked by the caller.
__device__ __forceinline__ uint32_t sample_theta(const float *sc, int n, int sel, SelShared &sm)
{
    constexpr int kPer = kSampleMax / kSelectThreads;
    const int half = n >> 1;
    const int ns = ((half < kSampleMax ? half : kSampleMax) / kWave) * kWave;  // n > kCandCap: ns >= 6144
    const int nch = ns / kWave;
    uint32_t slo = 0xFFFFFFFFu, shi = 0u;
    float f[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int i = threadIdx.x + u * kSelectThreads;
        const int ch = i / kWave;
        f[u] = i < ns ? sc[(int)((int64_t)ch * n / nch) + i % kWave] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int i = threadIdx.x + u * kSelectThreads;
        if (i < ns) {
            sm.cs[i] = f[u];
            slo = min(slo, score_key(f[u]));
            shi = max(shi, score_key(f[u]));
        }
    }
    const WaveTotals st = wave_totals(0, wave_min(slo), wave_max(shi), sm);
    const float expect = (float)sel * (float)ns / (float)n;
    int r = (int)ceilf(expect + 4.f * sqrtf(expect)) + 8;
    r = r < ns ? r : ns;
    return rank_bin_floor(ns, r, st.lo, st.hi, [&](int i) { return score_key(sm.cs[i]); }, sm);
}

// The scores >= theta among positions [b, e) of a row (b a multiple of 4),
// counted and then, if there are at most `cap`, written in index order as
// dst(slot, score, position). Wave w walks the w-th contiguous segment in
// float4 steps; a segment of at most kRegSteps steps stays in registers
// between the two passes. Returns the count; kmax gets the largest key among
// them (in every thread).
template <typename Dst>
__device__ __forceinline__ int count_pack(const float *sc, int b, int e, uint32_t theta, int cap, Dst dst,
                                          SelShared &sm, uint32_t &kmax)
{
    const int wave = uniform(threadIdx.x / kWave), lane = lane_id();
    const int S = (e - b + kSelWaves * 256 - 1) / (kSelWaves * 256) * 256;
    const int b0 = b + wave * S;
    const int b1 = (b0 + S < e) ? b0 + S : e;
    const bool held = S <= kRegSteps * 256;
    float4 v[kRegSteps];
    int cnt = 0;
    uint32_t km = 0u;
    for (int i0 = b0; i0 < b1; i0 += kRegSteps * 256) {
        load_batch(sc, i0, b1, v);
#pragma unroll
        for (int q = 0; q < kRegSteps; ++q) {
            const int p = i0 + q * 256 + 4 * lane;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const uint32_t k = score_key(f4(v[q], x));
                const bool in = p + x < b1 && k >= theta;
                cnt += in ? 1 : 0;
                km = in ? max(km, k) : km;
            }
        }
    }
    const WaveTotals t = wave_totals(wave_sum(cnt), 0u, wave_max(km), sm);
    kmax = t.hi;
    if (t.total > cap)
        return t.total;
    int slot0 = t.off;
    for (int i0 = b0; i0 < b1; i0 += kRegSteps * 256) {
        if (!held)
            load_batch(sc, i0, b1, v);
#pragma unroll
        for (int q = 0; q < kRegSteps; ++q) {
            const int p = i0 + q * 256 + 4 * lane;
            bool in[4];
            uint64_t bm[4];
            int before = 0, mine = 0;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                in[x] = p + x < b1 && score_key(f4(v[q], x)) >= theta;
                bm[x] = ballot(in[x]);
                before += prefix_count(bm[x]);
            }
            int o = slot0 + before;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                if (in[x]) {
                    dst(o, f4(v[q], x), p + x);
                    ++o;
                }
                mine += __popcll(bm[x]);
            }
            slot0 += mine;
        }
    }
    lds_sync();
    return t.total;
}

// A row of at most kRegRow scores is read from global memory once: wave w
// holds its contiguous segment in registers, one score per lane per step of
// 64 positions, and the sample, the count and the pack all work on those
// registers. The sample is every kSampleEvery-th step of each wave (at most
// 8192 scores, packed into LDS); it gives the key theta as in sample_theta. Counting and packing compare floats with the float of
// theta, which orders finite scores exactly as their keys do once a theta of
// +0 is lowered to -0 (both zeros then pass, as their keys do). Padding
// positions hold -inf and never pass, because theta lies within the key range
// of finite sampled scores (a row holding -inf takes the exact path instead).
// Returns the number of scores >= theta; if it is at most kCandCap they are
// packed into cs/cp in index order, with [lo, hi] their key range.
constexpr int kRegDw = 64;                         // steps per lane held in registers
constexpr int kRegRow = kSelectThreads * kRegDw;   // longest row held whole
constexpr int kSampleEvery = 8;

__device__ __forceinline__ int reg_stage(const float *sc, int n, int sel, SelShared &sm, uint32_t &lo, uint32_t &hi)
{
    const int wave = uniform(threadIdx.x / kWave), lane = lane_id();
    const int S = (n + kSelWaves * kWave - 1) / (kSelWaves * kWave) * kWave;  // positions per wave
    const int b0 = wave * S;
    const int len = uniform(max(0, min(S, n - b0)));  // this wave's positions
    float v[kRegDw];
#pragma unroll
    for (int q = 0; q < kRegDw; ++q) {
        const int o = q * kWave + lane;
        v[q] = o < len ? sc[b0 + o] : -__builtin_inff();
    }
    // the sample: wave totals give each wave its slice of cs
    int nsw = 0;
    uint32_t slo = 0xFFFFFFFFu, shi = 0u;
#pragma unroll
    for (int q = 0; q < kRegDw; q += kSampleEvery) {
        const int r = min(max(len - q * kWave, 0), kWave);
        nsw += r;
        if (lane < r) {
            const uint32_t k = score_key(v[q]);
            slo = min(slo, k);
            shi = max(shi, k);
        }
    }
    const WaveTotals st = wave_totals(nsw, wave_min(slo), wave_max(shi), sm);
    {
        int off = st.off;
#pragma unroll
        for (int q = 0; q < kRegDw; q += kSampleEvery) {
            const int r = min(max(len - q * kWave, 0), kWave);
            if (lane < r)
                sm.cs[off + lane] = v[q];
            off += r;
        }
    }
    lds_sync();
    const int ns = st.total;
    const float expect = (float)sel * (float)ns / (float)n;
    int rk = (int)ceilf(expect + 4.f * sqrtf(expect)) + 8;
    rk = rk < ns ? rk : ns;
    uint32_t theta = rank_bin_floor(ns, rk, st.lo, st.hi, [&](int i) { return score_key(sm.cs[i]); }, sm);
    if (theta == 0x80000000u)  // +0: lower to -0
        theta = 0x7FFFFFFFu;
    const float thf = key_score(theta);
    if (!(thf > -__builtin_inff()))
        return -1;

    int cnt = 0;
    float fm = -__builtin_inff();
#pragma unroll
    for (int q = 0; q < kRegDw; ++q) {
        cnt += __popcll(ballot(v[q] >= thf));
        fm = fmaxf(fm, v[q]);
    }
    const WaveTotals t = wave_totals(cnt, 0u, wave_max(score_key(fm)), sm);
    if (t.total > kCandCap)
        return t.total;
    int slot0 = t.off;
#pragma unroll
    for (int q = 0; q < kRegDw; ++q) {
        const bool in = v[q] >= thf;
        const uint64_t m = ballot(in);
        if (in) {
            const int o = slot0 + prefix_count(m);
            sm.cs[o] = v[q];
            sm.cp[o] = b0 + q * kWave + lane;
        }
        slot0 += __popcll(m);
    }
    lds_sync();
    lo = theta;
    hi = t.hi;
    return t.total;
}

// Key range of positions [0, n) of a row (for the exact path over the row).
__device__ __forceinline__ void row_range(const float *sc, int n, SelShared &sm, uint32_t &lo, uint32_t &hi)
{
    uint32_t a = 0xFFFFFFFFu, z = 0u;
    for (int i = threadIdx.x; i < n; i += kSelectThreads) {
        const uint32_t k = score_key(sc[i]);
        a = min(a, k);
        z = max(z, k);
    }
    const WaveTotals t = wave_totals(0, wave_min(a), wave_max(z), sm);
    lo = t.lo;
    hi = t.hi;
}

// Top selections of one score row: positions [0, npos), of which those with
// list[pos] <= lim (all of them without a list) are valid; valid positions
// form a prefix. Rows are 16-byte aligned and padded to a multiple of 4.
__device__ __forceinline__ void select_row(const SelRow &s, const SelOut *outs, int nout, SelShared &sm)
{
    const int lane = lane_id();
    const float *sc = s.sc;
    const int selmax = (nout > 1 && outs[1].sel > outs[0].sel) ? outs[1].sel : outs[0].sel;

    bool staged = true;
    bool identity = true;  // LDS entry i is row position i
    int n = s.npos, m;
    const int32_t *vlist = s.list;  // list still to be checked for validity
    if (vlist && n > kCandCap) {
        int v = 0;
        for (int i = threadIdx.x; i < s.npos; i += kSelectThreads)
            v += (vlist[i] >= 0 && vlist[i] <= s.lim) ? 1 : 0;
        n = wave_totals(wave_sum(v), 0u, 0u, sm).total;
        vlist = nullptr;
    }
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    if (n <= kCandCap) {
        // the whole row: one batched load, validity from the list on the way
        const RowSeg g = row_segment(n);
        int nv = 0;
        for (int i0 = g.b0; i0 < g.b1; i0 += kStageSteps * 256) {
            float4 v[kStageSteps];
            int4 lv[kStageSteps] = {};
            load_batch(sc, i0, g.b1, v);
            if (vlist) {
#pragma unroll
                for (int q = 0; q < kStageSteps; ++q) {
                    const int p = i0 + q * 256 + 4 * lane;
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const int px = p + x;
                        const int e = px < g.b1 ? vlist[px] : 0;
                        (x == 0 ? lv[q].x : x == 1 ? lv[q].y : x == 2 ? lv[q].z : lv[q].w) = e;
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < kStageSteps; ++q) {
                const int p = i0 + q * 256 + 4 * lane;
                if (p + 3 < g.b1)
                    *reinterpret_cast<float4 *>(&sm.cs[p]) = v[q];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int px = p + x;
                    const int e = x == 0 ? lv[q].x : x == 1 ? lv[q].y : x == 2 ? lv[q].z : lv[q].w;
                    if (px < g.b1 && (vlist == nullptr || (e >= 0 && e <= s.lim))) {
                        const float f = f4(v[q], x);
                        if (p + 3 >= g.b1)
                            sm.cs[px] = f;
                        lo = min(lo, score_key(f));
                        hi = max(hi, score_key(f));
                        ++nv;
                    }
                }
            }
        }
        const WaveTotals t = wave_totals(wave_sum(nv), wave_min(lo), wave_max(hi), sm);
        n = m = t.total;
        lo = t.lo;
        hi = t.hi;
    } else if (n <= kRegRow) {
        m = reg_stage(sc, n, selmax, sm, lo, hi);
        if (m < selmax || m > kCandCap)
            staged = false;
        else
            identity = false;
    } else {
        const uint32_t theta = sample_theta(sc, n, selmax, sm);
        uint32_t km;
        m = count_pack(sc, 0, n, theta, kCandCap,
                       [&](int o, float f, int pos) {
                           sm.cs[o] = f;
                           sm.cp[o] = pos;
                       },
                       sm, km);
        if (m < selmax || m > kCandCap) {
            staged = false;
        } else {
            identity = false;
            lo = theta;
            hi = km;
        }
    }
    if (!staged)
        row_range(sc, n, sm, lo, hi);  // exact selection on the row in global memory

#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (j >= nout)
            break;
        const SelOut &o = outs[j];
        if (staged) {
            const Cut c = block_radix_cut(m, o.sel, lo, hi, [&](int i) { return score_key(sm.cs[i]); }, sm);
            if (identity)
                block_emit(m, c, o, s.list, [&](int i) { return sm.cs[i]; }, [&](int i) { return i; }, sm);
            else
                block_emit(m, c, o, s.list, [&](int i) { return sm.cs[i]; }, [&](int i) { return sm.cp[i]; }, sm);
        } else {
            const Cut c = block_radix_cut(n, o.sel, lo, hi, [&](int i) { return score_key(sc[i]); }, sm);
            block_emit(n, c, o, s.list, [&](int i) { return sc[i]; }, [&](int i) { return i; }, sm);
        }
    }
}

// Row r of batch item bi of a selection pass: its scores, validity, and the
// outputs of its selections.
__device__ __forceinline__ bool select_geometry(const SplitSelectParams &p, int bi, int64_t r, SelRow &s,
                                                SelOut (&outs)[2])
{
    const Req rq = request_of(p.req, bi, p.L, p.q_len, p.g, p.m0);
    const int64_t off = rq.L - rq.q_len;
    s.sc = p.scores + ((int64_t)bi * p.nrows + r) * p.rowlen;
    int32_t *o1, *o2 = nullptr;
    float *s1, *s2 = nullptr;
    int fan1 = 1, fan2 = 0;
    if (p.mode == kProxy) {
        const int64_t m = rq.m0 + r;
        if (m >= rq.G)
            return false;
        const int64_t r0 = m * p.g;
        const int64_t r1 = (r0 + p.g < rq.q_len) ? r0 + p.g : rq.q_len;
        const int64_t mrow = rq.q_off + r0;
        const int64_t grow = rq.g_off + m;
        s.list = nullptr;
        s.lim = p.glim ? p.glim[grow] : (int)(off + r1 - 1);
        s.npos = s.lim + 1;
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
        int64_t rr = r;
        if (p.mode == kDense) {
            if (r >= dense_rows(rq, p.g, p.guard_rows))
                return false;
            s.list = nullptr;
            s.lim = (int)(off + rr);
            s.npos = s.lim + 1;
        } else {
            rr = dense_rows(rq, p.g, 1) + r;
            if (rr >= rq.q_len)
                return false;
            s.lim = (int)(off + rr);
            const int64_t m = rr / p.g;
            const int64_t r1 = ((m + 1) * p.g < rq.q_len) ? (m + 1) * p.g : rq.q_len;
            const int64_t t_last = off + r1 - 1;
            s.list = p.cand + (rq.g_off + m) * p.c;
            s.npos = p.cand_n ? p.cand_n[rq.g_off + m] : (int)((p.c < t_last + 1) ? p.c : t_last + 1);
        }
        const int64_t row = rq.q_off + rr;
        o1 = p.o1_idx + row * p.sel;
        s1 = p.o1_score ? p.o1_score + row * p.sel : nullptr;
    }
    outs[0] = SelOut{p.sel, o1, s1, fan1};
    outs[1] = SelOut{p.sel2, o2, s2, fan2};
    return true;
}

__global__ __launch_bounds__(kSelectThreads) void split_select_kernel(SplitSelectParams p)
{
    __shared__ SelShared sm;
    const int bi = blockIdx.y;
    const int64_t r = blockIdx.x;
    SelRow s;
    SelOut outs[2];
    if (!select_geometry(p, bi, r, s, outs))
        return;  // no such row in this request
    select_row(s, outs, p.sel2 > 0 ? 2 : 1, sm);
}

// ------------------------------------------------------------- launchers
template <int H, int D>
static hipError_t launch_split_score_t(const SplitScoreParams &prm, int mr, dim3 grid, hipStream_t stream)
{
    const dim3 block(kSplitWaves * kWave);
    if (prm.mode == kRefine && mr == 2)
        hipLaunchKernelGGL((split_score_kernel<H, D, true, 2>), grid, block, 0, stream, prm);
    else if (prm.mode == kRefine)
        hipLaunchKernelGGL((split_score_kernel<H, D, true, 1>), grid, block, 0, stream, prm);
    else
        hipLaunchKernelGGL((split_score_kernel<H, D, false, 1>), grid, block, 0, stream, prm);
    return hipGetLastError();
}

hipError_t launch_split_score(int H, int D, const SplitScoreParams &prm, int mr, dim3 grid, hipStream_t stream)
{
    if (prm.chunk % (32 * kSplitWaves) != 0 || (prm.mode == kRefine && prm.chunk / kSplitWaves > kSplitSpanMax))
        return hipErrorInvalidValue;
    if (mr != 1 && !(mr == 2 && prm.mode == kRefine && prm.g % 2 == 0))
        return hipErrorInvalidValue;
    if (H == 64 && D == 128)
        return launch_split_score_t<64, 128>(prm, mr, grid, stream);
    if (H == 4 && D == 32)
        return launch_split_score_t<4, 32>(prm, mr, grid, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_split_select(const SplitSelectParams &prm, hipStream_t stream)
{

    hipLaunchKernelGGL(split_select_kernel, dim3((unsigned)prm.nrows, (unsigned)prm.B),
                       dim3(kSelectThreads), 0, stream, prm);
    return hipGetLastError();
}

}  // namespace dsaidx
