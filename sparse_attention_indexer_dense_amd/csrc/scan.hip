// scan.hip - fused score + select kernels for many query rows (prefill shape),
// and the group-proxy pooling kernel.
//
// One workgroup owns NW rows (one per wave) that share a stream of key tiles.
// Per stage (128 keys for 8-wave workgroups, 64 or 32 for the smaller Refine
// ones), the keys are staged in LDS once for all NW rows. Each wave computes,
// for its row and 32 keys at a time, the 64-head score tile
// S[j][s] = q_j . k_s with bf16 MFMA 32x32x16 (fp32 accumulate), then the
// epilogue I(s) = sum_j w_j * max(0, S[j][s]) in registers (Eq. (1) of the
// PIVOT paper, arXiv 2607.24593, as described in its observation-O3
// paragraph); then, per 64 keys, the causal mask and a threshold filter: a
// key is kept only if its score beats a running threshold below which it
// provably cannot reach the row's top-sel. Kept (score, index) pairs go, in index order, to a
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

// Keys per LDS stage: 128 (four 32-key MFMA N-tiles) for 8-wave workgroups,
// 64 for 4-wave ones (two workgroups then share a CU).
template <int NW>
struct ScanStage {
    static constexpr int KEYS = NW >= 8 ? 128 : (NW >= 4 ? 64 : 32);
};

// LDS histogram increment for use while key DMA is in flight. Written as
// inline asm because the compiler's wait insertion cannot tell an LDS atomic
// from the DMA's LDS writes and would make every increment wait for all
// outstanding memory traffic (the key DMA of the next stage included). LDS
// operations of a wave execute in order, so later reads of the bin see it.
__device__ __forceinline__ void lds_inc(uint32_t *p)
{
    const uint32_t a = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint32_t *)p);
    asm volatile("ds_add_u32 %0, %1" : : "v"(a), "v"(1u) : "memory");
}

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
__device__ __forceinline__ Level1 level1(const uint32_t *h, RowState st, int sel)
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

// Visit buf[0..nbuf) in index order, 64 entries per wave step, with the loads
// of sixteen steps issued together so that passes are not latency-bound.
// f(entry, valid) runs once per step and lane.
template <typename F>
__device__ __forceinline__ void buffer_pass(const Entry *buf, int nbuf, F &&f)
{
    constexpr int U = 16;
    const int lane = lane_id();
    for (int base = 0; base < nbuf; base += U * kWave) {
        Entry e[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * kWave + lane;
            e[u].score = 0.f;
            e[u].idx = -1;
            if (i < nbuf)
                e[u] = buf[i];
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            f(e[u], base + u * kWave + lane < nbuf);
    }
}

// Finish a cut with levels 2 and 3 (passes over the buffer); h is scratch.
__device__ __forceinline__ Cut finish_cut(const Entry *buf, int nbuf, uint32_t *h, Level1 a)
{
    Cut c;
    if (a.all || a.r1 == a.h1) {
        c.kgt = (int64_t)a.b1 * (1ll << 21) - 1;
        c.keq = 0u;
        c.req = 0;
        return c;
    }
    clear_hist<kBins2>(h);
    buffer_pass(buf, nbuf, [&](const Entry &e, bool v) {
        const uint32_t key = score_key(e.score);
        if (v && (int)(key >> 21) == a.b1)
            atomicAdd(&h[(key >> 10) & (kBins2 - 1)], 1u);
    });
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
    buffer_pass(buf, nbuf, [&](const Entry &e, bool v) {
        const uint32_t key = score_key(e.score);
        if (v && (key >> 10) == pre)
            atomicAdd(&h[key & (kBins3 - 1)], 1u);
    });
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
__device__ __forceinline__ void emit(const Entry *buf, int nbuf, Cut c, int sel,
                     int32_t *oidx, float *osc, int fan, int64_t fstride)
{
    const int lane = lane_id();
    int emitted = 0, eqseen = 0;
    buffer_pass(buf, nbuf, [&](const Entry &e, bool v) {
        const uint32_t key = score_key(e.score);
        const bool eq = v && c.req > 0 && key == c.keq;
        const uint64_t meq = ballot(eq);
        const int er = eqseen + prefix_count(meq);
        const bool in = v && ((int64_t)key > c.kgt || (eq && er < c.req));
        const uint64_t min_ = ballot(in);
        const int pos = emitted + prefix_count(min_);
        if (in && pos < sel) {
            for (int f = 0; f < fan; ++f) {
                oidx[f * fstride + pos] = e.idx;
                if (osc)
                    osc[f * fstride + pos] = e.score;
            }
        }
        emitted += __popcll(min_);
        eqseen += __popcll(meq);
    });
    for (int x = emitted + lane; x < sel; x += kWave) {
        for (int f = 0; f < fan; ++f) {
            oidx[f * fstride + x] = -1;
            if (osc)
                osc[f * fstride + x] = -__builtin_inff();
        }
    }
}

// Keep only the top-`sel` entries of the buffer (stable, in place) and rebuild
// the level-1 histogram from them; returns the new state. Used when a buffer
// is about to overflow. (State travels by value so it stays in registers.)
__device__ __noinline__ RowState compact(Entry *buf, uint32_t *h, RowState st, int sel)
{
    __threadfence_block();
    Level1 a = level1(h, st, sel);
    Cut c = finish_cut(buf, st.nbuf, h, a);
    int kept = 0, eqseen = 0;
    // every write lands at or below the index of the entry it moves, and the
    // loads of a batch precede its writes: no entry is overwritten unread
    buffer_pass(buf, st.nbuf, [&](const Entry &e, bool v) {
        const uint32_t key = score_key(e.score);
        const bool eq = v && c.req > 0 && key == c.keq;
        const uint64_t meq = ballot(eq);
        const int er = eqseen + prefix_count(meq);
        const bool in = v && ((int64_t)key > c.kgt || (eq && er < c.req));
        const uint64_t min_ = ballot(in);
        const int pos = kept + prefix_count(min_);
        if (in)
            buf[pos] = e;
        kept += __popcll(min_);
        eqseen += __popcll(meq);
    });
    __threadfence_block();
    clear_hist<kBins1>(h);
    for (int i = lane_id(); i < kept; i += kWave)
        atomicAdd(&h[bin1(score_key(buf[i].score))], 1u);
    st.nbuf = kept;
    st.count_ge = kept;
    st.b = a.b1;
    if (c.req > 0)
        st.theta_exact = key_score(c.keq);
    else
        st.theta_exact = (c.kgt + 1 < (4ll << 21)) ? -__builtin_inff() : key_score((uint32_t)(c.kgt + 1));
    st.theta = fmaxf(st.theta_exact, bin1_floor(st.b));
    return st;
}

// ------------------------------------------------------------- block plans
struct WaveRow {
    bool valid;
    const uint16_t *q;
    const float *w;
    int lim;      // last eligible key index (< 2^31)
    int32_t *o1;
    float *s1;
    int fan1;
    int32_t *o2;
    float *s2;
    int fan2;
};

struct BlockKeys {
    const uint16_t *Kb;   // keys of this request
    const int32_t *list;  // candidate list (kRefine) or nullptr (prefix)
    int nkeys;            // list length, or number of prefix keys (< 2^31); 0: idle block
    int L;                // keys of the request
};

// Block j of a launch: request j % B, and the (j / B)-th of that request's
// blocks, longest first. Requests with fewer blocks than the largest one
// leave the remaining ones idle (no rows, no keys).
template <int H, int D, int NW, int MODE>
__device__ __forceinline__ void plan_block(const ScanParams &p, int64_t j, int wave,
                                           WaveRow &wr, BlockKeys &bk)
{
    const int bi = (int)(j % p.B);
    const int64_t jj = j / p.B;
    const Req rq = request_of(p.req, bi, p.L, p.q_len, p.g, p.m0);
    const int64_t off = rq.L - rq.q_len;  // position of query row 0
    wr.o2 = nullptr;
    wr.s2 = nullptr;
    wr.fan2 = 0;
    bk.Kb = p.K + rq.key_off * D;
    bk.L = (int)rq.L;
    if (MODE == kDense) {
        const int64_t rows = dense_rows(rq, p.g, p.guard_rows);
        const int64_t rb = (rows + NW - 1) / NW - 1 - jj;
        const int64_t r = rb * NW + wave;
        const int64_t rlast = (rb * NW + NW < rows ? rb * NW + NW : rows) - 1;
        wr.valid = rb >= 0 && r < rows;
        const int64_t row = rq.q_off + r;
        wr.q = p.Q + row * H * D;
        wr.w = p.W + row * H;
        wr.lim = (int)(off + r);
        wr.o1 = p.o1_idx + row * p.sel;
        wr.s1 = p.o1_score ? p.o1_score + row * p.sel : nullptr;
        wr.fan1 = 1;
        bk.list = nullptr;
        bk.nkeys = rb >= 0 ? (int)(off + rlast + 1) : 0;
    } else if (MODE == kProxy) {
        const int64_t rb = (rq.G - rq.m0 + NW - 1) / NW - 1 - jj;
        const int64_t m = rq.m0 + rb * NW + wave;
        const int64_t mlast = (rq.m0 + rb * NW + NW < rq.G ? rq.m0 + rb * NW + NW : rq.G) - 1;
        wr.valid = rb >= 0 && m < rq.G;
        const int64_t grow = rq.g_off + m;
        const int64_t r0 = m * p.g;
        const int64_t r1 = (r0 + p.g < rq.q_len) ? r0 + p.g : rq.q_len;
        wr.q = p.Q + grow * H * D;
        wr.w = p.W + grow * H;
        wr.lim = (int)(off + r1 - 1);
        const int64_t r1last = ((mlast + 1) * p.g < rq.q_len) ? (mlast + 1) * p.g : rq.q_len;
        bk.nkeys = rb >= 0 ? (int)(off + r1last) : 0;
        if (p.glim) {
            // chunk summaries: the chunks complete at the group's last
            // position (a non-decreasing limit over the groups)
            bk.Kb = p.K + (int64_t)bi * p.krows * D;
            bk.L = (int)p.krows;
            wr.lim = wr.valid ? p.glim[grow] : -1;
            bk.nkeys = rb >= 0 ? p.glim[rq.g_off + mlast] + 1 : 0;
        }
        // output 1: candidate rows [groups][sel] or the member rows
        if (p.o1_members) {
            const int64_t row = rq.q_off + r0;
            wr.o1 = p.o1_idx + row * p.sel;
            wr.s1 = p.o1_score ? p.o1_score + row * p.sel : nullptr;
            wr.fan1 = (int)(r1 - r0);
        } else {
            wr.o1 = p.o1_idx + grow * p.sel;
            wr.s1 = p.o1_score ? p.o1_score + grow * p.sel : nullptr;
            wr.fan1 = 1;
        }
        if (p.sel2 > 0) {
            const int64_t row = rq.q_off + r0;
            wr.o2 = p.o2_idx + row * p.sel2;
            wr.s2 = p.o2_score ? p.o2_score + row * p.sel2 : nullptr;
            wr.fan2 = (int)(r1 - r0);
        }
        bk.list = nullptr;
    } else {  // kRefine
        const int64_t m = rq.G - 1 - jj / p.member_chunks;
        const int chunk = (int)(jj % p.member_chunks);
        const bool live = m >= rq.m0;
        const int64_t r0 = m * p.g;
        const int64_t r1 = (r0 + p.g < rq.q_len) ? r0 + p.g : rq.q_len;
        const int64_t r = r0 + (int64_t)chunk * NW + wave;
        wr.valid = live && r < r1;
        const int64_t row = rq.q_off + r;
        wr.q = p.Q + row * H * D;
        wr.w = p.W + row * H;
        wr.lim = (int)(off + r);
        wr.o1 = p.o1_idx + row * p.sel;
        wr.s1 = p.o1_score ? p.o1_score + row * p.sel : nullptr;
        wr.fan1 = 1;
        const int64_t t_last = off + r1 - 1;
        // a block without a live group (m < 0 past a request's groups, or an
        // empty request) reads no keys, but the branch-free list loads still
        // touch entry 0: point it at the first candidate row, which exists
        bk.list = p.cand + (live ? (rq.g_off + m) * p.c : 0);
        bk.nkeys = live ? (p.cand_n ? p.cand_n[rq.g_off + m] : (int)((p.c < t_last + 1) ? p.c : t_last + 1)) : 0;
    }
}

// ------------------------------------------------------------------ kernel
// Global->LDS DMA through a buffer resource (MUBUF buffer_load ... lds): lane
// l writes 16 bytes at LDS address lds + 16*l from byte voffset of the range
// [base, base + bytes); base and bytes must be wave-uniform.
__device__ __forceinline__ void buffer_load_lds16(const unsigned char *base, int bytes, unsigned char *lds,
                                                  int voffset)
{
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char *>(base), (short)0, bytes, kBufferRsrcWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)lds, 16, voffset, 0, 0, 0);
}

// Keys of one stage live in LDS as rows of 2*D bytes whose 16-byte chunks are
// XOR-swizzled by the row index (chunk c of row n sits at slot c ^ (n % CHUNKS)),
// so that the 32 rows one MFMA B-fragment read touches spread over all banks.
// Stages are filled by global->LDS DMA (global_load_lds_dwordx4): lane l of a
// DMA instruction writes the l-th 16 bytes of a 1 KiB span, so it fetches the
// global chunk that belongs in that slot. A candidate list (Refine) travels the
// same way, one int per lane, into a per-stage LDS array.
template <int D, int NW, int STAGE>
struct StageDma {
    static constexpr int ROWB = 2 * D;
    static constexpr int CHUNKS = ROWB / 16;
    static constexpr int RPI = kWave / CHUNKS;                  // key rows per DMA instruction
    static constexpr int PER_STAGE = STAGE * ROWB / 1024;       // DMA instructions per stage
    static constexpr int PER_WAVE = (PER_STAGE + NW - 1) / NW;  // per wave
};

// Prefix scans (dense rows, proxies): DMA of stage t's keys, rows
// t*STAGE .. t*STAGE+STAGE-1. A full stage's rows are contiguous: slot j of
// lane l fetches the 16 bytes at stage base + j * NW*RPI*ROWB + loff, where
// loff (this lane's row-in-slot and swizzled chunk, the same for every j
// because NW*RPI is a multiple of CHUNKS) is fixed for the whole kernel. No
// index arithmetic, bounds checks or branches per DMA. The last, partial
// stage of a row block fetches the stage's first row for slots past the
// prefix (the causal mask never admits them).
//
// These DMAs are buffer loads (MUBUF) through a resource based at the stage's
// first key row and spanning the stage: with the global (FLAT-encoded) form
// in flight, the compiler treats LDS completions as unordered and makes every
// B-fragment read of the stage wait for all of a tile's reads (lgkmcnt(0))
// before its first MFMA; with buffer loads it waits for each fragment only.
template <int D, int NW, int STAGE>
__device__ __forceinline__ void stage_issue_prefix(unsigned char *kbuf, const BlockKeys &bk, int t, uint32_t loff,
                                                   int wave, int lane)
{
    using SD = StageDma<D, NW, STAGE>;
    static_assert((NW * SD::RPI) % SD::CHUNKS == 0, "slot offsets must not change the swizzle");
    const int row0 = t * STAGE;
    const unsigned char *sb = reinterpret_cast<const unsigned char *>(bk.Kb) + (int64_t)row0 * SD::ROWB;
    if (row0 + STAGE <= bk.nkeys) {
#pragma unroll
        for (int j = 0; j < SD::PER_WAVE; ++j) {
            const int i = wave + NW * j;
            if (SD::PER_STAGE % NW == 0 || i < SD::PER_STAGE)
                buffer_load_lds16(sb, STAGE * SD::ROWB, kbuf + i * 1024, (int)(loff + j * NW * SD::RPI * SD::ROWB));
        }
    } else {
        // the last, partial stage: slots past the prefix fetch the stage's
        // first row again (the causal mask never admits them)
#pragma unroll
        for (int j = 0; j < SD::PER_WAVE; ++j) {
            const int i = wave + NW * j;
            if (SD::PER_STAGE % NW == 0 || i < SD::PER_STAGE) {
                const int n = i * SD::RPI + lane / SD::CHUNKS;
                const int rn = (row0 + n < bk.nkeys) ? n : 0;
                const int c = (lane % SD::CHUNKS) ^ (n & (SD::CHUNKS - 1));
                buffer_load_lds16(sb, STAGE * SD::ROWB, kbuf + i * 1024, rn * SD::ROWB + c * 16);
            }
        }
    }
}

// Refine: the list entries of this wave's DMA slots of stage t, loaded
// without branches (a clamped index for slots past the list) so that the
// compiler can count the loads in flight exactly; ok[j] marks the slots that
// hold a key.
template <int D, int NW, int STAGE>
__device__ __forceinline__ void stage_list_keys(const BlockKeys &bk, int t, int ntiles, int wave, int lane,
                                                int (&raw)[StageDma<D, NW, STAGE>::PER_WAVE],
                                                bool (&ok)[StageDma<D, NW, STAGE>::PER_WAVE])
{
    using SD = StageDma<D, NW, STAGE>;
#pragma unroll
    for (int j = 0; j < SD::PER_WAVE; ++j) {
        const int i = wave + NW * j;
        const int pp = t * STAGE + i * SD::RPI + lane / SD::CHUNKS;
        ok[j] = (SD::PER_STAGE % NW == 0 || i < SD::PER_STAGE) && t < ntiles && pp < bk.nkeys;
        raw[j] = bk.list[ok[j] ? pp : 0];
    }
}

// Refine: DMA of stage t's keys (no branches: a slot without a key fetches
// row 0, which the filter never admits) and of its list entries.
template <int D, int NW, int STAGE>
__device__ __forceinline__ void stage_issue_list(unsigned char *kbuf, int32_t *lbuf, const BlockKeys &bk, int L,
                                                 int t, const int (&raw)[StageDma<D, NW, STAGE>::PER_WAVE],
                                                 const bool (&ok)[StageDma<D, NW, STAGE>::PER_WAVE], int wave,
                                                 int lane)
{
    using SD = StageDma<D, NW, STAGE>;
#pragma unroll
    for (int j = 0; j < SD::PER_WAVE; ++j) {
        const int i = wave + NW * j;
        // every wave owns PER_WAVE slots when NW divides the stage's DMA count
        if (SD::PER_STAGE % NW == 0 || i < SD::PER_STAGE) {
            const int n = i * SD::RPI + lane / SD::CHUNKS;
            const int c = (lane % SD::CHUNKS) ^ (n & (SD::CHUNKS - 1));
            const int key = (ok[j] && raw[j] >= 0 && raw[j] < L) ? raw[j] : 0;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(bk.Kb + (int64_t)key * D + c * 8),
                (__attribute__((address_space(3))) void *)(kbuf + i * 1024), 16, 0, 0);
        }
    }
    if (wave == NW - 1) {
#pragma unroll
        for (int h0 = 0; h0 < STAGE; h0 += kWave) {
            const int pp = t * STAGE + h0 + lane;
            if (h0 + lane < STAGE)
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void *)(bk.list + (pp < bk.nkeys ? pp : 0)),
                    (__attribute__((address_space(3))) void *)(lbuf + h0), 4, 0, 0);
        }
    }
}

// Two waves per SIMD: one 8-wave workgroup, or two 4-wave workgroups, per CU.
template <int H, int D, int NW, int MODE>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void scan_select_kernel(ScanParams p)
{
    using S = Shape<H, D>;
    constexpr int STAGE = ScanStage<NW>::KEYS;
    using SD = StageDma<D, NW, STAGE>;
    constexpr int MB = S::MB, KS = S::KS, ROWB = S::ROWB, CHUNKS = S::CHUNKS;
    constexpr int STAGE_BYTES = STAGE * ROWB;
    constexpr int TILES = STAGE / 32;

    __shared__ __align__(1024) unsigned char kA[STAGE_BYTES];
    __shared__ __align__(1024) unsigned char kB[STAGE_BYTES];
    __shared__ __align__(16) int32_t lA[MODE == kRefine ? STAGE : 1];
    __shared__ __align__(16) int32_t lB[MODE == kRefine ? STAGE : 1];
    __shared__ uint32_t hist_all[NW * kBins1];

    const int tid = threadIdx.x;
    const int wave = uniform(tid / kWave);  // wave-uniform (SGPR)
    const int lane = tid % kWave;
    const int half = lane >> 5;
    const int col = lane & 31;
    uint32_t *h = hist_all + wave * kBins1;
    Entry *buf = p.slots + ((int64_t)blockIdx.x * NW + wave) * p.cap;

    // this lane's byte offset within slot 0 of a stage of contiguous keys
    // (row within the slot, XOR-swizzled chunk)
    uint32_t loff;
    {
        const int n = wave * SD::RPI + lane / SD::CHUNKS;
        loff = (uint32_t)(n * SD::ROWB + (((lane % SD::CHUNKS) ^ (n & (SD::CHUNKS - 1))) * 16));
    }

    // lane-constant LDS byte offsets of this lane's B-fragment chunks in a stage
    uint32_t koff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        koff[ks] = (uint32_t)(col * ROWB + (((half * KS + ks) ^ (col & (CHUNKS - 1))) * 16));

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

        const int nkeys = bk.nkeys;
        const int lim = wr.valid ? wr.lim : -1;
        // prefix keys: positions above `last` are never eligible for this row
        const int last = (nkeys - 1 < lim) ? nkeys - 1 : lim;
        const int ntiles = (nkeys + STAGE - 1) / STAGE;

        // MFMA score tile of 32 keys (tile nt of the stage in kb)
        // (all K fragments of the tile are read before its first MFMA; the
        // scheduling barrier keeps the compiler from sinking the reads back
        // next to their MFMAs, where each would wait out the LDS latency)
        // (Refine, with its candidate-list bookkeeping, reads them in two
        // halves to stay within the register budget)
        auto mfma_tile = [&](const unsigned char *kb, int nt, f32x16 (&acc)[MB]) {
            constexpr int KB = (MODE == kRefine && KS > 4) ? KS / 2 : KS;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[mb] = f32x16{};
#pragma unroll
            for (int k0 = 0; k0 < KS; k0 += KB) {
                bf16x8 kf[KB];
#pragma unroll
                for (int ks = 0; ks < KB; ++ks)
                    kf[ks] = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const u32x4 *>(kb + koff[k0 + ks] + nt * 32 * ROWB));
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < KB; ++ks)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][k0 + ks], kf[ks], acc[mb], 0, 0, 0);
            }
        };
        // epilogue: ReLU, head weights, and the sum over this lane's heads (the
        // other half-wave's heads are added when two tiles are combined)
        auto epilogue = [&](const f32x16 (&acc)[MB]) {
            float part[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                part[mb] = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    part[mb] = fmaf(wv[mb][r], relu(acc[mb][r]), part[mb]);
            }
            float s = part[0];
#pragma unroll
            for (int mb = 1; mb < MB; ++mb)
                s += part[mb];
            return s;
        };
        // raise the threshold bin while the bins above it hold >= sel entries:
        // a step or two by walking, a longer jump by searching all bins at once
        auto advance = [&]() {
            int bb = st.b, cg = st.count_ge, hv = uniform((int)h[bb]);
            if (cg - hv < p.sel)
                return;
            for (int step = 0; step < 2 && cg - hv >= p.sel && bb < kBins1 - 1; ++step) {
                cg -= hv;
                ++bb;
                hv = uniform((int)h[bb]);
            }
            if (cg - hv >= p.sel) {
                int x, above;
                find_bin<kBins1>(h, p.sel, x, above);
                bb = x;
                hv = uniform((int)h[x]);
                cg = above + hv;
            }
            st.b = bb;
            st.count_ge = cg;
            st.theta = fmaxf(st.theta_exact, bin1_floor(st.b));
        };
        // causal mask and threshold filter of the tile pair pr of stage t: lane
        // l owns key position t*STAGE + 64*pr + l (tile 2pr in lanes 0..31,
        // tile 2pr+1 in lanes 32..63). A stage of one tile pairs it with
        // nothing: its upper lanes are masked.
        auto filter = [&](float total, const int32_t *lb, int t, int pr) {
            const int p0 = t * STAGE + pr * 64;
            const bool in_stage = STAGE >= 64 || lane < STAGE;
            int key;
            bool ok;
            // bitwise ands: the lane-varying conditions need no branch or exec
            // mask change
            if (MODE == kRefine) {
                key = lb[STAGE >= 64 ? pr * 64 + lane : (in_stage ? lane : 0)];
                ok = in_stage & (lane < nkeys - p0) & (key >= 0) & (key <= lim);
            } else {
                key = p0 + lane;
                ok = in_stage & (lane <= last - p0);
            }
            const bool adm = ok & (total > st.theta);
            const uint64_t m = ballot(adm);
            if (m) {
                if (adm) {
                    Entry e;
                    e.score = total;
                    e.idx = key;
                    buf[st.nbuf + prefix_count(m)] = e;
                    lds_inc(&h[bin1(score_key(total))]);
                }
                const int cnt = __popcll(m);
                st.nbuf += cnt;
                st.count_ge += cnt;
            }
        };

        // after a stage: raise the threshold (once per stage: a lag of at
        // most one stage of keys), and compact a nearly full buffer
        auto stage_end = [&]() {
            if (!wr.valid)
                return;
            if (st.count_ge >= p.sel)
                advance();
            if (st.nbuf > p.cap - STAGE)
                st = compact(buf, h, st, p.sel);
        };

        // the active tiles of a stage, software-pipelined: the MFMAs of tile
        // nt+1 are issued next to the epilogue of tile nt so that the matrix
        // pipe and the VALU work at the same time. The two waves sharing a
        // SIMD start a stage together; the issue arbiter favours the older
        // one, which then waits at the stage barrier while the other finishes
        // alone. Each wave therefore raises its priority by the tiles it has
        // left, so that the one behind is served first and both finish
        // together.
        auto compute = [&](const unsigned char *kb, const int32_t *lb, int t) {
            if (!wr.valid)
                return;
            const int pf = t * STAGE;
            const int span = (MODE == kRefine) ? nkeys - pf : last - pf + 1;
            const int ntl = span <= 0 ? 0 : (span >= STAGE ? TILES : (span + 31) / 32);
            if (ntl == 0)
                return;
            f32x16 a0[MB], a1[MB];
            mfma_tile(kb, 0, a0);
            float s0 = 0.f;  // lane partial of the pair's first tile
#pragma unroll
            for (int nt = 0; nt < TILES; ++nt) {
                if (nt >= ntl)
                    break;
                wave_priority(TILES - 1 - nt);
                float s;
                if (nt + 1 < ntl) {
                    if (nt & 1) {
                        mfma_tile(kb, nt + 1, a0);
                        s = epilogue(a1);
                    } else {
                        mfma_tile(kb, nt + 1, a1);
                        s = epilogue(a0);
                    }
                    // interleave: one MFMA per four VALU ops
#pragma unroll
                    for (int q = 0; q < KS * MB; ++q) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                    }
                } else {
                    s = (nt & 1) ? epilogue(a1) : epilogue(a0);
                }
                // one filter per tile pair, all 64 lanes holding a key; a
                // pair missing its second tile adds nothing for it (its
                // lanes are past the stage's last key)
                if (nt & 1)
                    filter(half_wave_sum2(s0, s) + 0.0f, lb, t, nt >> 1);
                else if (nt + 1 >= ntl)
                    filter(half_wave_sum2(s, 0.f) + 0.0f, lb, t, nt >> 1);
                else
                    s0 = s;
            }
            wave_priority(0);
            stage_end();
        };

        // key indices of this wave's DMA slots, one stage ahead
        int keys[SD::PER_WAVE];
        bool kok[SD::PER_WAVE];
        auto fetch_keys = [&](int t) {
            if constexpr (MODE == kRefine)
                stage_list_keys<D, NW, STAGE>(bk, t, ntiles, wave, lane, keys, kok);
        };
        auto issue = [&](unsigned char *kb, int32_t *lb, int t) {
            if constexpr (MODE == kRefine)
                stage_issue_list<D, NW, STAGE>(kb, lb, bk, bk.L, t, keys, kok, wave, lane);
            else
                stage_issue_prefix<D, NW, STAGE>(kb, bk, t, loff, wave, lane);
        };

        fetch_keys(0);
        if (ntiles > 0)
            issue(kA, lA, 0);
        fetch_keys(1);
        __syncthreads();
        // two stages per trip so that each LDS buffer is a distinct object at
        // every access (the DMA into one overlaps the MFMA reads of the other)
        for (int t = 0; t < ntiles; t += 2) {
            if (t + 1 < ntiles)
                issue(kB, lB, t + 1);
            fetch_keys(t + 2);
            compute(kA, lA, t);
            __syncthreads();
            if (t + 1 >= ntiles)
                break;
            if (t + 2 < ntiles)
                issue(kA, lA, t + 2);
            fetch_keys(t + 3);
            compute(kB, lB, t + 1);
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
        __syncthreads();
    }
}

// -------------------------------------------------------------- pooling
// Proxy of group m (PIVOT, experimental setup: mean pooling per head, within
// a window; ablation: endpoint proxies): the averaged members' queries summed
// in row order in fp32, divided by their count (IEEE division), rounded to
// bf16 nearest-even; weights likewise in fp32.
template <int H, int D>
__global__ __launch_bounds__(256) void pool_kernel(PoolParams p)
{
    const int64_t m = blockIdx.x;
    const int bi = blockIdx.y;
    const Req rq = request_of(p.req, bi, p.L, p.q_len, p.g, p.m0);
    if (m < rq.m0 || m >= rq.G)
        return;  // guarded, or beyond the request's groups
    const int64_t grp = rq.g_off + m;
    const int64_t g0 = m * p.g;
    const int64_t g1 = (g0 + p.g < rq.q_len) ? g0 + p.g : rq.q_len;
    // the members averaged: a window ending at the group's last row, or one
    // endpoint member
    int64_t r0 = g0, r1 = g1;
    if (p.proxy == 1) {
        r1 = g0 + 1;
    } else if (p.proxy == 2) {
        r0 = g1 - 1;
    } else if (p.window > 0 && p.window < g1 - g0) {
        r0 = g1 - p.window;
    }
    const float n = (float)(r1 - r0);
    const uint16_t *Qb = p.Q + rq.q_off * H * D;
    const float *Wb = p.W + rq.q_off * H;
    // a few groups spread each proxy over gridDim.z workgroups; the member
    // loads are unrolled so that several are in flight at once
    for (int x = (blockIdx.z * blockDim.x + threadIdx.x) * 8; x < H * D; x += gridDim.z * blockDim.x * 8) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
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
    if (blockIdx.z == 0) {
        for (int jh = threadIdx.x; jh < H; jh += blockDim.x) {
            float acc = 0.f;
#pragma unroll 4
            for (int64_t r = r0; r < r1; ++r)
                acc += Wb[r * H + jh];
            p.Wp[grp * H + jh] = __fdiv_rn(acc, n);
        }
    }
}

// ------------------------------------------------------------- launchers
template <int H, int D, int NW, int MODE>
static hipError_t launch_scan(const ScanParams &prm, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL((scan_select_kernel<H, D, NW, MODE>), dim3(grid), dim3(NW * kWave), 0, stream, prm);
    return hipGetLastError();
}

template <int H, int D>
static hipError_t launch_pool_t(const PoolParams &prm, hipStream_t stream)
{
    // one workgroup per (group, request) and, when there are few groups (a
    // decode step), one per 2048 proxy elements; gmax = the largest request's
    // groups
    const unsigned zc = (prm.gmax * prm.B <= 1024) ? (unsigned)((H * D / 8 + 255) / 256) : 1u;
    hipLaunchKernelGGL((pool_kernel<H, D>), dim3((unsigned)prm.gmax, (unsigned)prm.B, zc), dim3(256), 0, stream,
                       prm);
    return hipGetLastError();
}

size_t scan_lds_bytes(int H, int D, int NW)
{
    (void)H;
    const int stage = NW >= 8 ? ScanStage<8>::KEYS : (NW >= 4 ? ScanStage<4>::KEYS : ScanStage<1>::KEYS);
    return 2 * (size_t)stage * 2 * D + (size_t)NW * kBins1 * 4;
}

hipError_t launch_scan_select(int H, int D, int NW, int mode, const ScanParams &prm, int grid,
                              hipStream_t stream)
{
#define DSAIDX_SCAN_CASE(HH, DD, NN, MM)                                   \
    if (H == HH && D == DD && NW == NN && mode == MM)                      \
        return launch_scan<HH, DD, NN, MM>(prm, grid, stream);
    DSAIDX_SCAN_CASE(64, 128, 8, kDense)
    DSAIDX_SCAN_CASE(64, 128, 8, kProxy)
    DSAIDX_SCAN_CASE(64, 128, 1, kRefine)
    DSAIDX_SCAN_CASE(64, 128, 4, kRefine)
    DSAIDX_SCAN_CASE(64, 128, 8, kRefine)
    DSAIDX_SCAN_CASE(4, 32, 8, kDense)
    DSAIDX_SCAN_CASE(4, 32, 8, kProxy)
    DSAIDX_SCAN_CASE(4, 32, 1, kRefine)
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
