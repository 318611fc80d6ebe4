// refine.hip - PIVOT-Refine (PIVOT paper, abstract and Method: every member of
// a group re-scores the group's candidates that are causal for it, with its
// own query and weights, and keeps its own top-k) for groups of at most four
// members and at most 4608 candidates, with the members' scores kept on chip.
//
// One workgroup per CU (the LDS below), looping over groups, eight waves:
// wave (member m, half h) scores tiles 2h and 2h+1 of every 128-key stage for
// member m. A group's candidate list is staged in LDS once, and each member's
// query rows pass through LDS on the way to the MFMA A fragments (so that
// their loads are contiguous). Each stage's candidate keys are gathered with
// plain 16-byte loads into registers two stages ahead (each wave loads an
// eighth of a stage), then written to an LDS stage buffer (XOR-swizzled
// rows, as in scan.hip) that all eight waves read their MFMA B fragments
// from. The score tile and its epilogue are those of scan.hip's Refine mode
// (same fragment order, same additions), so the scores are the same bits.
// Every score goes to the member's row in LDS (4096 or 4608 floats), and
// after the last stage the member's two waves select the exact top-k of its
// causal candidates from that row (a radix cut over the row's key range,
// ties to the lower index) and write it in ascending index order. No candidate
// buffer goes to global memory: the kernel writes the outputs only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "kernels.h"

namespace dsaidx {

constexpr int kRefMembers = 4;                 // members per group (g <= 4)
constexpr int kRefHalves = 2;                  // waves per member
constexpr int kRefWaves = kRefMembers * kRefHalves;
constexpr int kRefStage = 128;                 // keys per stage: two 32-key tiles per wave
constexpr int kRefRing = 2;                    // stages gathered ahead (registers)
constexpr int kRefXch = 8;  // words of LDS per member for its two waves' exchanges

// List capacities the kernel is built for (candidates per group): one for
// the common c <= 4096, one for the key-chunk path's lists of (nsel + 1)
// 64-key chunks; the LDS is 64 KiB + 20 bytes per entry of capacity.
constexpr int kRefCapSmall = 4096;
static_assert(kRefineLdsCandMax == 4608 && kRefineLdsCandMax % kRefStage == 0 &&
                  kRefCapSmall % kRefStage == 0, "whole stages");

// Exact top-`sel` of the n scores r[0..n) (LDS) of one row, ties to the lower
// index, by the row's two waves (hv = 0, 1), written to oidx/osc in ascending
// index order (list[x] is the key index of entry x) and padded with -1 / -inf
// up to sel. Every wave of the workgroup calls it (its barriers are the
// workgroup's); a wave of an absent member passes active = false.
//
// Wave hv holds entries x = (hv * NQ + q) * 64 + lane, q < NQ, as
// order-preserving keys in registers. The cut is a radix select over the
// row's own key range [kmin, kmax] rather than over fixed bit fields: level 1
// splits the range into at most 2048 bins of 2^s keys, each later level
// splits the boundary bin of the one before into 2048 (the last into single
// keys), and a level ends the search as soon as its boundary bin is wholly
// in. Scores of one row share few exponents, so fixed top-bit bins would pile
// most keys into a handful of bins, and the LDS atomics of a bin serialise.
// Both waves count into the member's histogram h and both read it back; xch
// carries the range and wave 0's counts. The emit pass takes 16 entries per
// lane at a time: their list indices, then every selected entry's output slot
// (ballots, no branches), then the writes; wave 1 starts after wave 0's share.
template <int NQ>  // row entries per lane per wave
__device__ __forceinline__ void member_select(const float *r, const int32_t *list, int n, int sel, uint32_t *h,
                                              uint32_t *xch, int hv, bool active, int32_t *oidx, float *osc)
{
    const int lane = lane_id();
    const int e0 = hv * NQ;  // this wave's first entry block
    uint32_t key[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
        key[q] = score_key(r[(e0 + q) * kWave + lane]);  // (past n: unused)
    auto valid = [&](int q) { return active && (e0 + q) * kWave + lane < n; };

    // the key range of the row
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
        if (valid(q)) {
            lo = min(lo, key[q]);
            hi = max(hi, key[q]);
        }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (active && lane == 0) {
        xch[2 * hv] = lo;
        xch[2 * hv + 1] = hi;
    }
    __syncthreads();
    lo = min(xch[0], xch[2]);
    hi = max(xch[1], xch[3]);

    Cut c{-1, 0u, 0};  // every key when n <= sel
    bool done = !(active && n > sel);
    uint64_t width = (uint64_t)(hi - lo) + 1;  // keys in [lo, lo + width)
    int sh = 0;
    while ((width - 1) >> sh >= (uint64_t)kBins1)
        ++sh;
    int need = sel;
    // at most three levels: sh <= 21 at level 1, <= 10 at level 2, 0 at 3
    for (int level = 0; level < 3; ++level) {
        if (!done)
#pragma unroll
            for (int b = 0; b < kBins1 / kRefHalves / kWave; ++b)
                h[(hv * (kBins1 / kRefHalves)) + b * kWave + lane] = 0u;
        __syncthreads();
        if (!done) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const uint32_t d = key[q] - lo;  // wraps below lo: out of range
                if (valid(q) && key[q] >= lo && (uint64_t)d < width)
                    atomicAdd(&h[d >> sh], 1u);
            }
        }
        __syncthreads();
        if (!done) {
            int b, above;
            find_bin<kBins1>(h, need, b, above);
            need -= above;
            const uint32_t base = lo + ((uint32_t)b << sh);
            if (sh == 0) {
                c.kgt = (int64_t)base;
                c.keq = base;
                c.req = need;
                done = true;
            } else if (need == uniform((int)h[b])) {
                c.kgt = (int64_t)base - 1;
                done = true;
            } else {
                lo = base;
                width = (uint64_t)1 << sh;
                sh = sh > 11 ? sh - 11 : 0;
            }
        }
        __syncthreads();
    }

    // Without a partial take of equal keys (req = 0) an entry is in iff its
    // key is above kgt, one 32-bit compare (kgt = -1: every entry).
    const bool partial = c.req > 0;
    const bool every = c.kgt < 0;
    const uint32_t thr = (uint32_t)c.kgt;
    // wave 0's share: its selected entries and its entries equal to keq
    if (active && hv == 0) {
        int ngt = 0, neq = 0;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            ngt += __popcll(ballot(valid(q) && (every || key[q] > thr)));
            if (partial)
                neq += __popcll(ballot(valid(q) && key[q] == c.keq));
        }
        if (lane == 0) {
            xch[4] = (uint32_t)ngt;
            xch[5] = (uint32_t)neq;
        }
    }
    __syncthreads();
    if (!active)
        return;
    int emitted = 0, eqseen = 0;
    if (hv == 1) {
        eqseen = (int)xch[5];
        emitted = (int)xch[4] + min(eqseen, c.req);
    }
    constexpr int EQ = 16;
#pragma unroll
    for (int q0 = 0; q0 < NQ; q0 += EQ) {
        if ((e0 + q0) * kWave < n) {
            int32_t idx[EQ];
            int slot[EQ];
#pragma unroll
            for (int e = 0; e < EQ; ++e)  // (past n: an unused entry)
                idx[e] = (q0 + e < NQ) ? list[(e0 + q0 + e) * kWave + lane] : -1;
            if (!partial) {
#pragma unroll
                for (int e = 0; e < EQ; ++e) {
                    const int q = q0 + e;
                    slot[e] = -1;
                    if (q >= NQ)
                        continue;
                    const bool in = valid(q) && (every || key[q] > thr);
                    const uint64_t min_ = ballot(in);
                    slot[e] = in ? emitted + prefix_count(min_) : -1;
                    emitted += __popcll(min_);
                }
            } else {
#pragma unroll
                for (int e = 0; e < EQ; ++e) {
                    const int q = q0 + e;
                    slot[e] = -1;
                    if (q >= NQ)
                        continue;
                    const bool v = valid(q);
                    const bool eq = v && key[q] == c.keq;
                    const uint64_t meq = ballot(eq);
                    const int er = eqseen + prefix_count(meq);
                    const bool in = v && (key[q] > thr || (eq && er < c.req));
                    const uint64_t min_ = ballot(in);
                    slot[e] = in ? emitted + prefix_count(min_) : -1;
                    emitted += __popcll(min_);
                    eqseen += __popcll(meq);
                }
            }
#pragma unroll
            for (int e = 0; e < EQ; ++e)
                if (q0 + e < NQ && slot[e] >= 0 && slot[e] < sel) {
                    oidx[slot[e]] = idx[e];
                    if (osc)
                        osc[slot[e]] = key_score(key[q0 + e < NQ ? q0 + e : 0]);
                }
        }
    }
    if (hv == 1)
        for (int x = emitted + lane; x < sel; x += kWave) {
            oidx[x] = -1;
            if (osc)
                osc[x] = -__builtin_inff();
        }
}

// Group j of the launch (request j % B, its (j / B)-th longest group), with
// lists of at most CAP candidates.
template <int H, int D, int CAP>
__device__ __forceinline__ void refine_group(const RefineLdsParams &p, int64_t j)
{
    using S = Shape<H, D>;
    constexpr int MB = S::MB, KS = S::KS, ROWB = S::ROWB, CHUNKS = S::CHUNKS;
    constexpr int KB = KS > 4 ? KS / 2 : KS;     // B fragments read per half tile
    constexpr int STAGE_BYTES = kRefStage * ROWB;
    constexpr int LPW = STAGE_BYTES / 1024 / kRefWaves;  // 1 KiB gathers per wave per stage
    static_assert(LPW >= 1 && STAGE_BYTES % (1024 * kRefWaves) == 0, "stage split over the waves");
    constexpr int RPL = 1024 / ROWB;              // key rows per 1 KiB gather

    // two stage buffers; after the last stage the same bytes hold one level
    // histogram and the exchange words per member
    constexpr int SELB = kRefMembers * (kBins1 + kRefXch) * 4;
    constexpr int KBUF = (2 * STAGE_BYTES > SELB) ? 2 * STAGE_BYTES : SELB;
    __shared__ __align__(1024) unsigned char kbuf[KBUF];
    __shared__ __align__(16) int32_t lst[CAP];
    __shared__ __align__(16) float rows[kRefMembers][CAP];

    const int bi = (int)(j % p.B);
    const Req rq = request_of(p.req, bi, p.L, p.q_len, p.g, p.m0);
    const int64_t m = rq.G - 1 - j / p.B;  // longest groups first
    if (m < rq.m0)
        return;  // (the whole workgroup) a guarded group, or none: nothing to do
    // (an opaque copy of the thread index, so that what the loop over groups
    // could hoist out of this body is recomputed per group instead of held in
    // registers through the selection)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wave = uniform(tid / kWave);
    const int lane = tid % kWave;
    const int half = lane >> 5;
    const int col = lane & 31;
    const int mem = wave % kRefMembers;
    const int hv = wave / kRefMembers;

    const int64_t off = rq.L - rq.q_len;
    const int64_t r0 = m * p.g;
    const int64_t r1 = (r0 + p.g < rq.q_len) ? r0 + p.g : rq.q_len;
    const int nmem = (int)(r1 - r0);
    const int64_t t_last = off + r1 - 1;
    // the group's list: its first min(c, t_last + 1) entries, or cand_n[g]
    // of them (key-chunk lists); at least one either way (c >= k >= 1, and a
    // key-chunk list holds a selected chunk or the keys after the last one),
    // which the clamped gather index below relies on
    const int ncand = p.cand_n ? p.cand_n[rq.g_off + m] : (int)((p.c < t_last + 1) ? p.c : t_last + 1);
    const int32_t *clist = p.cand + (rq.g_off + m) * p.c;
    const unsigned char *Kb = reinterpret_cast<const unsigned char *>(p.K + rq.key_off * D);
    // the candidate list (eight entries per thread at most) and the member's
    // query and weights are loaded together, then the list goes to LDS
    constexpr int NT = kRefWaves * kWave;
    constexpr int LPT = CAP / NT;
    int32_t lv[LPT];
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
        const int x = tid + i * NT;
        lv[i] = (x < ncand) ? clist[x] : 0;
    }

    const bool live = mem < nmem;
    const int64_t row = rq.q_off + r0 + (live ? mem : 0);
    const unsigned char *qrow = reinterpret_cast<const unsigned char *>(p.Q + row * H * D);
    const float *wrow = p.W + row * H;

    // the member's query rows go through LDS (the member's score row, unused
    // until the first stage's scores): the member's two waves load them with
    // contiguous 16-byte loads (a fragment-order load would touch a different
    // row, so a different cache line, in every lane), each row's chunks
    // XOR-swizzled by the row so that the fragment reads spread over the banks
    constexpr int QCH = H * CHUNKS;  // 16-byte chunks of one member's query
    constexpr int QPL = (QCH + kRefHalves * kWave - 1) / (kRefHalves * kWave);
    unsigned char *qst = reinterpret_cast<unsigned char *>(rows[mem]);
    u32x4 qv[QPL];
#pragma unroll
    for (int i = 0; i < QPL; ++i) {
        const int ch = (i * kRefHalves + hv) * kWave + lane;
        qv[i] = u32x4{0u, 0u, 0u, 0u};
        if (live && ch < QCH)
            qv[i] = *reinterpret_cast<const u32x4 *>(qrow + ch * 16);
    }
    // weights per accumulator row (zero for an absent member)
    float wv[MB][16];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int hr = mb * 32 + 8 * r4 + 4 * half;  // rows hr .. hr + 3
            if constexpr (H % 32 == 0) {
                const float4 w4 = live ? *reinterpret_cast<const float4 *>(wrow + hr) : float4{0.f, 0.f, 0.f, 0.f};
                wv[mb][4 * r4 + 0] = w4.x;
                wv[mb][4 * r4 + 1] = w4.y;
                wv[mb][4 * r4 + 2] = w4.z;
                wv[mb][4 * r4 + 3] = w4.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    wv[mb][4 * r4 + e] = (live && hr + e < H) ? wrow[hr + e] : 0.f;
            }
        }
#pragma unroll
    for (int i = 0; i < QPL; ++i) {
        const int ch = (i * kRefHalves + hv) * kWave + lane;
        const int hr = ch / CHUNKS;
        if (ch < QCH)
            *reinterpret_cast<u32x4 *>(qst + hr * ROWB + (((ch % CHUNKS) ^ (hr & (CHUNKS - 1))) * 16)) = qv[i];
    }
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
        const int x = tid + i * NT;
        if (x < ncand)
            lst[x] = lv[i];
    }
    __syncthreads();

    // the member's query as A fragments (scan.hip's chunk order: lane (col,
    // half) holds head col's chunks half * KS .. half * KS + KS - 1)
    bf16x8 qa[MB][KS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int head = mb * 32 + col;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (head < H)
                v = *reinterpret_cast<const u32x4 *>(qst + head * ROWB +
                                                     ((((half * KS + ks)) ^ (head & (CHUNKS - 1))) * 16));
            qa[mb][ks] = __builtin_bit_cast(bf16x8, v);
        }
    }
    // lane-constant LDS offsets of this lane's B-fragment chunks in a stage
    uint32_t koff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        koff[ks] = (uint32_t)(col * ROWB + (((half * KS + ks) ^ (col & (CHUNKS - 1))) * 16));

    // gather slot u of this wave: key row n = (wave * LPW + u) * RPL + lane /
    // (ROWB / 16) of the stage, 16-byte chunk lane % (ROWB / 16); it lands in
    // LDS at the XOR-swizzled chunk of that row
    const int nst = (ncand + kRefStage - 1) / kRefStage;
    u32x4 ring[kRefRing][LPW];
    auto gather = [&](int t, u32x4 (&g)[LPW]) {
#pragma unroll
        for (int u = 0; u < LPW; ++u) {
            const int n = (wave * LPW + u) * RPL + lane / CHUNKS;
            // past the list: a clamped entry of it (loaded, never used), so
            // that the load needs no branch
            const int x = min(t * kRefStage + n, ncand - 1);
            const int key = lst[x];
            g[u] = *reinterpret_cast<const u32x4 *>(Kb + (int64_t)key * ROWB + (lane % CHUNKS) * 16);
        }
    };
    auto put = [&](unsigned char *kb, const u32x4 (&g)[LPW]) {
#pragma unroll
        for (int u = 0; u < LPW; ++u) {
            const int n = (wave * LPW + u) * RPL + lane / CHUNKS;
            const int c = (lane % CHUNKS) ^ (n & (CHUNKS - 1));
            *reinterpret_cast<u32x4 *>(kb + n * ROWB + c * 16) = g[u];
        }
    };
    auto mfma_tile = [&](const unsigned char *kb, int nt, f32x16 (&acc)[MB]) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            acc[mb] = f32x16{};
#pragma unroll
        for (int k0 = 0; k0 < KS; k0 += KB) {
            bf16x8 kf[KB];
#pragma unroll
            for (int ks = 0; ks < KB; ++ks)
                kf[ks] = __builtin_bit_cast(bf16x8,
                                            *reinterpret_cast<const u32x4 *>(kb + koff[k0 + ks] + nt * 32 * ROWB));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < KB; ++ks)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][k0 + ks], kf[ks], acc[mb], 0, 0, 0);
        }
    };
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
    // the wave's two tiles of stage t: their 64 scores (lane l holds key
    // t*128 + 64*hv + l) into the member's row. The MFMAs of tile 0 of stage
    // t run next to the epilogue of tile 1 of stage t - 1 (kept in accB across
    // the barrier), and the MFMAs of tile 1 next to the epilogue of tile 0.
    float *myrow = rows[mem];
    f32x16 accA[MB], accB[MB];
    float s0 = 0.f;  // tile 0's lane partials of the stage being finished
    auto interleave = [&]() {
#pragma unroll
        for (int q = 0; q < KS * MB; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
    };
    auto store_pair = [&](int t, float a, float b) {
        const float total = half_wave_sum2(a, b) + 0.0f;
        const int x = t * kRefStage + 64 * hv + lane;
        if (x < ncand)
            myrow[x] = total;
    };
    auto compute = [&](const unsigned char *kb, int t) {
        if (!live)
            return;
        wave_priority(1);
        mfma_tile(kb, 2 * hv, accA);
        if (t > 0) {
            const float s1 = epilogue(accB);
            interleave();
            store_pair(t - 1, s0, s1);
        }
        wave_priority(0);
        mfma_tile(kb, 2 * hv + 1, accB);
        s0 = epilogue(accA);
        interleave();
    };

    // stages: t's keys (gathered two stages ago) into LDS buffer t % 2, the
    // gather of stage t + 2 into the freed registers, one barrier, then the
    // MFMAs. Two stages per trip, so that buffers and ring slots are
    // compile-time, and an even number of stages (a last stage past the list
    // stores nothing): with no exit between the two halves, the wait for a
    // ring slot leaves the other slot's loads in flight.
    const int nst2 = (nst + 1) & ~1;
#pragma unroll
    for (int s = 0; s < kRefRing; ++s)
        gather(s, ring[s]);
    for (int t = 0; t < nst2; t += 2) {
        put(kbuf, ring[0]);
        gather(t + 2, ring[0]);
        __syncthreads();
        compute(kbuf, t);
        put(kbuf + STAGE_BYTES, ring[1]);
        gather(t + 3, ring[1]);
        __syncthreads();
        compute(kbuf + STAGE_BYTES, t + 1);
    }
    if (live)
        store_pair(nst2 - 1, s0, epilogue(accB));
    __syncthreads();

    // selection: both waves of each member over its causal candidates, a
    // prefix of the ascending list (at most the last nmem - 1 entries lie
    // after the member's position); the stage buffers become the members'
    // histograms and exchange words
    const int pos = (int)(off + r0 + mem);
    int ncaus = live ? ncand : 0;
    while (ncaus > 0 && lst[ncaus - 1] > pos)
        --ncaus;
    uint32_t *h = reinterpret_cast<uint32_t *>(kbuf) + mem * kBins1;
    uint32_t *xch = reinterpret_cast<uint32_t *>(kbuf) + kRefMembers * kBins1 + mem * kRefXch;
    int32_t *oidx = p.out_idx + row * p.k;
    float *osc = p.out_score ? p.out_score + row * p.k : nullptr;
    member_select<CAP / kWave / kRefHalves>(myrow, lst, ncaus, p.k, h, xch, hv, live, oidx, osc);
}

// Persistent workgroups: each takes groups j = blockIdx.x, + gridDim.x, ...;
// the barrier between two groups keeps the next group's list and stage
// writes behind the last selection's reads.
template <int H, int D, int CAP>
__global__ __launch_bounds__(kRefWaves * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void refine_lds_kernel(RefineLdsParams p)
{
    // workgroups are dealt to the 8 XCDs round-robin; let the ones of one XCD
    // take consecutive groups (neighbouring groups share most candidates)
    const int G8 = gridDim.x / 8;
    const int64_t b = (gridDim.x % 8 == 0) ? (int64_t)(blockIdx.x % 8) * G8 + blockIdx.x / 8 : blockIdx.x;
    for (int64_t j = b; j < p.nwork; j += gridDim.x) {
        refine_group<H, D, CAP>(p, j);
        __syncthreads();
    }
}

template <int H, int D>
static void launch_refine_lds_t(const RefineLdsParams &prm, int grid, hipStream_t stream)
{
    const dim3 block(kRefWaves * kWave);
    if (prm.c <= kRefCapSmall)
        hipLaunchKernelGGL((refine_lds_kernel<H, D, kRefCapSmall>), dim3((unsigned)grid), block, 0, stream, prm);
    else
        hipLaunchKernelGGL((refine_lds_kernel<H, D, kRefineLdsCandMax>), dim3((unsigned)grid), block, 0, stream,
                           prm);
}

hipError_t launch_refine_lds(int H, int D, const RefineLdsParams &prm, int grid, hipStream_t stream)
{
    if (prm.g > kRefMembers || prm.c > kRefineLdsCandMax || prm.nwork < 1 || grid < 1)
        return hipErrorInvalidValue;
    if (H == 64 && D == 128)
        launch_refine_lds_t<64, 128>(prm, grid, stream);
    else if (H == 4 && D == 32)
        launch_refine_lds_t<4, 32>(prm, grid, stream);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace dsaidx
