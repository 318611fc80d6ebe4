// abi.cpp - the C entry points of dsaidx.h: argument validation, workspace
// layout and the choice between the two kernel families.
//
//  - many rows (prefill): fused scan+select kernels (scan.hip), persistent
//    workgroups, one candidate buffer per (workgroup, wave) in the workspace;
//  - few rows (decode): split-key scoring into per-row score vectors, then a
//    per-row exact select (split.hip).
// PIVOT runs pool -> proxy scan (top-c and/or top-k) -> Refine on the
// candidates, each stage picking its family from its own row count.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cstdio>
#include <string>

#include "../../include/dsaidx.h"
#include "kernels.h"

using namespace dsaidx;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...)
{
    char msg[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, sizeof msg, fmt, ap);
    va_end(ap);
    g_last_error = msg;
    return status;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(DSAIDX_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Rows per batch item at or below which a stage uses the split-key kernels.
constexpr int64_t kSplitRowsMax = 64;
// Persistent workgroups of the scan kernels: at most as many as fit at once
// on the 256 CUs of an MI355X (LDS decides: one 8-wave or two 4-wave
// workgroups per CU); the workspace holds one set of row buffers per slot.
constexpr int64_t kCus = 256;
constexpr size_t kLdsPerCu = 160 * 1024;
constexpr int64_t kMaxSel = 1 << 20;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Score rows of the split-key path are padded to a multiple of 64 floats.
int64_t score_row(int64_t n) { return ceil_div(n, 64) * 64; }

bool supported(int H, int D) { return (H == 64 && D == 128) || (H == 4 && D == 32); }

// Entries per row buffer. A row admits about sel * (1 + ln(n / sel)) keys
// while its threshold rises (plus the width of a histogram bin), so a buffer
// of 16 sel entries is compacted only on adversarial inputs; it never needs
// more than the row's keys plus one stage.
int scan_cap(int64_t sel, int64_t L)
{
    int64_t cap = std::max<int64_t>(16 * sel, sel + 4096);
    cap = std::min<int64_t>(cap, L + 128);
    cap = std::max<int64_t>(cap, sel + 128);
    return (int)ceil_div(cap, 64) * 64;
}

int num_cus()
{
    static thread_local int cached_dev = -1;
    static thread_local int cached_cus = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    if (dev != cached_dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cached_dev = dev;
        cached_cus = cus;
    }
    return cached_cus;
}

int64_t scan_slots(int H, int D, int NW)
{
    const size_t lds = scan_lds_bytes(H, D, NW);
    return kCus * std::max<int64_t>(1, (int64_t)(kLdsPerCu / lds));
}

int scan_grid(int H, int D, int NW, int64_t nblocks)
{
    const size_t lds = scan_lds_bytes(H, D, NW);
    const int per_cu = std::max<int>(1, (int)(kLdsPerCu / lds));
    int64_t grid = (int64_t)std::max(1, num_cus()) * per_cu;
    grid = std::min<int64_t>(grid, scan_slots(H, D, NW));
    grid = std::min<int64_t>(grid, nblocks);
    return (int)std::max<int64_t>(grid, 1);
}

// Workspace layout of one call.
struct Plan {
    int mode;
    int64_t G;
    bool split_scan, split_refine;
    int nw_scan, nw_refine;
    int cap_scan, cap_refine;
    int sel, sel2;
    size_t off_proxy_q, off_proxy_w, off_cand, off_slots, off_scores, total;
};

// Fills `pl`; returns DSAIDX_OK or an error status (message set).
int make_plan(int mode, int B, int64_t L, int64_t q_len, int H, int D, int64_t g, int64_t c,
              int64_t k, bool have_cand, Plan &pl)
{
    if (B < 1 || B > 65535)
        return fail(DSAIDX_EINVAL, "B=%d must be in [1, 65535]", B);
    if (L < 1 || L >= (int64_t)INT32_MAX)
        return fail(DSAIDX_EINVAL, "L=%lld must be in [1, 2^31-1)", (long long)L);
    if (q_len < 1 || q_len > L)
        return fail(DSAIDX_EINVAL, "q_len=%lld must be in [1, L=%lld]", (long long)q_len, (long long)L);
    if (k < 1 || k > kMaxSel)
        return fail(DSAIDX_EINVAL, "k=%lld must be in [1, 2^20]", (long long)k);
    if (!supported(H, D))
        return fail(DSAIDX_EUNSUPPORTED, "(H_I, d_I) = (%d, %d) has no kernel; supported: (64, 128), (4, 32)", H, D);
    pl = Plan{};
    pl.mode = mode;
    size_t off = 0;
    if (mode == DSAIDX_DENSE) {
        pl.split_scan = q_len <= kSplitRowsMax;
        pl.sel = (int)k;
        pl.sel2 = 0;
        pl.nw_scan = 8;
        pl.cap_scan = scan_cap(k, L);
        if (pl.split_scan) {
            pl.off_scores = off;
            off += align_up((size_t)B * q_len * score_row(L) * sizeof(float));
        } else {
            pl.off_slots = off;
            off += align_up((size_t)scan_slots(H, D, pl.nw_scan) * pl.nw_scan * pl.cap_scan * sizeof(Entry));
        }
        pl.total = off;
        return DSAIDX_OK;
    }
    if (g < 1)
        return fail(DSAIDX_EINVAL, "g=%lld must be >= 1", (long long)g);
    const bool need_c = (mode == DSAIDX_REFINE) || have_cand;
    if (need_c && (c < k || c > kMaxSel))
        return fail(DSAIDX_EINVAL, "c=%lld must be in [k=%lld, 2^20]", (long long)c, (long long)k);
    pl.G = ceil_div(q_len, g);
    pl.split_scan = pl.G <= kSplitRowsMax;
    pl.nw_scan = 8;
    if (mode == DSAIDX_REUSE) {
        pl.sel = (int)(have_cand ? c : k);
        pl.sel2 = have_cand ? (int)k : 0;
    } else {
        pl.sel = (int)c;
        pl.sel2 = 0;
    }
    pl.cap_scan = scan_cap(pl.sel, L);
    pl.off_proxy_q = off;
    off += align_up((size_t)B * pl.G * H * D * sizeof(uint16_t));
    pl.off_proxy_w = off;
    off += align_up((size_t)B * pl.G * H * sizeof(float));
    if (mode == DSAIDX_REFINE && !have_cand) {
        pl.off_cand = off;
        off += align_up((size_t)B * pl.G * c * sizeof(int32_t));
    }
    // scan stage
    size_t scan_bytes = pl.split_scan
        ? (size_t)B * pl.G * score_row(L) * sizeof(float)
        : (size_t)scan_slots(H, D, pl.nw_scan) * pl.nw_scan * pl.cap_scan * sizeof(Entry);
    size_t refine_bytes = 0;
    if (mode == DSAIDX_REFINE) {
        pl.split_refine = q_len <= kSplitRowsMax;
        pl.nw_refine = g <= 4 ? 4 : 8;
        pl.cap_refine = (int)ceil_div(c + 128, 64) * 64;
        refine_bytes = pl.split_refine
            ? (size_t)B * q_len * score_row(c) * sizeof(float)
            : (size_t)scan_slots(H, D, pl.nw_refine) * pl.nw_refine * pl.cap_refine * sizeof(Entry);
    }
    // the scan's buffers/scores and Refine's are used one after the other
    pl.off_slots = off;
    pl.off_scores = off;
    off += align_up(std::max(scan_bytes, refine_bytes));
    pl.total = off;
    return DSAIDX_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_ptrs(const void *Q, const float *W, const void *K, const int32_t *out_idx, const float *out_score,
               const int32_t *out_cand, const void *ws, size_t need)
{
    if (!Q || !W || !K || !out_idx)
        return fail(DSAIDX_EINVAL, "Q, W, K and out_idx must not be NULL");
    if (!aligned(Q, 16) || !aligned(K, 16))
        return fail(DSAIDX_EINVAL, "Q and K must be 16-byte aligned");
    if (!aligned(W, 4) || !aligned(out_idx, 4) || (out_score && !aligned(out_score, 4)) ||
        (out_cand && !aligned(out_cand, 4)))
        return fail(DSAIDX_EINVAL, "W and the outputs must be 4-byte aligned");
    if (need > 0 && !ws)
        return fail(DSAIDX_EINVAL, "ws must not be NULL (%zu bytes needed)", need);
    if (ws && !aligned(ws, 16))
        return fail(DSAIDX_EINVAL, "ws must be 16-byte aligned");
    return DSAIDX_OK;
}

// Positions per workgroup of split_score_kernel: one round of workgroups (one
// per CU, four waves each) covers all rows, each wave a contiguous span of at
// least 128 positions (to amortise loading its query row); a span that reads
// a candidate list is capped by the list's LDS buffer.
int64_t split_chunk(int64_t rows_total, int64_t npos, bool list)
{
    const int64_t waves = (int64_t)std::max(1, num_cus()) * kSplitWaves;
    int64_t per_wave = ceil_div(ceil_div(rows_total * npos, waves), 32) * 32;
    per_wave = std::max<int64_t>(per_wave, 128);
    if (list)
        per_wave = std::min<int64_t>(per_wave, kSplitSpanMax);
    return per_wave * kSplitWaves;
}

// Score + select `nrows` rows per batch item with the split-key kernels.
int run_split(int mode, const uint16_t *Q, const float *W, const uint16_t *K, const int32_t *cand, int B,
              int64_t L, int64_t q_len, int64_t g, int64_t c, int64_t G, int64_t nrows, int64_t rowlen,
              int H, int D, int sel, int sel2, int32_t *o1, float *s1, int o1_members, int32_t *o2, float *s2,
              float *scores, hipStream_t stream)
{
    SplitScoreParams sp{};
    sp.Q = Q;
    sp.W = W;
    sp.K = K;
    sp.cand = cand;
    sp.mode = mode;
    sp.B = B;
    sp.L = L;
    sp.q_len = q_len;
    sp.g = g;
    sp.c = c;
    sp.G = G;
    sp.nrows = nrows;
    sp.rowlen = rowlen;
    const int64_t npos_max = (mode == kRefine) ? std::min<int64_t>(c, L) : L;
    sp.chunk = split_chunk((int64_t)B * nrows, npos_max, mode == kRefine);
    sp.scores = scores;
    dim3 grid((unsigned)ceil_div(npos_max, sp.chunk), (unsigned)nrows, (unsigned)B);
    hipError_t e = launch_split_score(H, D, sp, grid, stream);
    if (e != hipSuccess)
        return hip_fail(e, "split score launch");
    SplitSelectParams ss{};
    ss.scores = scores;
    ss.cand = cand;
    ss.mode = mode;
    ss.B = B;
    ss.L = L;
    ss.q_len = q_len;
    ss.g = g;
    ss.c = c;
    ss.G = G;
    ss.nrows = nrows;
    ss.rowlen = rowlen;
    ss.sel = sel;
    ss.sel2 = sel2;
    ss.o1_idx = o1;
    ss.o1_score = s1;
    ss.o1_members = o1_members;
    ss.o2_idx = o2;
    ss.o2_score = s2;
    e = launch_split_select(ss, stream);
    if (e != hipSuccess)
        return hip_fail(e, "split select launch");
    return DSAIDX_OK;
}

ScanParams scan_base(const uint16_t *Q, const float *W, const uint16_t *K, int B, int64_t L, int64_t q_len,
                     int64_t g, int64_t c, int64_t G)
{
    ScanParams p{};
    p.Q = Q;
    p.W = W;
    p.K = K;
    p.B = B;
    p.L = L;
    p.q_len = q_len;
    p.g = g;
    p.c = c;
    p.G = G;
    return p;
}

int run_pivot(int mode, const void *Qv, const float *W, const void *Kv, int B, int64_t L, int64_t q_len,
              int H, int D, int64_t g, int64_t c, int64_t k, int32_t *out_idx, float *out_score,
              int32_t *out_cand, void *ws, size_t ws_bytes, hipStream_t stream)
{
    Plan pl;
    int s = make_plan(mode, B, L, q_len, H, D, g, c, k, out_cand != nullptr, pl);
    if (s != DSAIDX_OK)
        return s;
    s = check_ptrs(Qv, W, Kv, out_idx, out_score, out_cand, ws, pl.total);
    if (s != DSAIDX_OK)
        return s;
    if (ws_bytes < pl.total)
        return fail(DSAIDX_EWORKSPACE, "workspace of %zu bytes is below the %zu needed", ws_bytes, pl.total);
    const uint16_t *Q = static_cast<const uint16_t *>(Qv);
    const uint16_t *K = static_cast<const uint16_t *>(Kv);
    unsigned char *wsb = static_cast<unsigned char *>(ws);
    uint16_t *Qp = reinterpret_cast<uint16_t *>(wsb + pl.off_proxy_q);
    float *Wp = reinterpret_cast<float *>(wsb + pl.off_proxy_w);
    const int64_t G = pl.G;

    // 1. proxies
    PoolParams pp{};
    pp.Q = Q;
    pp.W = W;
    pp.B = B;
    pp.q_len = q_len;
    pp.g = g;
    pp.G = G;
    pp.Qp = Qp;
    pp.Wp = Wp;
    hipError_t e = launch_pool(H, D, pp, stream);
    if (e != hipSuccess)
        return hip_fail(e, "pool launch");

    // 2. proxy scan: outputs per mode
    int32_t *cand = out_cand;
    if (mode == DSAIDX_REFINE && !cand)
        cand = reinterpret_cast<int32_t *>(wsb + pl.off_cand);
    int32_t *o1;
    float *s1;
    int o1_members;
    int32_t *o2 = nullptr;
    float *s2 = nullptr;
    if (mode == DSAIDX_REUSE && !out_cand) {
        o1 = out_idx;
        s1 = out_score;
        o1_members = 1;
    } else {
        o1 = cand;
        s1 = nullptr;
        o1_members = 0;
        if (mode == DSAIDX_REUSE) {
            o2 = out_idx;
            s2 = out_score;
        }
    }
    if (pl.split_scan) {
        s = run_split(kProxy, Qp, Wp, K, nullptr, B, L, q_len, g, c, G, G, score_row(L), H, D, pl.sel, pl.sel2, o1, s1,
                      o1_members, o2, s2, reinterpret_cast<float *>(wsb + pl.off_scores), stream);
        if (s != DSAIDX_OK)
            return s;
    } else {
        ScanParams p = scan_base(Qp, Wp, K, B, L, q_len, g, c, G);
        p.nblk_per_batch = ceil_div(G, pl.nw_scan);
        p.nblocks = p.nblk_per_batch * B;
        p.sel = pl.sel;
        p.sel2 = pl.sel2;
        p.o1_idx = o1;
        p.o1_score = s1;
        p.o1_members = o1_members;
        p.o2_idx = o2;
        p.o2_score = s2;
        p.slots = reinterpret_cast<Entry *>(wsb + pl.off_slots);
        p.cap = pl.cap_scan;
        e = launch_scan_select(H, D, pl.nw_scan, kProxy, p, scan_grid(H, D, pl.nw_scan, p.nblocks), stream);
        if (e != hipSuccess)
            return hip_fail(e, "proxy scan launch");
    }
    if (mode == DSAIDX_REUSE)
        return DSAIDX_OK;

    // 3. Refine on the candidates
    if (pl.split_refine) {
        return run_split(kRefine, Q, W, K, cand, B, L, q_len, g, c, G, q_len, score_row(c), H, D, (int)k, 0, out_idx,
                         out_score, 0, nullptr, nullptr, reinterpret_cast<float *>(wsb + pl.off_scores), stream);
    }
    ScanParams p = scan_base(Q, W, K, B, L, q_len, g, c, G);
    p.cand = cand;
    p.member_chunks = ceil_div(g, pl.nw_refine);
    p.nblocks = (int64_t)B * G * p.member_chunks;
    p.sel = (int)k;
    p.sel2 = 0;
    p.o1_idx = out_idx;
    p.o1_score = out_score;
    p.slots = reinterpret_cast<Entry *>(wsb + pl.off_slots);
    p.cap = pl.cap_refine;
    e = launch_scan_select(H, D, pl.nw_refine, kRefine, p, scan_grid(H, D, pl.nw_refine, p.nblocks), stream);
    if (e != hipSuccess)
        return hip_fail(e, "refine launch");
    return DSAIDX_OK;
}

}  // namespace

extern "C" {

size_t indexer_workspace_bytes(int mode, int B, int64_t L, int64_t q_len, int H_I, int d_I, int g, int c, int k)
{
    if (mode != DSAIDX_DENSE && mode != DSAIDX_REUSE && mode != DSAIDX_REFINE) {
        fail(DSAIDX_EINVAL, "unknown mode %d", mode);
        return 0;
    }
    Plan pl;
    // For Reuse the candidate output may or may not be requested; size for both.
    const bool have_cand = mode == DSAIDX_REUSE && c >= k;
    if (make_plan(mode, B, L, q_len, H_I, d_I, g, c, k, have_cand, pl) != DSAIDX_OK)
        return 0;
    size_t total = pl.total;
    if (mode == DSAIDX_REUSE) {
        Plan p2;
        if (make_plan(mode, B, L, q_len, H_I, d_I, g, c, k, false, p2) == DSAIDX_OK)
            total = std::max(total, p2.total);
    }
    return total;
}

int indexer_dense(const void *Qv, const float *W, const void *Kv, int B, int64_t L, int64_t q_len, int H_I,
                  int d_I, int k, int32_t *out_idx, float *out_score, void *ws, size_t ws_bytes,
                  hipStream_t stream)
{
    Plan pl;
    int s = make_plan(DSAIDX_DENSE, B, L, q_len, H_I, d_I, 1, 0, k, false, pl);
    if (s != DSAIDX_OK)
        return s;
    s = check_ptrs(Qv, W, Kv, out_idx, out_score, nullptr, ws, pl.total);
    if (s != DSAIDX_OK)
        return s;
    if (ws_bytes < pl.total)
        return fail(DSAIDX_EWORKSPACE, "workspace of %zu bytes is below the %zu needed", ws_bytes, pl.total);
    const uint16_t *Q = static_cast<const uint16_t *>(Qv);
    const uint16_t *K = static_cast<const uint16_t *>(Kv);
    unsigned char *wsb = static_cast<unsigned char *>(ws);
    if (pl.split_scan) {
        return run_split(kDense, Q, W, K, nullptr, B, L, q_len, 1, 0, q_len, q_len, score_row(L), H_I, d_I, k, 0, out_idx,
                         out_score, 0, nullptr, nullptr, reinterpret_cast<float *>(wsb + pl.off_scores), stream);
    }
    ScanParams p = scan_base(Q, W, K, B, L, q_len, 1, 0, q_len);
    p.nblk_per_batch = ceil_div(q_len, pl.nw_scan);
    p.nblocks = p.nblk_per_batch * B;
    p.sel = k;
    p.sel2 = 0;
    p.o1_idx = out_idx;
    p.o1_score = out_score;
    p.slots = reinterpret_cast<Entry *>(wsb + pl.off_slots);
    p.cap = pl.cap_scan;
    hipError_t e = launch_scan_select(H_I, d_I, pl.nw_scan, kDense, p,
                                      scan_grid(H_I, d_I, pl.nw_scan, p.nblocks), stream);
    if (e != hipSuccess)
        return hip_fail(e, "dense scan launch");
    return DSAIDX_OK;
}

int indexer_pivot_reuse(const void *Q, const float *W, const void *K, int B, int64_t L, int64_t q_len, int H_I,
                        int d_I, int g, int c, int k, int32_t *out_idx, float *out_score, int32_t *out_cand,
                        void *ws, size_t ws_bytes, hipStream_t stream)
{
    return run_pivot(DSAIDX_REUSE, Q, W, K, B, L, q_len, H_I, d_I, g, c, k, out_idx, out_score, out_cand, ws,
                     ws_bytes, stream);
}

int indexer_pivot_refine(const void *Q, const float *W, const void *K, int B, int64_t L, int64_t q_len, int H_I,
                         int d_I, int g, int c, int k, int32_t *out_idx, float *out_score, int32_t *out_cand,
                         void *ws, size_t ws_bytes, hipStream_t stream)
{
    return run_pivot(DSAIDX_REFINE, Q, W, K, B, L, q_len, H_I, d_I, g, c, k, out_idx, out_score, out_cand, ws,
                     ws_bytes, stream);
}

const char *indexer_last_error(void) { return g_last_error.c_str(); }

const char *indexer_version(void) { return "dsaidx 0.1.0 gfx950"; }

}  // extern "C"
