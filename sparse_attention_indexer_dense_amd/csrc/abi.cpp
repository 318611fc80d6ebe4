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
#include <mutex>
#include <string>
#include <vector>

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
// Rows of one split-score launch (its grid's y dimension).
constexpr int64_t kGridYMax = 65535;
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

// ------------------------------------------------------------------ batches
// A batch of requests: uniform (B requests of L keys and q_len queries, no
// descriptors: the kernels derive each request's geometry) or of variable
// length (per-request descriptors uploaded to the workspace). A request's
// groups never reach into another request. `guard` sends the groups whose
// causal prefix (t_last + 1 keys) is at most guard keys to the dense pass.
struct Batch {
    int B = 0;
    bool varlen = false;
    std::vector<ReqDesc> req;  // varlen only
    int64_t L = 0, q_len = 0;  // uniform values; varlen: the largest request's
    int64_t m0 = 0;            // uniform: guarded groups per request
    int64_t g = 1;
    int proxy = DSAIDX_PROXY_MEAN;
    int64_t window = 0;
    int64_t total_q = 0, total_G = 0, total_keys = 0;
    int64_t max_G = 0;
    int64_t max_dense_rows = 0;    // PIVOT: rows of guarded groups (largest request)
    int64_t max_pivot_groups = 0;  // PIVOT: unguarded groups (largest request)
    int64_t max_refine_rows = 0;   // PIVOT: rows of unguarded groups (largest request)
};

// Groups of a request whose causal prefix holds at most `guard` keys: group m
// ends at position off + min((m + 1) g, q_len) - 1.
int64_t guarded_groups(int64_t L, int64_t q_len, int64_t g, int64_t guard)
{
    const int64_t G = ceil_div(q_len, g);
    if (guard >= L)
        return G;
    const int64_t off = L - q_len;
    if (guard < off + std::min(g, q_len))
        return 0;
    return std::min<int64_t>((guard - off) / g, G - 1);
}

void finish_batch(Batch &b, const int64_t *Ls, const int64_t *qs, int64_t guard)
{
    b.total_q = b.total_G = b.total_keys = 0;
    b.max_G = b.max_dense_rows = b.max_pivot_groups = b.max_refine_rows = 0;
    for (int i = 0; i < b.B; ++i) {
        const int64_t L = Ls ? Ls[i] : b.L, q = qs ? qs[i] : b.q_len;
        const int64_t G = ceil_div(q, b.g);
        const int64_t m0 = guarded_groups(L, q, b.g, guard);
        const int64_t rg = std::min(m0 * b.g, q);
        if (b.varlen) {
            ReqDesc d;
            d.key_off = b.total_keys;
            d.q_off = b.total_q;
            d.g_off = b.total_G;
            d.L = L;
            d.q_len = q;
            d.m0 = m0;
            b.req.push_back(d);
        } else {
            b.m0 = m0;
        }
        b.total_keys += L;
        b.total_q += q;
        b.total_G += G;
        b.max_G = std::max(b.max_G, G);
        b.max_dense_rows = std::max(b.max_dense_rows, rg);
        b.max_pivot_groups = std::max(b.max_pivot_groups, G - m0);
        b.max_refine_rows = std::max(b.max_refine_rows, q - rg);
    }
}

// A request may be empty (q_len = 0, and then L may be 0 as well): it has no
// query rows and contributes nothing.
int check_sizes(int64_t L, int64_t q_len, const char *what, int i)
{
    if (L < 0 || L >= (int64_t)INT32_MAX)
        return fail(DSAIDX_EINVAL, "%s%d: L=%lld must be in [0, 2^31-1)", what, i, (long long)L);
    if (q_len < 0 || q_len > L)
        return fail(DSAIDX_EINVAL, "%s%d: q_len=%lld must be in [0, L=%lld]", what, i, (long long)q_len,
                    (long long)L);
    return DSAIDX_OK;
}

int uniform_batch(int B, int64_t L, int64_t q_len, int64_t g, Batch &b)
{
    if (B < 1 || B > 65535)
        return fail(DSAIDX_EINVAL, "B=%d must be in [1, 65535]", B);
    int s = check_sizes(L, q_len, "request ", 0);
    if (s != DSAIDX_OK)
        return s;
    b = Batch{};
    b.B = B;
    b.L = L;
    b.q_len = q_len;
    b.g = g;
    finish_batch(b, nullptr, nullptr, 0);
    return DSAIDX_OK;
}

int varlen_batch(int B, const int64_t *L, const int64_t *q_len, int64_t g, const dsaidx_pivot_opts *opts, Batch &b)
{
    const int64_t guard = opts ? opts->guard : 0;
    const int proxy = opts ? opts->proxy : DSAIDX_PROXY_MEAN;
    const int64_t window = opts ? opts->window : 0;
    if (proxy != DSAIDX_PROXY_MEAN && proxy != DSAIDX_PROXY_FIRST && proxy != DSAIDX_PROXY_LAST)
        return fail(DSAIDX_EINVAL, "unknown proxy strategy %d", proxy);
    if (window < 0)
        return fail(DSAIDX_EINVAL, "window=%lld must be >= 0", (long long)window);
    if (B < 1 || B > 65535)
        return fail(DSAIDX_EINVAL, "B=%d must be in [1, 65535]", B);
    if (!L || !q_len)
        return fail(DSAIDX_EINVAL, "L and q_len (host arrays of B lengths) must not be NULL");
    if (guard < 0)
        return fail(DSAIDX_EINVAL, "guard=%lld must be >= 0", (long long)guard);
    b = Batch{};
    b.B = B;
    b.varlen = true;
    b.g = g;
    b.proxy = proxy;
    b.window = window;
    for (int i = 0; i < B; ++i) {
        const int s = check_sizes(L[i], q_len[i], "request ", i);
        if (s != DSAIDX_OK)
            return s;
        b.L = std::max(b.L, L[i]);
        b.q_len = std::max(b.q_len, q_len[i]);
    }
    b.req.reserve(B);
    finish_batch(b, L, q_len, guard);
    if (b.total_keys >= ((int64_t)1 << 40) || b.total_q >= ((int64_t)1 << 40))
        return fail(DSAIDX_EINVAL, "batch too large");
    return DSAIDX_OK;
}

// ------------------------------------------------------------------ plans
// Workspace layout of one call. The stages of a call run one after the
// other on the stream, so the scan buffers or score rows of the dense pass,
// the proxy scan and Refine share one region.
struct Plan {
    int mode;
    bool dense_pass, pivot_pass;      // PIVOT: some groups guarded / unguarded
    bool split_dense, split_scan, split_refine;
    bool refine_lds;                  // Refine re-score with the members' scores in LDS (refine.hip)
    int nw_scan, nw_refine;
    int cap_dense, cap_scan, cap_refine;
    int sel, sel2;
    size_t off_desc, off_proxy_q, off_proxy_w, off_cand, off_work, total;
};

int check_common(int H, int D, int64_t k)
{
    if (k < 1 || k > kMaxSel)
        return fail(DSAIDX_EINVAL, "k=%lld must be in [1, 2^20]", (long long)k);
    if (!supported(H, D))
        return fail(DSAIDX_EUNSUPPORTED, "(H_I, d_I) = (%d, %d) has no kernel; supported: (64, 128), (4, 32)", H, D);
    return DSAIDX_OK;
}

size_t scan_bytes(int H, int D, int NW, int cap)
{
    return (size_t)scan_slots(H, D, NW) * NW * cap * sizeof(Entry);
}

// Fills `pl`; returns DSAIDX_OK or an error status (message set).
int make_plan(int mode, const Batch &b, int H, int D, int64_t c, int64_t k, bool have_cand, Plan &pl)
{
    int s = check_common(H, D, k);
    if (s != DSAIDX_OK)
        return s;
    pl = Plan{};
    pl.mode = mode;
    size_t off = 0;
    if (b.varlen) {
        pl.off_desc = off;
        off += align_up((size_t)b.B * sizeof(ReqDesc));
    }
    const int64_t L = b.L;
    pl.nw_scan = 8;
    if (mode == DSAIDX_DENSE) {
        pl.dense_pass = true;
        pl.split_dense = b.q_len <= kSplitRowsMax;
        pl.sel = (int)k;
        pl.cap_dense = scan_cap(k, L);
        pl.off_work = off;
        off += align_up(pl.split_dense ? (size_t)b.B * b.q_len * score_row(L) * sizeof(float)
                                       : scan_bytes(H, D, pl.nw_scan, pl.cap_dense));
        pl.total = off;
        return DSAIDX_OK;
    }
    const int64_t g = b.g;
    if (g < 1)
        return fail(DSAIDX_EINVAL, "g=%lld must be >= 1", (long long)g);
    const bool need_c = (mode == DSAIDX_REFINE) || have_cand;
    if (need_c && (c < k || c > kMaxSel))
        return fail(DSAIDX_EINVAL, "c=%lld must be in [k=%lld, 2^20]", (long long)c, (long long)k);
    pl.dense_pass = b.max_dense_rows > 0;
    pl.pivot_pass = b.max_pivot_groups > 0;
    size_t work = 0;
    if (pl.dense_pass) {
        pl.split_dense = b.max_dense_rows <= kSplitRowsMax;
        pl.cap_dense = scan_cap(k, L);
        work = std::max(work, pl.split_dense ? (size_t)b.B * b.max_dense_rows * score_row(L) * sizeof(float)
                                             : scan_bytes(H, D, pl.nw_scan, pl.cap_dense));
    }
    if (mode == DSAIDX_REUSE) {
        pl.sel = (int)(have_cand ? c : k);
        pl.sel2 = have_cand ? (int)k : 0;
    } else {
        pl.sel = (int)c;
        pl.sel2 = 0;
    }
    if (pl.pivot_pass) {
        pl.split_scan = b.max_pivot_groups <= kSplitRowsMax;
        pl.cap_scan = scan_cap(pl.sel, L);
        pl.off_proxy_q = off;
        off += align_up((size_t)b.total_G * H * D * sizeof(uint16_t));
        pl.off_proxy_w = off;
        off += align_up((size_t)b.total_G * H * sizeof(float));
        if (mode == DSAIDX_REFINE && !have_cand) {
            pl.off_cand = off;
            off += align_up((size_t)b.total_G * c * sizeof(int32_t));
        }
        work = std::max(work, pl.split_scan ? (size_t)b.B * b.max_pivot_groups * score_row(L) * sizeof(float)
                                            : scan_bytes(H, D, pl.nw_scan, pl.cap_scan));
        if (mode == DSAIDX_REFINE) {
            pl.split_refine = b.max_refine_rows <= kSplitRowsMax;
            pl.refine_lds = !pl.split_refine && g <= 4 && c <= kRefineLdsCandMax;
            pl.nw_refine = g <= 4 ? 4 : 8;
            pl.cap_refine = (int)ceil_div(c + 128, 64) * 64;
            if (pl.split_refine)
                work = std::max(work, (size_t)b.B * b.max_refine_rows * score_row(c) * sizeof(float));
            else if (!pl.refine_lds)
                work = std::max(work, scan_bytes(H, D, pl.nw_refine, pl.cap_refine));
        }
    }
    pl.off_work = off;
    off += align_up(work);
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
// per CU, four waves each) covers all rows, each wave at least 128 positions
// (to amortise loading its query row): a contiguous span when it reads a
// candidate list (capped by the list's LDS buffer), else the same number of
// 32-key tiles dealt over the row's waves in turn.
int64_t split_chunk(int64_t rows_total, int64_t npos, bool list)
{
    const int64_t waves = (int64_t)std::max(1, num_cus()) * kSplitWaves;
    int64_t per_wave = ceil_div(ceil_div(rows_total * npos, waves), 32) * 32;
    per_wave = std::max<int64_t>(per_wave, 128);
    if (list)
        per_wave = std::min<int64_t>(per_wave, kSplitSpanMax);
    // spread the row evenly over the workgroups it needs
    const int64_t nchunks = ceil_div(npos, per_wave * kSplitWaves);
    per_wave = ceil_div(ceil_div(ceil_div(npos, nchunks), kSplitWaves), 32) * 32;
    return per_wave * kSplitWaves;
}

// Everything a launch needs to know about the batch and its pass.
struct Pass {
    const Batch *b;
    const ReqDesc *req;  // device descriptors (varlen) or nullptr
    int64_t c;
    int guard_rows;      // dense pass over the rows of guarded groups
    const int32_t *glim = nullptr;    // chunk summaries: last complete chunk per group
    int64_t krows = 0;                // summaries per request
    const int32_t *cand_n = nullptr;  // keys per candidate list
};

// Score + select `nrows` rows per request with the split-key kernels.
int run_split(int mode, const Pass &ps, const uint16_t *Q, const float *W, const uint16_t *K, const int32_t *cand,
              int64_t nrows, int64_t rowlen, int H, int D, int sel, int sel2, int32_t *o1, float *s1,
              int o1_members, int32_t *o2, float *s2, float *scores, hipStream_t stream)
{
    const Batch &b = *ps.b;
    SplitScoreParams sp{};
    sp.Q = Q;
    sp.W = W;
    sp.K = K;
    sp.cand = cand;
    sp.req = ps.req;
    sp.mode = mode;
    sp.B = b.B;
    sp.L = b.L;
    sp.q_len = b.q_len;
    sp.g = (mode == kDense && !ps.guard_rows) ? 1 : b.g;
    sp.c = ps.c;
    sp.G = ceil_div(b.q_len, sp.g);
    sp.m0 = (mode == kDense && !ps.guard_rows) ? 0 : b.m0;
    sp.guard_rows = ps.guard_rows;
    sp.nrows = nrows;
    sp.rowlen = rowlen;
    const int64_t npos_max = (mode == kRefine) ? std::min<int64_t>(ps.c, b.L) : (ps.glim ? ps.krows : b.L);
    // Refine member rows of one group share its candidate list: with an even
    // g each wave scores two of them on every gathered key tile
    const int mr = (mode == kRefine && sp.g % 2 == 0) ? 2 : 1;
    const int64_t nunits = ceil_div(nrows, mr);  // row units per batch item
    sp.chunk = split_chunk((int64_t)b.B * nunits, npos_max, mode == kRefine);
    sp.scores = scores;
    sp.glim = ps.glim;
    sp.krows = ps.krows;
    sp.cand_n = ps.cand_n;
    hipError_t e = hipSuccess;
    for (int64_t r0 = 0; r0 < nrows; r0 += kGridYMax * mr) {
        sp.row0 = r0;
        dim3 grid((unsigned)ceil_div(npos_max, sp.chunk),
                  (unsigned)std::min<int64_t>(kGridYMax, ceil_div(nrows - r0, mr)), (unsigned)b.B);
        e = launch_split_score(H, D, sp, mr, grid, stream);
        if (e != hipSuccess)
            return hip_fail(e, "split score launch");
    }
    SplitSelectParams ss{};
    ss.scores = scores;
    ss.cand = cand;
    ss.req = ps.req;
    ss.mode = mode;
    ss.B = b.B;
    ss.L = b.L;
    ss.q_len = b.q_len;
    ss.g = sp.g;
    ss.c = ps.c;
    ss.G = sp.G;
    ss.m0 = sp.m0;
    ss.guard_rows = ps.guard_rows;
    ss.nrows = nrows;
    ss.rowlen = rowlen;
    ss.sel = sel;
    ss.sel2 = sel2;
    ss.o1_idx = o1;
    ss.o1_score = s1;
    ss.o1_members = o1_members;
    ss.o2_idx = o2;
    ss.o2_score = s2;
    ss.glim = ps.glim;
    ss.cand_n = ps.cand_n;
    e = launch_split_select(ss, stream);
    if (e != hipSuccess)
        return hip_fail(e, "split select launch");
    return DSAIDX_OK;
}

ScanParams scan_base(const Pass &ps, int mode, const uint16_t *Q, const float *W, const uint16_t *K)
{
    const Batch &b = *ps.b;
    ScanParams p{};
    p.Q = Q;
    p.W = W;
    p.K = K;
    p.req = ps.req;
    p.B = b.B;
    p.L = b.L;
    p.q_len = b.q_len;
    p.g = (mode == kDense && !ps.guard_rows) ? 1 : b.g;
    p.c = ps.c;
    p.G = ceil_div(b.q_len, p.g);
    p.m0 = (mode == kDense && !ps.guard_rows) ? 0 : b.m0;
    p.guard_rows = ps.guard_rows;
    p.glim = ps.glim;
    p.krows = ps.krows;
    p.cand_n = ps.cand_n;
    return p;
}

// Dense top-k for the rows of every request (all rows, or those of guarded
// groups), through the split or the scan kernels.
int run_dense(const Plan &pl, const Pass &ps, const uint16_t *Q, const float *W, const uint16_t *K, int H, int D,
              int64_t k, int32_t *out_idx, float *out_score, unsigned char *wsb, hipStream_t stream)
{
    const Batch &b = *ps.b;
    const int64_t rows = ps.guard_rows ? b.max_dense_rows : b.q_len;
    if (pl.split_dense)
        return run_split(kDense, ps, Q, W, K, nullptr, rows, score_row(b.L), H, D, (int)k, 0, out_idx, out_score, 0,
                         nullptr, nullptr, reinterpret_cast<float *>(wsb + pl.off_work), stream);
    ScanParams p = scan_base(ps, kDense, Q, W, K);
    p.nblk_per_batch = ceil_div(rows, pl.nw_scan);
    p.nblocks = p.nblk_per_batch * b.B;
    p.sel = (int)k;
    p.sel2 = 0;
    p.o1_idx = out_idx;
    p.o1_score = out_score;
    p.slots = reinterpret_cast<Entry *>(wsb + pl.off_work);
    p.cap = pl.cap_dense;
    hipError_t e = launch_scan_select(H, D, pl.nw_scan, kDense, p, scan_grid(H, D, pl.nw_scan, p.nblocks), stream);
    if (e != hipSuccess)
        return hip_fail(e, "dense scan launch");
    return DSAIDX_OK;
}

// The request descriptors of a variable-length batch, written to the
// workspace by a small kernel that receives them as launch arguments.
int upload_desc(const Batch &b, ReqDesc *dst, hipStream_t stream)
{
    for (int i0 = 0; i0 < b.B; i0 += kDescChunk) {
        DescChunk ch{};
        ch.n = std::min(kDescChunk, b.B - i0);
        ch.first = i0;
        for (int i = 0; i < ch.n; ++i)
            ch.d[i] = b.req[i0 + i];
        hipError_t e = launch_set_desc(ch, dst, stream);
        if (e != hipSuccess)
            return hip_fail(e, "descriptor launch");
    }
    return DSAIDX_OK;
}

int run_pivot(int mode, const Batch &b, const void *Qv, const float *W, const void *Kv, int H, int D, int64_t c,
              int64_t k, int32_t *out_idx, float *out_score, int32_t *out_cand, void *ws, size_t ws_bytes,
              hipStream_t stream)
{
    Plan pl;
    int s = make_plan(mode, b, H, D, c, k, out_cand != nullptr, pl);
    if (s != DSAIDX_OK)
        return s;
    if (b.total_q == 0)
        return DSAIDX_OK;  // no query rows: nothing to read or write
    s = check_ptrs(Qv, W, Kv, out_idx, out_score, out_cand, ws, pl.total);
    if (s != DSAIDX_OK)
        return s;
    if (ws_bytes < pl.total)
        return fail(DSAIDX_EWORKSPACE, "workspace of %zu bytes is below the %zu needed", ws_bytes, pl.total);
    const uint16_t *Q = static_cast<const uint16_t *>(Qv);
    const uint16_t *K = static_cast<const uint16_t *>(Kv);
    unsigned char *wsb = static_cast<unsigned char *>(ws);
    Pass ps{&b, nullptr, c, 0};
    if (b.varlen) {
        ReqDesc *d = reinterpret_cast<ReqDesc *>(wsb + pl.off_desc);
        s = upload_desc(b, d, stream);
        if (s != DSAIDX_OK)
            return s;
        ps.req = d;
    }
    hipError_t e;

    // 0. guarded groups: dense rows; no candidates
    if (pl.dense_pass) {
        Pass pd = ps;
        pd.guard_rows = 1;
        s = run_dense(pl, pd, Q, W, K, H, D, k, out_idx, out_score, wsb, stream);
        if (s != DSAIDX_OK)
            return s;
        if (out_cand) {
            e = launch_fill_guarded(ps.req, b.B, b.L, b.q_len, b.g, b.m0, b.max_G, c, out_cand, stream);
            if (e != hipSuccess)
                return hip_fail(e, "candidate fill launch");
        }
    }
    if (!pl.pivot_pass)
        return DSAIDX_OK;
    uint16_t *Qp = reinterpret_cast<uint16_t *>(wsb + pl.off_proxy_q);
    float *Wp = reinterpret_cast<float *>(wsb + pl.off_proxy_w);

    // 1. proxies of the unguarded groups
    PoolParams pp{};
    pp.Q = Q;
    pp.W = W;
    pp.req = ps.req;
    pp.B = b.B;
    pp.L = b.L;
    pp.q_len = b.q_len;
    pp.g = b.g;
    pp.m0 = b.m0;
    pp.gmax = b.max_G;
    pp.proxy = b.proxy;
    pp.window = b.window;
    pp.Qp = Qp;
    pp.Wp = Wp;
    e = launch_pool(H, D, pp, stream);
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
        s = run_split(kProxy, ps, Qp, Wp, K, nullptr, b.max_pivot_groups, score_row(b.L), H, D, pl.sel, pl.sel2, o1,
                      s1, o1_members, o2, s2, reinterpret_cast<float *>(wsb + pl.off_work), stream);
        if (s != DSAIDX_OK)
            return s;
    } else {
        ScanParams p = scan_base(ps, kProxy, Qp, Wp, K);
        p.nblk_per_batch = ceil_div(b.max_pivot_groups, pl.nw_scan);
        p.nblocks = p.nblk_per_batch * b.B;
        p.sel = pl.sel;
        p.sel2 = pl.sel2;
        p.o1_idx = o1;
        p.o1_score = s1;
        p.o1_members = o1_members;
        p.o2_idx = o2;
        p.o2_score = s2;
        p.slots = reinterpret_cast<Entry *>(wsb + pl.off_work);
        p.cap = pl.cap_scan;
        e = launch_scan_select(H, D, pl.nw_scan, kProxy, p, scan_grid(H, D, pl.nw_scan, p.nblocks), stream);
        if (e != hipSuccess)
            return hip_fail(e, "proxy scan launch");
    }
    if (mode == DSAIDX_REUSE)
        return DSAIDX_OK;

    // 3. Refine on the candidates
    if (pl.split_refine) {
        return run_split(kRefine, ps, Q, W, K, cand, b.max_refine_rows, score_row(c), H, D, (int)k, 0, out_idx,
                         out_score, 0, nullptr, nullptr, reinterpret_cast<float *>(wsb + pl.off_work), stream);
    }
    if (pl.refine_lds) {
        RefineLdsParams rp{};
        rp.Q = Q;
        rp.W = W;
        rp.K = K;
        rp.cand = cand;
        rp.req = ps.req;
        rp.B = b.B;
        rp.L = b.L;
        rp.q_len = b.q_len;
        rp.g = b.g;
        rp.c = c;
        rp.m0 = b.m0;
        rp.k = (int)k;
        rp.out_idx = out_idx;
        rp.out_score = out_score;
        rp.nwork = (int64_t)b.B * b.max_pivot_groups;
        // one workgroup per CU (the kernel's LDS), each looping over groups
        const int grid = (int)std::min<int64_t>(rp.nwork, std::max(1, num_cus()));
        e = launch_refine_lds(H, D, rp, grid, stream);
        if (e != hipSuccess)
            return hip_fail(e, "refine launch");
        return DSAIDX_OK;
    }
    ScanParams p = scan_base(ps, kRefine, Q, W, K);
    p.cand = cand;
    p.member_chunks = ceil_div(b.g, pl.nw_refine);
    p.nblk_per_batch = b.max_pivot_groups * p.member_chunks;
    p.nblocks = p.nblk_per_batch * b.B;
    p.sel = (int)k;
    p.sel2 = 0;
    p.o1_idx = out_idx;
    p.o1_score = out_score;
    p.slots = reinterpret_cast<Entry *>(wsb + pl.off_work);
    p.cap = pl.cap_refine;
    e = launch_scan_select(H, D, pl.nw_refine, kRefine, p, scan_grid(H, D, pl.nw_refine, p.nblocks), stream);
    if (e != hipSuccess)
        return hip_fail(e, "refine launch");
    return DSAIDX_OK;
}

int run_dense_call(const Batch &b, const void *Qv, const float *W, const void *Kv, int H, int D, int k,
                   int32_t *out_idx, float *out_score, void *ws, size_t ws_bytes, hipStream_t stream)
{
    Plan pl;
    int s = make_plan(DSAIDX_DENSE, b, H, D, 0, k, false, pl);
    if (s != DSAIDX_OK)
        return s;
    if (b.total_q == 0)
        return DSAIDX_OK;  // no query rows: nothing to read or write
    s = check_ptrs(Qv, W, Kv, out_idx, out_score, nullptr, ws, pl.total);
    if (s != DSAIDX_OK)
        return s;
    if (ws_bytes < pl.total)
        return fail(DSAIDX_EWORKSPACE, "workspace of %zu bytes is below the %zu needed", ws_bytes, pl.total);
    unsigned char *wsb = static_cast<unsigned char *>(ws);
    Pass ps{&b, nullptr, 0, 0};
    if (b.varlen) {
        ReqDesc *d = reinterpret_cast<ReqDesc *>(wsb + pl.off_desc);
        s = upload_desc(b, d, stream);
        if (s != DSAIDX_OK)
            return s;
        ps.req = d;
    }
    return run_dense(pl, ps, static_cast<const uint16_t *>(Qv), W, static_cast<const uint16_t *>(Kv), H, D, k,
                     out_idx, out_score, wsb, stream);
}

size_t workspace_for(int mode, const Batch &b, int H, int D, int64_t c, int64_t k)
{
    Plan pl;
    // For Reuse the candidate output may or may not be requested; size for both.
    const bool have_cand = mode == DSAIDX_REUSE && c >= k;
    if (make_plan(mode, b, H, D, c, k, have_cand, pl) != DSAIDX_OK)
        return 0;
    size_t total = pl.total;
    if (mode == DSAIDX_REUSE) {
        Plan p2;
        if (make_plan(mode, b, H, D, c, k, false, p2) == DSAIDX_OK)
            total = std::max(total, p2.total);
    }
    return total;
}

// ------------------------------------------------------------ key chunks
// Workspace of indexer_chunk_refine: proxies, chunk limits, list lengths,
// selected chunks and candidate lists (unless the caller takes them), and
// one region shared by the coarse scan and Refine.
struct ChunkPlan {
    bool split_scan = false, split_refine = false;
    bool dense_pass = false, split_dense = false;  // guarded groups' rows
    int cap_dense = 0;
    bool refine_lds = false;  // Refine on refine.hip (groups of 2-4 rows, short lists)
    int nw_refine = 4;
    int cap_scan = 0, cap_refine = 0;
    int64_t G = 0, cw = 0;
    size_t off_proxy_q = 0, off_proxy_w = 0, off_glim = 0, off_cn = 0, off_chunks = 0, off_cand = 0;
    size_t off_work = 0, total = 0;
};

constexpr int64_t kMaxCandWidth = (int64_t)1 << 22;

int make_chunk_plan(const Batch &b, int H, int D, int64_t nc, int64_t nsel, int64_t max_chunk, int64_t k,
                    bool have_chunks, bool have_cand, ChunkPlan &pl)
{
    int s = check_common(H, D, k);
    if (s != DSAIDX_OK)
        return s;
    if (b.g < 1)
        return fail(DSAIDX_EINVAL, "g=%lld must be >= 1", (long long)b.g);
    if (nc < 1 || nc > b.L)
        return fail(DSAIDX_EINVAL, "nc=%lld must be in [1, L=%lld]", (long long)nc, (long long)b.L);
    if (nsel < 1 || nsel > kMaxSel)
        return fail(DSAIDX_EINVAL, "nsel=%lld must be in [1, 2^20]", (long long)nsel);
    if (max_chunk < 1)
        return fail(DSAIDX_EINVAL, "max_chunk=%lld must be >= 1", (long long)max_chunk);
    pl = ChunkPlan{};
    pl.cw = (nsel + 1) * max_chunk;
    if (pl.cw > kMaxCandWidth)
        return fail(DSAIDX_EINVAL, "(nsel + 1) * max_chunk = %lld exceeds 2^22", (long long)pl.cw);
    if (pl.cw < k)
        return fail(DSAIDX_EINVAL, "(nsel + 1) * max_chunk = %lld must be >= k=%lld", (long long)pl.cw,
                    (long long)k);
    pl.G = ceil_div(b.q_len, b.g);
    const int64_t groups = (int64_t)b.B * pl.G;
    size_t off = 0;
    pl.off_proxy_q = off;
    off += align_up((size_t)groups * H * D * sizeof(uint16_t));
    pl.off_proxy_w = off;
    off += align_up((size_t)groups * H * sizeof(float));
    pl.off_glim = off;
    off += align_up((size_t)groups * sizeof(int32_t));
    pl.off_cn = off;
    off += align_up((size_t)groups * sizeof(int32_t));
    if (!have_chunks) {
        pl.off_chunks = off;
        off += align_up((size_t)groups * nsel * sizeof(int32_t));
    }
    if (!have_cand) {
        pl.off_cand = off;
        off += align_up((size_t)groups * pl.cw * sizeof(int32_t));
    }
    // groups past the guard (all of them without one) take the chunk path
    pl.split_scan = b.max_pivot_groups <= kSplitRowsMax;
    pl.cap_scan = scan_cap(nsel, nc);
    size_t work = pl.split_scan ? (size_t)b.B * b.max_pivot_groups * score_row(nc) * sizeof(float)
                                : scan_bytes(H, D, 8, pl.cap_scan);
    // guarded groups: their rows in a dense pass (the same region)
    pl.dense_pass = b.max_dense_rows > 0;
    if (pl.dense_pass) {
        pl.split_dense = b.max_dense_rows <= kSplitRowsMax;
        // (a guarded row's prefix ends at the last guarded row)
        pl.cap_dense = scan_cap(k, b.L - b.q_len + b.max_dense_rows);
        work = std::max(work, pl.split_dense ? (size_t)b.B * b.max_dense_rows * score_row(b.L) * sizeof(float)
                                             : scan_bytes(H, D, 8, pl.cap_dense));
    }
    // one row per group: every row has a list of its own, so each one-wave
    // workgroup streams its own list (several per CU)
    pl.split_refine = b.max_refine_rows <= kSplitRowsMax;
    pl.refine_lds = !pl.split_refine && b.g >= 2 && b.g <= 4 && pl.cw <= kRefineLdsCandMax;
    pl.nw_refine = b.g == 1 ? 1 : (b.g <= 4 ? 4 : 8);
    pl.cap_refine = (int)ceil_div(pl.cw + 128, 64) * 64;
    if (pl.split_refine)
        work = std::max(work, (size_t)b.B * b.max_refine_rows * score_row(pl.cw) * sizeof(float));
    else if (!pl.refine_lds)
        work = std::max(work, scan_bytes(H, D, pl.nw_refine, pl.cap_refine));
    pl.off_work = off;
    off += align_up(work);
    pl.total = off;
    return DSAIDX_OK;
}

int chunk_batch(int B, int64_t L, int64_t q_len, int g, const dsaidx_pivot_opts *opts, Batch &b)
{
    if (g < 1)
        return fail(DSAIDX_EINVAL, "g=%d must be >= 1", g);
    if (L < 1 || q_len < 1)
        return fail(DSAIDX_EINVAL, "the chunk path needs L >= 1 and q_len >= 1 (L=%lld, q_len=%lld)",
                    (long long)L, (long long)q_len);
    int s = uniform_batch(B, L, q_len, g, b);
    if (s != DSAIDX_OK)
        return s;
    if (opts) {
        if (opts->proxy != DSAIDX_PROXY_MEAN && opts->proxy != DSAIDX_PROXY_FIRST && opts->proxy != DSAIDX_PROXY_LAST)
            return fail(DSAIDX_EINVAL, "unknown proxy strategy %d", opts->proxy);
        if (opts->window < 0)
            return fail(DSAIDX_EINVAL, "window=%d must be >= 0", opts->window);
        if (opts->guard < 0)
            return fail(DSAIDX_EINVAL, "guard=%lld must be >= 0", (long long)opts->guard);
        b.proxy = opts->proxy;
        b.window = opts->window;
        if (opts->guard > 0)
            finish_batch(b, nullptr, nullptr, opts->guard);  // guarded groups: m0, dense rows
    }
    return DSAIDX_OK;
}

int run_chunk_refine(const Batch &b, const void *Qv, const float *W, const void *Kv, const void *Kbarv,
                     const int32_t *cend, int64_t nc, int H, int D, int64_t nsel, int64_t max_chunk, int64_t k,
                     int32_t *out_idx, float *out_score, int32_t *out_chunks, int32_t *out_cand, void *ws,
                     size_t ws_bytes, hipStream_t stream)
{
    ChunkPlan pl;
    int s = make_chunk_plan(b, H, D, nc, nsel, max_chunk, k, out_chunks != nullptr, out_cand != nullptr, pl);
    if (s != DSAIDX_OK)
        return s;
    s = check_ptrs(Qv, W, Kv, out_idx, out_score, out_cand, ws, pl.total);
    if (s != DSAIDX_OK)
        return s;
    if (!Kbarv || !cend)
        return fail(DSAIDX_EINVAL, "Kbar and cend must not be NULL");
    if (!aligned(Kbarv, 16) || !aligned(cend, 4) || (out_chunks && !aligned(out_chunks, 4)))
        return fail(DSAIDX_EINVAL, "Kbar must be 16-byte aligned, cend and out_chunks 4-byte aligned");
    if (ws_bytes < pl.total)
        return fail(DSAIDX_EWORKSPACE, "workspace of %zu bytes is below the %zu needed", ws_bytes, pl.total);
    const uint16_t *Q = static_cast<const uint16_t *>(Qv);
    const uint16_t *K = static_cast<const uint16_t *>(Kv);
    const uint16_t *Kbar = static_cast<const uint16_t *>(Kbarv);
    unsigned char *wsb = static_cast<unsigned char *>(ws);
    uint16_t *Qp = reinterpret_cast<uint16_t *>(wsb + pl.off_proxy_q);
    float *Wp = reinterpret_cast<float *>(wsb + pl.off_proxy_w);
    int32_t *glim = reinterpret_cast<int32_t *>(wsb + pl.off_glim);
    int32_t *cn = reinterpret_cast<int32_t *>(wsb + pl.off_cn);
    int32_t *chunks = out_chunks ? out_chunks : reinterpret_cast<int32_t *>(wsb + pl.off_chunks);
    int32_t *cand = out_cand ? out_cand : reinterpret_cast<int32_t *>(wsb + pl.off_cand);
    float *work = reinterpret_cast<float *>(wsb + pl.off_work);
    hipError_t e;

    // 0. guarded groups (the first m0 of each request): dense rows, chunk and
    // candidate rows -1
    if (pl.dense_pass) {
        Plan dp{};
        dp.split_dense = pl.split_dense;
        dp.nw_scan = 8;
        dp.cap_dense = pl.cap_dense;
        dp.off_work = pl.off_work;
        Pass pd{&b, nullptr, 0, 1};
        s = run_dense(dp, pd, Q, W, K, H, D, k, out_idx, out_score, wsb, stream);
        if (s != DSAIDX_OK)
            return s;
        e = launch_fill_guarded(nullptr, b.B, b.L, b.q_len, b.g, b.m0, b.m0, nsel, chunks, stream);
        if (e != hipSuccess)
            return hip_fail(e, "chunk fill launch");
        if (out_cand) {
            e = launch_fill_guarded(nullptr, b.B, b.L, b.q_len, b.g, b.m0, b.m0, pl.cw, out_cand, stream);
            if (e != hipSuccess)
                return hip_fail(e, "candidate fill launch");
        }
    }
    if (b.max_pivot_groups == 0)
        return DSAIDX_OK;  // every group guarded

    // 1. proxies
    PoolParams pp{};
    pp.Q = Q;
    pp.W = W;
    pp.B = b.B;
    pp.L = b.L;
    pp.q_len = b.q_len;
    pp.g = b.g;
    pp.m0 = b.m0;
    pp.gmax = pl.G;
    pp.proxy = b.proxy;
    pp.window = b.window;
    pp.Qp = Qp;
    pp.Wp = Wp;
    e = launch_pool(H, D, pp, stream);
    if (e != hipSuccess)
        return hip_fail(e, "pool launch");

    // 2. chunks complete at each group's last position
    e = launch_chunk_limits(b.B, b.L, b.q_len, b.g, cend, nc, glim, stream);
    if (e != hipSuccess)
        return hip_fail(e, "chunk limit launch");

    // 3. coarse scan of the summaries: top-nsel chunks per group
    Pass ps{&b, nullptr, 0, 0};
    ps.glim = glim;
    ps.krows = nc;
    if (pl.split_scan) {
        s = run_split(kProxy, ps, Qp, Wp, Kbar, nullptr, b.max_pivot_groups, score_row(nc), H, D, (int)nsel, 0, chunks,
                      nullptr, 0, nullptr, nullptr, work, stream);
        if (s != DSAIDX_OK)
            return s;
    } else {
        ScanParams p = scan_base(ps, kProxy, Qp, Wp, Kbar);
        p.nblk_per_batch = ceil_div(b.max_pivot_groups, 8);
        p.nblocks = p.nblk_per_batch * b.B;
        p.sel = (int)nsel;
        p.sel2 = 0;
        p.o1_idx = chunks;
        p.o1_score = nullptr;
        p.o1_members = 0;
        p.slots = reinterpret_cast<Entry *>(work);
        p.cap = pl.cap_scan;
        e = launch_scan_select(H, D, 8, kProxy, p, scan_grid(H, D, 8, p.nblocks), stream);
        if (e != hipSuccess)
            return hip_fail(e, "coarse scan launch");
    }

    // 4. candidate lists
    ChunkExpandParams xp{};
    xp.chunks = chunks;
    xp.cend = cend;
    xp.glim = glim;
    xp.L = b.L;
    xp.q_len = b.q_len;
    xp.g = b.g;
    xp.nc = nc;
    xp.nsel = (int)nsel;
    xp.cw = pl.cw;
    xp.cand = cand;
    xp.cand_n = cn;
    e = launch_chunk_expand(xp, (int64_t)b.B * pl.G, stream);
    if (e != hipSuccess)
        return hip_fail(e, "expansion launch");
    if (out_cand && b.m0 > 0) {
        // (a guarded group's list, from its -1 chunk row, is its tail only)
        e = launch_fill_guarded(nullptr, b.B, b.L, b.q_len, b.g, b.m0, b.m0, pl.cw, out_cand, stream);
        if (e != hipSuccess)
            return hip_fail(e, "candidate fill launch");
    }

    // 5. Refine on the lists
    Pass pr{&b, nullptr, pl.cw, 0};
    pr.cand_n = cn;
    if (pl.split_refine)
        return run_split(kRefine, pr, Q, W, K, cand, b.max_refine_rows, score_row(pl.cw), H, D, (int)k, 0, out_idx,
                         out_score, 0, nullptr, nullptr, work, stream);
    if (pl.refine_lds) {
        // groups of two to four rows sharing a list: the members' scores and
        // selections on chip (a single row per list stays on the one-wave
        // scan workgroups below)
        RefineLdsParams rp{};
        rp.Q = Q;
        rp.W = W;
        rp.K = K;
        rp.cand = cand;
        rp.cand_n = cn;
        rp.req = nullptr;
        rp.B = b.B;
        rp.L = b.L;
        rp.q_len = b.q_len;
        rp.g = b.g;
        rp.c = pl.cw;
        rp.m0 = b.m0;
        rp.k = (int)k;
        rp.out_idx = out_idx;
        rp.out_score = out_score;
        rp.nwork = (int64_t)b.B * b.max_pivot_groups;
        const int grid = (int)std::min<int64_t>(rp.nwork, std::max(1, num_cus()));
        e = launch_refine_lds(H, D, rp, grid, stream);
        if (e != hipSuccess)
            return hip_fail(e, "refine launch");
        return DSAIDX_OK;
    }
    ScanParams p = scan_base(pr, kRefine, Q, W, K);
    p.cand = cand;
    p.member_chunks = ceil_div(b.g, pl.nw_refine);
    p.nblk_per_batch = b.max_pivot_groups * p.member_chunks;
    p.nblocks = p.nblk_per_batch * b.B;
    p.sel = (int)k;
    p.sel2 = 0;
    p.o1_idx = out_idx;
    p.o1_score = out_score;
    p.slots = reinterpret_cast<Entry *>(work);
    p.cap = pl.cap_refine;
    e = launch_scan_select(H, D, pl.nw_refine, kRefine, p, scan_grid(H, D, pl.nw_refine, p.nblocks), stream);
    if (e != hipSuccess)
        return hip_fail(e, "refine launch");
    return DSAIDX_OK;
}

// Workspace of the adaptive partition: split gains and merge losses, and,
// beyond kAdaptBlocksLds blocks per request, the space their sort runs in.
struct AdaptLayout {
    int64_t n, nfull, npair, g2, p2;
    size_t off_loss, off_gk, off_gi, off_lk, off_li, total;
};

int64_t pow2_at_least(int64_t x)
{
    int64_t p = 1;
    while (p < x)
        p <<= 1;
    return p;
}

AdaptLayout adapt_layout(int B, int64_t L, int64_t block)
{
    AdaptLayout a{};
    a.n = ceil_div(L, block);
    a.nfull = L / block;
    a.npair = a.nfull / 2;
    a.g2 = pow2_at_least(std::max<int64_t>(a.nfull, 1));
    a.p2 = pow2_at_least(std::max<int64_t>(a.npair, 1));
    size_t off = align_up((size_t)B * a.nfull * sizeof(double));
    a.off_loss = off;
    off += align_up((size_t)B * a.npair * sizeof(double));
    if (a.n > kAdaptBlocksLds) {
        a.off_gk = off;
        off += align_up((size_t)B * a.g2 * sizeof(double));
        a.off_gi = off;
        off += align_up((size_t)B * a.g2 * sizeof(int32_t));
        a.off_lk = off;
        off += align_up((size_t)B * a.p2 * sizeof(double));
        a.off_li = off;
        off += align_up((size_t)B * a.p2 * sizeof(int32_t));
    }
    a.total = off;
    return a;
}

int check_chunk_sizes(int B, int64_t L, int block)
{
    if (B < 1 || B > 65535)
        return fail(DSAIDX_EINVAL, "B=%d must be in [1, 65535]", B);
    if (L < 1 || L >= (int64_t)INT32_MAX)
        return fail(DSAIDX_EINVAL, "L=%lld must be in [1, 2^31-1)", (long long)L);
    if (block < 1)
        return fail(DSAIDX_EINVAL, "block=%d must be >= 1", block);
    return DSAIDX_OK;
}

// --------------------------------------------------- library-held scratch
// Scratch of indexer_pivot_refine_noalloc: a fixed device array, one copy per
// GPU, held until the process ends. In host code the array's name is only a
// stand-in for the symbol: its device address comes from hipGetSymbolAddress,
// once per device with that device current, and only that address is used.
static __device__ __align__(256) unsigned char scratch[DSAIDX_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the device `stream` runs on (which
// must be the current device, as for every launch of this library).
int scratch_address(hipStream_t stream, void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    int sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess)
        return hip_fail(e, "hipStreamGetDevice");
    if (sdev != dev)
        return fail(DSAIDX_EINVAL, "the stream belongs to device %d, the current device is %d", sdev, dev);
    if (dev < 0 || dev >= kMaxDevices)
        return fail(DSAIDX_EUNSUPPORTED, "device %d is beyond the %d devices the scratch table holds", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p)
            return fail(DSAIDX_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DSAIDX_OK;
}

}  // namespace

// ------------------------------------ key chunks, variable-length batches
// Request r of a variable-length chunk call: L[r] keys, q_len[r] queried
// positions, nc[r] chunks (nc may be NULL where the call has none), checked
// before anything is enqueued; each request then runs as a uniform batch of
// one on the caller's stream.
int check_chunk_varlen(int B, const int64_t *L, const int64_t *q_len, const int64_t *nc)
{
    if (B < 1 || B > 65535)
        return fail(DSAIDX_EINVAL, "B=%d must be in [1, 65535]", B);
    if (!L)
        return fail(DSAIDX_EINVAL, "L must not be NULL");
    for (int r = 0; r < B; ++r) {
        if (L[r] < 1 || L[r] >= (int64_t)INT32_MAX)
            return fail(DSAIDX_EINVAL, "request %d: L=%lld must be in [1, 2^31-1)", r, (long long)L[r]);
        if (q_len && (q_len[r] < 0 || q_len[r] > L[r]))
            return fail(DSAIDX_EINVAL, "request %d: q_len=%lld must be in [0, L=%lld]", r, (long long)q_len[r],
                        (long long)L[r]);
        if (nc && (nc[r] < 1 || nc[r] > L[r]))
            return fail(DSAIDX_EINVAL, "request %d: nc=%lld must be in [1, L=%lld]", r, (long long)nc[r],
                        (long long)L[r]);
    }
    return DSAIDX_OK;
}

extern "C" {

size_t indexer_workspace_bytes(dsaidx_mode mode, int B, int64_t L, int64_t q_len, int H_I, int d_I, int g, int c,
                               int k)
{
    if (mode != DSAIDX_DENSE && mode != DSAIDX_REUSE && mode != DSAIDX_REFINE) {
        fail(DSAIDX_EINVAL, "unknown mode %d", mode);
        return 0;
    }
    Batch b;
    if (uniform_batch(B, L, q_len, mode == DSAIDX_DENSE ? 1 : g, b) != DSAIDX_OK)
        return 0;
    return workspace_for(mode, b, H_I, d_I, c, k);
}

int indexer_dense(const void *Qv, const float *W, const void *Kv, int B, int64_t L, int64_t q_len, int H_I,
                  int d_I, int k, int32_t *out_idx, float *out_score, void *ws, size_t ws_bytes,
                  hipStream_t stream)
{
    Batch b;
    int s = uniform_batch(B, L, q_len, 1, b);
    if (s != DSAIDX_OK)
        return s;
    return run_dense_call(b, Qv, W, Kv, H_I, d_I, k, out_idx, out_score, ws, ws_bytes, stream);
}

int indexer_pivot_reuse(const void *Q, const float *W, const void *K, int B, int64_t L, int64_t q_len, int H_I,
                        int d_I, int g, int c, int k, int32_t *out_idx, float *out_score, int32_t *out_cand,
                        void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (g < 1)
        return fail(DSAIDX_EINVAL, "g=%d must be >= 1", g);
    Batch b;
    int s = uniform_batch(B, L, q_len, g, b);
    if (s != DSAIDX_OK)
        return s;
    return run_pivot(DSAIDX_REUSE, b, Q, W, K, H_I, d_I, c, k, out_idx, out_score, out_cand, ws, ws_bytes, stream);
}

int indexer_pivot_refine(const void *Q, const float *W, const void *K, int B, int64_t L, int64_t q_len, int H_I,
                         int d_I, int g, int c, int k, int32_t *out_idx, float *out_score, int32_t *out_cand,
                         void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (g < 1)
        return fail(DSAIDX_EINVAL, "g=%d must be >= 1", g);
    Batch b;
    int s = uniform_batch(B, L, q_len, g, b);
    if (s != DSAIDX_OK)
        return s;
    return run_pivot(DSAIDX_REFINE, b, Q, W, K, H_I, d_I, c, k, out_idx, out_score, out_cand, ws, ws_bytes, stream);
}

int indexer_pivot_refine_noalloc(const void *Q, const float *W, const void *K, int B, int64_t L, int64_t q_len,
                                 int H_I, int d_I, int g, int c, int k, int32_t *out_idx, float *out_score,
                                 int32_t *out_cand, hipStream_t stream)
{
    if (g < 1)
        return fail(DSAIDX_EINVAL, "g=%d must be >= 1", g);
    Batch b;
    int s = uniform_batch(B, L, q_len, g, b);
    if (s != DSAIDX_OK)
        return s;
    Plan pl;
    s = make_plan(DSAIDX_REFINE, b, H_I, d_I, c, k, out_cand != nullptr, pl);
    if (s != DSAIDX_OK)
        return s;
    if (pl.total > (size_t)DSAIDX_SCRATCH_BYTES)
        return fail(DSAIDX_EWORKSPACE,
                    "these sizes need %zu bytes of scratch, above the %zu the library holds per device",
                    pl.total, (size_t)DSAIDX_SCRATCH_BYTES);
    if (b.total_q == 0)
        return DSAIDX_OK;
    void *ws = nullptr;
    s = scratch_address(stream, &ws);
    if (s != DSAIDX_OK)
        return s;
    return run_pivot(DSAIDX_REFINE, b, Q, W, K, H_I, d_I, c, k, out_idx, out_score, out_cand, ws,
                     (size_t)DSAIDX_SCRATCH_BYTES, stream);
}

size_t indexer_varlen_workspace_bytes(dsaidx_mode mode, int B, const int64_t *L, const int64_t *q_len, int H_I, int d_I,
                                      int g, int c, int k, const dsaidx_pivot_opts *opts)
{
    if (mode != DSAIDX_DENSE && mode != DSAIDX_REUSE && mode != DSAIDX_REFINE) {
        fail(DSAIDX_EINVAL, "unknown mode %d", mode);
        return 0;
    }
    if (mode != DSAIDX_DENSE && g < 1) {
        fail(DSAIDX_EINVAL, "g=%d must be >= 1", g);
        return 0;
    }
    Batch b;
    if (varlen_batch(B, L, q_len, mode == DSAIDX_DENSE ? 1 : g, mode == DSAIDX_DENSE ? nullptr : opts, b) !=
        DSAIDX_OK)
        return 0;
    return workspace_for(mode, b, H_I, d_I, c, k);
}

int indexer_dense_varlen(const void *Q, const float *W, const void *K, int B, const int64_t *L,
                         const int64_t *q_len, int H_I, int d_I, int k, int32_t *out_idx, float *out_score,
                         void *ws, size_t ws_bytes, hipStream_t stream)
{
    Batch b;
    int s = varlen_batch(B, L, q_len, 1, nullptr, b);
    if (s != DSAIDX_OK)
        return s;
    return run_dense_call(b, Q, W, K, H_I, d_I, k, out_idx, out_score, ws, ws_bytes, stream);
}

int indexer_pivot_reuse_varlen(const void *Q, const float *W, const void *K, int B, const int64_t *L,
                               const int64_t *q_len, int H_I, int d_I, int g, int c, int k,
                               const dsaidx_pivot_opts *opts, int32_t *out_idx, float *out_score,
                               int32_t *out_cand, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (g < 1)
        return fail(DSAIDX_EINVAL, "g=%d must be >= 1", g);
    Batch b;
    int s = varlen_batch(B, L, q_len, g, opts, b);
    if (s != DSAIDX_OK)
        return s;
    return run_pivot(DSAIDX_REUSE, b, Q, W, K, H_I, d_I, c, k, out_idx, out_score, out_cand, ws, ws_bytes, stream);
}

int indexer_pivot_refine_varlen(const void *Q, const float *W, const void *K, int B, const int64_t *L,
                                const int64_t *q_len, int H_I, int d_I, int g, int c, int k,
                                const dsaidx_pivot_opts *opts, int32_t *out_idx, float *out_score,
                                int32_t *out_cand, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (g < 1)
        return fail(DSAIDX_EINVAL, "g=%d must be >= 1", g);
    Batch b;
    int s = varlen_batch(B, L, q_len, g, opts, b);
    if (s != DSAIDX_OK)
        return s;
    return run_pivot(DSAIDX_REFINE, b, Q, W, K, H_I, d_I, c, k, out_idx, out_score, out_cand, ws, ws_bytes, stream);
}

int indexer_chunks_fixed(int B, int64_t L, int block, int32_t *cend, hipStream_t stream)
{
    int s = check_chunk_sizes(B, L, block);
    if (s != DSAIDX_OK)
        return s;
    if (!cend || !aligned(cend, 4))
        return fail(DSAIDX_EINVAL, "cend must be a non-NULL 4-byte aligned pointer");
    hipError_t e = launch_chunk_fixed(B, L, block, ceil_div(L, block), cend, stream);
    return e == hipSuccess ? DSAIDX_OK : hip_fail(e, "chunk launch");
}

size_t indexer_chunks_adaptive_workspace_bytes(int B, int64_t L, int block)
{
    if (check_chunk_sizes(B, L, block) != DSAIDX_OK)
        return 0;
    return adapt_layout(B, L, block).total;
}

int indexer_chunks_adaptive(const void *K, int B, int64_t L, int d_I, int block, int32_t *cend, void *ws,
                            size_t ws_bytes, hipStream_t stream)
{
    int s = check_chunk_sizes(B, L, block);
    if (s != DSAIDX_OK)
        return s;
    if (block < 2 || block % 2)
        return fail(DSAIDX_EINVAL, "block=%d must be even", block);
    if (d_I != 128 && d_I != 32)
        return fail(DSAIDX_EUNSUPPORTED, "d_I=%d has no kernel; supported: 32, 128", d_I);
    const int64_t n = ceil_div(L, block);
    if (n > kAdaptBlocksMax)
        return fail(DSAIDX_EUNSUPPORTED, "%lld blocks per request exceed the %d the adaptive partition supports",
                    (long long)n, kAdaptBlocksMax);
    if (!K || !cend || !aligned(K, 16) || !aligned(cend, 4))
        return fail(DSAIDX_EINVAL, "K (16-byte aligned) and cend (4-byte aligned) must not be NULL");
    const size_t need = indexer_chunks_adaptive_workspace_bytes(B, L, block);
    if (need > 0 && (!ws || !aligned(ws, 16)))
        return fail(DSAIDX_EINVAL, "ws must be a non-NULL 16-byte aligned pointer (%zu bytes needed)", need);
    if (ws_bytes < need)
        return fail(DSAIDX_EWORKSPACE, "workspace of %zu bytes is below the %zu needed", ws_bytes, need);
    const AdaptLayout al = adapt_layout(B, L, block);
    unsigned char *wsb = static_cast<unsigned char *>(ws);
    ChunkAdaptParams p{};
    p.K = static_cast<const uint16_t *>(K);
    p.L = L;
    p.block = block;
    p.n = al.n;
    p.nfull = al.nfull;
    p.npair = al.npair;
    p.g2 = al.g2;
    p.p2 = al.p2;
    p.gain = reinterpret_cast<double *>(wsb);
    p.loss = reinterpret_cast<double *>(wsb + al.off_loss);
    if (al.n > kAdaptBlocksLds) {
        p.gk = reinterpret_cast<double *>(wsb + al.off_gk);
        p.gi = reinterpret_cast<int32_t *>(wsb + al.off_gi);
        p.lk = reinterpret_cast<double *>(wsb + al.off_lk);
        p.li = reinterpret_cast<int32_t *>(wsb + al.off_li);
    }
    p.cend = cend;
    hipError_t e = launch_chunk_adaptive(d_I, B, p, stream);
    return e == hipSuccess ? DSAIDX_OK : hip_fail(e, "adaptive chunk launch");
}

int indexer_chunk_means(const void *K, int B, int64_t L, int d_I, const int32_t *cend, int64_t nc, int64_t first,
                        void *Kbar, hipStream_t stream)
{
    int s = check_chunk_sizes(B, L, 1);
    if (s != DSAIDX_OK)
        return s;
    if (d_I != 128 && d_I != 32)
        return fail(DSAIDX_EUNSUPPORTED, "d_I=%d has no kernel; supported: 32, 128", d_I);
    if (nc < 1 || nc > L || first < 0 || first > nc)
        return fail(DSAIDX_EINVAL, "need 1 <= nc <= L and 0 <= first <= nc (nc=%lld, first=%lld)", (long long)nc,
                    (long long)first);
    if (!K || !cend || !Kbar || !aligned(K, 16) || !aligned(Kbar, 16) || !aligned(cend, 4))
        return fail(DSAIDX_EINVAL, "K, Kbar (16-byte aligned) and cend (4-byte aligned) must not be NULL");
    if (first == nc)
        return DSAIDX_OK;
    hipError_t e = launch_chunk_means(d_I, static_cast<const uint16_t *>(K), B, L, cend, nc, first,
                                      static_cast<uint16_t *>(Kbar), stream);
    return e == hipSuccess ? DSAIDX_OK : hip_fail(e, "summary launch");
}

size_t indexer_chunk_refine_workspace_bytes(int B, int64_t L, int64_t q_len, int H_I, int d_I, int g, int64_t nc,
                                            int nsel, int max_chunk, int k, const dsaidx_pivot_opts *opts)
{
    Batch b;
    if (chunk_batch(B, L, q_len, g, opts, b) != DSAIDX_OK)
        return 0;
    ChunkPlan pl;
    if (make_chunk_plan(b, H_I, d_I, nc, nsel, max_chunk, k, false, false, pl) != DSAIDX_OK)
        return 0;
    return pl.total;
}

int indexer_chunk_refine(const void *Q, const float *W, const void *K, const void *Kbar, const int32_t *cend,
                         int64_t nc, int B, int64_t L, int64_t q_len, int H_I, int d_I, int g, int nsel,
                         int max_chunk, int k, const dsaidx_pivot_opts *opts, int32_t *out_idx, float *out_score,
                         int32_t *out_chunks, int32_t *out_cand, void *ws, size_t ws_bytes, hipStream_t stream)
{
    Batch b;
    int s = chunk_batch(B, L, q_len, g, opts, b);
    if (s != DSAIDX_OK)
        return s;
    return run_chunk_refine(b, Q, W, K, Kbar, cend, nc, H_I, d_I, nsel, max_chunk, k, out_idx, out_score,
                            out_chunks, out_cand, ws, ws_bytes, stream);
}

int indexer_chunks_fixed_varlen(int B, const int64_t *L, int block, int32_t *cend, hipStream_t stream)
{
    int s = check_chunk_varlen(B, L, nullptr, nullptr);
    if (s != DSAIDX_OK)
        return s;
    if (block < 1)
        return fail(DSAIDX_EINVAL, "block=%d must be >= 1", block);
    if (!cend || !aligned(cend, 4))
        return fail(DSAIDX_EINVAL, "cend must be a non-NULL 4-byte aligned pointer");
    int64_t off = 0;
    for (int r = 0; r < B; ++r) {
        const int64_t n = ceil_div(L[r], block);
        hipError_t e = launch_chunk_fixed(1, L[r], block, n, cend + off, stream);
        if (e != hipSuccess)
            return hip_fail(e, "chunk launch");
        off += n;
    }
    return DSAIDX_OK;
}

size_t indexer_chunks_adaptive_varlen_workspace_bytes(int B, const int64_t *L, int block)
{
    if (check_chunk_varlen(B, L, nullptr, nullptr) != DSAIDX_OK)
        return 0;
    size_t need = 0;
    for (int r = 0; r < B; ++r) {
        const size_t n = indexer_chunks_adaptive_workspace_bytes(1, L[r], block);
        if (n == 0)
            return 0;
        need = std::max(need, n);
    }
    return need;
}

int indexer_chunks_adaptive_varlen(const void *K, int B, const int64_t *L, int d_I, int block, int32_t *cend,
                                   void *ws, size_t ws_bytes, hipStream_t stream)
{
    int s = check_chunk_varlen(B, L, nullptr, nullptr);
    if (s != DSAIDX_OK)
        return s;
    if (block < 2 || block % 2)
        return fail(DSAIDX_EINVAL, "block=%d must be even", block);
    if (d_I != 128 && d_I != 32)
        return fail(DSAIDX_EUNSUPPORTED, "d_I=%d has no kernel; supported: 32, 128", d_I);
    for (int r = 0; r < B; ++r)
        if (ceil_div(L[r], block) > kAdaptBlocksMax)
            return fail(DSAIDX_EUNSUPPORTED, "request %d: %lld blocks exceed the %d the adaptive partition supports",
                        r, (long long)ceil_div(L[r], block), kAdaptBlocksMax);
    if (!K || !cend || !aligned(K, 16) || !aligned(cend, 4))
        return fail(DSAIDX_EINVAL, "K (16-byte aligned) and cend (4-byte aligned) must not be NULL");
    const size_t need = indexer_chunks_adaptive_varlen_workspace_bytes(B, L, block);
    if (need > 0 && (!ws || !aligned(ws, 16)))
        return fail(DSAIDX_EINVAL, "ws must be a non-NULL 16-byte aligned pointer (%zu bytes needed)", need);
    if (ws_bytes < need)
        return fail(DSAIDX_EWORKSPACE, "workspace of %zu bytes is below the %zu needed", ws_bytes, need);
    const uint16_t *Kh = static_cast<const uint16_t *>(K);
    int64_t koff = 0, coff = 0;
    for (int r = 0; r < B; ++r) {
        // (the request's own call reuses ws: its launches follow the previous
        // request's on the same stream)
        s = indexer_chunks_adaptive(Kh + koff * d_I, 1, L[r], d_I, block, cend + coff, ws, ws_bytes, stream);
        if (s != DSAIDX_OK)
            return s;
        koff += L[r];
        coff += ceil_div(L[r], block);
    }
    return DSAIDX_OK;
}

int indexer_chunk_means_varlen(const void *K, int B, const int64_t *L, int d_I, const int32_t *cend,
                               const int64_t *nc, void *Kbar, hipStream_t stream)
{
    if (!nc)
        return fail(DSAIDX_EINVAL, "nc must not be NULL");
    int s = check_chunk_varlen(B, L, nullptr, nc);
    if (s != DSAIDX_OK)
        return s;
    if (d_I != 128 && d_I != 32)
        return fail(DSAIDX_EUNSUPPORTED, "d_I=%d has no kernel; supported: 32, 128", d_I);
    if (!K || !cend || !Kbar || !aligned(K, 16) || !aligned(Kbar, 16) || !aligned(cend, 4))
        return fail(DSAIDX_EINVAL, "K, Kbar (16-byte aligned) and cend (4-byte aligned) must not be NULL");
    const uint16_t *Kh = static_cast<const uint16_t *>(K);
    uint16_t *Kb = static_cast<uint16_t *>(Kbar);
    int64_t koff = 0, coff = 0;
    for (int r = 0; r < B; ++r) {
        s = indexer_chunk_means(Kh + koff * d_I, 1, L[r], d_I, cend + coff, nc[r], 0, Kb + coff * d_I, stream);
        if (s != DSAIDX_OK)
            return s;
        koff += L[r];
        coff += nc[r];
    }
    return DSAIDX_OK;
}

size_t indexer_chunk_refine_varlen_workspace_bytes(int B, const int64_t *L, const int64_t *q_len, int H_I, int d_I,
                                                   int g, const int64_t *nc, int nsel, int max_chunk, int k,
                                                   const dsaidx_pivot_opts *opts)
{
    if (!q_len || !nc) {
        fail(DSAIDX_EINVAL, "q_len and nc must not be NULL");
        return 0;
    }
    if (check_chunk_varlen(B, L, q_len, nc) != DSAIDX_OK)
        return 0;
    size_t need = 256;  // (no request with rows: nothing is used, but 0 means an error)
    for (int r = 0; r < B; ++r) {
        if (q_len[r] == 0)
            continue;
        const size_t n =
            indexer_chunk_refine_workspace_bytes(1, L[r], q_len[r], H_I, d_I, g, nc[r], nsel, max_chunk, k, opts);
        if (n == 0)
            return 0;
        need = std::max(need, n);
    }
    return need;
}

int indexer_chunk_refine_varlen(const void *Q, const float *W, const void *K, const void *Kbar,
                                const int32_t *cend, const int64_t *nc, int B, const int64_t *L,
                                const int64_t *q_len, int H_I, int d_I, int g, int nsel, int max_chunk, int k,
                                const dsaidx_pivot_opts *opts, int32_t *out_idx, float *out_score,
                                int32_t *out_chunks, int32_t *out_cand, void *ws, size_t ws_bytes,
                                hipStream_t stream)
{
    if (!q_len || !nc)
        return fail(DSAIDX_EINVAL, "q_len and nc must not be NULL");
    int s = check_chunk_varlen(B, L, q_len, nc);
    if (s != DSAIDX_OK)
        return s;
    // every request's plan and the pointers, before anything is enqueued
    size_t need = 0;
    bool any = false;
    for (int r = 0; r < B; ++r) {
        if (q_len[r] == 0)
            continue;
        Batch b;
        s = chunk_batch(1, L[r], q_len[r], g, opts, b);
        if (s != DSAIDX_OK)
            return s;
        ChunkPlan pl;
        s = make_chunk_plan(b, H_I, d_I, nc[r], nsel, max_chunk, k, out_chunks != nullptr, out_cand != nullptr, pl);
        if (s != DSAIDX_OK)
            return s;
        need = std::max(need, pl.total);
        any = true;
    }
    if (!any)
        return DSAIDX_OK;
    s = check_ptrs(Q, W, K, out_idx, out_score, out_cand, ws, need);
    if (s != DSAIDX_OK)
        return s;
    if (!Kbar || !cend)
        return fail(DSAIDX_EINVAL, "Kbar and cend must not be NULL");
    if (!aligned(Kbar, 16) || !aligned(cend, 4) || (out_chunks && !aligned(out_chunks, 4)))
        return fail(DSAIDX_EINVAL, "Kbar must be 16-byte aligned, cend and out_chunks 4-byte aligned");
    if (ws_bytes < need)
        return fail(DSAIDX_EWORKSPACE, "workspace of %zu bytes is below the %zu needed", ws_bytes, need);
    const uint16_t *Qh = static_cast<const uint16_t *>(Q);
    const uint16_t *Kh = static_cast<const uint16_t *>(K);
    const uint16_t *Kb = static_cast<const uint16_t *>(Kbar);
    const int64_t cw = (int64_t)(nsel + 1) * max_chunk;
    int64_t koff = 0, qoff = 0, coff = 0, goff = 0;
    for (int r = 0; r < B; ++r) {
        if (q_len[r] > 0) {
            Batch b;
            chunk_batch(1, L[r], q_len[r], g, opts, b);
            s = run_chunk_refine(b, Qh + qoff * H_I * d_I, W + qoff * H_I, Kh + koff * d_I, Kb + coff * d_I,
                                 cend + coff, nc[r], H_I, d_I, nsel, max_chunk, k, out_idx + qoff * k,
                                 out_score ? out_score + qoff * k : nullptr,
                                 out_chunks ? out_chunks + goff * nsel : nullptr,
                                 out_cand ? out_cand + goff * cw : nullptr, ws, ws_bytes, stream);
            if (s != DSAIDX_OK)
                return s;
        }
        koff += L[r];
        qoff += q_len[r];
        coff += nc[r];
        goff += ceil_div(q_len[r], g);
    }
    return DSAIDX_OK;
}

int indexer_sort_rows(int32_t *idx, float *score, int64_t rows, int k, hipStream_t stream)
{
    if (rows < 0 || rows >= ((int64_t)1 << 40))
        return fail(DSAIDX_EINVAL, "rows=%lld must be in [0, 2^40)", (long long)rows);
    if (k < 1 || k > kSortRowMax)
        return fail(DSAIDX_EINVAL, "k=%d must be in [1, %d]", k, kSortRowMax);
    if (!idx || !score || !aligned(idx, 4) || !aligned(score, 4))
        return fail(DSAIDX_EINVAL, "idx and score must be non-NULL 4-byte aligned pointers");
    if (rows == 0)
        return DSAIDX_OK;
    hipError_t e = launch_sort_rows(idx, score, rows, k, stream);
    return e == hipSuccess ? DSAIDX_OK : hip_fail(e, "sort launch");
}

const char *indexer_last_error(void) { return g_last_error.c_str(); }

const char *indexer_version(void) { return "dsaidx 0.4.0 gfx950"; }

}  // extern "C"
