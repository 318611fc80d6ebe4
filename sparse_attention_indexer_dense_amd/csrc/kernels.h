// kernels.h - launch parameters of the indexer kernels and their host-side
// launchers (internal to the library; the public interface is dsaidx.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsaidx {

enum { kDense = 0, kProxy = 1, kRefine = 2 };

// One request of a variable-length batch (a device array in the workspace).
// A group never spans two requests.
struct ReqDesc {
    int64_t key_off;  // first row of the request's keys in K
    int64_t q_off;    // first row of its queries in Q and W, and of its output rows
    int64_t g_off;    // first of its groups in the proxy and candidate rows
    int64_t L;        // keys
    int64_t q_len;    // queries: the last q_len positions
    int64_t m0;       // groups [0, m0) are guarded: their rows are scored as dense rows
};

// Geometry of request bi: from the descriptor array, or that of a uniform
// batch (B requests of L keys and q_len queries, m0 guarded groups each).
struct Req {
    int64_t key_off, q_off, g_off, L, q_len, G, m0;
};

__device__ __forceinline__ Req request_of(const ReqDesc *req, int bi, int64_t L, int64_t q_len, int64_t g,
                                          int64_t m0)
{
    Req r;
    if (req) {
        const ReqDesc d = req[bi];
        r.key_off = d.key_off;
        r.q_off = d.q_off;
        r.g_off = d.g_off;
        r.L = d.L;
        r.q_len = d.q_len;
        r.m0 = d.m0;
    } else {
        r.key_off = (int64_t)bi * L;
        r.q_off = (int64_t)bi * q_len;
        r.g_off = (int64_t)bi * ((q_len + g - 1) / g);
        r.L = L;
        r.q_len = q_len;
        r.m0 = m0;
    }
    r.G = (r.q_len + g - 1) / g;
    return r;
}

// Rows a dense pass covers in a request: all of them, or (guard_rows) those
// of its guarded groups.
__device__ __forceinline__ int64_t dense_rows(const Req &r, int64_t g, int guard_rows)
{
    if (!guard_rows)
        return r.q_len;
    const int64_t x = r.m0 * g;
    return x < r.q_len ? x : r.q_len;
}

// One kept (score, key index) pair of a row's candidate buffer.
struct Entry {
    float score;
    int32_t idx;
};

// Fused score + select over many rows (scan.hip).
struct ScanParams {
    const uint16_t *Q;     // kDense/kRefine: queries [B][q_len][H][D]; kProxy: proxies [B][G][H][D]
    const float *W;        // matching weights
    const uint16_t *K;     // keys [B][L][D]
    const int32_t *cand;   // kRefine: candidate lists [B][G][c]
    const ReqDesc *req;    // requests of a variable-length batch (nullptr: uniform)
    int B;
    int64_t L, q_len;      // uniform batch: keys and queries per request
    int64_t g, c, G;
    int64_t m0;            // uniform batch: guarded groups per request
    int guard_rows;        // kDense: only the rows of guarded groups
    int64_t nblk_per_batch;  // blocks per request (the largest request's count)
    int64_t nblocks;         // total blocks
    int64_t member_chunks;   // kRefine: member chunks per group
    int sel, sel2;           // selection sizes (sel2 = 0: none)
    int32_t *o1_idx;         // output of the sel selection
    float *o1_score;
    int o1_members;          // kProxy: 1 = write to every member row, 0 = one row per group
    int32_t *o2_idx;         // kProxy: output of the sel2 selection (member rows)
    float *o2_score;
    Entry *slots;            // per (workgroup, wave) candidate buffers
    int cap;                 // entries per buffer
    // key-chunk coarse stage (kProxy): K holds krows chunk summaries per
    // request and group row m scans summaries 0..glim[m] (nullptr: token keys)
    const int32_t *glim;
    int64_t krows;
    const int32_t *cand_n;   // kRefine: keys in each group's list (nullptr: min(c, t_last + 1))
};

// PIVOT-Refine with the members' scores in LDS (refine.hip): groups of at
// most four members and at most kRefineLdsCandMax candidates.
constexpr int kRefineLdsCandMax = 4608;

struct RefineLdsParams {
    const uint16_t *Q;     // queries [B][q_len][H][D]
    const float *W;
    const uint16_t *K;     // keys [B][L][D]
    const int32_t *cand;   // candidate lists [B][G][c] (or packed per request)
    const ReqDesc *req;    // requests of a variable-length batch (nullptr: uniform)
    int B;
    int64_t L, q_len, g, c, m0;
    int k;
    int32_t *out_idx;      // [rows][k]
    float *out_score;      // [rows][k] or nullptr
    int64_t nwork;         // groups of the launch: B x groups of the largest request
    const int32_t *cand_n; // keys in each group's list (nullptr: min(c, t_last + 1))
};

struct PoolParams {
    const uint16_t *Q;
    const float *W;
    const ReqDesc *req;
    int B;
    int64_t L, q_len, g, m0;
    int64_t gmax;  // groups of the largest request
    int proxy;     // 0: mean of `window` members ending at the last (0: all), 1: first, 2: last member
    int64_t window;
    uint16_t *Qp;  // [groups][H][D]
    float *Wp;     // [groups][H]
};

// Split-key scoring for few rows (split.hip): every workgroup scores a chunk
// of key positions for a group of rows and stores the fp32 scores.
struct SplitScoreParams {
    const uint16_t *Q;    // queries or proxies (as in ScanParams)
    const float *W;
    const uint16_t *K;
    const int32_t *cand;  // kRefine: candidate lists [B][G][c]
    const ReqDesc *req;
    int mode;
    int B;
    int64_t L, q_len, g, c, G, m0;
    int guard_rows;
    int64_t nrows;        // score rows per batch item (the largest request's count)
    int64_t rowlen;       // positions per score row (L, or c for kRefine)
    int64_t chunk;        // positions per workgroup
    int64_t row0;         // first row of this launch (grid y covers at most 65535 rows)
    float *scores;        // [B][nrows][rowlen]
    const int32_t *glim;  // as in ScanParams
    int64_t krows;
    const int32_t *cand_n;
};

struct SplitSelectParams {
    const float *scores;
    const int32_t *cand;
    const ReqDesc *req;
    int mode;
    int B;
    int64_t L, q_len, g, c, G, m0;
    int guard_rows;
    int64_t nrows, rowlen;
    int sel, sel2;
    int32_t *o1_idx;
    float *o1_score;
    int o1_members;
    int32_t *o2_idx;
    float *o2_score;
    const int32_t *glim;  // as in ScanParams
    const int32_t *cand_n;
};

// Key chunks (chunks.hip).
struct ChunkExpandParams {
    const int32_t *chunks;  // selected chunks [B][G][nsel], ascending, -1 after the last
    const int32_t *cend;    // chunk ends [B][nc]
    const int32_t *glim;    // last complete chunk of each group [B][G]
    int64_t L, q_len, g, nc;
    int nsel;
    int64_t cw;             // candidate row width
    int32_t *cand;          // [B][G][cw]
    int32_t *cand_n;        // [B][G]
};

// Adaptive chunking: at most this many blocks per request (its per-block
// flags are LDS bitmaps); up to kAdaptBlocksLds blocks the gains and losses
// are sorted in LDS, beyond that in the workspace.
constexpr int kAdaptBlocksMax = 1 << 18;
constexpr int kAdaptBlocksLds = 4096;

struct ChunkAdaptParams {
    const uint16_t *K;      // [B][L][D]
    int64_t L, block;
    int64_t n, nfull, npair;  // blocks, full blocks, aligned pairs of full blocks
    int64_t g2, p2;         // nfull and npair rounded up to powers of two
    double *gain;           // [B][nfull] split gains
    double *loss;           // [B][npair] merge losses
    double *gk;             // n > kAdaptBlocksLds: sort space [B][g2] gains, [B][g2] their blocks,
    int32_t *gi;            //   [B][p2] losses, [B][p2] their pairs (unused otherwise)
    double *lk;
    int32_t *li;
    int32_t *cend;          // [B][n]
};

constexpr int kSplitWaves = 4;
constexpr int kSplitSpanMax = 1024;  // key positions one wave of split_score_kernel covers
constexpr int kSelectThreads = 1024;

// Request descriptors travel to the workspace as launch arguments, in chunks.
constexpr int kDescChunk = 24;
struct DescChunk {
    int n, first;
    ReqDesc d[kDescChunk];
};

size_t scan_lds_bytes(int H, int D, int NW);
hipError_t launch_set_desc(const DescChunk &ch, ReqDesc *dst, hipStream_t stream);
// Candidate rows [groups][c] of guarded groups (not computed) set to -1.
hipError_t launch_fill_guarded(const ReqDesc *req, int B, int64_t L, int64_t q_len, int64_t g, int64_t m0,
                               int64_t gmax, int64_t c, int32_t *cand, hipStream_t stream);
hipError_t launch_scan_select(int H, int D, int NW, int mode, const ScanParams &prm, int grid,
                              hipStream_t stream);
hipError_t launch_pool(int H, int D, const PoolParams &prm, hipStream_t stream);
// grid workgroups (at most one per CU fits its LDS), each looping over the
// prm.nwork groups of the launch
hipError_t launch_refine_lds(int H, int D, const RefineLdsParams &prm, int grid, hipStream_t stream);
// mr: score rows per wave (2: Refine member rows paired over their group's
// candidate list; needs an even g)
hipError_t launch_split_score(int H, int D, const SplitScoreParams &prm, int mr, dim3 grid, hipStream_t stream);
hipError_t launch_split_select(const SplitSelectParams &prm, hipStream_t stream);
hipError_t launch_chunk_fixed(int B, int64_t L, int64_t block, int64_t nc, int32_t *cend, hipStream_t stream);
hipError_t launch_chunk_means(int D, const uint16_t *K, int B, int64_t L, const int32_t *cend, int64_t nc,
                              int64_t first, uint16_t *Kbar, hipStream_t stream);
hipError_t launch_chunk_limits(int B, int64_t L, int64_t q_len, int64_t g, const int32_t *cend, int64_t nc,
                               int32_t *glim, hipStream_t stream);
hipError_t launch_chunk_expand(const ChunkExpandParams &prm, int64_t groups, hipStream_t stream);
hipError_t launch_chunk_adaptive(int D, int B, const ChunkAdaptParams &prm, hipStream_t stream);
// Rows of k (index, score) pairs reordered in place into ranking order (sort.hip).
constexpr int kSortRowMax = 8192;
hipError_t launch_sort_rows(int32_t *idx, float *score, int64_t rows, int k, hipStream_t stream);

}  // namespace dsaidx
