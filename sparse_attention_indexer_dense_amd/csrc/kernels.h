// kernels.h - launch parameters of the indexer kernels and their host-side
// launchers (internal to the library; the public interface is dsaidx.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsaidx {

enum { kDense = 0, kProxy = 1, kRefine = 2 };

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
    int B;
    int64_t L, q_len;
    int64_t g, c, G;
    int64_t nblk_per_batch;  // kDense/kProxy: row blocks per batch item
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
};

struct PoolParams {
    const uint16_t *Q;
    const float *W;
    int B;
    int64_t q_len, g, G;
    uint16_t *Qp;  // [B][G][H][D]
    float *Wp;     // [B][G][H]
};

// Split-key scoring for few rows (split.hip): every workgroup scores a chunk
// of key positions for a group of rows and stores the fp32 scores.
struct SplitScoreParams {
    const uint16_t *Q;    // queries or proxies (as in ScanParams)
    const float *W;
    const uint16_t *K;
    const int32_t *cand;  // kRefine: candidate lists [B][G][c]
    int mode;
    int B;
    int64_t L, q_len, g, c, G;
    int64_t nrows;        // score rows per batch item
    int64_t rowlen;       // positions per score row (L, or c for kRefine)
    int64_t chunk;        // positions per workgroup
    float *scores;        // [B][nrows][rowlen]
};

struct SplitSelectParams {
    const float *scores;
    const int32_t *cand;
    int mode;
    int B;
    int64_t L, q_len, g, c, G;
    int64_t nrows, rowlen;
    int sel, sel2;
    int32_t *o1_idx;
    float *o1_score;
    int o1_members;
    int32_t *o2_idx;
    float *o2_score;
};

constexpr int kSplitWaves = 4;
constexpr int kSplitSpanMax = 1024;  // key positions one wave of split_score_kernel covers
constexpr int kSelectThreads = 1024;

size_t scan_lds_bytes(int H, int D, int NW);
hipError_t launch_scan_select(int H, int D, int NW, int mode, const ScanParams &prm, int grid,
                              hipStream_t stream);
hipError_t launch_pool(int H, int D, const PoolParams &prm, hipStream_t stream);
hipError_t launch_split_score(int H, int D, const SplitScoreParams &prm, dim3 grid, hipStream_t stream);
hipError_t launch_split_select(const SplitSelectParams &prm, hipStream_t stream);

}  // namespace dsaidx
