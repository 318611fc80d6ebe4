/*
 * dsaidx.h - C ABI of the DSA token indexer and of PIVOT query-group indexing
 * on AMD Instinct MI355X (gfx950).
 *
 * What is computed. For a query row t and a key s, the index score of the
 * DeepSeek-Sparse-Attention indexer is
 *
 *     I(t,s) = sum_{j < H_I} w[t][j] * max(0, q[t][j] . k[s])
 *
 * ("PIVOT: Efficient Query-Group Indexing for Token-Level Sparse Attention",
 * arXiv 2607.24593: Eq. (1), whose form the paper describes in its paragraph on
 * observation O3: a per-head ReLU of q_{t,j} . k_s summed over the indexer
 * heads; one key vector per token, shared by every head). Each query keeps
 * the k keys of its causal prefix with the highest scores (motivation
 * paragraph: every query is scored against the entire prefix).
 *
 * PIVOT (same paper, Method and abstract) splits the query rows into groups of
 * g consecutive rows (the last group may be shorter), averages each group into
 * one proxy query and proxy weights per head, scans the causal prefix once
 * with the proxy (up to the group's last position) and keeps c candidates.
 *   - Reuse: every member of the group receives the proxy's top-k.
 *   - Refine: every member re-scores the candidates that are causal for it
 *     with its own query and weights and keeps its own top-k.
 *
 * Conventions shared by every entry point.
 *   Shapes (row-major, contiguous, device memory):
 *     Q        [B][q_len][H_I][d_I]  bf16 (raw 16-bit patterns)
 *     W        [B][q_len][H_I]       fp32
 *     K        [B][L][d_I]           bf16
 *     out_idx  [B][q_len][k]         int32
 *     out_score[B][q_len][k]         fp32, may be NULL
 *     out_cand [B][G][c]             int32, may be NULL, G = ceil(q_len / g)
 *   The q_len query rows of a sequence are its last q_len positions: row r sits
 *   at position L - q_len + r and may select keys 0 .. L - q_len + r (its own
 *   key included). Prefill passes q_len = L; a decode step passes the few new
 *   rows whose keys are already in K.
 *   Ranking: a key outranks another when its score is higher, or when the
 *   scores are equal and its index is lower. A selection of size n is the
 *   first n keys under this ranking.
 *   Output rows hold the selected key indices in ascending index order, with
 *   their scores alongside; a row whose eligible keys number fewer than its
 *   selection size is completed with index -1 and score -inf.
 *   Scores are computed from the bf16 inputs with fp32 accumulation.
 *   Supported (H_I, d_I): (4, 32) and (64, 128). Other pairs return
 *   DSAIDX_EUNSUPPORTED.
 *   Sizes: 1 <= B <= 65535, 0 <= q_len <= L < 2^31, 1 <= k <= 2^20. A batch
 *   without query rows (q_len = 0) is valid: the other arguments are still
 *   checked, nothing is read, written or enqueued, and the pointers may be
 *   NULL.
 *
 * Memory ownership. Every pointer is caller-owned device memory (16-byte
 * aligned for Q, K and ws). The library allocates and frees nothing, never
 * synchronises the stream, and keeps no state between calls except the last
 * error message of the calling thread (and, for indexer_pivot_refine_noalloc
 * only, its fixed per-device scratch array). Work is enqueued on `stream`; results
 * are valid once the stream reaches that point. `ws` is scratch space of at
 * least indexer_workspace_bytes(...) bytes whose content on entry is
 * irrelevant; calls sharing one ws must not overlap in time.
 *
 * Errors. Every entry point returns a dsaidx_status and never throws.
 * Arguments are validated before anything is enqueued; on DSAIDX_EHIP a
 * launch failed and part of the work may have been enqueued. The message of
 * the last non-OK return on the calling thread is in indexer_last_error().
 */
#ifndef DSAIDX_H
#define DSAIDX_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSAIDX_OK = 0,
    DSAIDX_EINVAL = 1,       /* null pointer, size out of range, misalignment */
    DSAIDX_EUNSUPPORTED = 2, /* (H_I, d_I) without a kernel instantiation     */
    DSAIDX_EWORKSPACE = 3,   /* ws_bytes below indexer_workspace_bytes(...)   */
    DSAIDX_EHIP = 4          /* a HIP runtime call or kernel launch failed    */
} dsaidx_status;

typedef enum {
    DSAIDX_DENSE = 0,
    DSAIDX_REUSE = 1,
    DSAIDX_REFINE = 2
} dsaidx_mode;

/*
 * Workspace size in bytes that `mode` needs for these sizes on the current
 * HIP device (it depends on the device's compute-unit count). For
 * DSAIDX_DENSE, g and c are ignored. Returns 0 when the arguments are invalid
 * (the matching entry point would return DSAIDX_EINVAL or
 * DSAIDX_EUNSUPPORTED).
 */
size_t indexer_workspace_bytes(dsaidx_mode mode, int B, int64_t L, int64_t q_len,
                               int H_I, int d_I, int g, int c, int k);

/*
 * Dense DSA indexer (PIVOT paper, motivation paragraph and Eq. (1)): for each
 * query row, the top-k keys of its causal prefix.
 * Sizes as in the shared conventions above.
 */
int indexer_dense(const void *Q, const float *W, const void *K,
                  int B, int64_t L, int64_t q_len, int H_I, int d_I, int k,
                  int32_t *out_idx, float *out_score,
                  void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * PIVOT-Reuse (PIVOT paper, abstract and Method): every member row of a group
 * receives the top-k of the group's proxy scan (so the rows of one group are
 * identical, and early members may hold keys beyond their own position, which
 * the downstream attention masks). c is used only to fill out_cand with the
 * proxy's top-c when out_cand is not NULL; otherwise it is ignored.
 * Requires g >= 1 and, when out_cand is not NULL, k <= c <= 2^20 (the top-k
 * is then the first k of the top-c).
 */
int indexer_pivot_reuse(const void *Q, const float *W, const void *K,
                        int B, int64_t L, int64_t q_len, int H_I, int d_I,
                        int g, int c, int k,
                        int32_t *out_idx, float *out_score, int32_t *out_cand,
                        void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * PIVOT-Refine (PIVOT paper, abstract and Method): each member row re-scores
 * the group's top-c candidates that lie at or before its own position, with
 * its own query and weights, and keeps its top-k. out_cand, when not NULL,
 * receives the candidates. Requires g >= 1 and k <= c <= 2^20.
 */
int indexer_pivot_refine(const void *Q, const float *W, const void *K,
                         int B, int64_t L, int64_t q_len, int H_I, int d_I,
                         int g, int c, int k,
                         int32_t *out_idx, float *out_score, int32_t *out_cand,
                         void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * PIVOT-Refine exactly as indexer_pivot_refine, for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). Its scratch is an
 * array of DSAIDX_SCRATCH_BYTES bytes that the library holds on each GPU it
 * runs on until the process ends (placed when the library's code is loaded on
 * that device; the library calls no allocator). Sizes whose workspace (what
 * indexer_pivot_refine would need with the same arguments, at most
 * indexer_workspace_bytes(DSAIDX_REFINE, ...)) exceeds that return
 * DSAIDX_EWORKSPACE before anything is enqueued; a decode step of 32 requests
 * of 65536 keys (g = 2, c = 4096, k = 2048) needs about 9 MiB. `stream` must
 * belong to the current device. Every call on one GPU uses that GPU's single
 * copy of the scratch: calls that overlap in time on one GPU (other streams,
 * other threads) race and must be serialised by the caller. No content of the
 * scratch carries over from one call to the next. Outputs, ranking, padding,
 * shapes and errors as for indexer_pivot_refine.
 */
#define DSAIDX_SCRATCH_BYTES ((size_t)64 << 20)

int indexer_pivot_refine_noalloc(const void *Q, const float *W, const void *K,
                                 int B, int64_t L, int64_t q_len, int H_I, int d_I,
                                 int g, int c, int k,
                                 int32_t *out_idx, float *out_score, int32_t *out_cand,
                                 hipStream_t stream);

/*
 * Options of the variable-length PIVOT entry points (NULL: all defaults).
 *   guard   see below; 0 (default) turns the guard off.
 *   proxy   how a group becomes one proxy query and proxy weights (PIVOT
 *           paper, ablation on the proxy aggregation strategy, and the
 *           experimental setup's mean pooling within a local window):
 *             DSAIDX_PROXY_MEAN  (default) the per-head mean of `window`
 *                                consecutive members ending at the group's
 *                                last row; window 0, or a window at least
 *                                the group's size, averages the whole group;
 *             DSAIDX_PROXY_FIRST the first member's query and weights;
 *             DSAIDX_PROXY_LAST  the last member's query and weights.
 *           A mean is an fp32 sum in row order divided in fp32 by the member
 *           count and rounded to bf16 (nearest even); weights stay fp32.
 *   window  members averaged by DSAIDX_PROXY_MEAN (>= 0; ignored otherwise).
 */
typedef enum {
    DSAIDX_PROXY_MEAN = 0,
    DSAIDX_PROXY_FIRST = 1,
    DSAIDX_PROXY_LAST = 2
} dsaidx_proxy;

typedef struct {
    int64_t guard;
    int32_t proxy;
    int32_t window;
} dsaidx_pivot_opts;

/*
 * Batches of requests of different lengths (PIVOT paper, Method: query
 * groups are contiguous, never cross a request boundary, and the last group
 * of a request may be smaller), with an optional guard for short prefixes
 * (Results: PIVOT falls back to a dense scan for short groups so that it is
 * never slower than the dense indexer).
 *
 *   L, q_len  host arrays of B entries: request b has L[b] keys and its
 *             queries are its last q_len[b] positions (0 <= q_len[b] <= L[b]
 *             < 2^31). The arrays are read during the call only. A request
 *             with q_len[b] = 0 (L[b] may then be 0 too) has no rows, groups
 *             or candidate rows and takes no part in the call; if no request
 *             has queries, nothing is read, written or enqueued and the
 *             device pointers may be NULL.
 *   Packed layouts (device memory, requests in order, no padding):
 *     Q        [sum q_len][H_I][d_I]  bf16
 *     W        [sum q_len][H_I]       fp32
 *     K        [sum L][d_I]           bf16
 *     out_idx  [sum q_len][k]         int32
 *     out_score[sum q_len][k]         fp32, may be NULL
 *     out_cand [sum G][c]             int32, may be NULL; G[b] = ceil(q_len[b] / g)
 *   opts->guard  a group whose last position t_last satisfies t_last + 1 <= guard
 *             (its whole causal prefix holds at most `guard` keys) is scored
 *             densely: each of its rows receives its dense top-k, and its
 *             candidate row, if requested, is filled with -1. guard = 0 turns
 *             the guard off. For Refine, any guard <= c leaves the results
 *             unchanged (a group whose prefix fits in c keys has every key as
 *             a candidate, so Refine equals the dense indexer there) and only
 *             skips work; for Reuse the guarded rows change from the shared
 *             proxy selection to each row's own dense selection.
 *   Everything else (ranking, output order, padding, supported shapes,
 *   ownership, errors) is as for the uniform entry points. The call uploads
 *   B small request descriptors into ws through kernel launches on `stream`.
 */
size_t indexer_varlen_workspace_bytes(dsaidx_mode mode, int B, const int64_t *L, const int64_t *q_len,
                                      int H_I, int d_I, int g, int c, int k,
                                      const dsaidx_pivot_opts *opts);

int indexer_dense_varlen(const void *Q, const float *W, const void *K,
                         int B, const int64_t *L, const int64_t *q_len, int H_I, int d_I, int k,
                         int32_t *out_idx, float *out_score,
                         void *ws, size_t ws_bytes, hipStream_t stream);

int indexer_pivot_reuse_varlen(const void *Q, const float *W, const void *K,
                               int B, const int64_t *L, const int64_t *q_len, int H_I, int d_I,
                               int g, int c, int k, const dsaidx_pivot_opts *opts,
                               int32_t *out_idx, float *out_score, int32_t *out_cand,
                               void *ws, size_t ws_bytes, hipStream_t stream);

int indexer_pivot_refine_varlen(const void *Q, const float *W, const void *K,
                                int B, const int64_t *L, const int64_t *q_len, int H_I, int d_I,
                                int g, int c, int k, const dsaidx_pivot_opts *opts,
                                int32_t *out_idx, float *out_score, int32_t *out_cand,
                                void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Key-axis coarse stage: hierarchical indexing over chunks of keys.
 *
 * "Not All Tokens Deserve Equal Resolution: Score-Adaptive Indexing for
 * Sparse Attention in Long-Context LLMs" (SCALE), abstract: contiguous runs
 * of keys ("chunks") are represented by their mean key; a query scores the
 * summaries, keeps the best chunks and refines their keys with the
 * token-level indexer. Fixed blocks of 64 keys are the HISA-64 baseline;
 * SCALE re-partitions the keys under the same number of chunks.
 *
 * A partition of each request's L keys is given by its chunk ends
 *     cend [B][nc]  int32: chunk b holds keys [cend[b-1], cend[b]) (cend[-1] =
 *                   0); strictly ascending, cend[nc-1] = L.
 * The summaries are
 *     Kbar [B][nc][d_I]  bf16: per dimension, the fp32 sum of the chunk's keys
 *                   in index order divided (IEEE fp32) by the chunk's size,
 *                   rounded to bf16 nearest-even (a stated reading: the paper
 *                   gives no precision).
 * Uniform batches (B requests of L keys, the last q_len positions queried,
 * L >= 1 and q_len >= 1), and variable-length ones (the *_varlen calls
 * below).
 * ------------------------------------------------------------------------ */

/* Fixed blocks: cend[b] = min((b + 1) * block, L) for b < nc = ceil(L / block),
 * for each of the B requests. cend: [B][nc] device memory. */
int indexer_chunks_fixed(int B, int64_t L, int block, int32_t *cend, hipStream_t stream);

/* Score-adaptive chunks (the reading taken of SCALE's rule; the abstract gives
 * no procedure): start from fixed blocks of `block` keys (block even,
 * n = ceil(L / block) blocks, at most 262144 per request). The split gain of a
 * full block is the drop of the squared reconstruction error by the mean,
 * D(block) - D(first half) - D(second half); the merge loss of an aligned pair
 * of full blocks (2j, 2j+1) is D(pair) - D(2j) - D(2j+1). Splits are taken in
 * order of gain (highest first), merges in order of loss (lowest first), ties
 * to the lower number, a split and a merge together while the gain exceeds
 * the loss; a block of a merged pair is not split and a pair holding a split
 * block is not merged (such candidates are passed over). The partition keeps
 * n chunks of block/2, block or 2*block keys (the last one may be short).
 * D is evaluated in double precision in a fixed order (per dimension the sums
 * of x and x*x over the keys in index order, then sum over dimensions of
 * sum(x^2) - sum(x)^2 / n in dimension order), so the decisions are
 * reproducible. K: [B][L][d_I] bf16; cend: [B][n] int32. ws: scratch of
 * indexer_chunks_adaptive_workspace_bytes(B, L, block) bytes. */
size_t indexer_chunks_adaptive_workspace_bytes(int B, int64_t L, int block);
int indexer_chunks_adaptive(const void *K, int B, int64_t L, int d_I, int block, int32_t *cend,
                            void *ws, size_t ws_bytes, hipStream_t stream);

/* Summaries of chunks first .. nc-1 of every request (first > 0 refreshes only
 * the chunks that changed, e.g. after keys were appended to the last one).
 * K: [B][L][d_I] bf16; cend: [B][nc]; Kbar: [B][nc][d_I] bf16 (rows below
 * `first` are left untouched). */
int indexer_chunk_means(const void *K, int B, int64_t L, int d_I, const int32_t *cend, int64_t nc,
                        int64_t first, void *Kbar, hipStream_t stream);

/* Chunk-level candidates and token-level Refine. For each group of g query
 * rows (as for PIVOT: contiguous, the last one may be shorter; proxy by
 * opts->proxy and opts->window; g = 1 makes the proxy the row itself):
 *  1. the chunks complete at the group's last position t_last, those with
 *     cend <= t_last + 1, are scored by the proxy with I(t,s), the summary in
 *     place of the key; the nsel best are kept (ranking as above);
 *  2. the candidate list holds the keys of those chunks in index order, then
 *     the keys after the last complete chunk up to t_last (the chunk in
 *     progress has no summary yet and its keys are always kept), then -1, in
 *     a row of cw = (nsel + 1) * max_chunk entries;
 *  3. every member re-scores the candidates at or before its own position and
 *     keeps its top-k (out_idx, out_score as for the other entry points).
 * max_chunk: the largest chunk size in cend (block for fixed blocks, 2*block
 * for adaptive ones; a larger value only widens the rows); a larger chunk
 * makes the list exceed cw and is truncated. Requires cw >= k.
 * opts->guard (>= 0; PIVOT, results, the guardrail: short groups fall back to
 * the dense indexer): a group whose whole causal prefix holds at most `guard`
 * keys (t_last + 1 <= guard) is scored as dense rows instead, its out_chunks
 * and out_cand rows are -1.
 *   Kbar     [B][nc][d_I]     summaries (indexer_chunk_means)
 *   out_chunks [B][G][nsel]   int32, may be NULL: selected chunks, ascending, -1 after
 *   out_cand [B][G][cw]       int32, may be NULL: the candidate lists
 * ws: indexer_chunk_refine_workspace_bytes(...) bytes, with the call's opts
 * (NULL: the defaults; a guard adds the dense pass of the guarded rows). */
size_t indexer_chunk_refine_workspace_bytes(int B, int64_t L, int64_t q_len, int H_I, int d_I, int g,
                                            int64_t nc, int nsel, int max_chunk, int k,
                                            const dsaidx_pivot_opts *opts);
int indexer_chunk_refine(const void *Q, const float *W, const void *K, const void *Kbar,
                         const int32_t *cend, int64_t nc, int B, int64_t L, int64_t q_len,
                         int H_I, int d_I, int g, int nsel, int max_chunk, int k,
                         const dsaidx_pivot_opts *opts, int32_t *out_idx, float *out_score,
                         int32_t *out_chunks, int32_t *out_cand,
                         void *ws, size_t ws_bytes, hipStream_t stream);

/* Variable-length batches on the key-chunk path (the calls above for B
 * requests of their own lengths). Request r has L[r] >= 1 keys, q_len[r]
 * queried positions (0 <= q_len[r] <= L[r], the last q_len[r] of its keys) and
 * nc[r] chunks (1 <= nc[r] <= L[r]); L, q_len and nc are host arrays of B
 * entries. Device arrays are the requests' rows one after the other:
 *   K [sum L][d_I], Q [sum q_len][H_I][d_I], W [sum q_len][H_I],
 *   cend [sum nc] (each request's chunk ends counted from its own first key,
 *   as in the uniform form), Kbar [sum nc][d_I],
 *   out_idx, out_score [sum q_len][k], out_chunks [sum G_r][nsel],
 *   out_cand [sum G_r][cw] with G_r = ceil(q_len[r] / g), cw = (nsel + 1) * max_chunk.
 * Every size is checked before anything is enqueued (a request with
 * q_len[r] = 0 only advances the offsets); then each request runs as a
 * uniform batch of one, in order, on `stream`, with the launches of that
 * form, reusing ws: suited to batches of few long requests. Results equal
 * those of the uniform calls on each request alone. fixed: nc[r] =
 * ceil(L[r] / block) chunk ends per request; adaptive: as indexer_chunks_adaptive
 * per request (ws: the largest request's scratch). */
int indexer_chunks_fixed_varlen(int B, const int64_t *L, int block, int32_t *cend, hipStream_t stream);
size_t indexer_chunks_adaptive_varlen_workspace_bytes(int B, const int64_t *L, int block);
int indexer_chunks_adaptive_varlen(const void *K, int B, const int64_t *L, int d_I, int block, int32_t *cend,
                                   void *ws, size_t ws_bytes, hipStream_t stream);
int indexer_chunk_means_varlen(const void *K, int B, const int64_t *L, int d_I, const int32_t *cend,
                               const int64_t *nc, void *Kbar, hipStream_t stream);
size_t indexer_chunk_refine_varlen_workspace_bytes(int B, const int64_t *L, const int64_t *q_len, int H_I,
                                                   int d_I, int g, const int64_t *nc, int nsel, int max_chunk,
                                                   int k, const dsaidx_pivot_opts *opts);
int indexer_chunk_refine_varlen(const void *Q, const float *W, const void *K, const void *Kbar,
                                const int32_t *cend, const int64_t *nc, int B, const int64_t *L,
                                const int64_t *q_len, int H_I, int d_I, int g, int nsel, int max_chunk, int k,
                                const dsaidx_pivot_opts *opts, int32_t *out_idx, float *out_score,
                                int32_t *out_chunks, int32_t *out_cand,
                                void *ws, size_t ws_bytes, hipStream_t stream);

/* Rows of a selection in ranking order. The entry points above write each
 * output row in ascending index order (the order in which a sparse attention
 * gathers keys best); this call rewrites `rows` rows of k (index, score) pairs
 * in place so that each runs in ranking order instead: score descending,
 * equal scores by ascending index, the -1 padding (score -inf) last ("each
 * query keeps the k highest-scoring keys": PIVOT, motivation paragraph; the
 * tie rule is the reading stated at the top of this header).
 *   idx   [rows][k] int32, score [rows][k] fp32 (both required; e.g. out_idx
 *         and out_score of any entry point above, rows = B * q_len)
 *   k     1 .. 8192
 * A -0 score is written back as +0. Errors as above (EINVAL before launch). */
int indexer_sort_rows(int32_t *idx, float *score, int64_t rows, int k, hipStream_t stream);

/* Message of the last non-OK return on the calling thread ("" if none). */
const char *indexer_last_error(void);

/* Library version string, e.g. "dsaidx 0.4.0 gfx950". */
const char *indexer_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSAIDX_H */
