/*
 * oracle.c - plain CPU reference for the DSA token indexer and for PIVOT's
 * query-group variants (Reuse and Refine).
 *
 * TEST INFRASTRUCTURE ONLY. Its users are the test-suite, the smoke check and
 * the benchmark's CPU-baseline leg. The GPU library never includes, links or
 * calls this file, and this file includes nothing from the library.
 *
 * Arithmetic. Every bf16 or fp32 input is widened exactly to double. Scores
 * are accumulated in double, on one thread, in plain loop order. The one place
 * where fp32/bf16 rounding is part of the definition is the group proxy
 * (orc_proxy), whose rounding is a stated reading, not something the paper fixes.
 *
 * Sources. "PIVOT: Efficient Query-Group Indexing for Token-Level Sparse
 * Attention" (arXiv 2607.24593):
 *  - index score, Eq. (1): referred to in the motivation paragraph and in the
 *    paragraph on observation O3 (per-head ReLU of q_{t,j} . k_s, summed over
 *    the indexer heads). The display of Eq. (1) is missing from the page; the
 *    weighted form I(t,s) = sum_j w_{t,j} * max(0, q_{t,j} . k_s) is the
 *    reading taken, with one key vector per token shared by every head (the
 *    O3 paragraph writes k_s without a head index);
 *  - per-query top-k over the entire prefix: motivation paragraph;
 *  - contiguous query groups, short last group: Method, prefill grouping;
 *  - proxy by per-head mean pooling: experimental setup and the ablation on
 *    the proxy aggregation strategy;
 *  - one shared causal scan, candidate set of size c, Reuse and Refine:
 *    abstract and Method.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL 1

#define ORC_PROXY_MEAN 0
#define ORC_PROXY_FIRST 1
#define ORC_PROXY_LAST 2

int orc_proxy_ex(const uint16_t *Q, const float *W, int64_t q_len, int H, int d,
                 int64_t g, int64_t m, int proxy, int64_t window, uint16_t *qbar, float *wbar);

/* Exact widening of a bf16 bit pattern (the upper half of an fp32). */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even. Inputs are finite. */
static uint16_t float_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/*
 * Index score of one query row against keys 0..n-1 (Eq. (1) as read above):
 *   score[s] = sum_j w[j] * max(0, sum_e q[j][e] * K[s][e])
 * and the tolerance mass
 *   mass[s]  = sum_j |w[j]| * sum_e |q[j][e] * K[s][e]|,
 * a bound on the magnitude of every partial sum, used to size the rounding
 * tolerance of a low-precision implementation. q is [H][d] bf16, w is [H]
 * fp32, K is [n][d] bf16 (row-major). mass may be NULL.
 */
int orc_scores(const uint16_t *q, const float *w, const uint16_t *K,
               int H, int d, int64_t n, double *score, double *mass)
{
    if (!q || !w || !K || !score || H < 1 || d < 1 || n < 0)
        return ORC_EINVAL;
    double *qd = malloc(sizeof(double) * (size_t)H * (size_t)d);
    double *kd = malloc(sizeof(double) * (size_t)d);
    if (!qd || !kd) {
        free(qd);
        free(kd);
        return ORC_EINVAL;
    }
    for (int64_t i = 0; i < (int64_t)H * d; ++i)
        qd[i] = bf16_to_double(q[i]);
    for (int64_t s = 0; s < n; ++s) {
        for (int e = 0; e < d; ++e)
            kd[e] = bf16_to_double(K[s * d + e]);
        double total = 0.0, bound = 0.0;
        for (int j = 0; j < H; ++j) {
            double dot = 0.0, adot = 0.0;
            for (int e = 0; e < d; ++e) {
                double p = qd[(int64_t)j * d + e] * kd[e];
                dot += p;
                adot += fabs(p);
            }
            double relu = dot > 0.0 ? dot : 0.0;
            total += (double)w[j] * relu;
            bound += fabs((double)w[j]) * adot;
        }
        score[s] = total;
        if (mass)
            mass[s] = bound;
    }
    free(qd);
    free(kd);
    return ORC_OK;
}

typedef struct {
    double score;
    int64_t idx;
} orc_entry;

/*
 * Ranking used for every top-k and top-c: a outranks b when its score is
 * higher, or when the scores are equal and its index is lower. The paper
 * does not state a tie rule; this one makes every selection unique.
 */
static int outranks_first(const void *pa, const void *pb)
{
    const orc_entry *a = pa, *b = pb;
    if (a->score > b->score)
        return -1;
    if (a->score < b->score)
        return 1;
    if (a->idx < b->idx)
        return -1;
    if (a->idx > b->idx)
        return 1;
    return 0;
}

/*
 * Top-k of n scored keys: the first min(k, n) keys under the ranking above,
 * written in ranking order; the remaining k - min(k, n) slots get index -1
 * and score -inf. idx may be NULL, meaning key i has index i. out_score may
 * be NULL.
 */
int orc_select(const double *score, const int64_t *idx, int64_t n, int64_t k,
               int64_t *out_idx, double *out_score)
{
    if (!score || !out_idx || n < 0 || k < 1)
        return ORC_EINVAL;
    orc_entry *e = malloc(sizeof(orc_entry) * (size_t)(n > 0 ? n : 1));
    if (!e)
        return ORC_EINVAL;
    for (int64_t i = 0; i < n; ++i) {
        e[i].score = score[i];
        e[i].idx = idx ? idx[i] : i;
    }
    qsort(e, (size_t)n, sizeof(orc_entry), outranks_first);
    int64_t m = n < k ? n : k;
    for (int64_t i = 0; i < k; ++i) {
        out_idx[i] = i < m ? e[i].idx : -1;
        if (out_score)
            out_score[i] = i < m ? e[i].score : -INFINITY;
    }
    free(e);
    return ORC_OK;
}

/*
 * Dense indexer for selected query rows of one sequence. The q_len query rows
 * are the last q_len positions of a sequence of L keys, so row r sits at
 * position pos(r) = L - q_len + r and is scored against keys 0..pos(r)
 * (causal, the key at its own position included: "the entire prefix").
 * Q is [q_len][H][d] bf16, W is [q_len][H] fp32, K is [L][d] bf16.
 * Outputs are [nrows][k] in ranking order.
 */
int orc_dense_rows(const uint16_t *Q, const float *W, const uint16_t *K,
                   int64_t L, int64_t q_len, int H, int d, int64_t k,
                   const int64_t *rows, int64_t nrows,
                   int64_t *out_idx, double *out_score)
{
    if (!Q || !W || !K || !rows || !out_idx || L < 1 || q_len < 1 || q_len > L || k < 1)
        return ORC_EINVAL;
    double *sc = malloc(sizeof(double) * (size_t)L);
    if (!sc)
        return ORC_EINVAL;
    int rc = ORC_OK;
    for (int64_t i = 0; i < nrows && rc == ORC_OK; ++i) {
        int64_t r = rows[i];
        if (r < 0 || r >= q_len) {
            rc = ORC_EINVAL;
            break;
        }
        int64_t n = L - q_len + r + 1;
        rc = orc_scores(Q + r * H * d, W + r * H, K, H, d, n, sc, NULL);
        if (rc == ORC_OK)
            rc = orc_select(sc, NULL, n, k, out_idx + i * k,
                            out_score ? out_score + i * k : NULL);
    }
    free(sc);
    return rc;
}

/*
 * Proxy of query group m. Groups are contiguous runs of g query rows starting
 * at row 0; the last group holds the remaining q_len - m*g rows when g does not
 * divide q_len (Method: a group never crosses a request boundary and the last
 * group of a request may be smaller). The proxy is the per-head mean of the
 * members' queries and weights (mean pooling over the whole group).
 * Reading of the unstated precision: each query element is summed over the
 * members in row order in fp32, divided in fp32 by the member count, and
 * rounded to bf16 (nearest, ties to even); each weight is summed in fp32 and
 * divided in fp32. qbar is [H][d] bf16, wbar is [H] fp32.
 */
/* Mean of query rows [a, b) per head and dimension: fp32 sum in row order,
 * fp32 division by the row count, rounded to bf16 (nearest even); the
 * weights likewise, kept in fp32. */
static void mean_rows(const uint16_t *Q, const float *W, int H, int d, int64_t a, int64_t b,
                      uint16_t *qbar, float *wbar)
{
    float cnt = (float)(b - a);
    for (int64_t x = 0; x < (int64_t)H * d; ++x) {
        float acc = 0.0f;
        for (int64_t r = a; r < b; ++r)
            acc += bf16_to_float(Q[r * H * d + x]);
        qbar[x] = float_to_bf16_rne(acc / cnt);
    }
    for (int j = 0; j < H; ++j) {
        float acc = 0.0f;
        for (int64_t r = a; r < b; ++r)
            acc += W[r * H + j];
        wbar[j] = acc / cnt;
    }
}

int orc_proxy(const uint16_t *Q, const float *W, int64_t q_len, int H, int d,
              int64_t g, int64_t m, uint16_t *qbar, float *wbar)
{
    return orc_proxy_ex(Q, W, q_len, H, d, g, m, ORC_PROXY_MEAN, 0, qbar, wbar);
}

/*
 * Proxy of group m (rows r0 .. r1-1) under an aggregation strategy (PIVOT
 * paper, ablation on the proxy aggregation strategy, and the experimental
 * setup's mean pooling within a local window):
 *   ORC_PROXY_MEAN  - mean of the members in a window of `window` rows; the
 *                     reading taken for a window narrower than the group is
 *                     its last `window` members (those with the longest
 *                     prefixes); window 0, or one at least the group's size,
 *                     averages the whole group;
 *   ORC_PROXY_FIRST - the first member's query and weights (an endpoint proxy);
 *   ORC_PROXY_LAST  - the last member's.
 */
int orc_proxy_ex(const uint16_t *Q, const float *W, int64_t q_len, int H, int d,
                 int64_t g, int64_t m, int proxy, int64_t window, uint16_t *qbar, float *wbar)
{
    if (!Q || !W || !qbar || !wbar || g < 1 || m < 0 || m * g >= q_len || window < 0)
        return ORC_EINVAL;
    int64_t r0 = m * g;
    int64_t r1 = r0 + g < q_len ? r0 + g : q_len;
    int64_t a, b;
    if (proxy == ORC_PROXY_MEAN) {
        int64_t n = r1 - r0;
        int64_t wn = (window == 0 || window >= n) ? n : window;
        a = r1 - wn;
        b = r1;
    } else if (proxy == ORC_PROXY_FIRST) {
        a = r0;
        b = r0 + 1;
    } else if (proxy == ORC_PROXY_LAST) {
        a = r1 - 1;
        b = r1;
    } else {
        return ORC_EINVAL;
    }
    mean_rows(Q, W, H, d, a, b, qbar, wbar);
    return ORC_OK;
}

/* The candidate list handed to Refine: min(c, t_last+1) distinct keys in
 * [0, t_last], then -1 padding. */
static int valid_candidates(const int64_t *cand, int64_t c, int64_t t_last)
{
    int64_t want = c < t_last + 1 ? c : t_last + 1;
    char *seen = calloc((size_t)(t_last + 1), 1);
    if (!seen)
        return 0;
    int ok = 1;
    for (int64_t i = 0; i < c && ok; ++i) {
        int64_t s = cand[i];
        if (i < want) {
            if (s < 0 || s > t_last || seen[s])
                ok = 0;
            else
                seen[s] = 1;
        } else if (s != -1) {
            ok = 0;
        }
    }
    free(seen);
    return ok;
}

/*
 * PIVOT for selected groups of one sequence (same row/position convention as
 * orc_dense_rows; t_last(m) is the position of the group's last row).
 *  1. proxy (orc_proxy);
 *  2. one causal scan of the proxy over keys 0..t_last(m);
 *  3. candidates C_m = top-c of that scan;
 *  4. Reuse: R_m = top-k of the same scan, shared by every member;
 *  5. Refine: member i re-scores, with its own query and weights, the
 *     candidates that are causal for it, C_m restricted to [0, pos(i)], and
 *     keeps its own top-k.
 * cand_in, when not NULL, replaces C_m in step 5 by a given list ([ngroups][c],
 * checked as above); step 3's output still reports the oracle's own C_m.
 * Outputs: cand [ngroups][c], reuse [ngroups][k], refine [ngroups][g][k]
 * (rows of absent members of a short last group are all -1). Score outputs
 * may be NULL.
 */
int orc_pivot_groups_ex(const uint16_t *Q, const float *W, const uint16_t *K,
                        int64_t L, int64_t q_len, int H, int d,
                        int64_t g, int64_t c, int64_t k, int proxy, int64_t window,
                        const int64_t *groups, int64_t ngroups,
                        const int64_t *cand_in,
                        int64_t *cand_out, double *cand_score,
                        int64_t *reuse_out, double *reuse_score,
                        int64_t *refine_out, double *refine_score);

int orc_pivot_groups(const uint16_t *Q, const float *W, const uint16_t *K,
                     int64_t L, int64_t q_len, int H, int d,
                     int64_t g, int64_t c, int64_t k,
                     const int64_t *groups, int64_t ngroups,
                     const int64_t *cand_in,
                     int64_t *cand_out, double *cand_score,
                     int64_t *reuse_out, double *reuse_score,
                     int64_t *refine_out, double *refine_score)
{
    return orc_pivot_groups_ex(Q, W, K, L, q_len, H, d, g, c, k, ORC_PROXY_MEAN, 0, groups, ngroups,
                               cand_in, cand_out, cand_score, reuse_out, reuse_score, refine_out,
                               refine_score);
}

/* orc_pivot_groups with the proxy of orc_proxy_ex(proxy, window). */
int orc_pivot_groups_ex(const uint16_t *Q, const float *W, const uint16_t *K,
                        int64_t L, int64_t q_len, int H, int d,
                        int64_t g, int64_t c, int64_t k, int proxy, int64_t window,
                        const int64_t *groups, int64_t ngroups,
                        const int64_t *cand_in,
                        int64_t *cand_out, double *cand_score,
                        int64_t *reuse_out, double *reuse_score,
                        int64_t *refine_out, double *refine_score)
{
    if (!Q || !W || !K || !groups || !cand_out || !reuse_out || !refine_out ||
        L < 1 || q_len < 1 || q_len > L || g < 1 || c < 1 || k < 1)
        return ORC_EINVAL;
    int64_t ngroups_total = (q_len + g - 1) / g;
    uint16_t *qbar = malloc(sizeof(uint16_t) * (size_t)H * (size_t)d);
    float *wbar = malloc(sizeof(float) * (size_t)H);
    double *sc = malloc(sizeof(double) * (size_t)L);
    double *csc = malloc(sizeof(double) * (size_t)c);
    int64_t *cidx = malloc(sizeof(int64_t) * (size_t)c);
    int64_t *cur = malloc(sizeof(int64_t) * (size_t)c);
    if (!qbar || !wbar || !sc || !csc || !cidx || !cur) {
        free(qbar); free(wbar); free(sc); free(csc); free(cidx); free(cur);
        return ORC_EINVAL;
    }
    int rc = ORC_OK;
    for (int64_t gi = 0; gi < ngroups && rc == ORC_OK; ++gi) {
        int64_t m = groups[gi];
        if (m < 0 || m >= ngroups_total) {
            rc = ORC_EINVAL;
            break;
        }
        int64_t r0 = m * g;
        int64_t r1 = r0 + g < q_len ? r0 + g : q_len;
        int64_t t_last = L - q_len + r1 - 1;
        int64_t n = t_last + 1;

        rc = orc_proxy_ex(Q, W, q_len, H, d, g, m, proxy, window, qbar, wbar);
        if (rc != ORC_OK)
            break;
        rc = orc_scores(qbar, wbar, K, H, d, n, sc, NULL);
        if (rc != ORC_OK)
            break;
        rc = orc_select(sc, NULL, n, c, cand_out + gi * c,
                        cand_score ? cand_score + gi * c : NULL);
        if (rc != ORC_OK)
            break;
        rc = orc_select(sc, NULL, n, k, reuse_out + gi * k,
                        reuse_score ? reuse_score + gi * k : NULL);
        if (rc != ORC_OK)
            break;

        const int64_t *cand = cand_out + gi * c;
        if (cand_in) {
            cand = cand_in + gi * c;
            if (!valid_candidates(cand, c, t_last)) {
                rc = ORC_EINVAL;
                break;
            }
        }
        for (int64_t i = 0; i < g; ++i) {
            int64_t *orow = refine_out + (gi * g + i) * k;
            double *srow = refine_score ? refine_score + (gi * g + i) * k : NULL;
            int64_t r = r0 + i;
            if (r >= r1) {
                for (int64_t x = 0; x < k; ++x) {
                    orow[x] = -1;
                    if (srow)
                        srow[x] = -INFINITY;
                }
                continue;
            }
            int64_t pos = L - q_len + r;
            int64_t nc = 0;
            for (int64_t x = 0; x < c; ++x)
                if (cand[x] >= 0 && cand[x] <= pos)
                    cur[nc++] = cand[x];
            /* score the member against its causal candidates, one key at a time */
            for (int64_t x = 0; x < nc; ++x) {
                rc = orc_scores(Q + r * H * d, W + r * H, K + cur[x] * d, H, d, 1,
                                csc + x, NULL);
                if (rc != ORC_OK)
                    break;
                cidx[x] = cur[x];
            }
            if (rc != ORC_OK)
                break;
            rc = orc_select(csc, cidx, nc, k, orow, srow);
            if (rc != ORC_OK)
                break;
        }
    }
    free(qbar); free(wbar); free(sc); free(csc); free(cidx); free(cur);
    return rc;
}

/* ------------------------------------------------------------------------
 * Key-axis coarse stage: hierarchical indexing over contiguous key chunks.
 *
 * Sources. "Not All Tokens Deserve Equal Resolution: Score-Adaptive Indexing
 * for Sparse Attention in Long-Context LLMs" (SCALE), abstract: contiguous
 * regions of keys are represented by compact summaries, the summary of a
 * chunk is its mean key, candidates are chosen at chunk level and refined
 * with the token-level indexer; fixed-size blocks (HISA-64: one summary per
 * 64 keys) are the baseline, and SCALE re-partitions the keys under the same
 * chunk budget by splitting high-dispersion regions and merging homogeneous
 * neighbours. The PIVOT paper names the same token-axis approach (HISA) in
 * its experimental setup and results.
 *
 * Chunks are given by their exclusive ends cend[0..nc): chunk b holds keys
 * [cend[b-1], cend[b]) (cend[-1] = 0), ascending, cend[nc-1] = L.
 * ------------------------------------------------------------------------ */

static int valid_chunks(const int32_t *cend, int64_t nc, int64_t L)
{
    if (!cend || nc < 1 || cend[nc - 1] != L)
        return 0;
    int64_t prev = 0;
    for (int64_t b = 0; b < nc; ++b) {
        if (cend[b] <= prev)
            return 0;
        prev = cend[b];
    }
    return 1;
}

/*
 * Mean key of every chunk (the summary; SCALE abstract: the mean key is the
 * best single representative of a chunk in squared error). Reading of the
 * unstated precision, the same as for the query proxy: per dimension, an fp32
 * sum over the chunk's keys in index order, an fp32 division by the number of
 * keys, bf16 rounding (nearest, ties to even). kbar is [nc][d] bf16.
 */
int orc_chunk_means(const uint16_t *K, int64_t L, int d, const int32_t *cend, int64_t nc,
                    uint16_t *kbar)
{
    if (!K || !kbar || d < 1 || L < 1 || !valid_chunks(cend, nc, L))
        return ORC_EINVAL;
    for (int64_t b = 0; b < nc; ++b) {
        int64_t first = b == 0 ? 0 : cend[b - 1];
        int64_t end = cend[b];
        float nkeys = (float)(end - first);
        for (int e = 0; e < d; ++e) {
            float sum = 0.0f;
            for (int64_t s = first; s < end; ++s)
                sum += bf16_to_float(K[s * d + e]);
            kbar[b * d + e] = float_to_bf16_rne(sum / nkeys);
        }
    }
    return ORC_OK;
}

/*
 * Dispersion of keys [a, b): the squared reconstruction error of the chunk by
 * its (unrounded) mean, sum_s |k_s - mean|^2 = sum_e (sum_s k_se^2 -
 * (sum_s k_se)^2 / n). Computed in double in a fixed order (per dimension
 * the sums run over s in index order; the dimensions are then added in
 * order), so that any implementation taking the same steps gets the same
 * bits: the chunking below compares these values, and both sides of a
 * comparison must make the same decision.
 */
static double dispersion(const uint16_t *K, int d, int64_t a, int64_t b)
{
    double n = (double)(b - a);
    double total = 0.0;
    for (int e = 0; e < d; ++e) {
        double s1 = 0.0, s2 = 0.0;
        for (int64_t s = a; s < b; ++s) {
            double x = bf16_to_double(K[s * d + e]);
            s1 += x;
            s2 += x * x;
        }
        total += s2 - s1 * s1 / n;
    }
    return total;
}

typedef struct {
    double key;
    int64_t idx;
} orc_rank;

/* higher key first, then lower index */
static int rank_desc(const void *pa, const void *pb)
{
    const orc_rank *a = pa, *b = pb;
    if (a->key > b->key)
        return -1;
    if (a->key < b->key)
        return 1;
    return a->idx < b->idx ? -1 : (a->idx > b->idx ? 1 : 0);
}

/* lower key first, then lower index */
static int rank_asc(const void *pa, const void *pb)
{
    const orc_rank *a = pa, *b = pb;
    if (a->key < b->key)
        return -1;
    if (a->key > b->key)
        return 1;
    return a->idx < b->idx ? -1 : (a->idx > b->idx ? 1 : 0);
}

/*
 * Score-adaptive chunking under a fixed budget (SCALE abstract: split
 * high-dispersion regions into more chunks, merge homogeneous neighbours,
 * keep the number of chunks). The abstract gives no procedure; the reading
 * taken here:
 *  - start from fixed blocks of `block` keys (block even); blocks are numbered
 *    0..n-1, n = ceil(L / block), the last one short when block does not
 *    divide L; only full blocks take part below;
 *  - a split cuts a full block into its two halves; its gain is the drop in
 *    dispersion, G = D(block) - D(first half) - D(second half);
 *  - a merge joins the aligned pair of full blocks 2j, 2j+1 into one chunk;
 *    its loss is M = D(pair) - D(2j) - D(2j+1);
 *  - greedy: splits are taken in order of gain (highest first), merges in
 *    order of loss (lowest first), ties to the lower block or pair number;
 *    a block whose pair is merged cannot be split, and a pair with a split
 *    block cannot be merged (such candidates are passed over); one split and
 *    one merge are made together while the gain exceeds the loss (the total
 *    dispersion falls with every step), and the first step where it does
 *    not ends the procedure.
 * Every split adds a chunk and every merge removes one, so there are n chunks,
 * of block/2, block or 2*block keys (the last chunk may be short).
 * cend gets the n chunk ends in key order.
 */
int orc_chunk_adaptive(const uint16_t *K, int64_t L, int d, int64_t block, int32_t *cend)
{
    if (!K || !cend || L < 1 || d < 1 || block < 2 || block % 2 || L > 2147483647LL)
        return ORC_EINVAL;
    int64_t n = (L + block - 1) / block;
    int64_t nfull = L / block;
    int64_t npair = nfull / 2;
    orc_rank *gain = malloc(sizeof(orc_rank) * (size_t)(nfull > 0 ? nfull : 1));
    orc_rank *loss = malloc(sizeof(orc_rank) * (size_t)(npair > 0 ? npair : 1));
    char *split = calloc((size_t)(n > 0 ? n : 1), 1);
    char *merged = calloc((size_t)(npair > 0 ? npair : 1), 1);
    if (!gain || !loss || !split || !merged) {
        free(gain); free(loss); free(split); free(merged);
        return ORC_EINVAL;
    }
    int64_t h = block / 2;
    for (int64_t b = 0; b < nfull; ++b) {
        int64_t a = b * block;
        gain[b].key = dispersion(K, d, a, a + block) - dispersion(K, d, a, a + h) -
                      dispersion(K, d, a + h, a + block);
        gain[b].idx = b;
    }
    for (int64_t j = 0; j < npair; ++j) {
        int64_t a = 2 * j * block;
        loss[j].key = dispersion(K, d, a, a + 2 * block) - dispersion(K, d, a, a + block) -
                      dispersion(K, d, a + block, a + 2 * block);
        loss[j].idx = j;
    }
    qsort(gain, (size_t)nfull, sizeof(orc_rank), rank_desc);
    qsort(loss, (size_t)npair, sizeof(orc_rank), rank_asc);
    int64_t ia = 0, ib = 0;
    for (;;) {
        /* next split candidate: a block whose pair is not merged */
        while (ia < nfull && gain[ia].idx / 2 < npair && merged[gain[ia].idx / 2])
            ++ia;
        /* next merge candidate: a pair with no split block and not holding
         * the split candidate */
        while (ib < npair) {
            int64_t j = loss[ib].idx;
            int conflict = split[2 * j] || split[2 * j + 1] ||
                           (ia < nfull && gain[ia].idx / 2 == j);
            if (!conflict)
                break;
            ++ib;
        }
        if (ia >= nfull || ib >= npair || !(gain[ia].key > loss[ib].key))
            break;
        split[gain[ia].idx] = 1;
        merged[loss[ib].idx] = 1;
        ++ia;
        ++ib;
    }
    int64_t out = 0;
    for (int64_t b = 0; b < n; ++b) {
        int64_t a = b * block;
        if (b % 2 == 0 && b / 2 < npair && merged[b / 2]) {
            cend[out++] = (int32_t)(a + 2 * block);
            ++b;
        } else if (split[b]) {
            cend[out++] = (int32_t)(a + h);
            cend[out++] = (int32_t)(a + block);
        } else {
            cend[out++] = (int32_t)(a + block < L ? a + block : L);
        }
    }
    free(gain); free(loss); free(split); free(merged);
    return out == n ? ORC_OK : ORC_EINVAL;
}

/*
 * Chunk-level candidates and token-level refinement for selected groups of
 * one sequence (positions as in orc_dense_rows; groups and proxies as in
 * orc_pivot_groups_ex; g = 1 makes the proxy the query itself, i.e. plain
 * per-query hierarchical indexing):
 *  1. summaries kbar = orc_chunk_means;
 *  2. the chunks complete at the group's last position t_last, those with
 *     cend[b] <= t_last + 1, are scored by the proxy with the index score of
 *     Eq. (1), the summary standing in for the key;
 *  3. the top-nsel of them (ranking as everywhere) are the selected chunks,
 *     written in ascending chunk order, -1 padded ([ngroups][nsel]);
 *  4. the candidate list: the keys of the selected chunks in index order,
 *     then the keys after the last complete chunk up to t_last (the chunk in
 *     progress has no summary yet, and the reading taken is that its keys are
 *     always kept), then -1 up to width cw ([ngroups][cw]; an error if the
 *     list does not fit);
 *  5. Refine: member i scores the candidates at or before pos(i) with its own
 *     query and weights and keeps its top-k ([ngroups][g][k]).
 * Score outputs may be NULL.
 */
int orc_chunk_groups(const uint16_t *Q, const float *W, const uint16_t *K,
                     int64_t L, int64_t q_len, int H, int d, int64_t g, int proxy, int64_t window,
                     const int32_t *cend, int64_t nc, int64_t nsel, int64_t cw, int64_t k,
                     const int64_t *groups, int64_t ngroups,
                     int64_t *chunk_out, double *chunk_score, int64_t *cand_out,
                     int64_t *refine_out, double *refine_score)
{
    if (!Q || !W || !K || !groups || !chunk_out || !cand_out || !refine_out ||
        L < 1 || q_len < 1 || q_len > L || g < 1 || nsel < 1 || cw < 1 || k < 1 ||
        !valid_chunks(cend, nc, L))
        return ORC_EINVAL;
    int64_t ngroups_total = (q_len + g - 1) / g;
    uint16_t *kbar = malloc(sizeof(uint16_t) * (size_t)nc * (size_t)d);
    uint16_t *qbar = malloc(sizeof(uint16_t) * (size_t)H * (size_t)d);
    float *wbar = malloc(sizeof(float) * (size_t)H);
    double *csc = malloc(sizeof(double) * (size_t)nc);
    int64_t *sel = malloc(sizeof(int64_t) * (size_t)nsel);
    double *tsc = malloc(sizeof(double) * (size_t)cw);
    int64_t *tix = malloc(sizeof(int64_t) * (size_t)cw);
    if (!kbar || !qbar || !wbar || !csc || !sel || !tsc || !tix) {
        free(kbar); free(qbar); free(wbar); free(csc); free(sel); free(tsc); free(tix);
        return ORC_EINVAL;
    }
    int rc = orc_chunk_means(K, L, d, cend, nc, kbar);
    for (int64_t gi = 0; gi < ngroups && rc == ORC_OK; ++gi) {
        int64_t m = groups[gi];
        if (m < 0 || m >= ngroups_total) {
            rc = ORC_EINVAL;
            break;
        }
        int64_t r0 = m * g;
        int64_t r1 = r0 + g < q_len ? r0 + g : q_len;
        int64_t t_last = (L - q_len) + r1 - 1;  /* the group's last position */
        /* chunks complete at t_last form a prefix 0..ncomp-1 */
        int64_t ncomp = 0;
        while (ncomp < nc && cend[ncomp] <= t_last + 1)
            ++ncomp;

        rc = orc_proxy_ex(Q, W, q_len, H, d, g, m, proxy, window, qbar, wbar);
        if (rc != ORC_OK)
            break;
        rc = orc_scores(qbar, wbar, kbar, H, d, ncomp, csc, NULL);
        if (rc != ORC_OK)
            break;
        rc = orc_select(csc, NULL, ncomp, nsel, sel, NULL);
        if (rc != ORC_OK)
            break;
        /* selected chunks in ascending order, -1 last */
        int64_t nsc = ncomp < nsel ? ncomp : nsel;
        for (int64_t x = 1; x < nsc; ++x)
            for (int64_t y = x; y > 0 && sel[y - 1] > sel[y]; --y) {
                int64_t t = sel[y];
                sel[y] = sel[y - 1];
                sel[y - 1] = t;
            }
        int64_t *crow = chunk_out + gi * nsel;
        for (int64_t x = 0; x < nsel; ++x) {
            crow[x] = x < nsc ? sel[x] : -1;
            if (chunk_score)
                chunk_score[gi * nsel + x] = x < nsc ? csc[sel[x]] : -INFINITY;
        }
        /* expansion into keys */
        int64_t *trow = cand_out + gi * cw;
        int64_t nt = 0;
        for (int64_t x = 0; x < nsc && rc == ORC_OK; ++x) {
            int64_t b = sel[x];
            for (int64_t s = (b == 0 ? 0 : cend[b - 1]); s < cend[b]; ++s) {
                if (nt == cw) {
                    rc = ORC_EINVAL;
                    break;
                }
                trow[nt++] = s;
            }
        }
        for (int64_t s = (ncomp == 0 ? 0 : cend[ncomp - 1]); s <= t_last && rc == ORC_OK; ++s) {
            if (nt == cw) {
                rc = ORC_EINVAL;
                break;
            }
            trow[nt++] = s;
        }
        if (rc != ORC_OK)
            break;
        for (int64_t x = nt; x < cw; ++x)
            trow[x] = -1;

        /* token-level refinement of each member */
        for (int64_t i = 0; i < g && rc == ORC_OK; ++i) {
            int64_t *orow = refine_out + (gi * g + i) * k;
            double *srow = refine_score ? refine_score + (gi * g + i) * k : NULL;
            int64_t r = r0 + i;
            if (r >= r1) {
                for (int64_t x = 0; x < k; ++x) {
                    orow[x] = -1;
                    if (srow)
                        srow[x] = -INFINITY;
                }
                continue;
            }
            int64_t pos = L - q_len + r;
            int64_t nv = 0;
            for (int64_t x = 0; x < nt && rc == ORC_OK; ++x) {
                if (trow[x] > pos)
                    continue;
                rc = orc_scores(Q + r * H * d, W + r * H, K + trow[x] * d, H, d, 1, tsc + nv, NULL);
                tix[nv++] = trow[x];
            }
            if (rc == ORC_OK)
                rc = orc_select(tsc, tix, nv, k, orow, srow);
        }
    }
    free(kbar); free(qbar); free(wbar); free(csc); free(sel); free(tsc); free(tix);
    return rc;
}
