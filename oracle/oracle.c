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
