/*
 * qsa_oracle.c -- FP64 CPU reference for route-set grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library. It shares no
 * code, header, table or helper with the HIP library it checks.
 *
 * What it computes is the plain definition of the method, written out with
 * loops, in double precision:
 *
 *  - Route set. For query row (b, i) the set R(b, i) holds every route value r
 *    with 0 <= r < Skv, tested on the full integer width; duplicates count once
 *    and everything else is padding. ("nemo_automodel ... flex_qsa" page,
 *    `_routes_to_membership`; "... fa4_qsa" page, `_preprocess` and
 *    `fa4_sparse_gqa_attention`.)
 *  - Membership and tiles. memb[b, i, j] = 1 iff j is in R(b, i); 128 x 128
 *    tiles are absent (no member), full (all 128*128 cells members) or partial;
 *    per tile row and per tile column, the partial and the full tile indices in
 *    ascending order. ("fa4_qsa" page, `_block_kinds`, `_compact_blocks`;
 *    "flex_qsa" page, `_dense_blocks_to_ordered`.)
 *  - Block-bitmap selection. For packed tokens t, j in [0, T): key j is
 *    allowed for query t iff lo[t] <= j <= hi[t], 0 <= b < NB and
 *    sel_blocks[t, b] != 0, with b = blk_base[t] + floor((j - tok_base[t]) /
 *    block_size) (floor division, so a key before the query's token origin
 *    maps to an earlier block). This is the lookup of the cuDNN Frontend QSA
 *    page, section "Selection and components"; the per-block token spans
 *    (block_first, block_last) do not enter it.
 *  - Document-causal selection. Query i of batch row b, at global position
 *    p = q_global_start + i, is allowed key j iff q_doc[b, i] != 0,
 *    kv_doc[b, j] == q_doc[b, i] and j <= p: causal attention within the
 *    query's document, padding queries (document 0) attending to nothing.
 *    This is the "fa4" page's `document_causal_fa4_attention`, a query shard
 *    against the global keys.
 *  - Forward. For every query head h of KV group g = h / (Hq / Hkv):
 *    s_j = scale * <q, k_j> over j in R, lse = log sum_j exp(s_j),
 *    o = sum_j exp(s_j - lse) v_j; an empty R gives o = 0 and lse = -inf.
 *    ("Query Sparse Attention (QSA)" page of cuDNN Frontend, sections
 *    "Tensors" and "Selection and components".)
 *  - Backward. The equations of that section: P = exp(S - lse) on the allowed
 *    keys and 0 elsewhere, delta = sum(dO * O), dP = dO V^T,
 *    dS = P (dP - delta), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO, with
 *    dK and dV summed over the query heads that share a KV head.
 *
 * Inputs are double arrays (bf16 values are widened exactly by the caller).
 * Layouts: q, dO [B, Sq, Hq, D]; k, v [B, Skv, Hkv, D]; routes [B, Sq, W]
 * (int32 or int64); lse [B, Hq, Sq] when written for all rows.
 *
 * Every function has a "parity pin" in the CPU test suite: dense masked-softmax
 * brute force, closed forms, central finite differences and invariants.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t B, Sq, Skv, Hq, Hkv, D, W;
    int32_t route_is_i64;
    int32_t pad_;
    double scale;
    const void *routes;
    const double *q, *k, *v, *dout;
    /* Saved forward state for the backward, or NULL: out [B, Sq, Hq, D] and
     * lse [B, Hq, Sq]. The backward equations take O and LSE as inputs (the
     * forward's FP32 output and LSE); when these are NULL the oracle uses the
     * O and LSE of its own FP64 forward. */
    const double *o_saved, *lse_saved;
} orc_problem;

static int cmp_i64(const void *a, const void *b)
{
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

/* R(b, i) in ascending order; returns |R|. `keys` must hold W entries. */
static int64_t route_set_raw(const void *routes, int is_i64, int64_t W, int64_t Skv,
                             int64_t row, int64_t *keys)
{
    int64_t n = 0;
    for (int64_t w = 0; w < W; ++w) {
        int64_t r = is_i64 ? ((const int64_t *)routes)[row * W + w]
                           : (int64_t)((const int32_t *)routes)[row * W + w];
        if (r >= 0 && r < Skv) keys[n++] = r;
    }
    qsort(keys, (size_t)n, sizeof(int64_t), cmp_i64);
    int64_t m = 0;
    for (int64_t t = 0; t < n; ++t)
        if (m == 0 || keys[t] != keys[m - 1]) keys[m++] = keys[t];
    return m;
}

int64_t orc_route_set(const void *routes, int32_t is_i64, int64_t W, int64_t Skv, int64_t row,
                      int64_t *keys)
{
    return route_set_raw(routes, is_i64, W, Skv, row, keys);
}

/* memb[b, i, j] for j < Skv, zero in the padding columns up to `stride`. */
void orc_membership(const void *routes, int32_t is_i64, int64_t B, int64_t Sq, int64_t W,
                    int64_t Skv, int64_t stride, uint8_t *memb, uint8_t *has_routes)
{
    memset(memb, 0, (size_t)(B * Sq * stride));
    for (int64_t row = 0; row < B * Sq; ++row) {
        int any = 0;
        for (int64_t w = 0; w < W; ++w) {
            int64_t r = is_i64 ? ((const int64_t *)routes)[row * W + w]
                               : (int64_t)((const int32_t *)routes)[row * W + w];
            if (r >= 0 && r < Skv) {
                memb[row * stride + r] = 1;
                any = 1;
            }
        }
        has_routes[row] = (uint8_t)any;
    }
}

/*
 * Tile kinds and lists. cnt = members of the tile (rows and columns clipped to
 * the table); kind 0 if cnt == 0, 2 if cnt == tq * tk, else 1. Lists hold the
 * matching tile indices in ascending order, then -1.
 */
/* floor(a / d) for d > 0, also for negative a. */
static int64_t floor_div(int64_t a, int64_t d)
{
    int64_t q = a / d;
    if ((a % d) != 0 && a < 0) q -= 1;
    return q;
}

/* Byte membership [1, T, stride] and has_routes [1, T] of a block-bitmap
 * selection: every (t, j) evaluated with the lookup above. */
void orc_block_membership(const uint8_t *sel, int64_t T, int64_t NB, const int32_t *lo,
                          const int32_t *hi, const int32_t *blk_base, const int32_t *tok_base,
                          int64_t block_size, int64_t stride, uint8_t *memb, uint8_t *has)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < T; ++t) {
        uint8_t *row = memb + t * stride;
        int any = 0;
        for (int64_t j = 0; j < stride; ++j) {
            int allowed = 0;
            if (j < T && lo[t] <= j && j <= hi[t]) {
                const int64_t b = (int64_t)blk_base[t] + floor_div(j - (int64_t)tok_base[t], block_size);
                allowed = b >= 0 && b < NB && sel[t * NB + b] != 0;
            }
            row[j] = (uint8_t)allowed;
            any |= allowed;
        }
        has[t] = (uint8_t)any;
    }
}

/* Byte membership [B, Sq, stride] and has_routes [B, Sq] of document-causal
 * selection: every (b, i, j) tested as above. */
void orc_doc_membership(const int32_t *q_doc, const int32_t *kv_doc, int64_t B, int64_t Sq,
                        int64_t Skv, int64_t q_global_start, int64_t stride, uint8_t *memb,
                        uint8_t *has)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < B * Sq; ++r) {
        const int64_t b = r / Sq, i = r % Sq;
        const int32_t d = q_doc[r];
        const int64_t p = q_global_start + i;
        uint8_t *row = memb + r * stride;
        int any = 0;
        for (int64_t j = 0; j < stride; ++j) {
            const int allowed = j < Skv && d != 0 && kv_doc[b * Skv + j] == d && j <= p;
            row[j] = (uint8_t)allowed;
            any |= allowed;
        }
        has[r] = (uint8_t)any;
    }
}

void orc_tiles(const uint8_t *memb, int64_t B, int64_t Sq, int64_t Skv, int64_t stride,
               int64_t tq, int64_t tk, int32_t *kinds, int32_t *fwd_p_cnt, int32_t *fwd_p_idx,
               int32_t *fwd_f_cnt, int32_t *fwd_f_idx, int32_t *rev_p_cnt, int32_t *rev_p_idx,
               int32_t *rev_f_cnt, int32_t *rev_f_idx)
{
    int64_t nqt = (Sq + tq - 1) / tq, nkt = (Skv + tk - 1) / tk;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t r = 0; r < nqt; ++r)
            for (int64_t t = 0; t < nkt; ++t) {
                int64_t cnt = 0;
                for (int64_t i = r * tq; i < (r + 1) * tq && i < Sq; ++i)
                    for (int64_t j = t * tk; j < (t + 1) * tk && j < Skv; ++j)
                        cnt += memb[(b * Sq + i) * stride + j];
                kinds[(b * nqt + r) * nkt + t] = cnt == 0 ? 0 : (cnt == tq * tk ? 2 : 1);
            }
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t r = 0; r < nqt; ++r) {
            int32_t np_ = 0, nf = 0;
            int32_t *pi = fwd_p_idx + (b * nqt + r) * nkt, *fi = fwd_f_idx + (b * nqt + r) * nkt;
            for (int64_t t = 0; t < nkt; ++t) {
                int32_t kd = kinds[(b * nqt + r) * nkt + t];
                if (kd == 1) pi[np_++] = (int32_t)t;
                if (kd == 2) fi[nf++] = (int32_t)t;
            }
            for (int64_t t = np_; t < nkt; ++t) pi[t] = -1;
            for (int64_t t = nf; t < nkt; ++t) fi[t] = -1;
            fwd_p_cnt[b * nqt + r] = np_;
            fwd_f_cnt[b * nqt + r] = nf;
        }
        for (int64_t t = 0; t < nkt; ++t) {
            int32_t np_ = 0, nf = 0;
            int32_t *pi = rev_p_idx + (b * nkt + t) * nqt, *fi = rev_f_idx + (b * nkt + t) * nqt;
            for (int64_t r = 0; r < nqt; ++r) {
                int32_t kd = kinds[(b * nqt + r) * nkt + t];
                if (kd == 1) pi[np_++] = (int32_t)r;
                if (kd == 2) fi[nf++] = (int32_t)r;
            }
            for (int64_t r = np_; r < nqt; ++r) pi[r] = -1;
            for (int64_t r = nf; r < nqt; ++r) fi[r] = -1;
            rev_p_cnt[b * nkt + t] = np_;
            rev_f_cnt[b * nkt + t] = nf;
        }
    }
}

static double dot(const double *a, const double *b, int64_t n)
{
    double s = 0.0;
    for (int64_t d = 0; d < n; ++d) s += a[d] * b[d];
    return s;
}

/*
 * Forward of one query row for all heads. s must hold |R| doubles.
 * out [Hq, D], lse [Hq].
 */
static void forward_row(const orc_problem *P, int64_t b, int64_t i, const int64_t *keys,
                        int64_t n, double *s, double *out, double *lse)
{
    const int64_t D = P->D, Hq = P->Hq, Hkv = P->Hkv, G = Hq / Hkv;
    for (int64_t h = 0; h < Hq; ++h) {
        const int64_t g = h / G;
        double *o = out + h * D;
        for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
        if (n == 0) {
            lse[h] = -INFINITY;
            continue;
        }
        const double *qh = P->q + ((b * P->Sq + i) * Hq + h) * D;
        double m = -INFINITY;
        for (int64_t t = 0; t < n; ++t) {
            const double *kj = P->k + ((b * P->Skv + keys[t]) * Hkv + g) * D;
            s[t] = P->scale * dot(qh, kj, D);
            if (s[t] > m) m = s[t];
        }
        double l = 0.0;
        for (int64_t t = 0; t < n; ++t) l += exp(s[t] - m);
        lse[h] = m + log(l);
        for (int64_t t = 0; t < n; ++t) {
            const double p = exp(s[t] - lse[h]);
            const double *vj = P->v + ((b * P->Skv + keys[t]) * Hkv + g) * D;
            for (int64_t d = 0; d < D; ++d) o[d] += p * vj[d];
        }
    }
}

/* Forward for the listed flat rows (b * Sq + i): out [nrows, Hq, D], lse [nrows, Hq]. */
void orc_forward(const orc_problem *P, int64_t nrows, const int64_t *rows, double *out,
                 double *lse)
{
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)(P->W > 0 ? P->W : 1));
        double *s = (double *)malloc(sizeof(double) * (size_t)(P->W > 0 ? P->W : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < nrows; ++t) {
            const int64_t row = rows[t], b = row / P->Sq, i = row % P->Sq;
            const int64_t n = route_set_raw(P->routes, P->route_is_i64, P->W, P->Skv, row, keys);
            forward_row(P, b, i, keys, n, s, out + t * P->Hq * P->D, lse + t * P->Hq);
        }
        free(keys);
        free(s);
    }
}

/* Replace the row's O [Hq, D] and lse [Hq] by the saved ones, when given. */
static void use_saved(const orc_problem *P, int64_t b, int64_t i, double *o, double *lse)
{
    if (!P->o_saved) return;
    const int64_t Hq = P->Hq, D = P->D;
    for (int64_t x = 0; x < Hq * D; ++x) o[x] = P->o_saved[(b * P->Sq + i) * Hq * D + x];
    for (int64_t h = 0; h < Hq; ++h) lse[h] = P->lse_saved[(b * Hq + h) * P->Sq + i];
}

/*
 * Backward terms of one row: with the row's O and lse (its own forward's, or
 * the saved ones), for each key of R
 * and each head, p = exp(s - lse), dp = <dO, v>, ds = p (dp - delta).
 * Accumulates dq [Hq, D] (zeroed here) unless dq is NULL. When dk/dv are given ([nsel, Hkv, D]),
 * also adds the row's contributions to the selected keys sel[0..nsel) of batch b.
 */
static void backward_row(const orc_problem *P, int64_t b, int64_t i, const int64_t *keys,
                         int64_t n, double *s, double *o, double *lse, double *dq,
                         int64_t nsel, const int64_t *sel, double *dk, double *dv)
{
    const int64_t D = P->D, Hq = P->Hq, Hkv = P->Hkv, G = Hq / Hkv;
    forward_row(P, b, i, keys, n, s, o, lse);
    use_saved(P, b, i, o, lse);
    if (dq)
        for (int64_t x = 0; x < Hq * D; ++x) dq[x] = 0.0;
    if (n == 0) return;
    for (int64_t h = 0; h < Hq; ++h) {
        const int64_t g = h / G;
        const double *qh = P->q + ((b * P->Sq + i) * Hq + h) * D;
        const double *doh = P->dout + ((b * P->Sq + i) * Hq + h) * D;
        const double delta = dot(doh, o + h * D, D);
        for (int64_t t = 0; t < n; ++t) {
            const int64_t j = keys[t];
            const double *kj = P->k + ((b * P->Skv + j) * Hkv + g) * D;
            const double *vj = P->v + ((b * P->Skv + j) * Hkv + g) * D;
            const double p = exp(P->scale * dot(qh, kj, D) - lse[h]);
            const double dp = dot(doh, vj, D);
            const double ds = p * (dp - delta);
            if (dq)
                for (int64_t d = 0; d < D; ++d) dq[h * D + d] += P->scale * ds * kj[d];
            for (int64_t u = 0; u < nsel; ++u) {
                if (sel[u] != b * P->Skv + j) continue;
                for (int64_t d = 0; d < D; ++d) {
                    dk[(u * Hkv + g) * D + d] += P->scale * ds * qh[d];
                    dv[(u * Hkv + g) * D + d] += p * doh[d];
                }
            }
        }
    }
}

/* dq for the listed flat rows: dq [nrows, Hq, D]. */
void orc_backward_dq(const orc_problem *P, int64_t nrows, const int64_t *rows, double *dq)
{
#pragma omp parallel
    {
        const int64_t W1 = P->W > 0 ? P->W : 1;
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)W1);
        double *s = (double *)malloc(sizeof(double) * (size_t)W1);
        double *o = (double *)malloc(sizeof(double) * (size_t)(P->Hq * P->D));
        double *lse = (double *)malloc(sizeof(double) * (size_t)P->Hq);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < nrows; ++t) {
            const int64_t row = rows[t], b = row / P->Sq, i = row % P->Sq;
            const int64_t n = route_set_raw(P->routes, P->route_is_i64, P->W, P->Skv, row, keys);
            backward_row(P, b, i, keys, n, s, o, lse, dq + t * P->Hq * P->D, 0, NULL, NULL,
                         NULL);
        }
        free(keys);
        free(s);
        free(o);
        free(lse);
    }
}

/*
 * dk, dv for the listed flat keys (b * Skv + j): dk, dv [nkeys, Hkv, D].
 * Every query row of the keys' batches contributes when its route set holds
 * the key. Rows are split over threads; each thread sums its rows in ascending
 * order and the per-thread sums are added in thread order.
 */
void orc_backward_dkdv(const orc_problem *P, int64_t nkeys, const int64_t *keys_sel, double *dk,
                       double *dv)
{
    const int64_t per = nkeys * P->Hkv * P->D;
    memset(dk, 0, sizeof(double) * (size_t)per);
    memset(dv, 0, sizeof(double) * (size_t)per);
    int nthreads = 1;
#ifdef _OPENMP
    nthreads = omp_get_max_threads();
#endif
    double *acc_k = (double *)calloc((size_t)(per * nthreads), sizeof(double));
    double *acc_v = (double *)calloc((size_t)(per * nthreads), sizeof(double));
    const int64_t nrows = P->B * P->Sq;
#pragma omp parallel num_threads(nthreads)
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        const int64_t W1 = P->W > 0 ? P->W : 1;
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)W1);
        double *s = (double *)malloc(sizeof(double) * (size_t)W1);
        double *o = (double *)malloc(sizeof(double) * (size_t)(P->Hq * P->D));
        double *lse = (double *)malloc(sizeof(double) * (size_t)P->Hq);
#pragma omp for schedule(static)
        for (int64_t row = 0; row < nrows; ++row) {
            const int64_t b = row / P->Sq, i = row % P->Sq;
            const int64_t n = route_set_raw(P->routes, P->route_is_i64, P->W, P->Skv, row, keys);
            int hit = 0;
            for (int64_t u = 0; u < nkeys && !hit; ++u)
                for (int64_t t = 0; t < n; ++t)
                    if (keys_sel[u] == b * P->Skv + keys[t]) {
                        hit = 1;
                        break;
                    }
            if (!hit) continue;
            backward_row(P, b, i, keys, n, s, o, lse, NULL, nkeys, keys_sel, acc_k + tid * per,
                         acc_v + tid * per);
        }
        free(keys);
        free(s);
        free(o);
        free(lse);
    }
    for (int t = 0; t < nthreads; ++t)
        for (int64_t x = 0; x < per; ++x) {
            dk[x] += acc_k[t * per + x];
            dv[x] += acc_v[t * per + x];
        }
    free(acc_k);
    free(acc_v);
}

/*
 * Whole backward restricted to a set of query rows: dq of those rows and their
 * contributions to every dk, dv ([B, Skv, Hkv, D], zeroed here). With all rows
 * listed this is the full backward. out [nrows, Hq, D] and lse [nrows, Hq],
 * when not NULL, receive the rows' forward results (the oracle's own forward,
 * also when the backward runs on saved state). The rows are split over the threads in
 * contiguous blocks; each thread adds its rows' dk, dv terms in list order
 * into a sum of its own, and the threads' sums are added in thread order.
 */
void orc_backward_rows(const orc_problem *P, int64_t nrows, const int64_t *rows, double *dq,
                       double *dk, double *dv, double *out, double *lse_out)
{
    const int64_t D = P->D, Hq = P->Hq, Hkv = P->Hkv, G = Hq / Hkv;
    const int64_t W1 = P->W > 0 ? P->W : 1;
    const int64_t per = P->B * P->Skv * Hkv * D;
    memset(dk, 0, sizeof(double) * (size_t)per);
    memset(dv, 0, sizeof(double) * (size_t)per);
    int nthreads = 1;
#ifdef _OPENMP
    nthreads = omp_get_max_threads();
    if (nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;
#endif
    double *acc_k = nthreads > 1 ? (double *)calloc((size_t)(per * nthreads), sizeof(double)) : dk;
    double *acc_v = nthreads > 1 ? (double *)calloc((size_t)(per * nthreads), sizeof(double)) : dv;
#pragma omp parallel num_threads(nthreads)
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double *tk = acc_k + (nthreads > 1 ? tid * per : 0);
        double *tv = acc_v + (nthreads > 1 ? tid * per : 0);
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)W1);
        double *s = (double *)malloc(sizeof(double) * (size_t)W1);
        double *o = (double *)malloc(sizeof(double) * (size_t)(Hq * D));
        double *lse = (double *)malloc(sizeof(double) * (size_t)Hq);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < nrows; ++t) {
            const int64_t row = rows[t], b = row / P->Sq, i = row % P->Sq;
            const int64_t n = route_set_raw(P->routes, P->route_is_i64, P->W, P->Skv, row, keys);
            double *dqr = dq + t * Hq * D;
            forward_row(P, b, i, keys, n, s, o, lse);
            if (out)
                for (int64_t x = 0; x < Hq * D; ++x) out[t * Hq * D + x] = o[x];
            if (lse_out)
                for (int64_t h = 0; h < Hq; ++h) lse_out[t * Hq + h] = lse[h];
            use_saved(P, b, i, o, lse);
            for (int64_t x = 0; x < Hq * D; ++x) dqr[x] = 0.0;
            for (int64_t h = 0; h < Hq && n > 0; ++h) {
                const int64_t g = h / G;
                const double *qh = P->q + ((b * P->Sq + i) * Hq + h) * D;
                const double *doh = P->dout + ((b * P->Sq + i) * Hq + h) * D;
                const double delta = dot(doh, o + h * D, D);
                for (int64_t u = 0; u < n; ++u) {
                    const int64_t j = keys[u];
                    const double *kj = P->k + ((b * P->Skv + j) * Hkv + g) * D;
                    const double *vj = P->v + ((b * P->Skv + j) * Hkv + g) * D;
                    const double p = exp(P->scale * dot(qh, kj, D) - lse[h]);
                    const double ds = p * (dot(doh, vj, D) - delta);
                    double *dkj = tk + ((b * P->Skv + j) * Hkv + g) * D;
                    double *dvj = tv + ((b * P->Skv + j) * Hkv + g) * D;
                    for (int64_t d = 0; d < D; ++d) {
                        dqr[h * D + d] += P->scale * ds * kj[d];
                        dkj[d] += P->scale * ds * qh[d];
                        dvj[d] += p * doh[d];
                    }
                }
            }
        }
        free(keys);
        free(s);
        free(o);
        free(lse);
    }
    if (nthreads > 1) {
        for (int t = 0; t < nthreads; ++t)
            for (int64_t x = 0; x < per; ++x) {
                dk[x] += acc_k[t * per + x];
                dv[x] += acc_v[t * per + x];
            }
        free(acc_k);
        free(acc_v);
    }
}

int32_t orc_num_threads(void)
{
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}
