/*
 * Sanitizer driver for the oracle (built with gcc -fsanitize=address,undefined
 * together with oracle/qsa_oracle.c): runs every oracle function on small
 * seeded inputs, including empty rows, duplicate and out-of-range routes,
 * int64 routes with values beyond 2^31, ragged tiles and odd block metadata,
 * so that any out-of-bounds access or undefined arithmetic aborts the run.
 * Results are checked loosely (finite, consistent shapes); their values are
 * pinned by the Python tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t B, Sq, Skv, Hq, Hkv, D, W;
    int32_t route_is_i64;
    int32_t pad_;
    double scale;
    const void *routes;
    const double *q, *k, *v, *dout;
    const double *o_saved, *lse_saved;
} orc_problem;

int64_t orc_route_set(const void *routes, int32_t is_i64, int64_t W, int64_t Skv, int64_t row,
                      int64_t *keys);
void orc_membership(const void *routes, int32_t is_i64, int64_t B, int64_t Sq, int64_t W,
                    int64_t Skv, int64_t stride, uint8_t *memb, uint8_t *has);
void orc_block_membership(const uint8_t *sel, int64_t T, int64_t NB, const int32_t *lo,
                          const int32_t *hi, const int32_t *blk_base, const int32_t *tok_base,
                          int64_t block_size, int64_t stride, uint8_t *memb, uint8_t *has);
void orc_tiles(const uint8_t *memb, int64_t B, int64_t Sq, int64_t Skv, int64_t stride,
               int64_t tq, int64_t tk, int32_t *kinds, int32_t *fpc, int32_t *fpi, int32_t *ffc,
               int32_t *ffi, int32_t *rpc, int32_t *rpi, int32_t *rfc, int32_t *rfi);
void orc_forward(const orc_problem *P, int64_t nrows, const int64_t *rows, double *out,
                 double *lse);
void orc_backward_dq(const orc_problem *P, int64_t nrows, const int64_t *rows, double *dq);
void orc_backward_dkdv(const orc_problem *P, int64_t nkeys, const int64_t *keys, double *dk,
                       double *dv);
void orc_backward_rows(const orc_problem *P, int64_t nrows, const int64_t *rows, double *dq,
                       double *dk, double *dv, double *out, double *lse_out);

static uint64_t g_state = 0x9e3779b97f4a7c15ull;
static uint64_t next_u64(void)
{
    /* splitmix64 */
    uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
static double uniform(void) { return (double)(next_u64() >> 11) * (1.0 / 9007199254740992.0); }

static int check_finite(const double *x, int64_t n, const char *name)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) {
            fprintf(stderr, "%s[%lld] not finite\n", name, (long long)i);
            return 1;
        }
    return 0;
}

static int run_case(int64_t B, int64_t Sq, int64_t Skv, int64_t Hkv, int64_t W, int is_i64)
{
    const int64_t Hq = 12 * Hkv, D = 256, stride = (Skv + 127) / 128 * 128;
    int64_t *r64 = malloc(sizeof(int64_t) * B * Sq * W);
    int32_t *r32 = malloc(sizeof(int32_t) * B * Sq * W);
    for (int64_t s = 0; s < B * Sq * W; ++s) {
        const double u = uniform();
        int64_t v = (int64_t)(uniform() * Skv);
        if (u < 0.1) v = -1;
        else if (u < 0.15) v = Skv + 3;
        else if (u < 0.2) v = is_i64 ? ((int64_t)1 << 33) + 5 : -7;
        r64[s] = v;
        r32[s] = (int32_t)(v > INT32_MAX || v < INT32_MIN ? -1 : v);
    }
    for (int64_t x = 0; x < W; ++x) r64[x] = r32[x] = -1; /* an empty first row */
    const void *routes = is_i64 ? (const void *)r64 : (const void *)r32;

    int64_t *keys = malloc(sizeof(int64_t) * (W > 0 ? W : 1));
    for (int64_t row = 0; row < B * Sq; ++row) (void)orc_route_set(routes, is_i64, W, Skv, row, keys);

    uint8_t *memb = malloc((size_t)(B * Sq * stride));
    uint8_t *has = malloc((size_t)(B * Sq));
    orc_membership(routes, is_i64, B, Sq, W, Skv, stride, memb, has);
    const int64_t nqt = (Sq + 127) / 128, nkt = (Skv + 127) / 128;
    int32_t *kinds = malloc(4 * B * nqt * nkt), *fpc = malloc(4 * B * nqt),
            *fpi = malloc(4 * B * nqt * nkt), *ffc = malloc(4 * B * nqt),
            *ffi = malloc(4 * B * nqt * nkt), *rpc = malloc(4 * B * nkt),
            *rpi = malloc(4 * B * nkt * nqt), *rfc = malloc(4 * B * nkt),
            *rfi = malloc(4 * B * nkt * nqt);
    orc_tiles(memb, B, Sq, Skv, stride, 128, 128, kinds, fpc, fpi, ffc, ffi, rpc, rpi, rfc, rfi);

    double *q = malloc(sizeof(double) * B * Sq * Hq * D), *g = malloc(sizeof(double) * B * Sq * Hq * D);
    double *k = malloc(sizeof(double) * B * Skv * Hkv * D), *v = malloc(sizeof(double) * B * Skv * Hkv * D);
    for (int64_t x = 0; x < B * Sq * Hq * D; ++x) {
        q[x] = uniform() - 0.5;
        g[x] = uniform() - 0.5;
    }
    for (int64_t x = 0; x < B * Skv * Hkv * D; ++x) {
        k[x] = uniform() - 0.5;
        v[x] = uniform() - 0.5;
    }
    orc_problem P = {B, Sq, Skv, Hq, Hkv, D, W, is_i64, 0, 0.0625, routes, q, k, v, g, NULL, NULL};
    const int64_t nrows = B * Sq;
    int64_t *rows = malloc(sizeof(int64_t) * nrows);
    for (int64_t x = 0; x < nrows; ++x) rows[x] = x;
    double *out = malloc(sizeof(double) * B * Sq * Hq * D), *lse = malloc(sizeof(double) * B * Hq * Sq);
    orc_forward(&P, nrows, rows, out, lse);
    double *dq = malloc(sizeof(double) * B * Sq * Hq * D);
    orc_backward_dq(&P, nrows, rows, dq);
    int64_t *kk = malloc(sizeof(int64_t) * B * Skv);
    int64_t nk = 0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t j = 0; j < Skv; j += 3) kk[nk++] = b * Skv + j;
    double *dk = malloc(sizeof(double) * nk * Hkv * D), *dv = malloc(sizeof(double) * nk * Hkv * D);
    orc_backward_dkdv(&P, nk, kk, dk, dv);
    double *dq2 = malloc(sizeof(double) * B * Sq * Hq * D);
    double *dk2 = malloc(sizeof(double) * B * Skv * Hkv * D), *dv2 = malloc(sizeof(double) * B * Skv * Hkv * D);
    double *out2 = malloc(sizeof(double) * B * Sq * Hq * D), *lse2 = malloc(sizeof(double) * B * Hq * Sq);
    orc_backward_rows(&P, nrows, rows, dq2, dk2, dv2, out2, lse2);
    /* saved state: out [B, Sq, Hq, D] as the forward wrote it, lse moved from the
     * forward's [row, Hq] order to [B, Hq, Sq] */
    double *lse_t = malloc(sizeof(double) * B * Hq * Sq);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t i = 0; i < Sq; ++i)
            for (int64_t h = 0; h < Hq; ++h) lse_t[(b * Hq + h) * Sq + i] = lse[(b * Sq + i) * Hq + h];
    P.o_saved = out;
    P.lse_saved = lse_t;
    orc_backward_rows(&P, nrows, rows, dq2, dk2, dv2, NULL, NULL);

    int bad = check_finite(out, B * Sq * Hq * D, "out") | check_finite(dq, B * Sq * Hq * D, "dq") |
              check_finite(dk, nk * Hkv * D, "dk") | check_finite(dv, nk * Hkv * D, "dv") |
              check_finite(dk2, B * Skv * Hkv * D, "dk2");
    free(r64); free(r32); free(keys); free(memb); free(has); free(kinds); free(fpc); free(fpi);
    free(ffc); free(ffi); free(rpc); free(rpi); free(rfc); free(rfi); free(q); free(g); free(k);
    free(v); free(rows); free(out); free(lse); free(dq); free(kk); free(dk); free(dv); free(dq2);
    free(dk2); free(dv2); free(out2); free(lse2); free(lse_t);
    return bad;
}

static int run_blocks(int64_t T, int64_t NB)
{
    const int64_t stride = (T + 127) / 128 * 128;
    uint8_t *sel = malloc((size_t)(T * NB));
    int32_t *lo = malloc(4 * T), *hi = malloc(4 * T), *bb = malloc(4 * T), *tb = malloc(4 * T);
    for (int64_t x = 0; x < T * NB; ++x) sel[x] = uniform() < 0.3 ? (uint8_t)(1 + (next_u64() & 127)) : 0;
    for (int64_t t = 0; t < T; ++t) {
        lo[t] = (int32_t)(uniform() * (T + 40)) - 20;
        hi[t] = (int32_t)(uniform() * (T + 40)) - 20;
        bb[t] = (int32_t)(uniform() * (NB + 20)) - 10;
        tb[t] = (int32_t)(uniform() * (T + 60)) - 30;
    }
    lo[0] = INT32_MIN;
    hi[0] = INT32_MAX;
    bb[0] = INT32_MIN;
    tb[0] = INT32_MAX;
    uint8_t *memb = malloc((size_t)(T * stride)), *has = malloc((size_t)T);
    orc_block_membership(sel, T, NB, lo, hi, bb, tb, 4, stride, memb, has);
    free(sel); free(lo); free(hi); free(bb); free(tb); free(memb); free(has);
    return 0;
}

int main(void)
{
    int bad = 0;
    bad |= run_case(1, 130, 200, 1, 20, 0);
    bad |= run_case(2, 70, 129, 2, 9, 1);
    bad |= run_case(1, 5, 3, 1, 1, 0);
    bad |= run_blocks(200, 60);
    bad |= run_blocks(1, 1);
    if (bad) return 1;
    printf("oracle driver ok\n");
    return 0;
}
