/*
 * qsa.h -- C ABI of the MI355X (gfx950) route-set grouped-query attention
 * library (Query Sparse Attention, QSA).
 *
 * The operation. Each query row (b, i) attends exactly to the set R(b, i) of
 * key/value rows named by its routes: every route value r with 0 <= r < Skv,
 * tested on the full integer width, is a member; duplicates count once; -1 and
 * every other out-of-range value is padding. All query heads share the row's
 * set; query head h reads KV head h / 12. No causal or document mask is added:
 * the routes carry causality, documents and padding. A row with no member gives
 * exactly zero output, zero query gradient and lse = -inf. The selection
 * receives no gradient.
 *   Sources: "nemo_automodel ... qwen3_8_flash_next.flex_qsa" page (module
 *   summary, `_routes_to_membership`); "... fa4_qsa" page (`_preprocess`,
 *   `fa4_sparse_gqa_attention`); cuDNN Frontend "Query Sparse Attention (QSA)"
 *   page, sections "Tensors" and "Selection and components".
 *
 * Forward (per head, over j in R): s_j = scale <q, k_j>, lse = ln sum_j e^{s_j},
 * out_fp32 = sum_j e^{s_j - lse} v_j, out = bf16(out_fp32) (round to nearest
 * even). Backward: P = e^{S - lse} on members, delta = sum(grad_out * out_fp32),
 * dP = grad_out V^T, dS = P (dP - delta), dQ = scale dS K, dK = scale dS^T Q,
 * dV = P^T grad_out, with dK and dV summed over the 12 query heads of a KV head
 * (QSA page, "Selection and components", backward equations).
 *
 * Conventions for every call.
 *  - Tensor pointers are DEVICE pointers to contiguous row-major arrays;
 *    `dims` and `scale` are host values. Layouts:
 *      q, out, grad_out, dq    [B, Sq, Hq, 256]  bf16 (out_fp32: fp32)
 *      k, v, dk, dv            [B, Skv, Hkv, 256] bf16
 *      routes                  [B, Sq, W] int32, or int64 if route_is_i64
 *      lse                     [B, Hq, Sq] fp32, natural log
 *    (QSA page, "Tensors": FP32 out_fp32 and [Hq, T] LSE are the saved state.)
 *  - Alignment: 16 bytes for q, k, v, grad_out, out, out_fp32, dq, dk, dv and
 *    the workspace; 4 bytes for lse and int32 routes, 8 for int64 routes
 *    (QSA page, "Tensors": layouts are rejected before launch).
 *  - Shapes: B, Sq, Skv, W >= 1; D == 256; Hkv >= 1 and Hq == 12 * Hkv, so
 *    24Q/2KV runs as two independent 12Q/1KV groups; Skv <= 2^19 (the per-row
 *    route scatter holds one bit per key on chip); W <= 2^20. scale must be
 *    finite and > 0. All offsets are 64-bit, so B * Sq * Skv beyond 2^31 is
 *    supported ("flex_qsa" page, `_membership_flat_offset`).
 *  - Route VALUES are never read on the host and the host never waits on the
 *    device: every count stays on the device ("fa4_qsa" page, `_block_kinds`).
 *  - Ownership: the caller allocates every output and the workspace, whose
 *    size the matching *_workspace_bytes call returns. The library keeps no
 *    state between calls and writes every output element, so outputs need no
 *    clearing. Outputs must not overlap inputs or each other.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and
 *    the call returns without waiting for it. Calls that share a workspace
 *    must be ordered on one stream.
 *  - Errors: validation happens on the host before any launch and returns a
 *    status without touching the device; QSA_ERR_LAUNCH reports a failed
 *    launch. The error classes follow the "cudnn_qsa" page
 *    (`cudnn_sparse_gqa_attention`, Raises): value errors -> SHAPE, HEADS,
 *    HEADDIM, SCALE; type errors -> ROUTE_DTYPE; runtime errors -> DEVICE,
 *    LAUNCH.
 *  - Determinism: no kernel uses floating-point atomics; for fixed inputs the
 *    results are bitwise reproducible, and they do not depend on the order of
 *    the route slots, on duplicates or on which invalid value pads a slot.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qsa_status {
    QSA_OK = 0,
    QSA_ERR_NULL = 1,        /* a required pointer is NULL */
    QSA_ERR_SHAPE = 2,       /* a dimension < 1 or beyond the stated limits */
    QSA_ERR_HEADS = 3,       /* Hkv < 1 or Hq != 12 * Hkv */
    QSA_ERR_HEADDIM = 4,     /* D != 256 */
    QSA_ERR_SCALE = 5,       /* scale not finite or not > 0 */
    QSA_ERR_ALIGN = 6,       /* a pointer is not aligned as stated above */
    QSA_ERR_ROUTE_DTYPE = 7, /* route_is_i64 not 0 or 1, or an unknown flags bit */
    QSA_ERR_WORKSPACE = 8,   /* workspace NULL or smaller than required */
    QSA_ERR_DEVICE = 9,      /* no gfx950 device current, or a HIP runtime error */
    QSA_ERR_LAUNCH = 10      /* a kernel launch failed */
} qsa_status;

/* Bits of qsa_dims.flags.
 * QSA_FLAG_DETERMINISTIC: the same inputs give bitwise the same outputs on
 *   every call. Without it (the default), on calls with at least eight
 *   query rows per resident wave of the device (B * Sq * Hkv >= 64 * CUs),
 *   the gathered forward and dQ passes start each query row's walk over its
 *   key list at the point that the rows in flight have reached, so that they
 *   read the same key rows at about the same time; the sums are the same sums
 *   taken in another order, so out_fp32, lse and dq (and through them dk, dv)
 *   can differ in the last bits between calls, with the same accuracy.
 *   Smaller calls are bitwise reproducible either way. */
#define QSA_FLAG_DETERMINISTIC 1

typedef struct qsa_dims {
    int64_t B, Sq, Skv, Hq, Hkv, D, W;
    int32_t route_is_i64; /* 0: routes are int32, 1: int64 */
    int32_t flags;        /* QSA_FLAG_* bits; every other bit must be 0 */
} qsa_dims;

/* Sizes of the workspace each call needs (0 if `dims` is invalid). */
size_t qsa_forward_workspace_bytes(const qsa_dims *dims);
size_t qsa_backward_workspace_bytes(const qsa_dims *dims);
size_t qsa_preprocess_workspace_bytes(const qsa_dims *dims);

/*
 * Forward. Runs the route preprocessing (membership table, tile kinds, tile
 * lists, per-row sorted key lists) into the workspace, then the attention.
 * Outputs: out (bf16), out_fp32, lse. Empty rows: out = out_fp32 = +0,
 * lse = -inf. (QSA page, "Selection and components", forward paragraph.)
 */
qsa_status qsa_forward(const qsa_dims *dims, const void *q, const void *k, const void *v,
                       const void *routes, float scale, void *out, float *out_fp32, float *lse,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward. Takes the forward's out_fp32 and lse (not a re-cast of `out`) and
 * the same q, k, v, routes and scale; reruns the route preprocessing, computes
 * delta = sum(grad_out * out_fp32) per (row, head), then dq (query-major, from
 * the per-row key lists) and dk, dv (key-major, from the reverse tile lists and
 * the membership table; no atomics). Keys that no query selects get dk = dv = 0;
 * empty rows get dq = 0. (QSA page, "Selection and components", backward
 * paragraph and equations.)
 */
qsa_status qsa_backward(const qsa_dims *dims, const void *grad_out, const void *q, const void *k,
                        const void *v, const float *out_fp32, const float *lse,
                        const void *routes, float scale, void *dq, void *dk, void *dv,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Route preprocessing alone, for inspection and bit-exact checks. With
 * nQT = ceil(Sq / 128), nKT = ceil(Skv / 128), stride = nKT * 128:
 *   memb       uint8 [B, Sq, stride]  1 where j is in R(b, i), 0 elsewhere and in
 *                                     the padding columns j >= Skv
 *   has_routes uint8 [B, Sq]          |R(b, i)| > 0
 *   kinds      int32 [B, nQT, nKT]    per 128 x 128 tile: 0 absent, 1 partial,
 *                                     2 full (every cell a member; a ragged edge
 *                                     tile is therefore never full)
 *   fwd_p_cnt, fwd_f_cnt int32 [B, nQT]; fwd_p_idx, fwd_f_idx int32 [B, nQT, nKT]:
 *                                     per tile row, the partial / full tile
 *                                     columns in ascending order, then -1
 *   rev_p_cnt, rev_f_cnt int32 [B, nKT]; rev_p_idx, rev_f_idx int32 [B, nKT, nQT]:
 *                                     per tile column, the partial / full tile
 *                                     rows in ascending order, then -1
 *   row_keys   int32 [B, Sq, W]       R(b, i) in ascending order, then -1
 *                                     (optional: NULL skips it)
 *   row_cnt    int32 [B, Sq]          |R(b, i)| (optional)
 * ("fa4_qsa" page: `_preprocess`, `_block_kinds`, `_compact_blocks`;
 *  "flex_qsa" page: `_routes_to_membership`, `_dense_blocks_to_ordered`.)
 * Alignment: 16 bytes for memb, 4 bytes for the int32 arrays.
 */
qsa_status qsa_preprocess(const qsa_dims *dims, const void *routes, uint8_t *memb,
                          uint8_t *has_routes, int32_t *kinds, int32_t *fwd_p_cnt,
                          int32_t *fwd_p_idx, int32_t *fwd_f_cnt, int32_t *fwd_f_idx,
                          int32_t *rev_p_cnt, int32_t *rev_p_idx, int32_t *rev_f_cnt,
                          int32_t *rev_f_idx, int32_t *row_keys, int32_t *row_cnt,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Benchmark variants: identical work, plus event records between the launch
 * stages so a caller can time each kernel on the stream it runs on. `events`
 * holds n_events >= stages + 1 hipEvent_t handles created by the caller;
 * events[0] is recorded before the first launch and events[s + 1] after
 * stage s. Forward stages: 0 route preprocessing, 1 attention over the keys
 * of partial tiles (gathered), 2 attention over full tiles (dense) and the
 * output write. Backward stages: 0 route preprocessing, 1 delta, 2 dQ over
 * the keys of partial tiles (gathered), 3 dQ over full tiles (dense) and the
 * dQ write, 4 dK/dV partial sums of partial tiles per query segment, 5 dK/dV
 * partial sums of full tiles (dense), 6 the sum of the partials and the bf16
 * cast. events == NULL behaves exactly like the plain call; too few events
 * gives QSA_ERR_NULL.
 */
#define QSA_FORWARD_STAGES 3
#define QSA_BACKWARD_STAGES 7
qsa_status qsa_forward_timed(const qsa_dims *dims, const void *q, const void *k, const void *v,
                             const void *routes, float scale, void *out, float *out_fp32,
                             float *lse, void *workspace, size_t workspace_bytes, void *stream,
                             void *const *events, int32_t n_events);
qsa_status qsa_backward_timed(const qsa_dims *dims, const void *grad_out, const void *q,
                              const void *k, const void *v, const float *out_fp32,
                              const float *lse, const void *routes, float scale, void *dq,
                              void *dk, void *dv, void *workspace, size_t workspace_bytes,
                              void *stream, void *const *events, int32_t n_events);

/* Static description of a status code. */
const char *qsa_status_string(qsa_status status);

/* Library ABI version: (major << 16) | minor. */
int32_t qsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
