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
 *  - Shapes: B, Sq, Skv, W >= 1; D == 256; 1 <= Hkv <= 4096 and Hq == 12 *
 *    Hkv, so 24Q/2KV runs as two independent 12Q/1KV groups; Skv <= 2^19 (the
 *    per-row route scatter holds one bit per key on chip); W <= 2^20. scale
 *    must be finite and > 0. Grid and addressing limits: B, Sq and B * Sq <=
 *    2^24, B * Sq * Hq <= 2^26, B * Hkv * ceil(Skv / 128) * 128 <= 2^30; one
 *    batch row of Q (Sq * Hq * 512 bytes) and of K (Skv * Hkv * 512 bytes)
 *    each below 2^31 bytes, since the gathers use 32-bit offsets inside a
 *    batch row. Offsets across batch rows and tables are 64-bit, so B * Sq *
 *    Skv beyond 2^31 is supported ("flex_qsa" page,
 *    `_membership_flat_offset`). Larger shapes return QSA_ERR_SHAPE.
 *  - Route VALUES are never read on the host and the host never waits on the
 *    device: every count stays on the device ("fa4_qsa" page, `_block_kinds`).
 *  - Ownership: the caller allocates every output and the workspace, whose
 *    size the matching *_workspace_bytes call returns. The library keeps no
 *    data between calls (only per-device resources: cached device properties
 *    and the backward's second stream and its two events) and writes every
 *    output element, so outputs need no clearing. Outputs must not overlap inputs or each other.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and
 *    the call returns without waiting for it. Calls that share a workspace
 *    must be ordered on one stream. The backward calls run their dQ passes
 *    on a second stream of the library (one per device, default priority,
 *    created on the first backward call and kept until the process ends),
 *    forked from `stream` after the call's earlier work with an event and
 *    joined back into `stream` before its last kernel: work enqueued on
 *    `stream` after the call sees all its outputs, as if it had run on
 *    `stream` alone. The fork and join of one call are enqueued under a
 *    per-device lock, so calls from several host threads stay paired.
 *  - Errors: validation happens on the host before any launch and returns a
 *    status without touching the device; QSA_ERR_LAUNCH reports a failed
 *    launch. The error classes follow the "cudnn_qsa" page
 *    (`cudnn_sparse_gqa_attention`, Raises): value errors -> SHAPE, HEADS,
 *    HEADDIM, SCALE; type errors -> ROUTE_DTYPE; runtime errors -> DEVICE,
 *    LAUNCH.
 *  - Determinism: no kernel uses floating-point atomics. Two modes, chosen
 *    per call by QSA_FLAG_DETERMINISTIC (see below):
 *      with the flag, the same inputs give bitwise the same outputs on every
 *      call, and the outputs do not depend on the order of the route slots,
 *      on duplicates or on which invalid value pads a slot;
 *      without it (the default), calls with at least eight query rows per
 *      resident wave of the device (B * Sq * Hkv >= 64 * CUs) take the
 *      gathered sums in an order that depends on timing, so out_fp32, lse and
 *      the gradients can differ in their last bits between calls (same
 *      accuracy); smaller calls behave as with the flag. The default is about
 *      11 % faster on a 32768-token call (14.3 against 16.0 ms per plan build,
 *      forward and backward on MI355X).
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
    QSA_ERR_LAUNCH = 10,     /* a kernel launch failed */
    QSA_ERR_SCRATCH = 11,    /* qsa_forward_noalloc: the call needs more workspace than
                                the library's fixed device scratch holds */
    QSA_ERR_PLAN = 12        /* a plan not built by qsa_plan_build, edited so that its
                                buffer no longer fits its dims, or used on another device */
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
 * Route plan, built once and used by any number of forward, recomputed
 * forward and backward calls on the same routes (the mask object that the
 * "flex_qsa" page builds once per step and hands to both the checkpointed
 * forward and its recompute: `FlexQSAMask`, `build_flex_qsa_mask`, and the
 * `mask` argument of `flex_sparse_gqa_attention`).
 *
 * qsa_plan_build runs the route preprocessing of qsa_forward and
 * qsa_backward once (per-row sorted key lists, the membership bits the dK/dV
 * pass reads, tile kinds and forward and reverse tile lists) into plan_mem, a
 * caller-owned device buffer of at least qsa_plan_bytes(dims) bytes (16-byte
 * aligned), and fills the host struct *plan. The routes are not read again
 * after the build's kernels have run. The planned calls below read plan_mem
 * and never write it, so one plan serves calls on several streams once its
 * build is complete on each of them (order them after the build, e.g. with
 * an event).
 *
 * Ownership: plan_mem stays the caller's; the plan struct only records it.
 * The plan is valid while plan_mem holds what the build wrote and only on
 * the device that was current during the build. Freeing or overwriting
 * plan_mem, or changing the routes, needs a new build. qsa_plan_build clears
 * *plan first, so a failed build leaves a plan that every planned call
 * rejects with QSA_ERR_PLAN.
 *
 * The planned calls take the plan in place of dims and routes and compute
 * exactly what qsa_forward and qsa_backward compute from the same routes
 * (bitwise, with QSA_FLAG_DETERMINISTIC in the plan's dims); their own
 * workspace holds only per-call scratch (the sizes below, much smaller than
 * the plain calls'). The plan's dims, including flags, apply to every
 * planned call.
 */
#define QSA_PLAN_TAG 0x51534150u
typedef struct qsa_plan {
    qsa_dims dims;    /* the dims the plan was built for */
    void *mem;        /* the caller's device buffer holding the plan */
    size_t bytes;     /* its size as passed to qsa_plan_build */
    int32_t device;   /* HIP device current during the build */
    uint32_t tag;     /* QSA_PLAN_TAG after a successful build */
} qsa_plan;
size_t qsa_plan_bytes(const qsa_dims *dims);
size_t qsa_forward_planned_workspace_bytes(const qsa_dims *dims);
size_t qsa_backward_planned_workspace_bytes(const qsa_dims *dims);
qsa_status qsa_plan_build(const qsa_dims *dims, const void *routes, void *plan_mem,
                          size_t plan_bytes, qsa_plan *plan, void *stream);
qsa_status qsa_forward_planned(const qsa_plan *plan, const void *q, const void *k, const void *v,
                               float scale, void *out, float *out_fp32, float *lse,
                               void *workspace, size_t workspace_bytes, void *stream);
qsa_status qsa_backward_planned(const qsa_plan *plan, const void *grad_out, const void *q,
                                const void *k, const void *v, const float *out_fp32,
                                const float *lse, float scale, void *dq, void *dk, void *dv,
                                void *workspace, size_t workspace_bytes, void *stream);
/*
 * Block-bitmap selection over packed sequences: the Miles packed-training
 * interface of the cuDNN Frontend QSA page (sections "API" for the two
 * calls, "Tensors" for the layouts, "Selection and components" for the
 * lookup). T packed tokens are both the queries and the keys; NB blocks
 * cover all sequences. Key j is allowed for query t iff
 *     lo[t] <= j <= hi[t], 0 <= b < NB and sel_blocks[t, b] != 0,
 *     with b = blk_base[t] + floor((j - tok_base[t]) / block_size),
 * floor division for any sign. Everything else (forward, backward, empty
 * rows, no gradient for the selection) is as for route rows: a block
 * selection is expanded on the device into the same per-row key sets.
 *
 * Layouts (device pointers; int32 metadata 4-byte aligned, tensors as
 * above): q, out, grad_out, dq [T, Hq, 256]; k, v, dk, dv [T, Hkv, 256];
 * out_fp32 [T, Hq, 256]; lse [Hq, T]; sel_blocks uint8 [T, NB] (nonzero
 * selects); lo, hi, blk_base, tok_base int32 [T]; block_first, block_last
 * int32 [NB]. These are the shapes of qsa_dims with B = 1 and Sq = Skv = T.
 *
 * block_size must be 4. The metadata are a caller contract, as on that
 * page: nothing is read on the host, and invalid metadata give the
 * selection the lookup defines for them. The block spans block_first and
 * block_last are validated as pointers but not read: for a valid partition
 * they are what the lookup implies (block b of a sequence holds its tokens
 * tok_base + 4 (b - blk_base) .. + 3), and the lookup alone decides
 * membership.
 *
 * Memory: a row of a block selection can hold up to min(T, 4 NB) keys, and
 * the per-row key lists are sized for that (about 8 T min(T, 4 NB) bytes
 * in the plan, 8.6 GB at T = 32768 with NB = 8192).
 *
 * qsa_block_plan_build builds an ordinary qsa_plan (dims B = 1, Sq = Skv =
 * T, W = min(T, 4 NB), route_is_i64 = 0) for the planned calls and
 * qsa_plan_tables. qsa_block_forward and qsa_block_backward are the one-call
 * forms: each builds the plan at the start of its workspace, then runs the
 * planned call (so each call reads the current selection, as on that page).
 */
typedef struct qsa_block_dims {
    int64_t T;          /* packed tokens */
    int64_t NB;         /* blocks across all sequences, 1 <= NB <= 2^31 - 1 */
    int64_t Hq, Hkv, D; /* as in qsa_dims */
    int32_t block_size; /* must be 4 */
    int32_t flags;      /* QSA_FLAG_* bits */
} qsa_block_dims;
size_t qsa_block_plan_bytes(const qsa_block_dims *dims);
size_t qsa_block_forward_workspace_bytes(const qsa_block_dims *dims);
size_t qsa_block_backward_workspace_bytes(const qsa_block_dims *dims);
qsa_status qsa_block_plan_build(const qsa_block_dims *dims, const uint8_t *sel_blocks,
                                const int32_t *lo, const int32_t *hi, const int32_t *blk_base,
                                const int32_t *tok_base, const int32_t *block_first,
                                const int32_t *block_last, void *plan_mem, size_t plan_bytes,
                                qsa_plan *plan, void *stream);
qsa_status qsa_block_forward(const qsa_block_dims *dims, const void *q, const void *k,
                             const void *v, const uint8_t *sel_blocks, const int32_t *lo,
                             const int32_t *hi, const int32_t *blk_base, const int32_t *tok_base,
                             const int32_t *block_first, const int32_t *block_last, float scale,
                             void *out, float *out_fp32, float *lse, void *workspace,
                             size_t workspace_bytes, void *stream);
qsa_status qsa_block_backward(const qsa_block_dims *dims, const void *grad_out, const void *q,
                              const void *k, const void *v, const float *out_fp32,
                              const float *lse, const uint8_t *sel_blocks, const int32_t *lo,
                              const int32_t *hi, const int32_t *blk_base, const int32_t *tok_base,
                              const int32_t *block_first, const int32_t *block_last, float scale,
                              void *dq, void *dk, void *dv, void *workspace,
                              size_t workspace_bytes, void *stream);
/*
 * Document-causal attention: causal attention within documents, for a
 * contiguous query shard against the global keys (the "fa4" page,
 * `document_causal_fa4_attention`, and its module summary: packed documents
 * and context parallelism with contiguous shards). Query i of batch row b sits
 * at global position q_global_start + i and attends to key j iff
 *     q_doc_ids[b, i] != 0, kv_doc_ids[b, j] == q_doc_ids[b, i] and
 *     j <= q_global_start + i.
 * Document ids are 1-based; 0 marks padding: a padding query gets zero output
 * and gradients and lse = -inf, and a padding key is never attended. Any id
 * layout is taken as written (a document need not be one contiguous run).
 * Everything else is as for route rows: the document ids are expanded on the
 * device into the same per-row key sets, and a plan built from them serves
 * the planned calls and qsa_plan_tables.
 *
 * Layouts: q_doc_ids int32 [B, Sq], kv_doc_ids int32 [B, Skv] (device, 4-byte
 * aligned); tensors as for qsa_forward. q_global_start >= 0 (a shard's first
 * query position; 0 for self-attention over the whole sequence). The plan's
 * dims are B, Sq, Skv, Hq, Hkv, D with W = min(Skv, q_global_start + Sq), the
 * most keys a row can hold (per-row key lists sized for that: 4 bytes per key
 * slot and row).
 */
typedef struct qsa_doc_dims {
    int64_t B, Sq, Skv, Hq, Hkv, D; /* as in qsa_dims */
    int64_t q_global_start;         /* global position of query 0, >= 0 */
    int32_t flags;                  /* QSA_FLAG_* bits */
    int32_t reserved;               /* must be 0 (else QSA_ERR_ROUTE_DTYPE, as an unknown flag) */
} qsa_doc_dims;
size_t qsa_doc_plan_bytes(const qsa_doc_dims *dims);
size_t qsa_doc_forward_workspace_bytes(const qsa_doc_dims *dims);
size_t qsa_doc_backward_workspace_bytes(const qsa_doc_dims *dims);
qsa_status qsa_doc_plan_build(const qsa_doc_dims *dims, const int32_t *q_doc_ids,
                              const int32_t *kv_doc_ids, void *plan_mem, size_t plan_bytes,
                              qsa_plan *plan, void *stream);
qsa_status qsa_doc_forward(const qsa_doc_dims *dims, const void *q, const void *k, const void *v,
                           const int32_t *q_doc_ids, const int32_t *kv_doc_ids, float scale,
                           void *out, float *out_fp32, float *lse, void *workspace,
                           size_t workspace_bytes, void *stream);
qsa_status qsa_doc_backward(const qsa_doc_dims *dims, const void *grad_out, const void *q,
                            const void *k, const void *v, const float *out_fp32,
                            const float *lse, const int32_t *q_doc_ids,
                            const int32_t *kv_doc_ids, float scale, void *dq, void *dk, void *dv,
                            void *workspace, size_t workspace_bytes, void *stream);
/*
 * Copies of a built plan's tables, for inspection and bit-exact checks, in
 * the layouts qsa_preprocess documents, except that the membership comes bit
 * packed: mbits uint32 [B, Sq, stride / 32], bit (j % 32) of word j / 32 set
 * where j is in R(b, i). Every pointer is a device pointer to a buffer of
 * that size, 4-byte aligned, none may be NULL. Copies are enqueued on
 * `stream` after whatever the stream already holds; the plan is not changed.
 */
qsa_status qsa_plan_tables(const qsa_plan *plan, uint32_t *mbits, int32_t *kinds,
                           int32_t *fwd_p_cnt, int32_t *fwd_p_idx, int32_t *fwd_f_cnt,
                           int32_t *fwd_f_idx, int32_t *rev_p_cnt, int32_t *rev_p_idx,
                           int32_t *rev_f_cnt, int32_t *rev_f_idx, int32_t *row_keys,
                           int32_t *row_cnt, void *stream);
/*
 * Forward that allocates nothing, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). Same operation, arguments, validation and results as
 * qsa_forward, without the workspace arguments: the workspace is a fixed
 * device array of this library, QSA_NOALLOC_SCRATCH_BYTES (64 MiB) per
 * device, which each device holds from the first call until the process
 * ends. A call whose qsa_forward_workspace_bytes exceeds it returns
 * QSA_ERR_SCRATCH before touching the device. The call makes no device
 * allocation and no allocating library call. Every call on one device uses
 * that device's one array, so calls that overlap on one device (different
 * streams, or different host threads without ordering) race and give wrong
 * results: order them on one stream. The first call on each device looks up
 * the array's device address once (thread-safe).
 */
#define QSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
qsa_status qsa_forward_noalloc(const qsa_dims *dims, const void *q, const void *k, const void *v,
                               const void *routes, float scale, void *out, float *out_fp32,
                               float *lse, void *stream);

/*
 * Block selector (cuDNN Frontend QSA page, "Finding QSA attention and its
 * indexer"): the step that produces the route rows the calls above consume.
 *
 * Query t (0 <= t < Sq) of batch row b sits at position p = q_offset + t.
 * Its document starts at s = doc_start[b, t] and block j of the document
 * (tokens s + 4j .. s + 4j + 3, compression ratio four) is row
 * blk_base[b, t] + j of kbar[b]; with doc_start NULL every s is 0, with
 * blk_base NULL every base is 0. Block j is visible when it is complete
 * before the query's own block, j < (p - s) / 4 (integer division), and its
 * kbar row lies in [0, NB). A query with s < 0 or s > p is padding.
 *
 * Each visible block scores scale * sum over h < H of
 * relu(q_idx[b, t, h, :] . kbar[b, row, :]); each query keeps its top_k
 * visible blocks (all of them when fewer are visible), larger score first and,
 * between equal scores, the lower block number first (the pages leave the tie
 * rule open).
 *
 * Layouts (device memory, contiguous):
 *   q_idx      bf16 [B, Sq, H, D], 16-byte aligned
 *   kbar       bf16 [B, NB, D], 16-byte aligned
 *   doc_start  int32 [B, Sq] or NULL, 4-byte aligned
 *   blk_base   int32 [B, Sq] or NULL, 4-byte aligned
 * Outputs, each optional (NULL = not written), at least one not NULL:
 *   blocks     int32 [B, Sq, top_k]: the kept block numbers j in ascending
 *              order, then -1; padding queries: all -1. 4-byte aligned.
 *   routes     int32 [B, Sq, 4 top_k + 4], 16-byte aligned: route rows in the
 *              form qsa_forward takes (NeMo AutoModel QSA page,
 *              cudnn_sparse_gqa_attention): for the n-th kept block j, slots
 *              4n .. 4n+3 hold tokens s + 4j .. s + 4j + 3; slots up to 4 top_k
 *              hold -1; slots 4 top_k .. 4 top_k + 3 hold the query's own
 *              incomplete block, tokens s + 4((p - s) / 4) .. p, then -1.
 *              Padding queries: all -1.
 *   scores     float [B, Sq, NB] by kbar row: the score of every visible row,
 *              -inf elsewhere.
 * Shapes: B, Sq, NB >= 1; NB <= 32768; B * Sq < 2^31; 1 <= H <= 64; D = 128
 * (else QSA_ERR_HEADDIM); 1 <= top_k <= 4096; q_offset >= 0 and
 * q_offset + Sq < 2^31; flags = 0 (else QSA_ERR_ROUTE_DTYPE). scale finite and
 * > 0 (QSA_ERR_SCALE).
 * Workspace: qsa_select_workspace_bytes(dims) bytes (16-byte aligned; the
 * scores of every query, B * Sq * NB floats), or none when `scores` is given,
 * which then serves as that buffer. Work is enqueued on `stream`; the caller
 * owns every buffer; errors are returned before anything is enqueued.
 */
typedef struct {
    int64_t B, Sq, NB;
    int64_t q_offset;  /* position of query 0 of every batch row */
    int32_t H, D;      /* indexer heads and width */
    int32_t top_k;
    int32_t flags;
} qsa_select_dims;

size_t qsa_select_workspace_bytes(const qsa_select_dims *dims);
qsa_status qsa_select(const qsa_select_dims *dims, const void *q_idx, const void *kbar,
                      const int32_t *doc_start, const int32_t *blk_base, float scale,
                      int32_t *blocks, int32_t *routes, float *scores, void *workspace,
                      size_t workspace_bytes, void *stream);

/* Static description of a status code. */
const char *qsa_status_string(qsa_status status);

/* Library ABI version: (major << 16) | minor. */
int32_t qsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
