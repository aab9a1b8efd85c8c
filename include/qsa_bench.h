/*
 * qsa_bench.h -- timing variants of the QSA calls, for benchmarks and
 * profiling. NOT a stable ABI: the stage list changes with the kernels, and
 * these entry points may change or go away between library versions. Code
 * that computes attention uses qsa.h only.
 *
 * Each variant does exactly the work of its plain call (same validation, same
 * launches, same results) and in addition records caller-created HIP events
 * between the launch stages, so that a caller can time each kernel on the
 * stream it runs on. `events` holds n_events >= stages + 1 hipEvent_t
 * handles; events[0] is recorded before the first launch and events[s + 1]
 * after stage s. events == NULL behaves exactly like the plain call; too few
 * events gives QSA_ERR_NULL.
 *
 * Forward stages: 0 route preprocessing, 1 attention over the keys of
 * partial tiles (gathered), 2 attention over full tiles (dense) and the
 * output write.
 * Backward stages: 0 route preprocessing, 1 delta, 2 dQ over the keys of
 * partial tiles (gathered), 3 dQ over full tiles (dense) and the dQ write,
 * 4 dK/dV partial sums of partial tiles per query segment, 5 dK/dV partial
 * sums of full tiles (dense), 6 the sum of the partials and the bf16 cast.
 */
#ifndef QSA_BENCH_H
#define QSA_BENCH_H

#include "qsa.h"

#ifdef __cplusplus
extern "C" {
#endif

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

/* The same for the planned calls; their stage 0 only resets the walk clocks
 * (the plan replaces the preprocessing). */
qsa_status qsa_forward_planned_timed(const qsa_plan *plan, const void *q, const void *k,
                                     const void *v, float scale, void *out, float *out_fp32,
                                     float *lse, void *workspace, size_t workspace_bytes,
                                     void *stream, void *const *events, int32_t n_events);
qsa_status qsa_backward_planned_timed(const qsa_plan *plan, const void *grad_out, const void *q,
                                      const void *k, const void *v, const float *out_fp32,
                                      const float *lse, float scale, void *dq, void *dk,
                                      void *dv, void *workspace, size_t workspace_bytes,
                                      void *stream, void *const *events, int32_t n_events);

/* The selector with stage events: stage 0 the scores (with the -inf fill of
 * a caller's scores buffer), stage 1 the top-k selection and the outputs. */
#define QSA_SELECT_STAGES 2
qsa_status qsa_select_timed(const qsa_select_dims *dims, const void *q_idx, const void *kbar,
                            const int32_t *doc_start, const int32_t *blk_base, float scale,
                            int32_t *blocks, int32_t *routes, float *scores, void *workspace,
                            size_t workspace_bytes, void *stream, void *const *events,
                            int32_t n_events);

/*
 * Gather-rate probe: stages rows rows[0 .. n_rows) of `src` (device memory of
 * src_bytes < 2^31; row i occupies bytes [rows[i] * row_bytes, + row_bytes))
 * into LDS with the direct-to-LDS loads the gathered kernels use, and
 * discards them. row_bytes is 512 (K or V rows, two per load instruction,
 * as the gathered forward and dQ stage them; n_rows even) or 6144 (the 12
 * heads of one Q or dO row, as the gathered dK/dV stages them). `blocks` work
 * groups share the rows; `shape` picks the launch shape, 0 .. 3: four waves
 * with 32 KB of LDS each, eight with 16 KB, eight with 20 KB, four with
 * 16 KB (two work groups per CU). Row indices must lie inside `src`
 * (out-of-range offsets read zeros). Timing is the caller's (events around
 * the call).
 */
qsa_status qsa_bench_gather(const void *src, size_t src_bytes, const int32_t *rows,
                            int64_t n_rows, int32_t row_bytes, int32_t blocks, int32_t shape,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_BENCH_H */
