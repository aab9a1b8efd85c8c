// Kernel launchers for the host-only sanitizer build of api.cpp: that build
// checks argument validation and workspace arithmetic on a machine without
// a GPU, where no call gets past the device check, so no launcher runs.
// Each reports a failed launch if it ever did.
#include "common.h"

namespace qsa {
hipError_t launch_preprocess(const Problem &, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_walk_reset(const Problem &, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_partial_keys(const Problem &, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_row_keys(const Problem &, int32_t *, int32_t *, hipStream_t)
{
    return hipErrorLaunchFailure;
}
hipError_t launch_forward(const Problem &, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_forward_dense(const Problem &, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_dq_dense(const Problem &, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_dkdv_dense(const Problem &, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_delta(const Problem &, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_dq(const Problem &, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_dkdv(const Problem &, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_dkdv_reduce(const Problem &, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_select_fill(const SelectProblem &, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_select_scores(const SelectProblem &, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_select_topk(const SelectProblem &, hipStream_t) { return hipErrorLaunchFailure; }
}  // namespace qsa
