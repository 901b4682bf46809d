// First kernel of the decode step on the float32 path: the step's small
// per-sequence jobs (step_prep.h) in one launch, role = blockIdx.x.  The
// bf16 path folds the same jobs into the score kernel instead.
#include "step_prep.h"

namespace csa {

namespace {

constexpr int kPrepThreads = 256;

__global__ __launch_bounds__(kPrepThreads) void k_step_prep(PrepArgs a) {
    __shared__ float ybuf[kPrepMaxD];
    __shared__ float red[kPrepThreads / kWave];
    step_prep_role(a, blockIdx.x, blockIdx.y, ybuf, red);
}

}  // namespace

hipError_t launch_step_prep(const PrepArgs& a, hipStream_t s) {
    const int roles = !a.completes ? 1 : (a.main_wgs > 1 ? 1 + a.main_wgs : 3);
    hipLaunchKernelGGL(k_step_prep, dim3(roles, a.batch), dim3(kPrepThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace csa
