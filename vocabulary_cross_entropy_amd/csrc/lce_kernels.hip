// Fused linear cross-entropy (placeholder until the matrix-core kernels land).
#include "vce_device.h"
#include "vce_internal.h"

namespace vce {

bool lce_make_plan(int64_t M, int64_t H, int64_t V, LcePlan* plan) {
  (void)M; (void)H; (void)V; (void)plan;
  return false;
}

hipError_t launch_lce_forward(const LcePlan&, const LceFwdArgs&, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_lce_backward(const LcePlan&, const LceBwdArgs&, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_gemm_bf16(const void*, int, int64_t, const void*, int, int64_t, int64_t, int64_t,
                            int64_t, float*, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace vce
