// Fused kernel instances: float32 I/O, time-varying.
#define S5_INST_BF16 0
#define S5_INST_TV 1
#include "s5_fused_inst.h"

namespace s5 {

hipError_t launch_reduce_f32_tv(const FusedParams& q, const FusedPlan& p, hipStream_t s) {
  return dispatch<true>(q, p, s);
}

hipError_t launch_scan_f32_tv(const FusedParams& q, const FusedPlan& p, hipStream_t s) {
  return dispatch<false>(q, p, s);
}

}  // namespace s5
