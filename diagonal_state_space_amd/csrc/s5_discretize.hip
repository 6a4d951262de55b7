// Zero-order-hold discretisation of the diagonal S5 system (paper eq. 6;
// App. A `discretize`; abhik.ai review, row 2 "Integrate a held input exactly").
//
// Per mode p, in float64:
//   Delta = exp(log_delta[p]),  z = lambda[p]*Delta,
//   lambda_bar = exp(z),
//   gain = (exp(z) - 1)/lambda       (|z| >= 1e-4)
//        = Delta * sum_{n=0}^{8} z^n/(n+1)!   (|z| < 1e-4; removable singularity)
//   b_bar[p, :] = gain * b_tilde[p, :]
// Results are rounded to float32.
#include "s5_f64.h"
#include "s5_internal.h"

namespace s5 {

using f64::zd;

// One block per mode; threads stride over H.
__global__ void __launch_bounds__(256) k_discretize(int P, int H, const float2* __restrict__ lam,
                                                    const float2* __restrict__ b_tilde,
                                                    const float* __restrict__ log_delta,
                                                    float2* __restrict__ lam_bar_out,
                                                    float2* __restrict__ b_bar_out) {
  const int p = blockIdx.x;
  if (p >= P) return;
  const zd l = {static_cast<double>(lam[p].x), static_cast<double>(lam[p].y)};
  zd lb, g;
  f64::zoh(l, exp(static_cast<double>(log_delta[p])), lb, g);
  if (threadIdx.x == 0) lam_bar_out[p] = make_float2(static_cast<float>(lb.re), static_cast<float>(lb.im));
  for (int h = threadIdx.x; h < H; h += blockDim.x) {
    const float2 bt = b_tilde[static_cast<size_t>(p) * H + h];
    const zd b = f64::zmul(g, {static_cast<double>(bt.x), static_cast<double>(bt.y)});
    b_bar_out[static_cast<size_t>(p) * H + h] = make_float2(static_cast<float>(b.re), static_cast<float>(b.im));
  }
}

hipError_t launch_discretize(int P, int H, const float2* lam, const float2* b_tilde, const float* log_delta,
                             float2* lam_bar, float2* b_bar, hipStream_t stream) {
  hipLaunchKernelGGL(k_discretize, dim3(P), dim3(256), 0, stream, P, H, lam, b_tilde, log_delta, lam_bar, b_bar);
  return hipGetLastError();
}

}  // namespace s5
