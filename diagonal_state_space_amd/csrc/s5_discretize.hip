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
#include "s5_internal.h"

namespace s5 {

struct zd {
  double re, im;
};

__device__ __forceinline__ zd zmul(zd a, zd b) {
  return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re};
}

__device__ __forceinline__ zd zdiv(zd a, zd b) {
  const double den = b.re * b.re + b.im * b.im;
  return {(a.re * b.re + a.im * b.im) / den, (a.im * b.re - a.re * b.im) / den};
}

__device__ __forceinline__ zd zexp(zd z) {
  const double e = exp(z.re);
  double s, c;
  sincos(z.im, &s, &c);
  return {e * c, e * s};
}

// Gain (exp(z) - 1)/lambda for z = lambda*delta, float64.
__device__ __forceinline__ zd zoh_gain(zd lam, double delta, zd lam_bar) {
  const zd z = {lam.re * delta, lam.im * delta};
  if (sqrt(z.re * z.re + z.im * z.im) < 1e-4) {
    zd term = {1.0, 0.0};
    zd phi = {1.0, 0.0};
    for (int n = 1; n <= 8; ++n) {
      term = zmul(term, z);
      term.re /= (n + 1);
      term.im /= (n + 1);
      phi.re += term.re;
      phi.im += term.im;
    }
    return {delta * phi.re, delta * phi.im};
  }
  return zdiv({lam_bar.re - 1.0, lam_bar.im}, lam);
}

// One block per mode; threads stride over H.
// Outputs (any may be null): lam_bar[P], b_bar[P,H], pow_out[P] = lam_bar^pow_n
// (exp(pow_n*z) evaluated directly), inv_lam[P] = 1/lambda.
__global__ void __launch_bounds__(256) k_discretize(int P, int H, const float2* __restrict__ lam,
                                                    const float2* __restrict__ b_tilde,
                                                    const float* __restrict__ log_delta,
                                                    float2* __restrict__ lam_bar_out,
                                                    float2* __restrict__ b_bar_out,
                                                    float2* __restrict__ pow_out, int pow_n,
                                                    float2* __restrict__ inv_lam_out) {
  const int p = blockIdx.x;
  if (p >= P) return;
  const zd l = {static_cast<double>(lam[p].x), static_cast<double>(lam[p].y)};
  const double delta = exp(static_cast<double>(log_delta[p]));
  const zd z = {l.re * delta, l.im * delta};
  const zd lb = zexp(z);
  const zd g = zoh_gain(l, delta, lb);
  if (threadIdx.x == 0) {
    if (lam_bar_out) lam_bar_out[p] = make_float2(static_cast<float>(lb.re), static_cast<float>(lb.im));
    if (pow_out) {
      const zd pw = zexp({z.re * pow_n, z.im * pow_n});
      pow_out[p] = make_float2(static_cast<float>(pw.re), static_cast<float>(pw.im));
    }
    if (inv_lam_out) {
      const zd il = zdiv({1.0, 0.0}, l);
      inv_lam_out[p] = make_float2(static_cast<float>(il.re), static_cast<float>(il.im));
    }
  }
  if (b_bar_out) {
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
      const float2 bt = b_tilde[static_cast<size_t>(p) * H + h];
      const zd b = zmul(g, {static_cast<double>(bt.x), static_cast<double>(bt.y)});
      b_bar_out[static_cast<size_t>(p) * H + h] =
          make_float2(static_cast<float>(b.re), static_cast<float>(b.im));
    }
  }
}

hipError_t launch_discretize(int P, int H, const float2* lam, const float2* b_tilde,
                             const float* log_delta, float2* lam_bar, float2* b_bar,
                             float2* pow_out, int pow_n, float2* inv_lam, hipStream_t stream) {
  hipLaunchKernelGGL(k_discretize, dim3(P), dim3(256), 0, stream, P, H, lam, b_tilde, log_delta,
                     lam_bar, b_bar, pow_out, pow_n, inv_lam);
  return hipGetLastError();
}

// 1/lambda per mode in float64 (time-varying path; lambda = 0 gives inf, which
// the per-step small-|z| branch never reads).
__global__ void k_inv_lambda(int P, const float2* __restrict__ lam, float2* __restrict__ out) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= P) return;
  const zd l = {static_cast<double>(lam[p].x), static_cast<double>(lam[p].y)};
  const zd il = zdiv({1.0, 0.0}, l);
  out[p] = make_float2(static_cast<float>(il.re), static_cast<float>(il.im));
}

hipError_t launch_inv_lambda(int P, const float2* lam, float2* out, hipStream_t stream) {
  hipLaunchKernelGGL(k_inv_lambda, dim3((P + 255) / 256), dim3(256), 0, stream, P, lam, out);
  return hipGetLastError();
}

}  // namespace s5
