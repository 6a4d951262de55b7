// One recurrent step of the S5 layer for a batch of sequences: the online
// (streaming / generation) form, which keeps only the current state
// (abhik.ai review, "Associative scans preserve the recurrence": streaming
// keeps one state per layer; papercache notes Sec. 3.3):
//   x <- Lambda_bar x + B_bar u,   y = Re(C~ x) + D u   (paper eq. 2, 5).
// One workgroup per sequence; the whole step is a few hundred kilobytes of
// parameter reads, so it is latency-bound and runs on the vector units.
#include "s5_common.h"
#include "s5_f64.h"
#include "s5_internal.h"

namespace s5 {

namespace {

constexpr int kStepThreads = 512;   // >= S5_MAX_H outputs, >= 2 S5_MAX_P

using f64::zd;


// lanes per row of a sum: the 512 threads spread over `rows` rows, a power
// of two from 1 to 8, the lanes of a row adjacent
__device__ __forceinline__ int lanes_per_row(int rows) {
  int k = 1;
  while (k < 8 && rows * (2 * k) <= kStepThreads) k *= 2;
  return k;
}

// sum over the k adjacent lanes of a row (k a power of two <= 8)
__device__ __forceinline__ float row_sum(float v, int k) {
  for (int o = 1; o < k; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__global__ void __launch_bounds__(kStepThreads) k_step(StepArgs q) {
  __shared__ float s_u[kStepThreads];
  __shared__ float2 s_bu[kStepThreads / 2];
  __shared__ float2 s_x[kStepThreads / 2];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const size_t ub = static_cast<size_t>(b) * q.H;
  for (int h = t; h < q.H; h += kStepThreads)
    s_u[h] = q.bf16_io ? bf16_to_f32(static_cast<const uint16_t*>(q.u)[ub + h]) : static_cast<const float*>(q.u)[ub + h];
  __syncthreads();

  // drive: the k lanes of mode p sum B~[p, h] u[h] over h = part, part + k, ...
  const int kd = lanes_per_row(q.P);
  const int p = t / kd;
  const int part = t - p * kd;
  {
    float re = 0.0f, im = 0.0f;
    if (p < q.P) {
      const float2* row = q.b_tilde + static_cast<size_t>(p) * q.H;
#pragma unroll 16
      for (int h = part; h < q.H; h += kd) {
        const float2 bt = row[h];
        re = fmaf(bt.x, s_u[h], re);
        im = fmaf(bt.y, s_u[h], im);
      }
    }
    re = row_sum(re, kd);   // every lane takes part (the shuffles span the wave)
    im = row_sum(im, kd);
    if (p < q.P && part == 0) s_bu[p] = make_float2(re, im);
  }
  __syncthreads();

  // state update of mode t, in place
  if (t < q.P) {
    const cf bu = {s_bu[t].x, s_bu[t].y};
    const size_t xi = static_cast<size_t>(b) * q.P + t;
    cf a, g;
    if (q.delta != nullptr) {
      // per-step interval: float32, as the time-varying forward pass
      const cf lam = {q.lam[t].x, q.lam[t].y};
      const float dt = q.delta[xi];
      if (q.bilinear) {
        bilinear_step(lam, dt, a, g);
      } else {
        const bool zero = static_cast<double>(lam.re) * lam.re + static_cast<double>(lam.im) * lam.im < 1e-60;
        const zd il = zero ? zd{0.0, 0.0} : f64::zdiv({1.0, 0.0}, {lam.re, lam.im});
        const float hrev = static_cast<float>(static_cast<double>(lam.im) / (4.0 * 3.14159265358979323846));
        zoh_step(lam, {static_cast<float>(il.re), static_cast<float>(il.im)}, hrev, zero ? 1.0f : 0.0f, dt, a, g);
      }
    } else {
      zd a64, g64;
      f64::discretize({q.lam[t].x, q.lam[t].y}, exp(static_cast<double>(q.log_delta[t])), q.bilinear, a64, g64);
      a = {static_cast<float>(a64.re), static_cast<float>(a64.im)};
      g = {static_cast<float>(g64.re), static_cast<float>(g64.im)};
    }
    const float2 x0 = q.x[xi];
    const cf xn = cfma(a, {x0.x, x0.y}, cmul(g, bu));
    q.x[xi] = make_float2(xn.re, xn.im);
    s_x[t] = make_float2(xn.re, xn.im);
  }
  __syncthreads();

  // readout: the k lanes of feature h sum Re(C~[h, m] x[m]) over m = part, part + k, ...
  const int kr = lanes_per_row(q.H);
  const int h = t / kr;
  const int rp = t - h * kr;
  float acc = 0.0f;
  if (h < q.H) {
    const float2* row = q.c_tilde + static_cast<size_t>(h) * q.P;
#pragma unroll 16
    for (int m = rp; m < q.P; m += kr) {
      const float2 c = row[m];
      const float2 xv = s_x[m];
      acc = fmaf(c.x, xv.x, fmaf(-c.y, xv.y, acc));
    }
  }
  acc = row_sum(acc, kr);
  if (h < q.H && rp == 0) {
    float yv = fmaf(q.d[h], s_u[h], q.c_scale * acc);
    if (q.gelu != 0) yv = gelu_form(yv, q.gelu);
    if (q.bf16_io) {
      static_cast<uint16_t*>(q.y)[ub + h] = f32_to_bf16(yv);
    } else {
      static_cast<float*>(q.y)[ub + h] = yv;
    }
  }
}

}  // namespace

hipError_t launch_step(const StepArgs& a, hipStream_t stream) {
  if (a.B <= 0) return hipSuccess;
  if (a.H > kStepThreads || a.P > kStepThreads / 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_step, dim3(static_cast<unsigned>(a.B)), dim3(kStepThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace s5
