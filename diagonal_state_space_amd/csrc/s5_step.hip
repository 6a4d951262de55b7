// One recurrent step of the S5 layer for a batch of sequences: the online
// (streaming / generation) form, which keeps only the current state
// (abhik.ai review, "Associative scans preserve the recurrence": streaming
// keeps one state per layer; papercache notes Sec. 3.3):
//   x <- Lambda_bar x + B_bar u,   y = Re(C~ x) + D u   (paper eq. 2, 5).
// One workgroup per sequence; the whole step is a few hundred kilobytes of
// parameter reads, so it is latency-bound and runs on the vector units.
#include "s5_common.h"
#include "s5_internal.h"

namespace s5 {

namespace {

constexpr int kStepThreads = 512;   // >= S5_MAX_H outputs, >= 2 S5_MAX_P

struct zd {
  double re, im;
};
__device__ __forceinline__ zd zmul(zd a, zd b) { return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re}; }
__device__ __forceinline__ zd zdiv(zd a, zd b) {
  const double den = b.re * b.re + b.im * b.im;
  return {(a.re * b.re + a.im * b.im) / den, (a.im * b.re - a.re * b.im) / den};
}

// float64 discretisation of one mode for interval dt: zero-order hold
// (Lambda_bar = e^z, gain = (e^z - 1)/lambda, 9-term phi1 series for
// |z| < 1e-4) or bilinear (w = 1/(1 - z/2), Lambda_bar = 2w - 1, gain = dt w)
__device__ void disc_mode64(zd lam, double dt, bool bilinear, zd& abar, zd& gain) {
  const zd z = {lam.re * dt, lam.im * dt};
  if (bilinear) {
    const zd w = zdiv({1.0, 0.0}, {1.0 - 0.5 * z.re, -0.5 * z.im});
    abar = {2.0 * w.re - 1.0, 2.0 * w.im};
    gain = {dt * w.re, dt * w.im};
    return;
  }
  const double e = exp(z.re);
  double sn, cs;
  sincos(z.im, &sn, &cs);
  abar = {e * cs, e * sn};
  if (sqrt(z.re * z.re + z.im * z.im) < 1e-4) {
    zd term = {1.0, 0.0}, phi = {1.0, 0.0};
    for (int n = 1; n <= 8; ++n) {
      term = zmul(term, z);
      term.re /= (n + 1);
      term.im /= (n + 1);
      phi.re += term.re;
      phi.im += term.im;
    }
    gain = {dt * phi.re, dt * phi.im};
  } else {
    gain = zdiv({abar.re - 1.0, abar.im}, lam);
  }
}

__device__ __forceinline__ float gelu_step(float v) { return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f)); }

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
        const zd il = zdiv({1.0, 0.0}, {lam.re, lam.im});
        const float hrev = static_cast<float>(static_cast<double>(lam.im) / (4.0 * 3.14159265358979323846));
        zoh_step(lam, {static_cast<float>(il.re), static_cast<float>(il.im)}, hrev, dt, a, g);
      }
    } else {
      zd a64, g64;
      disc_mode64({q.lam[t].x, q.lam[t].y}, exp(static_cast<double>(q.log_delta[t])), q.bilinear, a64, g64);
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
    if (q.gelu) yv = gelu_step(yv);
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
