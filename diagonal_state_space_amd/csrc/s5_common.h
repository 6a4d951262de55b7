// Shared device helpers for the S5 kernels (gfx950). Internal header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s5 {

// ---- bfloat16 storage conversions ------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even; NaN stays NaN (quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t x = __float_as_uint(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((x >> 16) | 0x40u);
  x += 0x7fffu + ((x >> 16) & 1u);
  return static_cast<uint16_t>(x >> 16);
}

// ---- complex float helpers --------------------------------------------------
struct cf {
  float re, im;
};

__device__ __forceinline__ cf cmul(cf a, cf b) {
  return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re};
}

// a * x + b
__device__ __forceinline__ cf cfma(cf a, cf x, cf b) {
  return {fmaf(a.re, x.re, fmaf(-a.im, x.im, b.re)), fmaf(a.re, x.im, fmaf(a.im, x.re, b.im))};
}

// sin and cos of 2*pi*t for t in revolutions, any finite t: quarter-turn
// reduction to |x| <= pi/4 (f = t - q/4 is exact: for |t| > 1/8, q/4 is a
// multiple of ulp(t) and |f| <= 1/8 < |t|; otherwise q = 0), then Taylor
// polynomials (truncation below 3e-8 absolute; relative accuracy is kept for
// small t). The quadrant count q = rint(4t) is reduced modulo 4 while still a
// float (exactly: both terms are integers and their difference is in
// [-2, 2]), so that its conversion to an integer cannot saturate.
__device__ __forceinline__ void sincos_rev(float t, float& s, float& c) {
  const float qf = rintf(4.0f * t);               // quadrant count
  const float f = fmaf(-0.25f, qf, t);            // exact: |f| <= 1/8
  const float x = 6.28318530717958647692f * f;
  const float x2 = x * x;
  float sp = fmaf(x2, 2.7557319e-6f, -1.98412698e-4f);
  sp = fmaf(x2, sp, 8.33333333e-3f);
  sp = fmaf(x2, sp, -1.66666667e-1f);
  const float sx = fmaf(x * x2, sp, x);
  float cp = fmaf(x2, 2.48015873e-5f, -1.38888889e-3f);
  cp = fmaf(x2, cp, 4.16666667e-2f);
  cp = fmaf(x2, cp, -0.5f);
  const float cx = fmaf(x2, cp, 1.0f);
  // quadrant q (mod 4): odd q swaps the pair; bit 1 of q flips the sine's
  // sign, bit 1 of q + 1 the cosine's (exact, and without branches)
  const int q = __float2int_rz(fmaf(-4.0f, rintf(0.25f * qf), qf));   // -2..2
  const bool swap = (q & 1) != 0;
  const float s0 = swap ? cx : sx;
  const float c0 = swap ? sx : cx;
  s = __uint_as_float(__float_as_uint(s0) ^ (static_cast<uint32_t>(q & 2) << 30));
  c = __uint_as_float(__float_as_uint(c0) ^ (static_cast<uint32_t>((q + 1) & 2) << 30));
}

// e^r - 1: degree-8 Taylor polynomial for |r| < 1/2 (truncation < 3e-9
// relative), exp(r) - 1 otherwise (no cancellation there).
__device__ __forceinline__ float expm1_small(float r) {
  // both forms, then a select: a branch would split the wave's scan loop
  float p = fmaf(r, 2.48015873e-5f, 1.98412698e-4f);
  p = fmaf(r, p, 1.38888889e-3f);
  p = fmaf(r, p, 8.33333333e-3f);
  p = fmaf(r, p, 4.16666667e-2f);
  p = fmaf(r, p, 1.66666667e-1f);
  p = fmaf(r, p, 0.5f);
  const float series = fmaf(r * r, p, r);
  const float direct = __expf(r) - 1.0f;
  return fabsf(r) < 0.5f ? series : direct;
}

// Zero-order hold of one mode for a per-step interval dt >= 0 (the
// time-varying path), with the half-angle taken in revolutions:
//   w/2 = Im(lam) dt / 2 = 2 pi th,  th = dt * Im(lam)/(4 pi) = dt * hrev.
// Whole turns of th drop out exactly in the quarter-turn reduction, so the
// angle's only error is the rounding of th itself, the same as rounding w.
// Then as zoh_f32:
//   abar - 1 = (expm1(r)(1 - 2 s^2) - 2 s^2,  e^r 2 s c),  gain = (abar - 1)/lam.
// SEL computes the small-|z| form on every lane and selects it (no branch in
// the caller's loop); otherwise it sits behind a branch that waves skip when
// no lane needs it. Both give the same values.
template <bool SEL = false>
__device__ __forceinline__ void zoh_step(cf lam, cf inv_lam, float hrev, float dt, cf& abar, cf& gain) {
  const float r = lam.re * dt;
  const float th = hrev * dt;
  float s, c;
  sincos_rev(th, s, c);
  const float em1 = expm1_small(r);
  const float er = em1 + 1.0f;
  const float two_s2 = 2.0f * s * s;
  const float cosw = 1.0f - two_s2;
  const float sinw = 2.0f * s * c;
  abar = {er * cosw, er * sinw};
  const cf am1 = {fmaf(em1, cosw, -two_s2), er * sinw};
  gain = cmul(am1, inv_lam);
  // |z| < 1e-4 (also covers lam = 0): dt * (1 + z/2 + z^2/6)
  const float w = lam.im * dt;
  const bool tiny = fabsf(r) + fabsf(w) < 1e-4f;
  if (SEL || tiny) {
    const float hr = 0.5f * r + (r * r - w * w) * (1.0f / 6.0f);
    const float hi = 0.5f * w + (2.0f * r * w) * (1.0f / 6.0f);
    gain = {tiny ? dt * (1.0f + hr) : gain.re, tiny ? dt * hi : gain.im};
  }
}

// Bilinear map of one mode for a per-step interval dt >= 0, z = lam dt:
// w = 1/(1 - z/2), abar = (1 + z/2)/(1 - z/2) = 2 w - 1, gain = dt w.
// (|1 - z/2| >= 1 for Re lam <= 0.)
__device__ __forceinline__ void bilinear_step(cf lam, float dt, cf& abar, cf& gain) {
  const float br = fmaf(-0.5f * dt, lam.re, 1.0f);
  const float bi = -0.5f * dt * lam.im;
  const float inv = 1.0f / fmaf(br, br, bi * bi);
  const cf w = {br * inv, -bi * inv};
  abar = {fmaf(2.0f, w.re, -1.0f), 2.0f * w.im};
  gain = {dt * w.re, dt * w.im};
}

// one per-step discretisation: bilinear when `bil`, else zero-order hold
template <bool SEL = false>
__device__ __forceinline__ void disc_step(bool bil, cf lam, cf inv_lam, float hrev, float dt, cf& abar, cf& gain) {
  if (bil) {
    bilinear_step(lam, dt, abar, gain);
  } else {
    zoh_step<SEL>(lam, inv_lam, hrev, dt, abar, gain);
  }
}

// ---- GELU epilogue forms -------------------------------------------------------
// Exact form: GELU(v) = v Phi(v), Phi the standard normal distribution
// function, with erf from Abramowitz & Stegun's formula 7.1.26 (Handbook of
// Mathematical Functions; absolute error below 1.5e-7): for z >= 0,
// erf(z) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2) with
// t = 1/(1 + p z). With z = |v|/sqrt2, Phi(|v|) = 1 - q/2 and Phi(-|v|) = q/2
// for q = 1 - erf(z). Branch-free.
__device__ __forceinline__ float gelu_erf(float v) {
  const float z = fabsf(v) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
  float poly = fmaf(t, 1.061405429f, -1.453152027f);
  poly = fmaf(t, poly, 1.421413741f);
  poly = fmaf(t, poly, -0.284496736f);
  poly = fmaf(t, poly, 0.254829592f);
  const float half_q = 0.5f * t * poly * __expf(-z * z);
  return v * (v >= 0.0f ? 1.0f - half_q : half_q);
}

// Tanh form: v/2 (1 + tanh(k)), k = sqrt(2/pi) (v + 0.044715 v^3), the
// approximation that the App. A listing's library GELU applies by default.
// Since (1 + tanh k)/2 = 1/(1 + e^-2k), it is v / (1 + e^-2k); for v -> -inf
// the exponential overflows to inf and the result is -0.
__device__ __forceinline__ float gelu_tanh(float v) {
  const float k2 = v * fmaf(0.0713548162726f, v * v, 1.5957691216057f);   // 2k
  return v * __builtin_amdgcn_rcpf(1.0f + __expf(-k2));
}

// GELU form code: 0 none, 1 exact (erf), 2 tanh
__device__ __forceinline__ float gelu_form(float v, int form) { return form == 2 ? gelu_tanh(v) : gelu_erf(v); }

// ---- MFMA operand types and helpers ----------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ uint4 as_u4(bf16x8 v) { return __builtin_bit_cast(uint4, v); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint4 ldg16(const uint4* p) { return *p; }

// Write 8 float values as bf16 hi (and lo if `lo` is non-null) fragments.
__device__ __forceinline__ void put_frag(const float (&v)[8], uint4* hi, uint4* lo) {
  f32x8 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = v[i];
  const bf16x8 h = __builtin_convertvector(f, bf16x8);
  *hi = as_u4(h);
  if (lo) {
    const f32x8 back = __builtin_convertvector(h, f32x8);
    *lo = as_u4(__builtin_convertvector(f - back, bf16x8));
  }
}

}  // namespace s5
