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

// e^r - 1 for r <= 0 (Re(lambda) <= 0 and dt >= 0): degree-6 Taylor
// polynomial for r > -1/8 (truncation below 1e-9 relative), exp(r) - 1
// otherwise (no cancellation there: |e^r - 1| > 0.117). Both forms are
// computed and one selected: a branch would split the caller's scan loop.
__device__ __forceinline__ float expm1_neg(float r, float er) {
  float p = fmaf(r, 1.98412698e-4f, 1.38888889e-3f);
  p = fmaf(r, p, 8.33333333e-3f);
  p = fmaf(r, p, 4.16666667e-2f);
  p = fmaf(r, p, 1.66666667e-1f);
  p = fmaf(r, p, 0.5f);
  const float series = fmaf(r * r, p, r);
  return r > -0.125f ? series : er - 1.0f;
}

// abar - 1 of the zero-order hold of one mode for a per-step interval dt >= 0
// (the time-varying path), with the half-angle taken in turns:
//   w/2 = Im(lam) dt / 2 = 2 pi th,  th = dt * Im(lam)/(4 pi) = dt * hrev.
// Whole turns of th drop out exactly (th - rint(th), any finite th), so the
// angle's only error is the rounding of th itself, the same as rounding w;
// the sine and cosine of the remaining fraction come from the hardware's
// transcendental unit, which takes its argument in turns (measured on this
// chip: absolute error below 1.3e-7 over a turn, relative error below 9e-7
// for small angles).
// With s, c = sin, cos(w/2) and r = Re(lam) dt:
//   abar - 1 = ((e^r - 1)(1 - 2 s^2) - 2 s^2,  e^r 2 s c)
// has no cancellation (for Re(lam) <= 0 the two terms of the real part have
// the same sign while cos w >= 0, and otherwise the real part is below -1).
__device__ __forceinline__ cf zoh_am1(float lam_re, float hrev, float dt) {
  const float r = lam_re * dt;
  const float th = hrev * dt;
  const float f = th - rintf(th);                 // exact: whole turns dropped, |f| <= 1/2
  const float s = __builtin_amdgcn_sinf(f);       // hardware sine and cosine of 2 pi f
  const float c = __builtin_amdgcn_cosf(f);
  const float er = __expf(r);
  const float em1 = expm1_neg(r, er);
  const float two_s2 = 2.0f * s * s;
  return {fmaf(em1, 1.0f - two_s2, -two_s2), er * (2.0f * s * c)};
}

// Zero-order hold for the single-step kernel, which drives with B~ u: abar and
// the gain (abar - 1)/lam (dt at lambda = 0: inv_lam = 0, fz = 1, the
// removable singularity, where abar - 1 = 0).
__device__ __forceinline__ void zoh_step(cf lam, cf inv_lam, float hrev, float fz, float dt, cf& abar, cf& gain) {
  const cf am1 = zoh_am1(lam.re, hrev, dt);
  abar = {1.0f + am1.re, am1.im};
  gain = {fmaf(am1.re, inv_lam.re, fmaf(-am1.im, inv_lam.im, fz * dt)), fmaf(am1.re, inv_lam.im, am1.im * inv_lam.re)};
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

// abar - 1 = z w of the bilinear map (no cancellation for small z, unlike 2w - 2).
__device__ __forceinline__ cf bilinear_am1(cf lam, float dt) {
  const float zr = lam.re * dt, zi = lam.im * dt;
  const float br = fmaf(-0.5f, zr, 1.0f);
  const float bi = -0.5f * zi;
  const float inv = 1.0f / fmaf(br, br, bi * bi);
  return {fmaf(zr, br, zi * bi) * inv, fmaf(zi, br, -zr * bi) * inv};
}

// per-mode constants of the fused kernels' per-step discretisation: lambda
// and the half-angle turns per unit interval Im(lambda)/(4 pi)
struct StepMode {
  cf lam;
  float hrev;
};

// The fused kernels' per-step discretisation, as am1 = abar - 1. Both maps
// have gain = (abar - 1)/lambda (zero-order hold by definition; bilinear:
// abar - 1 = z w and gain = dt w), so with the drive packed from B~/lambda,
// bu = (B~/lambda) u, one step is
//   x <- abar x + gain B~u = x + am1 (x + bu)           (step_am1)
// and needs neither abar nor the gain. lambda = 0 is packed as a tiny
// negative real lambda, for which x + am1 (x + bu) is x + dt B~u to float
// precision.
__device__ __forceinline__ cf disc_am1(bool bil, const StepMode& m, float dt) {
  return bil ? bilinear_am1(m.lam, dt) : zoh_am1(m.lam.re, m.hrev, dt);
}

__device__ __forceinline__ cf step_am1(cf am1, cf x, cf bu) {
  return cfma(am1, {x.re + bu.re, x.im + bu.im}, x);
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
