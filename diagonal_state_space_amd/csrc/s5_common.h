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

// Zero-order hold of one mode in float32 for an interval dt >= 0:
//   abar = exp(lam*dt),  gain = (abar - 1)/lam.
// abar - 1 is formed without cancellation from s = sin(w/2), c = cos(w/2),
// w = Im(lam)*dt:  cos(w) - 1 = -2 s^2,  sin(w) = 2 s c,  so
//   abar - 1 = (expm1(r)(1 - 2 s^2) - 2 s^2,  e^r 2 s c),   r = Re(lam)*dt.
// `inv_lam` is 1/lam, computed once per mode. For |lam*dt| < 1e-4 the gain is
// dt*(1 + z/2 + z^2/6), the leading terms of dt*phi1(z) (phi1(z) = (e^z-1)/z),
// which also covers lam = 0 (gain = dt).
__device__ __forceinline__ void zoh_f32(cf lam, cf inv_lam, float dt, cf& abar, cf& gain) {
  const float r = lam.re * dt;
  const float w = lam.im * dt;
  if (fabsf(r) + fabsf(w) < 1e-4f) {
    const float er = expf(r);
    float sw, cw;
    sincosf(w, &sw, &cw);
    abar = {er * cw, er * sw};
    // z/2 + z^2/6
    const float hr = 0.5f * r + (r * r - w * w) * (1.0f / 6.0f);
    const float hi = 0.5f * w + (2.0f * r * w) * (1.0f / 6.0f);
    gain = {dt * (1.0f + hr), dt * hi};
    return;
  }
  float s, c;
  sincosf(0.5f * w, &s, &c);
  const float em1 = expm1f(r);
  const float er = em1 + 1.0f;
  const float two_s2 = 2.0f * s * s;
  const float cosw = 1.0f - two_s2;
  const float sinw = 2.0f * s * c;
  abar = {er * cosw, er * sinw};
  const cf am1 = {fmaf(em1, cosw, -two_s2), er * sinw};
  gain = cmul(am1, inv_lam);
}

}  // namespace s5
