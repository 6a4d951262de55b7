// Float64 complex arithmetic and the per-mode discretisations in float64,
// shared by the parameter packing, the discretisation entry point and the
// single-step kernel. Internal header.
#pragma once

#include <hip/hip_runtime.h>

namespace s5 {
namespace f64 {

struct zd {
  double re, im;
};

__device__ __forceinline__ zd zmul(zd a, zd b) { return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re}; }

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

__device__ __forceinline__ zd zlog(zd z) { return {log(sqrt(z.re * z.re + z.im * z.im)), atan2(z.im, z.re)}; }

// Zero-order hold of one mode over an interval dt >= 0 (paper eq. 6; App. A
// `discretize`): z = lambda dt, abar = e^z, gain = (e^z - 1)/lambda. For
// |z| < 1e-4 the gain is dt times the Taylor series of phi1(z) = (e^z - 1)/z
// through z^8 (the abhik.ai review's guard, row 2 "Integrate a held input
// exactly"): the singularity at lambda = 0 is removable, with gain -> dt.
__device__ __forceinline__ void zoh(zd lam, double dt, zd& abar, zd& gain) {
  const zd z = {lam.re * dt, lam.im * dt};
  abar = zexp(z);
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

// Bilinear map of one mode (S4 notes, "Discretization and the step size"; the
// diagonal case of (I - dt/2 A)^-1 (I + dt/2 A) and (I - dt/2 A)^-1 dt B):
// w = 1/(1 - z/2), abar = (1 + z/2)/(1 - z/2) = 2 w - 1, gain = dt w.
__device__ __forceinline__ void bilinear(zd lam, double dt, zd& abar, zd& gain) {
  const zd w = zdiv({1.0, 0.0}, {1.0 - 0.5 * lam.re * dt, -0.5 * lam.im * dt});
  abar = {2.0 * w.re - 1.0, 2.0 * w.im};
  gain = {dt * w.re, dt * w.im};
}

__device__ __forceinline__ void discretize(zd lam, double dt, bool bil, zd& abar, zd& gain) {
  if (bil) {
    bilinear(lam, dt, abar, gain);
  } else {
    zoh(lam, dt, abar, gain);
  }
}

}  // namespace f64
}  // namespace s5
