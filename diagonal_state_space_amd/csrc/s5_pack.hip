// Parameter packing for the fused S5 forward kernels: discretisation in
// float64 (zero-order hold: paper eq. 6, App. A `discretize`, abhik.ai review
// row 2; or bilinear: intuitivepapers S4 notes, "Discretization and the step
// size"), the MFMA operand layouts of B_bar and C', and the per-mode
// constants.
#include "s5_common.h"
#include "s5_f64.h"
#include "s5_fused.h"

namespace s5 {

namespace {

using f64::zd;

// lambda of the per-step discretisation: a tiny negative real value in place
// of |lambda| < 1e-20, so that B~/lambda stays finite (the kernels step with
// x + (abar - 1)(x + (B~/lambda) u), which for such lambda is x + dt B~u to
// float precision, the lambda = 0 step)
__device__ __forceinline__ zd step_lambda(float2 l) {
  const zd lam = {l.x, l.y};
  return lam.re * lam.re + lam.im * lam.im < 1e-40 ? zd{-1e-20, 0.0} : lam;
}

__global__ void __launch_bounds__(256) k_pack(FusedParams q, int split) {
  const int KS = q.Hpad / 32;
  const int K2 = 2 * q.Ppad / 32;
  const int nb = (q.Ppad / 16) * 2 * KS * 64;  // B_bar fragment lanes
  const int nc = (q.Hpad / 16) * K2 * 64;      // C' fragment lanes
  const int nm = q.Ppad;                        // per-mode values
  // (bidirectional form: the backward scan's C' too, from the columns P
  // further on, into cpack_b; gated activation: the gate's W, split into bf16
  // hi and lo planes, into gpack)
  const int nc2 = q.cpack_b != nullptr ? nc : 0;
  const int ng = q.gpack != nullptr ? (q.Hpad / 16) * KS * 64 : 0;
  const int g0 = nb + nc + nm + nc2;
  const int total = g0 + ng;
  for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += gridDim.x * blockDim.x) {
    if (idx >= g0) {
      // fragment (ht*KS + s), lane l: row j = 16 ht + l%16 (gate output j),
      // k = 32 s + 8(l/16) + i (input feature k); zero past H
      const int e = idx - g0;
      const int l = e & 63;
      const int f = e >> 6;
      const int s = f % KS;
      const int j = 16 * (f / KS) + (l & 15);
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = 32 * s + 8 * (l >> 4) + i;
        v[i] = j < q.H && k < q.H ? q.glu_w[static_cast<size_t>(j) * q.H + k] : 0.0f;
      }
      put_frag(v, q.gpack + e, q.gpack + ng + e);
      continue;
    }
    if (idx < nb) {
      // fragment ((j*2 + c)*KS + s), lane l: row m = l%16 (mode 16j+m), k = 8(l/16)+i
      const int l = idx & 63;
      const int f = idx >> 6;
      const int s = f % KS;
      const int c = (f / KS) & 1;
      const int j = f / (2 * KS);
      const int p = 16 * j + (l & 15);
      float v[8];
      zd g = {0.0, 0.0};
      if (p < q.P) {
        if (!q.time_varying) {
          zd abar;
          f64::discretize({q.lam[p].x, q.lam[p].y}, exp(static_cast<double>(q.log_delta[p])), q.bilinear,
                          abar, g);
        } else {
          g = f64::zdiv({1.0, 0.0}, step_lambda(q.lam[p]));   // per-step: the drive gives (B~/lambda) u
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int h = 32 * s + 8 * (l >> 4) + i;
        double val = 0.0;
        if (p < q.P && h < q.H) {
          const float2 bt = q.b_tilde[static_cast<size_t>(p) * q.H + h];
          const zd b = f64::zmul(g, {bt.x, bt.y});
          val = c == 0 ? b.re : b.im;
        }
        v[i] = static_cast<float>(val);
      }
      put_frag(v, q.bpack + idx, split ? q.bpack + nb + idx : nullptr);
    } else if (idx < nb + nc || idx >= nb + nc + nm) {
      // fragment (ht*K2 + s), lane l: row h = 16 ht + l%16, k = 32 s + 8(l/16) + i,
      // k = 2p + comp with comp 0 -> Re C~, comp 1 -> -Im C~
      const bool second = idx >= nb + nc + nm;
      const int e = second ? idx - nb - nc - nm : idx - nb;
      const int c_off = second ? q.c_off + q.P : q.c_off;
      uint4* cp = second ? q.cpack_b : q.cpack;
      const int l = e & 63;
      const int f = e >> 6;
      const int s = f % K2;
      const int ht = f / K2;
      const int h = 16 * ht + (l & 15);
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = 32 * s + 8 * (l >> 4) + i;
        const int p = k >> 1;
        float val = 0.0f;
        if (h < q.H && p < q.P) {
          const float2 ct = q.c_tilde[static_cast<size_t>(h) * q.c_ld + c_off + p];
          val = q.c_scale * ((k & 1) ? -ct.y : ct.x);
        }
        v[i] = val;
      }
      put_frag(v, cp + e, split ? cp + nc + e : nullptr);
    } else if (idx < nb + nc + nm) {
      const int p = idx - nb - nc;
      ModeParams mp{};
      if (p < q.P) {
        const zd lam = {q.lam[p].x, q.lam[p].y};
        mp.lam = make_float2(q.lam[p].x, q.lam[p].y);
        if (q.time_varying) {
          const zd ls = step_lambda(q.lam[p]);
          mp.lam = make_float2(static_cast<float>(ls.re), static_cast<float>(ls.im));
          mp.hrev = static_cast<float>(ls.im / (4.0 * 3.14159265358979323846));
        } else {
          const double dt = exp(static_cast<double>(q.log_delta[p]));
          // log of Lambda_bar: z itself for zero-order hold
          zd z = {lam.re * dt, lam.im * dt};
          if (q.bilinear) {
            zd ab, g;
            f64::bilinear(lam, dt, ab, g);
            z = f64::zlog(ab);
          }
          const zd a = f64::zexp(z);
          const zd as = f64::zexp({z.re * q.Lseg, z.im * q.Lseg});
          const double m = (q.L - 1) % q.Lseg + 1;
          const zd al = f64::zexp({z.re * m, z.im * m});
          mp.alast = make_float2(static_cast<float>(al.re), static_cast<float>(al.im));
          mp.abar = make_float2(static_cast<float>(a.re), static_cast<float>(a.im));
          mp.aseg = make_float2(static_cast<float>(as.re), static_cast<float>(as.im));
          const double nr = static_cast<double>(fused::kStreams) * q.Lseg;
          const zd ar = f64::zexp({z.re * nr, z.im * nr});
          mp.arange = make_float2(static_cast<float>(ar.re), static_cast<float>(ar.im));
        }
      }
      q.modes[p] = mp;
    }
  }
}


}  // namespace

hipError_t launch_pack(const FusedParams& q, hipStream_t stream) {
  if (q.dry) return hipSuccess;
  const int KS = q.Hpad / 32, K2 = 2 * q.Ppad / 32;
  const int nc = (q.Hpad / 16) * K2 * 64;
  const int total = (q.Ppad / 16) * 2 * KS * 64 + nc + q.Ppad + (q.cpack_b != nullptr ? nc : 0) +
                    (q.gpack != nullptr ? (q.Hpad / 16) * KS * 64 : 0);
  const int blocks = (total + 255) / 256 < 1024 ? (total + 255) / 256 : 1024;
  hipLaunchKernelGGL(k_pack, dim3(blocks), dim3(256), 0, stream, q, q.bf16_io ? 0 : 1);
  return hipGetLastError();
}

}  // namespace s5
