// S5 forward path, first version: chunked two-pass scan on the vector ALUs.
//
//   1. discretisation (float64)                  k_discretize
//   2. per-chunk aggregate of the recurrence     k_chunk_aggregate
//      (drive b_k = B_bar u_k, then x = a x + b over the chunk from zero)
//   3. exclusive scan of the chunk aggregates    k_chunk_carry
//      with the operator (a2,b2) o (a1,b1) = (a2 a1, a2 b1 + b2) (App. H)
//   4. per-chunk recurrence from the carried-in state and the readout
//      y_k = Re(C~ x_k) + D u_k                  k_chunk_output
//
// All arithmetic is float32 except the discretisation.
#include "s5_common.h"
#include "s5_internal.h"

namespace s5 {

namespace {

constexpr int kChunk = 16;     // tokens per chunk
constexpr int kThreads = 256;  // threads per block

template <bool BF16>
__device__ __forceinline__ float load_io(const void* p, size_t i) {
  if constexpr (BF16) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

template <bool BF16>
__device__ __forceinline__ void store_io(void* p, size_t i, float v) {
  if constexpr (BF16) {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  } else {
    static_cast<float*>(p)[i] = v;
  }
}

struct Params {
  int B, L, H, P, nch;
  const void* u;
  const float2* bmat;     // B_bar (time-invariant) or B~ (time-varying), [P, H]
  const float2* c_tilde;  // [H, P]
  const float* d;         // [H]
  const float* delta;     // [B, L, P] (time-varying)
  const float2* lam;      // continuous lambda [P]
  const float2* lam_bar;  // [P] (time-invariant)
  const float2* pow_T;    // lam_bar^kChunk [P] (time-invariant)
  const float2* inv_lam;  // 1/lambda [P] (time-varying)
  float2* agg;            // [B, nch, P] chunk end state from zero
  float2* agg_a;          // [B, nch, P] chunk transition product (time-varying)
  float2* carry;          // [B, nch, P] state entering the chunk
  void* y;
};

template <bool BF16>
__device__ void load_u_tile(const Params& q, int b, int t0, int tc, float* u_s) {
  for (int i = threadIdx.x; i < kChunk * q.H; i += kThreads) {
    const int t = i / q.H;
    u_s[i] = (t < tc) ? load_io<BF16>(q.u, (static_cast<size_t>(b) * q.L + t0) * q.H + i) : 0.0f;
  }
}

// drive[t] = sum_h bmat[p, h] * u[t, h] for the kChunk tokens of the tile.
__device__ __forceinline__ void drive_tile(const Params& q, int p, const float* u_s, cf (&bu)[kChunk]) {
#pragma unroll
  for (int t = 0; t < kChunk; ++t) bu[t] = {0.0f, 0.0f};
  const float2* row = q.bmat + static_cast<size_t>(p) * q.H;
  for (int h = 0; h < q.H; ++h) {
    const float2 bm = row[h];
#pragma unroll
    for (int t = 0; t < kChunk; ++t) {
      const float uv = u_s[t * q.H + h];
      bu[t].re = fmaf(bm.x, uv, bu[t].re);
      bu[t].im = fmaf(bm.y, uv, bu[t].im);
    }
  }
}

template <bool TV, bool BF16>
__global__ void __launch_bounds__(kThreads) k_chunk_aggregate(Params q) {
  extern __shared__ float smem[];
  float* u_s = smem;
  const int c = blockIdx.x, b = blockIdx.y;
  const int t0 = c * kChunk;
  const int tc = min(kChunk, q.L - t0);
  load_u_tile<BF16>(q, b, t0, tc, u_s);
  __syncthreads();
  for (int p = threadIdx.x; p < q.P; p += kThreads) {
    cf bu[kChunk];
    drive_tile(q, p, u_s, bu);
    cf x = {0.0f, 0.0f};
    cf acc_a = {1.0f, 0.0f};
    const cf lam = {q.lam[p].x, q.lam[p].y};
    const cf inv = TV ? cf{q.inv_lam[p].x, q.inv_lam[p].y} : cf{0.0f, 0.0f};
    const cf lb = TV ? cf{0.0f, 0.0f} : cf{q.lam_bar[p].x, q.lam_bar[p].y};
#pragma unroll
    for (int t = 0; t < kChunk; ++t) {
      if (t < tc) {
        if constexpr (TV) {
          const float dt = q.delta[(static_cast<size_t>(b) * q.L + t0 + t) * q.P + p];
          cf a, g;
          zoh_f32(lam, inv, dt, a, g);
          x = cfma(a, x, cmul(g, bu[t]));
          acc_a = cmul(a, acc_a);
        } else {
          x = cfma(lb, x, bu[t]);
        }
      }
    }
    const size_t o = (static_cast<size_t>(b) * q.nch + c) * q.P + p;
    q.agg[o] = make_float2(x.re, x.im);
    if constexpr (TV) q.agg_a[o] = make_float2(acc_a.re, acc_a.im);
  }
}

template <bool TV>
__global__ void __launch_bounds__(kThreads) k_chunk_carry(Params q) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= q.B * q.P) return;
  const int b = i / q.P, p = i % q.P;
  cf s = {0.0f, 0.0f};
  const cf pw = TV ? cf{1.0f, 0.0f} : cf{q.pow_T[p].x, q.pow_T[p].y};
  for (int c = 0; c < q.nch; ++c) {
    const size_t o = (static_cast<size_t>(b) * q.nch + c) * q.P + p;
    q.carry[o] = make_float2(s.re, s.im);
    const cf a = TV ? cf{q.agg_a[o].x, q.agg_a[o].y} : pw;
    s = cfma(a, s, {q.agg[o].x, q.agg[o].y});
  }
}

template <bool TV, bool BF16>
__global__ void __launch_bounds__(kThreads) k_chunk_output(Params q) {
  extern __shared__ float smem[];
  float* u_s = smem;
  float2* x_s = reinterpret_cast<float2*>(smem + kChunk * q.H);
  const int c = blockIdx.x, b = blockIdx.y;
  const int t0 = c * kChunk;
  const int tc = min(kChunk, q.L - t0);
  load_u_tile<BF16>(q, b, t0, tc, u_s);
  __syncthreads();
  for (int p = threadIdx.x; p < q.P; p += kThreads) {
    cf bu[kChunk];
    drive_tile(q, p, u_s, bu);
    const size_t o = (static_cast<size_t>(b) * q.nch + c) * q.P + p;
    cf x = {q.carry[o].x, q.carry[o].y};
    const cf lam = {q.lam[p].x, q.lam[p].y};
    const cf inv = TV ? cf{q.inv_lam[p].x, q.inv_lam[p].y} : cf{0.0f, 0.0f};
    const cf lb = TV ? cf{0.0f, 0.0f} : cf{q.lam_bar[p].x, q.lam_bar[p].y};
#pragma unroll
    for (int t = 0; t < kChunk; ++t) {
      if (t < tc) {
        if constexpr (TV) {
          const float dt = q.delta[(static_cast<size_t>(b) * q.L + t0 + t) * q.P + p];
          cf a, g;
          zoh_f32(lam, inv, dt, a, g);
          x = cfma(a, x, cmul(g, bu[t]));
        } else {
          x = cfma(lb, x, bu[t]);
        }
        x_s[t * q.P + p] = make_float2(x.re, x.im);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < tc * q.H; i += kThreads) {
    const int t = i / q.H, h = i % q.H;
    const float2* crow = q.c_tilde + static_cast<size_t>(h) * q.P;
    const float2* xr = x_s + t * q.P;
    float acc = 0.0f;
    for (int p = 0; p < q.P; ++p) {
      const float2 cc = crow[p];
      const float2 xv = xr[p];
      acc = fmaf(cc.x, xv.x, acc);
      acc = fmaf(-cc.y, xv.y, acc);
    }
    acc = fmaf(q.d[h], u_s[i], acc);
    store_io<BF16>(q.y, (static_cast<size_t>(b) * q.L + t0) * q.H + i, acc);
  }
}

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Layout {
  size_t lam_bar, pow_T, inv_lam, bmat, agg, agg_a, carry, total;
};

Layout layout(const ForwardArgs& a) {
  const size_t nch = (static_cast<size_t>(a.L) + kChunk - 1) / kChunk;
  const size_t f2 = sizeof(float2);
  Layout l{};
  size_t off = 0;
  l.lam_bar = off; off += align_up(a.P * f2);
  l.pow_T = off;   off += align_up(a.P * f2);
  l.inv_lam = off; off += align_up(a.P * f2);
  l.bmat = off;    off += a.time_varying ? 0 : align_up(static_cast<size_t>(a.P) * a.H * f2);
  const size_t agg = align_up(static_cast<size_t>(a.B) * nch * a.P * f2);
  l.agg = off;     off += agg;
  l.agg_a = off;   off += a.time_varying ? agg : 0;
  l.carry = off;   off += agg;
  l.total = off;
  return l;
}

template <bool TV, bool BF16>
hipError_t run(const Params& q, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const dim3 grid(q.nch, q.B);
  const size_t sm_agg = kChunk * q.H * sizeof(float);
  const size_t sm_out = sm_agg + kChunk * q.P * sizeof(float2);
  if (ev_start) (void)hipEventRecord(ev_start, stream);
  hipLaunchKernelGGL((k_chunk_aggregate<TV, BF16>), grid, dim3(kThreads), sm_agg, stream, q);
  hipLaunchKernelGGL((k_chunk_carry<TV>), dim3((q.B * q.P + kThreads - 1) / kThreads),
                     dim3(kThreads), 0, stream, q);
  hipLaunchKernelGGL((k_chunk_output<TV, BF16>), grid, dim3(kThreads), sm_out, stream, q);
  if (ev_stop) (void)hipEventRecord(ev_stop, stream);
  return hipGetLastError();
}

}  // namespace

size_t forward_workspace_bytes(const ForwardArgs& a) { return layout(a).total; }

hipError_t launch_forward(const ForwardArgs& a, void* ws, hipStream_t stream, hipEvent_t ev_start,
                          hipEvent_t ev_stop) {
  const Layout l = layout(a);
  char* base = static_cast<char*>(ws);
  Params q{};
  q.B = a.B; q.L = a.L; q.H = a.H; q.P = a.P;
  q.nch = (a.L + kChunk - 1) / kChunk;
  q.u = a.u;
  q.c_tilde = a.c_tilde;
  q.d = a.d;
  q.delta = a.delta;
  q.lam = a.lam;
  q.lam_bar = reinterpret_cast<float2*>(base + l.lam_bar);
  q.pow_T = reinterpret_cast<float2*>(base + l.pow_T);
  q.inv_lam = reinterpret_cast<float2*>(base + l.inv_lam);
  q.agg = reinterpret_cast<float2*>(base + l.agg);
  q.agg_a = a.time_varying ? reinterpret_cast<float2*>(base + l.agg_a) : nullptr;
  q.carry = reinterpret_cast<float2*>(base + l.carry);
  q.y = a.y;
  hipError_t e;
  if (a.time_varying) {
    q.bmat = a.b_tilde;
    e = launch_inv_lambda(a.P, a.lam, const_cast<float2*>(q.inv_lam), stream);
  } else {
    float2* bbar = reinterpret_cast<float2*>(base + l.bmat);
    q.bmat = bbar;
    e = launch_discretize(a.P, a.H, a.lam, a.b_tilde, a.log_delta, const_cast<float2*>(q.lam_bar),
                          bbar, const_cast<float2*>(q.pow_T), kChunk, nullptr, stream);
  }
  if (e != hipSuccess) return e;
  if (a.time_varying) {
    return a.bf16_io ? run<true, true>(q, stream, ev_start, ev_stop)
                     : run<true, false>(q, stream, ev_start, ev_stop);
  }
  return a.bf16_io ? run<false, true>(q, stream, ev_start, ev_stop)
                   : run<false, false>(q, stream, ev_start, ev_stop);
}

}  // namespace s5
