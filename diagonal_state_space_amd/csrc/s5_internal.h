// Internal launcher declarations shared by the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "s5_fused.h"

namespace s5 {

// Zero-order-hold discretisation (float64 inside): lam_bar [P], b_bar [P, H].
hipError_t launch_discretize(int P, int H, const float2* lam, const float2* b_tilde,
                             const float* log_delta, float2* lam_bar, float2* b_bar, hipStream_t stream);

// Arguments of one forward call after validation on the host.
struct ForwardArgs {
  int B, L, H, P;
  bool bf16_io;
  bool time_varying;
  const void* u;
  const float2* lam;
  const float2* b_tilde;
  const float2* c_tilde;
  const float* d;          // [H], or null (no feedthrough)
  const float* log_delta;  // time-invariant
  const float* delta;      // time-varying [B, L, P]
  void* y;
  const float2* x0 = nullptr;   // [B, P] state before step 0 (null: zero)
  float2* xlast = nullptr;      // [B, P] out: state after step L-1 (null: not written)
  int c_ld = 0;                 // row stride of c_tilde (0: P)
  int c_off = 0;                // first column of c_tilde read
  float c_scale = 1.0f;         // readout factor (2: half-spectrum storage)
  bool bilinear = false;        // bilinear discretisation
  bool rev = false;             // reverse time (the backward scan)
  bool accum = false;           // add the result to y
  int gelu = 0;                 // GELU of the final y: 0 no, 1 exact form, 2 tanh form
  bool bidir = false;           // bidirectional form: forward and backward scans, c_tilde [H, 2P]
  const float* glu_w = nullptr;     // gated activation in the output pass (bf16, H <= 128), or null
  const float* glu_bias = nullptr;  // [H] or null
  int glu_variant = 0;              // 1: GELU(y) * gate, 2: y * gate
};

// One recurrent step for B sequences (validated on the host): x [B, P] in
// place, y [B, H]; exactly one of log_delta [P] and delta [B, P].
struct StepArgs {
  int B, H, P;
  bool bf16_io;
  bool bilinear;
  int gelu;   // 0 no GELU, 1 exact form, 2 tanh form
  float c_scale;
  const void* u;
  const float2* lam;
  const float2* b_tilde;
  const float2* c_tilde;
  const float* d;
  const float* log_delta;
  const float* delta;
  float2* x;
  void* y;
};

hipError_t launch_step(const StepArgs& a, hipStream_t stream);

// Gated activation over T tokens of H features (validated on the host):
// out = (variant 1: GELU(y); 2: y) * sigma(W GELU(y) + bias); H <= 256.
struct GluArgs {
  int T, H;
  bool bf16_io;
  int variant;
  const void* y;
  const float* w;      // [H, H] row-major: output j reads w[j, :]
  const float* bias;   // [H] or null
  void* out;
};

hipError_t launch_glu(const GluArgs& a, hipStream_t stream);

// Launch plan and workspace layout for these sizes, computed once per call;
// false when no compiled kernel instance covers them.
bool forward_layout(const ForwardArgs& a, ForwardLayout& l);

// Zero-length sequences: the final state is the initial one (x0, or zero when
// x0 is null); n = B*P complex values.
hipError_t launch_state_passthrough(const float2* x0, float2* xlast, int64_t n, hipStream_t stream);

// bf16 <-> float32 copies of n elements (float32 -> bf16 rounds to nearest
// even; NaN and infinities carry through), for bf16 I/O computed with the
// float32-operand arithmetic
hipError_t launch_widen_bf16(const void* in, float* out, int64_t n, hipStream_t stream);
hipError_t launch_narrow_bf16(const float* in, void* out, int64_t n, hipStream_t stream);

// Enqueue the whole forward path on `stream` using `ws` (l.total bytes,
// 256-byte aligned), with the layout forward_layout gave for `a`. ev[2k] /
// ev[2k+1] are recorded around the k-th kernel launch for k < nev/2: packing,
// pass 1, pass 2; for the bidirectional form then the backward scan's
// packing, its own pass 1 (an empty pair where the forward pass 1 computed
// its aggregates) and its pass 2.
// With dry = true nothing is launched or recorded and ws may be null: the
// result says whether every launch of the plan has a compiled kernel instance
// (hipErrorInvalidValue where one is missing), so a caller can refuse the
// call before it enqueues anything.
hipError_t launch_forward(const ForwardArgs& a, const ForwardLayout& l, void* ws, hipStream_t stream,
                          const hipEvent_t* ev, int nev, bool dry = false);

}  // namespace s5
