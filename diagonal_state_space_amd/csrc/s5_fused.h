// Internal interface of the fused S5 forward kernels (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s5 {

namespace fused {
constexpr int kStreams = 16;   // token streams per workgroup (the MFMA N columns)
constexpr int kBlock = 1024;   // one LDS block: 64 lanes x 16 bytes

// LDS bytes of one u tile (KS K-steps x R steps; float32 keeps 32 bytes per
// lane) and of one x tile (K2 mode tiles x R steps; float32 keeps hi and lo).
__host__ __device__ constexpr size_t u_tile_bytes(int KS, int R, bool bf16) {
  return static_cast<size_t>(KS) * R * (bf16 ? 1 : 2) * kBlock;
}
__host__ __device__ constexpr size_t x_tile_bytes(int K2, int R, bool bf16) {
  return static_cast<size_t>(K2) * R * (bf16 ? 1 : 2) * kBlock;
}
// LDS bytes of the per-mode constants (abar, or lambda and hrev for the
// time-varying path) and optionally D (16-byte aligned: Ppad is a multiple of 64).
__host__ __device__ constexpr size_t mode_table_bytes(int Ppad, int Hpad, bool tv, bool with_d) {
  return static_cast<size_t>(Ppad) * (tv ? 12 : 8) + (with_d ? static_cast<size_t>(Hpad) * 4 : 0);
}
// chunks between two barriers of the eight-wave pass 1 (u tiles of two such
// groups in LDS; the chunk count is padded to a multiple of it). Smaller for
// the time-varying step, whose per-token constants leave fewer registers, and
// for more than four drive K-steps, whose weights do.
__host__ __device__ constexpr int reduce_group(bool bf16, bool tv, int ks) {
  return tv ? (bf16 ? 1 : 2) : (bf16 && ks <= 4 ? 4 : 2);
}
}  // namespace fused

// Per-mode constants written by the packing kernel.
struct ModeParams {
  float2 lam;      // continuous eigenvalue (time-varying: -1e-20 where |lambda| < 1e-20)
  float2 abar;     // exp(lambda Delta)                         (time-invariant)
  float2 aseg;     // exp(Lseg lambda Delta): one whole stream   (time-invariant)
  float hrev;      // Im(lambda) / (4 pi): half-angle turns per unit interval  (time-varying)
  float2 alast;    // abar^m, m = ((L-1) mod Lseg) + 1: the stream holding token
                   // L-1, from its first token through L-1  (time-invariant)
  float2 arange;   // exp(16 Lseg lambda Delta): one whole workgroup range   (time-invariant)
};

// One forward call, as the kernels see it.
//
// Work split: sequence b is cut into Q workgroup ranges of 16 streams; stream
// t of range qq holds the Lseg consecutive tokens starting at
// (16 qq + t) Lseg, and is processed in chunks of R tokens (Lseg = R nck).
// The 16 streams of a workgroup are the 16 columns of every MFMA tile.
struct FusedParams {
  int B, L, H, P;
  int Hpad, Ppad;  // H rounded up to 32, P rounded up to 64
  int R;           // tokens of one stream per chunk
  int nck;         // chunks per stream
  int Lseg;        // tokens per stream (R * nck)
  int Q;           // workgroup ranges per sequence
  bool bf16_io, time_varying;
  const void* u;
  void* y;
  const float2* lam;
  const float2* b_tilde;
  const float2* c_tilde;
  const float* d;     // [H], or null: no feedthrough
  const float* log_delta;
  const float* delta;
  const float2* x0;   // [B, P] state before step 0, or null (zero)
  float2* xlast;      // [B, P] out: state after step L-1, or null
  // options (the last four only in the extended kernel instances)
  int c_ld, c_off;    // C~ row stride and first column (bidirectional halves)
  float c_scale;      // 2 for half-spectrum storage, else 1
  int bilinear;       // bilinear instead of zero-order hold discretisation
  int rev;            // reverse time: token k is row L-1-k of u and y
  int accum;          // y += the readout (D u included when d is given)
  int gelu;           // y = GELU(y) after the sum: 0 no, 1 exact form, 2 tanh form
  // workspace
  uint4* bpack;       // drive operand fragments (hi plane, then lo plane for float32 I/O):
                      // B_bar, or B~/lambda for the time-varying path
  uint4* cpack;       // readout operand fragments (hi, then lo)
  uint4* cpack_b;     // the backward scan's (bidirectional form; null otherwise)
  ModeParams* modes;  // [Ppad]
  float2* sagg;       // [B*Q][16][Ppad] stream state from a zero start
  float2* sagg_a;     // [B*Q][16][Ppad] stream transition product (time-varying)
  float2* tot;        // [B*Q][Ppad] workgroup range state from a zero start
  float2* tot_a;      // [B*Q][Ppad] workgroup range transition product
  float2* cap;        // [B][2][Ppad] state (from zero) and transition product of the
                      // stream holding token L-1, from its first token through L-1
  // bidirectional form (time-invariant)
  int both;           // pass 1 also writes the backward scan's aggregates (sagg_b, tot_b, tot_a_b)
  int ypart;          // pass 2 writes y (D u included) as float32 into yp (the forward half)
  float* yp;          // [B, L, H] float32 forward half of y; the backward pass adds it
  float2* sagg_b;     // backward scan's stream and range aggregates, indexed as the
  float2* tot_b;      // backward pass sees its ranges (range qq mirrors forward range
  float2* tot_a_b;    // Q-1-qq, stream t mirrors stream 15-t)
  // gated activation in the output pass (symmetric kernel, bf16 I/O)
  const float* glu_w;     // [H, H] float32, output j reads row j; null: no gate
  const float* glu_bias;  // [H] or null
  int glu_variant;        // 1: GELU(y) * gate, 2: y * gate
  uint4* gpack;           // the gate's W as A-operand fragments, bf16 hi plane then lo plane
                          // ([Hpad/16][Hpad/32][64 lanes] each); null: no gate
  // host only: walk the launch sequence and its instance dispatch without
  // launching anything (whether every launch has a compiled kernel)
  int dry;
};

// Launch plan of one call: chunk size, stream length, grid and LDS bytes.
struct FusedPlan {
  int R = 0, nck = 0, Lseg = 0, Q = 0;
  bool keep = false;        // pass 1 holds B_bar in registers (eight-wave kernel)
  bool keep_scan = false;   // pass 2 holds B_bar and C' in registers (wave-specialized kernel)
  bool scan8 = false;       // pass 2 on the symmetric eight-wave kernel (with keep_scan)
  int ks = 0;               // its drive K-steps (Hpad / 32)
  int group = 1;            // nck is a multiple of this (reduce_group with `keep`)
  bool both = false;        // the eight-wave pass 1 can sum the backward scan's aggregates too
  size_t lds_reduce = 0, lds_scan = 0, lds_reduce_ws = 0;
};

// Plan and workspace layout of one forward call (byte offsets into the
// 256-byte aligned workspace; total = bytes needed).
struct ForwardLayout {
  FusedPlan plan;
  int Ppad = 0, Hpad = 0;
  size_t bpack = 0, cpack = 0, modes = 0, sagg = 0, sagg_a = 0, tot = 0, tot_a = 0, cap = 0, total = 0;
  size_t sagg_b = 0, tot_b = 0, tot_a_b = 0, yp = 0, cpack_b = 0;   // bidirectional form (yp: bf16 I/O)
  size_t gpack = 0;   // the gate's packed W (gated activation in the output pass)
};

// R and `keep` for these sizes (R = 0: no compiled instance fits).
void fused_shape(bool bf16_io, bool time_varying, int Ppad, int Hpad, bool gate, FusedPlan& p);
// Fill in nck, Lseg and Q for B sequences of length L (features H, modes P)
// on `ncu` compute units.
void fused_split(int B, int L, int H, int P, int ncu, FusedPlan& p);

hipError_t launch_pack(const FusedParams& q, hipStream_t stream);

// Pass 1 (stream and range aggregates) and pass 2 (states and outputs).
hipError_t launch_reduce(const FusedParams& q, const FusedPlan& p, hipStream_t stream);
hipError_t launch_scan(const FusedParams& q, const FusedPlan& p, hipStream_t stream);

// Per-kind entry points (one translation unit each).
hipError_t launch_reduce_bf16_ti(const FusedParams& q, const FusedPlan& p, hipStream_t s);
hipError_t launch_scan_bf16_ti(const FusedParams& q, const FusedPlan& p, hipStream_t s);
hipError_t launch_reduce_bf16_tv(const FusedParams& q, const FusedPlan& p, hipStream_t s);
hipError_t launch_scan_bf16_tv(const FusedParams& q, const FusedPlan& p, hipStream_t s);
hipError_t launch_reduce_f32_ti(const FusedParams& q, const FusedPlan& p, hipStream_t s);
hipError_t launch_scan_f32_ti(const FusedParams& q, const FusedPlan& p, hipStream_t s);
hipError_t launch_reduce_f32_tv(const FusedParams& q, const FusedPlan& p, hipStream_t s);
hipError_t launch_scan_f32_tv(const FusedParams& q, const FusedPlan& p, hipStream_t s);

}  // namespace s5
