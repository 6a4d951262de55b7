// Internal interface of the fused S5 forward kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s5 {

// Per-mode constants written by the packing kernel.
struct ModeParams {
  float2 lam;      // continuous eigenvalue
  float2 inv_lam;  // 1/lambda
  float2 abar;     // exp(lambda Delta)            (time-invariant)
  float2 abar_R;   // exp(R lambda Delta), R = T/16 (time-invariant)
  float2 abar_T;   // exp(T lambda Delta)          (time-invariant)
  float hrev;      // Im(lambda) / (4 pi): half-angle turns per unit interval
  float pad_;
};

struct FusedParams {
  int B, L, H, P;
  int Hpad, Ppad;  // H rounded up to 32, P rounded up to 64
  int T, R;        // tokens per chunk, tokens per lane run (T/16)
  int nch;         // chunks per sequence
  int nflags;      // B * nch
  bool bf16_io, time_varying;
  unsigned spin_limit;  // bound on look-back polling (never reached in a correct run)
  const void* u;
  void* y;
  const float2* lam;
  const float2* b_tilde;
  const float2* c_tilde;
  const float* d;
  const float* log_delta;
  const float* delta;
  // workspace
  uint4* bpack;       // drive operand fragments (hi plane, then lo plane for float32 I/O)
  uint4* cpack;       // readout operand fragments (hi, then lo)
  ModeParams* modes;  // [Ppad]
  unsigned* flags;    // [B * nch] 0 none, 1 aggregate, 2 inclusive
  unsigned* ticket;   // chunk ticket counter
  float2* agg;        // [B * nch * Ppad] chunk state from zero carry-in
  float2* agg_a;      // [B * nch * Ppad] chunk transition product (time-varying)
  float2* incl;       // [B * nch * Ppad] state at the end of the chunk
};

// Tokens per chunk for these sizes (64, or 32 where registers / LDS require).
int fused_chunk_tokens(bool bf16_io, bool time_varying, int Ppad, int Hpad);
size_t fused_lds_bytes(bool bf16_io, bool time_varying, int T, int Ppad, int Hpad);

hipError_t launch_pack(const FusedParams& q, hipStream_t stream);
hipError_t launch_fused(const FusedParams& q, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);

}  // namespace s5
