// Instances and dispatch of the fused kernels for one I/O type and one kind
// (time-invariant or time-varying). Included once by each of four translation
// units, which define S5_INST_BF16 and S5_INST_TV (0 or 1) and compile in
// parallel.
#pragma once

#include "s5_fused_kernels.h"

#if !defined(S5_INST_BF16) || !defined(S5_INST_TV)
#error "define S5_INST_BF16 and S5_INST_TV before including s5_fused_inst.h"
#endif

namespace s5 {
namespace {

constexpr bool kBF16 = S5_INST_BF16 != 0;
constexpr bool kTV = S5_INST_TV != 0;

// Register-resident weights are compiled where they fit: float32 I/O doubles
// every operand, so there only up to two mode tiles per wave.
constexpr int kKeepMaxMPW = kBF16 ? 4 : 2;

// the symmetric pass-2 kernel, instanced for 1..4 drive K-steps (H <= 128)
// and the time-varying step
template <int MPW, int KS>
hipError_t scan8_ks(const FusedParams& q, const FusedPlan& p, hipStream_t s) {
  // instances whose LDS (four u tiles, two x tiles, the mode table, and for
  // the gate (bf16 I/O, at most four K-steps) its ring of two-plane g tiles,
  // multipliers and bias) fits
  constexpr size_t lds = 4 * fused::u8_tile_bytes(KS, 2, kBF16) + 2 * fused::x_tile_bytes(4 * MPW, 2, kBF16) +
                         fused::mode_table_bytes(64 * MPW, 32 * KS, kTV, true) +
                         (kBF16 && KS <= 4 ? (4 * KS + 8 * ((2 * KS + 7) / 8)) * 2 * fused::kBlock + 128 * KS : 0);
  if constexpr (lds > 160 * 1024) {
    return hipErrorInvalidValue;
  } else {
    return fused::launch_scan8_t<MPW, KS, kTV, kBF16>(q, p, s);
  }
}

template <int MPW>
hipError_t scan8(const FusedParams& q, const FusedPlan& p, hipStream_t s) {
  // the plan takes it for the time-varying step with at most two mode tiles
  // per wave, and for time-invariant bf16 I/O with 5..8 drive K-steps
  if constexpr (MPW > kKeepMaxMPW) {
    return hipErrorInvalidValue;
  } else if constexpr (kTV) {
    if constexpr (MPW > 2) {
      return hipErrorInvalidValue;
    } else {
      switch (p.ks) {
        case 1: return scan8_ks<MPW, 1>(q, p, s);
        case 2: return scan8_ks<MPW, 2>(q, p, s);
        case 3: return scan8_ks<MPW, 3>(q, p, s);
        case 4: return scan8_ks<MPW, 4>(q, p, s);
        default: return hipErrorInvalidValue;
      }
    }
  } else if constexpr (kBF16) {
    switch (p.ks) {   // (1..4: the gate only)
      case 1: return scan8_ks<MPW, 1>(q, p, s);
      case 2: return scan8_ks<MPW, 2>(q, p, s);
      case 3: return scan8_ks<MPW, 3>(q, p, s);
      case 4: return scan8_ks<MPW, 4>(q, p, s);
      case 5: return scan8_ks<MPW, 5>(q, p, s);
      case 6: return scan8_ks<MPW, 6>(q, p, s);
      case 7: return scan8_ks<MPW, 7>(q, p, s);
      case 8: return scan8_ks<MPW, 8>(q, p, s);
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
}

template <bool REDUCE, int MPW, int R, bool KEEP>
hipError_t one(const FusedParams& q, const FusedPlan& p, hipStream_t s) {
  if constexpr (KEEP && (MPW > kKeepMaxMPW || R != 2)) {
    return hipErrorInvalidValue;
  } else if constexpr (!REDUCE && KEEP) {
    if (p.scan8) return scan8<MPW>(q, p, s);
    return fused::launch_scan_t<MPW, R, kTV, kBF16, KEEP>(q, p, s);
  } else if constexpr (REDUCE) {
    return fused::launch_reduce_t<MPW, R, kTV, kBF16, KEEP>(q, p, s);
  } else {
    return fused::launch_scan_t<MPW, R, kTV, kBF16, KEEP>(q, p, s);
  }
}

template <bool REDUCE, int R, bool KEEP>
hipError_t by_mpw(const FusedParams& q, const FusedPlan& p, hipStream_t s) {
  switch (q.Ppad / 64) {
    case 1: return one<REDUCE, 1, R, KEEP>(q, p, s);
    case 2: return one<REDUCE, 2, R, KEEP>(q, p, s);
    case 3: return one<REDUCE, 3, R, KEEP>(q, p, s);
    case 4: return one<REDUCE, 4, R, KEEP>(q, p, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool REDUCE>
hipError_t dispatch(const FusedParams& q, const FusedPlan& p, hipStream_t s) {
  if (q.bf16_io != kBF16 || q.time_varying != kTV) return hipErrorInvalidValue;
  const bool keep = REDUCE ? p.keep : (p.keep_scan || p.scan8);
  if (p.R == 2) return keep ? by_mpw<REDUCE, 2, true>(q, p, s) : by_mpw<REDUCE, 2, false>(q, p, s);
  if constexpr (!kBF16) {
    if (p.R == 1 && !keep) return by_mpw<REDUCE, 1, false>(q, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace s5
