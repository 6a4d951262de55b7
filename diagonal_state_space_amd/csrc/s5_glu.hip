// Gated activation after the S5 layer (wikillm notes, "Paper vs code": GLU
// variant and dense gate bias; the pseudocode's half_glu1 step):
//   g = GELU(y),  gate = sigma(W g + b),  out = g * gate   (variant 1)
//                                         out = y * gate   (variant 2)
// with a dense H x H matrix W. The product W g runs on the matrix cores:
// per workgroup eight waves, wave w holding the operand fragments of output
// tiles w, w + 8, ... of W for all K-steps in registers (loaded once), and a
// persistent loop over tiles of 64 tokens whose GELU(y) is staged in LDS as
// B operands, with the epilogue's multiplier (GELU(y) or y, float32) beside
// them. Both operands are split into bf16 hi and lo parts and three products
// summed (W_hi g_hi + W_hi g_lo + W_lo g_hi), for either I/O type: the gate's
// slope times |g| amplifies the rounding of W g, so single bf16 products
// lose accuracy once |y| grows past a few units. The epilogue adds the bias, applies the logistic gate and the
// multiplier and stores the result, all in the same pass.
#include <algorithm>

#include "s5_common.h"
#include "s5_internal.h"

namespace s5 {

namespace {

constexpr int kGluWaves = 8;
constexpr int kGluThreads = 64 * kGluWaves;
constexpr int kGluNT = 4;             // 16-column MFMA tiles (tokens) per pass
constexpr int kGluTokens = 16 * kGluNT;
// register-held W: K-steps of 32 features and output tiles of 16 per wave,
// for H <= 128 (SMALL) and H <= 256
template <bool SMALL>
constexpr int glu_ks() { return SMALL ? 4 : 8; }
template <bool SMALL>
constexpr int glu_mt() { return SMALL ? 1 : 2; }


// 8 consecutive elements of y from element index idx (zeros past `count`);
// vec: one 16-byte (bf16) or two 16-byte (float32) loads
template <bool BF16>
__device__ __forceinline__ void load8(const GluArgs& q, size_t idx, int count, bool vec, float (&v)[8]) {
  if (vec && count >= 8) {
    if constexpr (BF16) {
      const uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q.y) + idx);
      const uint32_t wv[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(wv[i] << 16);
        v[2 * i + 1] = __uint_as_float(wv[i] & 0xffff0000u);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(q.y) + idx);
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (BF16) {
        v[i] = i < count ? bf16_to_f32(static_cast<const uint16_t*>(q.y)[idx + i]) : 0.0f;
      } else {
        v[i] = i < count ? static_cast<const float*>(q.y)[idx + i] : 0.0f;
      }
    }
  }
}

template <bool BF16, bool SMALL>
__global__ void __launch_bounds__(kGluThreads) k_glu(GluArgs q) {
  constexpr int NP = 2;   // hi and lo planes of both operands
  constexpr int kGluMaxKS = glu_ks<SMALL>();
  constexpr int kGluMaxMT = glu_mt<SMALL>();
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int KS = (q.H + 31) >> 5;
  const int HM = (q.H + 15) >> 4;
  const int Hpad = 32 * KS;
  const int mstride = Hpad + 4;   // float32 row stride of the multipliers (padded off the bank period)
  // whole 8-element groups are aligned 16-byte units when the row length allows
  const bool vec = BF16 ? (q.H % 8 == 0) : (q.H % 4 == 0);

  // W fragments of this wave's output tiles: row j = 16 m + l%16,
  // inputs 32 s + 8 (l/16) + 0..7
  bf16x8 wf[kGluMaxMT][kGluMaxKS][NP];
#pragma unroll
  for (int mt = 0; mt < kGluMaxMT; ++mt) {
    const int m = w + kGluWaves * mt;
    const int j = 16 * m + (l & 15);
#pragma unroll
    for (int s = 0; s < kGluMaxKS; ++s) {
      f32x8 f;
      const int k0 = 32 * s + 8 * (l >> 4);
      if (m < HM && s < KS && j < q.H && k0 + 8 <= q.H && q.H % 4 == 0) {
        // whole row segment, 16-byte aligned: two vector loads
        const float4* p = reinterpret_cast<const float4*>(q.w + static_cast<size_t>(j) * q.H + k0);
        const float4 a = p[0], b = p[1];
        f = f32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int k = k0 + i;
          f[i] = (m < HM && s < KS && j < q.H && k < q.H) ? q.w[static_cast<size_t>(j) * q.H + k] : 0.0f;
        }
      }
      const bf16x8 hi = __builtin_convertvector(f, bf16x8);
      wf[mt][s][0] = hi;
      wf[mt][s][1] = __builtin_convertvector(f - __builtin_convertvector(hi, f32x8), bf16x8);
    }
  }

  // LDS: the tile's GELU(y) as B-operand blocks (s, nt, pl) of 64 lanes x 16
  // bytes (lane l: token 16 nt + l%16, inputs 32 s + 8 (l/16) + 0..7), then
  // the epilogue's multiplier (variant 1: GELU(y), 2: y) as float32
  // [64 tokens][Hpad + 4]
  auto gblk = [&](int s, int nt, int pl) { return smem + ((s * kGluNT + nt) * NP + pl) * 1024; };
  float* s_mul = reinterpret_cast<float*>(smem + kGluNT * KS * NP * 1024);
  const int ntiles = (q.T + kGluTokens - 1) / kGluTokens;
  // y of a tile for this wave's staging blocks blk = w + 8 c (c < kBlk),
  // loaded one tile ahead of its use
  constexpr int kBlk = kGluNT * kGluMaxKS / kGluWaves;
  float ynext[kBlk][8];
  auto fetch = [&](int tile) {
#pragma unroll
    for (int c = 0; c < kBlk; ++c) {
      const int blk = w + kGluWaves * c;
      const int tok = tile * kGluTokens + 16 * (blk % kGluNT) + (l & 15);
      const int k0 = 32 * (blk / kGluNT) + 8 * (l >> 4);
      const int count = (blk < kGluNT * KS && tile < ntiles && tok < q.T) ? min(8, q.H - k0) : 0;
      load8<BF16>(q, static_cast<size_t>(tok) * q.H + k0, count, vec, ynext[c]);
    }
  };
  fetch(blockIdx.x);
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int t0 = tile * kGluTokens;
#pragma unroll
    for (int c = 0; c < kBlk; ++c) {
      const int blk = w + kGluWaves * c;
      if (blk >= kGluNT * KS) break;   // wave-uniform
      const int s = blk / kGluNT, nt = blk % kGluNT;
      const int tl = 16 * nt + (l & 15);
      const int k0 = 32 * s + 8 * (l >> 4);
      float yv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) yv[i] = ynext[c][i];
      f32x8 f;
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = gelu_erf(yv[i]);
      const bf16x8 hi = __builtin_convertvector(f, bf16x8);
      *reinterpret_cast<uint4*>(gblk(s, nt, 0) + l * 16) = as_u4(hi);
      *reinterpret_cast<uint4*>(gblk(s, nt, 1) + l * 16) =
          as_u4(__builtin_convertvector(f - __builtin_convertvector(hi, f32x8), bf16x8));
      float4* dst = reinterpret_cast<float4*>(s_mul + tl * mstride + k0);
      if (q.variant == 1) {
        dst[0] = make_float4(f[0], f[1], f[2], f[3]);
        dst[1] = make_float4(f[4], f[5], f[6], f[7]);
      } else {
        dst[0] = make_float4(yv[0], yv[1], yv[2], yv[3]);
        dst[1] = make_float4(yv[4], yv[5], yv[6], yv[7]);
      }
    }
    __syncthreads();   // g tile and multipliers complete
    fetch(tile + gridDim.x);   // the next tile's y, in flight during this tile's products
#pragma unroll
    for (int mt = 0; mt < kGluMaxMT; ++mt) {
      const int m = w + kGluWaves * mt;
      if (m >= HM) break;   // wave-uniform
      f32x4 acc[kGluNT];
#pragma unroll
      for (int nt = 0; nt < kGluNT; ++nt) acc[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < kGluMaxKS; ++s) {
        if (s >= KS) break;
#pragma unroll
        for (int nt = 0; nt < kGluNT; ++nt) {
          const bf16x8 b0 = as_bf16x8(*reinterpret_cast<const uint4*>(gblk(s, nt, 0) + l * 16));
          const bf16x8 b1 = as_bf16x8(*reinterpret_cast<const uint4*>(gblk(s, nt, 1) + l * 16));
          acc[nt] = mfma(wf[mt][s][0], b1, acc[nt]);
          acc[nt] = mfma(wf[mt][s][1], b0, acc[nt]);
          acc[nt] = mfma(wf[mt][s][0], b0, acc[nt]);
        }
      }
      // lane (t, g): token 16 nt + t, outputs j0 = 16 m + 4 g .. j0 + 3
      const int j0 = 16 * m + 4 * (l >> 4);
      float bj[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) bj[r] = (q.bias != nullptr && j0 + r < q.H) ? q.bias[j0 + r] : 0.0f;
#pragma unroll
      for (int nt = 0; nt < kGluNT; ++nt) {
        const int tl = 16 * nt + (l & 15);
        const int tok = t0 + tl;
        if (tok >= q.T || j0 >= q.H) continue;
        const float4 mv = *reinterpret_cast<const float4*>(s_mul + tl * mstride + j0);
        const float mul[4] = {mv.x, mv.y, mv.z, mv.w};
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gate = __builtin_amdgcn_rcpf(1.0f + __expf(-(acc[nt][r] + bj[r])));
          o[r] = mul[r] * gate;
        }
        const size_t idx = static_cast<size_t>(tok) * q.H + j0;
        if (j0 + 4 <= q.H && (q.H % 4 == 0)) {
          if constexpr (BF16) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            const f32x4 ov = {o[0], o[1], o[2], o[3]};
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(q.out) + idx) =
                __builtin_bit_cast(uint2, __builtin_convertvector(ov, bf16x4));
          } else {
            *reinterpret_cast<float4*>(static_cast<float*>(q.out) + idx) = make_float4(o[0], o[1], o[2], o[3]);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (j0 + r >= q.H) break;
            if constexpr (BF16) {
              static_cast<uint16_t*>(q.out)[idx + r] = f32_to_bf16(o[r]);
            } else {
              static_cast<float*>(q.out)[idx + r] = o[r];
            }
          }
        }
      }
    }
    __syncthreads();   // every wave is done with the tile's LDS
  }
}

}  // namespace

size_t glu_lds_bytes(int H, bool bf16_io) {
  const size_t ks = (H + 31) / 32;
  (void)bf16_io;   // (two operand planes for either I/O type)
  return ks * kGluNT * 2 * 1024 + static_cast<size_t>(kGluTokens) * (32 * ks + 4) * sizeof(float);
}

// one launch of instance Kern; its first launch lifts the dynamic LDS limit
// (up to 128 KB at H = 256 with float32 I/O)
template <auto Kern>
hipError_t glu_go(const GluArgs& a, int grid, size_t lds, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(Kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(Kern, dim3(grid), dim3(kGluThreads), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_glu(const GluArgs& a, hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  if (a.H > 32 * glu_ks<false>()) return hipErrorInvalidValue;
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  const int ntiles = (a.T + kGluTokens - 1) / kGluTokens;
  const bool small = a.H <= 128;
  // every workgroup reads and converts W once, so the grid stays at two
  // workgroups per CU (measured: 4 and 8 per CU were slower); the large
  // instance (W of up to 256 KB) takes at least four tiles per workgroup
  int grid = ntiles < 2 * ncu ? ntiles : 2 * ncu;
  if (!small) grid = std::max(std::min(ntiles, ncu), std::min(grid, (ntiles + 3) / 4));
  const size_t lds = glu_lds_bytes(a.H, a.bf16_io);
  if (a.bf16_io) return small ? glu_go<k_glu<true, true>>(a, grid, lds, stream) : glu_go<k_glu<true, false>>(a, grid, lds, stream);
  return small ? glu_go<k_glu<false, true>>(a, grid, lds, stream) : glu_go<k_glu<false, false>>(a, grid, lds, stream);
}

}  // namespace s5
