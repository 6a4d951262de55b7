// Pass 2 of the fused S5 forward path with eight symmetric waves (gfx950).
// Included by s5_fused_kernels.h after the helpers it uses.
//
// Every wave does, for each chunk, the same three kinds of work on its own
// share: the drive (B_bar u on MFMA) and the scan of its mode tiles
// j = w + 8 m, the readout (C' x on MFMA) of its h-tiles ht = w + 8 e with
// their D u feedthrough and y stores, and a share of staging the next u tiles.
// Both waves of a SIMD therefore mix matrix-core and vector work, and the y
// epilogue of chunk i-1 is issued beside the readout MFMAs of chunk i (it
// needs only that chunk's sums, kept in registers across the barrier), so the
// epilogue's vector work and stores hide under matrix-core work instead of
// following it. The drive's K-step count KS (Hpad = 32 KS) is a template
// parameter: no MFMA multiplies padding.
//
// LDS: four u tiles (tile c in buffer c & 3: staged in iteration c-2, driven
// in iteration c-1, its feedthrough read in iteration c+1), two x tiles and
// the per-mode table with D. Float32 u is staged as three bf16 planes hi,
// lo = bf16(u - hi), lo2 = bf16(u - hi - lo): u = hi + lo + lo2 exactly (each
// residual is exact in float32 and has at most 16, then 8, significant
// bits), so the drive's operands hi and lo are split once per tile and the
// feedthrough still reads u exactly.
#pragma once

namespace s5 {
namespace fused {

constexpr int kW8 = 2 * kWaves;   // waves of the symmetric kernel

// bytes of one u tile (KS K-steps x R steps; one bf16 plane, or three for float32 u)
__host__ __device__ constexpr size_t u8_tile_bytes(int KS, int R, bool bf16) {
  return static_cast<size_t>(KS) * R * (bf16 ? 1 : 3) * kBlock;
}

template <int R, bool BF16, int NB>
__device__ __forceinline__ void stash8(const FusedParams& q, const UStage<NB>& st, lds_byte* ub, int w, int l) {
  const int nblk = (q.Hpad >> 5) * R * (BF16 ? 1 : 2);
#pragma unroll
  for (int e = 0; e < NB; ++e) {
    const int blk = w + kW8 * e;
    if (blk >= nblk) {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): see stash_u
      continue;
    }
    if constexpr (BF16) {
      lds_st<uint4>(ub + blk * kBlock + l * 16, st.v[e]);
    } else {
      // half-block: elements 4 half .. 4 half + 3 of fragment f = s R + n
      const int half = blk & 1;
      const int f = blk >> 1;
      const f32x4 v = {__uint_as_float(st.v[e].x), __uint_as_float(st.v[e].y), __uint_as_float(st.v[e].z),
                       __uint_as_float(st.v[e].w)};
      const bf16x4 hi = __builtin_convertvector(v, bf16x4);
      const f32x4 r1 = v - __builtin_convertvector(hi, f32x4);
      const bf16x4 lo = __builtin_convertvector(r1, bf16x4);
      const bf16x4 lo2 = __builtin_convertvector(r1 - __builtin_convertvector(lo, f32x4), bf16x4);
      lds_byte* p = ub + (f * 3) * kBlock + l * 16 + 8 * half;
      lds_st<uint2>(p, __builtin_bit_cast(uint2, hi));
      lds_st<uint2>(p + kBlock, __builtin_bit_cast(uint2, lo));
      lds_st<uint2>(p + 2 * kBlock, __builtin_bit_cast(uint2, lo2));
    }
  }
}

// y already in memory for the wave's readout outputs of chunk i (the backward
// scan adds to it), loaded an iteration ahead of its use (see load_y_old)
template <int R, bool BF16, bool VEC, int ET>
__device__ __forceinline__ void load_y_old8(const FusedParams& q, __amdgpu_buffer_rsrc_t yr, const RowMap& rm, int i,
                                            int w, const Lane& ln, YOld<BF16>& o) {
  static_assert(R <= 2 && ET <= kKeepHT, "YOld holds two steps of two h-tiles");
  constexpr int esz = BF16 ? 2 : 4;
#pragma unroll
  for (int e = 0; e < ET; ++e) {
    const int h0 = 16 * (w + kW8 * e) + 4 * ln.g;
#pragma unroll
    for (int n = 0; n < R; ++n) {
      const int roff = rm(rel_row<R>(q, ln.t, i, n)) * q.H;
      if constexpr (VEC) {
        const int off = h0 < q.H ? (roff + h0) * esz : kBufferOOB;
        if constexpr (BF16) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b64(yr, off, 0, 0);
          o.v[e][n] = make_uint2(v[0], v[1]);
        } else {
          const auto v = __builtin_amdgcn_raw_buffer_load_b128(yr, off, 0, 0);
          o.v[e][n] = make_uint4(v[0], v[1], v[2], v[3]);
        }
      } else {
        uint32_t v4[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int off = h0 + m < q.H ? (roff + h0 + m) * esz : kBufferOOB;
          v4[m] = BF16 ? static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(yr, off, 0, 0))
                       : __builtin_amdgcn_raw_buffer_load_b32(yr, off, 0, 0);
        }
        if constexpr (BF16) {
          o.v[e][n] = make_uint2(v4[0] | (v4[1] << 16), v4[2] | (v4[3] << 16));
        } else {
          o.v[e][n] = make_uint4(v4[0], v4[1], v4[2], v4[3]);
        }
      }
    }
  }
}

// drive operand fragments of K-step s: [plane][n] (hi, and lo for float32 u)
template <int R, bool BF16>
__device__ __forceinline__ void get_u8(const lds_byte* ub, int s, int l, bf16x8 (&uf)[BF16 ? 1 : 2][R]) {
#pragma unroll
  for (int n = 0; n < R; ++n) {
    if constexpr (BF16) {
      uf[0][n] = as_bf16x8(lds_ld<uint4>(ub + (s * R + n) * kBlock + l * 16));
    } else {
      uf[0][n] = as_bf16x8(lds_ld<uint4>(ub + ((s * R + n) * 3) * kBlock + l * 16));
      uf[1][n] = as_bf16x8(lds_ld<uint4>(ub + ((s * R + n) * 3 + 1) * kBlock + l * 16));
    }
  }
}

// u of the readout lane's 4 outputs, features 16 ht + 4 g + 0..3 of token
// (t, n): K-step ht/2, lane t + 16 (2 (ht & 1) + g/2), elements 4 (g & 1)..+3
template <int R, bool BF16>
__device__ __forceinline__ void u_for_y8(const lds_byte* ub, int ht, int n, int t, int g, float (&uv)[4]) {
  const int s = ht >> 1;
  const int lp = t + 16 * (2 * (ht & 1) + (g >> 1));
  const int off = lp * 16 + 8 * (g & 1);
  auto four = [](uint2 p, float (&o)[4]) {
    o[0] = __uint_as_float(p.x << 16);
    o[1] = __uint_as_float(p.x & 0xffff0000u);
    o[2] = __uint_as_float(p.y << 16);
    o[3] = __uint_as_float(p.y & 0xffff0000u);
  };
  if constexpr (BF16) {
    four(lds_ld<uint2>(ub + (s * R + n) * kBlock + off), uv);
  } else {
    const lds_byte* p = ub + ((s * R + n) * 3) * kBlock + off;
    float hi[4], lo[4], lo2[4];
    four(lds_ld<uint2>(p), hi);
    four(lds_ld<uint2>(p + kBlock), lo);
    four(lds_ld<uint2>(p + 2 * kBlock), lo2);
#pragma unroll
    for (int r = 0; r < 4; ++r) uv[r] = (hi[r] + lo[r]) + lo2[r];   // exact: u itself
  }
}

// Delta of chunk i for the lane's 4 modes of each of the wave's tiles
template <int MT, int NT, int R>
__device__ __forceinline__ void load_delta8(const FusedParams& q, int b, int qq, int i, int w, const Lane& ln,
                                            float4 (&dl)[MT][R]) {
  const bool vec = (q.P & 3) == 0;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int pm0 = 16 * (w + kW8 * m) + 4 * ln.g;
#pragma unroll
    for (int n = 0; n < R; ++n) {
      const int tok = tok_of<R>(q, qq, ln.t, i, n);
      float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (w + kW8 * m < NT && tok < q.L && pm0 < q.P) {
        const float* dp = q.delta + range_row0(q, b, qq) * q.P +
                          (rel_row<R>(q, ln.t, i, n) * static_cast<uint32_t>(q.P) + pm0);
        if (vec) {
          const float4 x = *reinterpret_cast<const float4*>(dp);
          v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = pm0 + r < q.P ? dp[r] : 0.0f;
        }
      }
      dl[m][n] = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// state entering the lane's stream for the wave's tiles (see stream_start)
template <int MT, int NT, bool TV>
__device__ __forceinline__ void stream_start8(const FusedParams& q, int bq, int w, const Lane& ln,
                                              const S5_LDS pf2* s_c0, cf (&st)[MT][4]) {
  float2 xv[MT][4], av[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = w + kW8 * m;
      const int pm = 16 * j + 4 * ln.g + r;
      xv[m][r] = make_float2(0.0f, 0.0f);
      av[m][r] = make_float2(1.0f, 0.0f);
      if (j < NT) {
        const size_t si = (static_cast<size_t>(bq) * kStreams + ln.t) * q.Ppad + pm;
        xv[m][r] = q.sagg[si];
        av[m][r] = TV ? q.sagg_a[si] : q.modes[pm].aseg;
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = w + kW8 * m;
      cf X = {xv[m][r].x, xv[m][r].y};
      cf A = {av[m][r].x, av[m][r].y};
      row_scan(A, X);
      const cf Ae = {row_shr<1>(A.re, 1.0f), row_shr<1>(A.im, 0.0f)};
      const cf Xe = {row_shr<1>(X.re, 0.0f), row_shr<1>(X.im, 0.0f)};
      st[m][r] = j < NT ? cfma(Ae, ld_pf2(s_c0 + (16 * j + 4 * ln.g + r)), Xe) : cf{0.0f, 0.0f};
    }
  }
}

// the state after token L-1 for the wave's modes (see write_final_state)
template <int R, int MT, int NT, bool TV>
__device__ __forceinline__ void write_final_state8(const FusedParams& q, int b, const LastTok& lt, int w,
                                                   const Lane& ln, const cf (&st)[MT][4]) {
  if (ln.t != lt.t) return;
  const float2* c = q.cap + static_cast<size_t>(b) * 2 * q.Ppad;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = w + kW8 * m;
      const int pm = 16 * j + 4 * ln.g + r;
      if (j >= NT || pm >= q.P) continue;
      const cf X = {c[pm].x, c[pm].y};
      cf A;
      if constexpr (TV) {
        A = {c[q.Ppad + pm].x, c[q.Ppad + pm].y};
      } else {
        const float2 al = q.modes[pm].alast;
        A = {al.x, al.y};
      }
      const cf x = cfma(A, st[m][r], X);
      q.xlast[static_cast<size_t>(b) * q.P + pm] = make_float2(x.re, x.im);
    }
}

// Scan of mode tile j (slot m) of one chunk from its drive sums acc, then its
// x tile fragments (bf16 hi [+ lo]) into LDS.
template <int MT, int NT, int R, bool TV, bool BF16>
__device__ __forceinline__ void scan_tile8(bool bil, int j, int m, f32x4 (&acc)[2][R], const ModeTable& mtab,
                                           const Lane& ln, const float4 (&dl)[TV ? MT : 1][TV ? R : 1],
                                           cf (&st)[MT][4], lds_byte* xb) {
  constexpr int K2 = NT;   // readout K-steps = mode tiles
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int pm = 16 * j + 4 * ln.g + r;
    cf x = st[m][r];
    if constexpr (TV) {
      const StepMode sm = mtab.step_mode(pm);
#pragma unroll
      for (int n = 0; n < R; ++n) {
        x = step_am1(disc_am1(bil, sm, f4_at(dl[m][n], r)), x, {acc[0][n][r], acc[1][n][r]});
        acc[0][n][r] = x.re;
        acc[1][n][r] = x.im;
      }
    } else {
      const cf ab = ld_pf2(mtab.ab + pm);
#pragma unroll
      for (int n = 0; n < R; ++n) {
        x = cfma(ab, x, {acc[0][n][r], acc[1][n][r]});
        acc[0][n][r] = x.re;
        acc[1][n][r] = x.im;
      }
    }
    st[m][r] = x;
  }
#pragma unroll
  for (int n = 0; n < R; ++n) {
    float v[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[2 * r] = acc[0][n][r];
      v[2 * r + 1] = acc[1][n][r];
    }
    const int blk = j * R + n;
    uint4 hi, lo;
    put_frag(v, &hi, BF16 ? nullptr : &lo);
    lds_st<uint4>(xb + blk * kBlock + ln.l * 16, hi);
    if constexpr (!BF16) lds_st<uint4>(xb + (K2 * R + blk) * kBlock + ln.l * 16, lo);
  }
}

// Drive, scan and x tile of the wave's mode tiles for one chunk (u tile ub,
// x tile xb). Tile by tile, so that one tile's scan runs beside the next
// tile's MFMAs. bf16: the chunk's u fragments are read once for all tiles.
template <int MT, int NT, int KS, int R, bool TV, bool BF16, bool ONCE = true>
__device__ __forceinline__ void drive_scan8(bool bil, int w, const bf16x8 (&bw)[KS][MT][2][BF16 ? 1 : 2],
                                            const lds_byte* ub, const ModeTable& mtab, const Lane& ln,
                                            const float4 (&dl)[TV ? MT : 1][TV ? R : 1], cf (&st)[MT][4],
                                            lds_byte* xb) {
  constexpr int NP = BF16 ? 1 : 2;
  constexpr bool kOnce = ONCE && BF16 && MT > 1;
  bf16x8 ua[kOnce ? KS : 1][NP][R];
  if constexpr (kOnce) {
#pragma unroll
    for (int s = 0; s < KS; ++s) get_u8<R, BF16>(ub, s, ln.l, ua[s]);
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int j = w + kW8 * m;
    if ((NT % kW8) != 0 && j >= NT) continue;   // wave-uniform
    f32x4 acc[2][R];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int n = 0; n < R; ++n) acc[cc][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // (read per K-step: one K-step ahead of its MFMAs)
    bf16x8 uq[kOnce ? 1 : 2][NP][R];
    if constexpr (!kOnce) get_u8<R, BF16>(ub, 0, ln.l, uq[0]);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8 uk[NP][R];
      if constexpr (kOnce) {
#pragma unroll
        for (int pl = 0; pl < NP; ++pl)
#pragma unroll
          for (int n = 0; n < R; ++n) uk[pl][n] = ua[s][pl][n];
      } else {
        if (s + 1 < KS) get_u8<R, BF16>(ub, s + 1, ln.l, uq[(s + 1) & 1]);
#pragma unroll
        for (int pl = 0; pl < NP; ++pl)
#pragma unroll
          for (int n = 0; n < R; ++n) uk[pl][n] = uq[s & 1][pl][n];
      }
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int n = 0; n < R; ++n) {
          acc[cc][n] = mfma(bw[s][m][cc][0], uk[0][n], acc[cc][n]);
          if constexpr (NP == 2) {
            acc[cc][n] = mfma(bw[s][m][cc][0], uk[1][n], acc[cc][n]);
            acc[cc][n] = mfma(bw[s][m][cc][1], uk[0][n], acc[cc][n]);
          }
        }
    }
    scan_tile8<MT, NT, R, TV, BF16>(bil, j, m, acc, mtab, ln, dl, st, xb);
  }
}

// The drive with B_bar streamed from L2 (bf16, time-invariant, more than four
// K-steps), tile by tile: the fragments of (tile, K-step) step t + kBW are
// loaded at step t, the first kBW steps' come in bwin (loaded by the caller
// ahead of the chunk); each tile's scan follows its MFMAs.
// B_bar fragment (tile j, component cc, K-step s) of the lane from the packed
// operand's buffer descriptor: the lane's 16 bytes at a wave-uniform offset
// (one scalar offset per load, where 64-bit addresses would take two vector
// registers each)
template <int KS>
__device__ __forceinline__ bf16x8 ld_bfrag8(__amdgpu_buffer_rsrc_t br, int j, int cc, int s, int l) {
  const int soff = __builtin_amdgcn_readfirstlane(((j * 2 + cc) * KS + s) * kBlock);
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(br, l * 16, soff, 0);
  return as_bf16x8(make_uint4(v[0], v[1], v[2], v[3]));
}

template <int MT, int NT, int KS, int R, int kBW>
__device__ __forceinline__ void drive_scan8_sb(int w, __amdgpu_buffer_rsrc_t br, const bf16x8 (&bwin)[kBW][2],
                                               const lds_byte* ub, const ModeTable& mtab, const Lane& ln,
                                               cf (&st)[MT][4], lds_byte* xb) {
  constexpr int T = MT * KS;   // (tile, K-step) steps
  bf16x8 bq[T][2];
#pragma unroll
  for (int t = 0; t < kBW && t < T; ++t) {
    bq[t][0] = bwin[t][0];
    bq[t][1] = bwin[t][1];
  }
  const float4 dl[1][1] = {};
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int j = w + kW8 * m;
    if ((NT % kW8) != 0 && j >= NT) continue;   // wave-uniform
    f32x4 acc[2][R];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int n = 0; n < R; ++n) acc[cc][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    bf16x8 uq[2][1][R];
    get_u8<R, true>(ub, 0, ln.l, uq[0]);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int t = m * KS + s;
      const int tn = t + kBW;   // the step loaded now
      if (tn < T) {
        const int jn = w + kW8 * (tn / KS);
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
          bq[tn][cc] = jn < NT ? ld_bfrag8<KS>(br, jn, cc, tn % KS, ln.l) : as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
      }
      if (s + 1 < KS) get_u8<R, true>(ub, s + 1, ln.l, uq[(s + 1) & 1]);
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int n = 0; n < R; ++n) acc[cc][n] = mfma(bq[t][cc], uq[s & 1][0][n], acc[cc][n]);
      // each step's loads beside its MFMAs (left alone, the scheduler issues
      // every load of the chunk first and runs out of registers)
      if (tn < T) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
      if (s + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * R, 0);
    }
    scan_tile8<MT, NT, R, false, true>(false, j, m, acc, mtab, ln, dl, st, xb);
  }
}

// B_bar fragments of the streamed drive's first kBW (tile, K-step) steps
template <int MT, int NT, int KS, int kBW>
__device__ __forceinline__ void get_bwin8(__amdgpu_buffer_rsrc_t br, int w, int l, bf16x8 (&b)[kBW][2]) {
#pragma unroll
  for (int t = 0; t < kBW; ++t) {
    const int j = w + kW8 * (t / KS);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
      b[t][cc] = t < MT * KS && j < NT ? ld_bfrag8<KS>(br, j, cc, t % KS, l) : as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
  }
}

template <int MPW, int KS, bool TV, bool BF16, int XM>
__global__ void __launch_bounds__(2 * kThreads, 1) k_scan8(FusedParams q) {
  constexpr bool EXT = XM != 0;   // options of the extended entry point
  constexpr int R = 2;
  constexpr int NP = BF16 ? 1 : 2;
  constexpr int NT = 4 * MPW;                   // mode tiles (= readout K-steps)
  constexpr int K2 = NT;
  constexpr int MT = (NT + kW8 - 1) / kW8;      // mode tiles per wave, at most
  constexpr int HT = 2 * KS;                    // h-tiles
  constexpr int ET = (HT + kW8 - 1) / kW8;      // h-tiles per wave, at most
  constexpr bool kAcc = XM == 3;                // backward scan: add to y
  // More than four drive K-steps (H > 128, bf16): the weights of both
  // products exceed the registers; C' stays, B_bar is streamed from L2 (see
  // drive_scan8_sb), its first kBW K-steps loaded at the top of the iteration
  // before the drive, so that they arrive during the readout.
  constexpr bool SB = KS > 4;
  constexpr int kBW = MPW >= 4 ? 2 : MPW == 3 ? 3 : 4;   // (what the registers allow)
  static_assert(!SB || (BF16 && !TV), "the streamed drive is built for time-invariant bf16 I/O");
  // XM = 5: the gated activation in this pass (bf16 I/O, H <= 128). Chunk c's
  // y (D u included), rounded to bf16 as the layer would store it (so that
  // the gate sees the same input as after a separate layer call), gives
  // g = GELU(y), written as B-operand fragments (the
  // layout of a bf16 u tile, inputs = features) split into a bf16 hi and lo
  // plane, into a ring of two g tiles, and the multiplier (g or y, float32)
  // into LDS; after the next barrier every wave forms W g for its h-tiles on
  // the matrix cores from three products (W_hi g_hi + W_hi g_lo + W_lo g_hi:
  // float32-level accuracy, since the gate's slope times |g| amplifies any
  // rounding of W or g) and stores y = multiplier * sigma(W g + bias): one
  // store of y, after the gate. W_hi stays in registers; W_lo is read from L2
  // once per chunk (at the end of the previous iteration).
  constexpr bool GATE = XM == 5;
  static_assert(!GATE || (BF16 && !SB), "the fused gate is built for bf16 I/O with H <= 128");
  extern __shared__ __align__(16) unsigned char smem[];
  if (q.Ppad != 64 * MPW || q.Hpad != 32 * KS || q.R != R) return;   // dispatch mismatch: do nothing
  Lane ln = lane_ids();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & (kW8 - 1);
  ln.w = w;
  const int bq = blockIdx.x;
  const int b = bq / q.Q;
  const int qq = bq - b * q.Q;
  const bool bil = EXT && q.bilinear;
  const RowMap rmap = row_map<XM == 3>(q, qq);
  constexpr int ut = static_cast<int>(u8_tile_bytes(KS, R, BF16));
  constexpr int xt = static_cast<int>(x_tile_bytes(K2, R, BF16));
  lds_byte* lds = (lds_byte*)smem;
  lds_byte* xlds = lds + 4 * ut;
  const ModeTable mtab = fill_mode_table<TV>(q, xlds + 2 * xt, true);
  // the gate's ring of two g tiles (hi and lo planes), after the mode table,
  // then its multipliers and the bias
  constexpr int gt = static_cast<int>(KS * R * kBlock);   // one plane of one g tile
  lds_byte* glds = xlds + 2 * xt + mode_table_bytes(64 * MPW, 32 * KS, TV, true);
  S5_LDS pf2* s_c0 = reinterpret_cast<S5_LDS pf2*>(xlds + xt);   // free until x tile 1
  if (threadIdx.x < static_cast<unsigned>(q.Ppad)) range_carry<EXT, TV>(q, b, qq, threadIdx.x, s_c0);

  // weights: B_bar fragments of the wave's mode tiles, C' fragments of its h-tiles
  bf16x8 bw[SB ? 1 : KS][MT][2][NP];
  bf16x8 cw[ET][K2][NP];
  {
    const int nb = (q.Ppad / 16) * 2 * KS * 64;
    const int nc = (q.Hpad / 16) * K2 * 64;
    if constexpr (!SB) {
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int pl = 0; pl < NP; ++pl) {
              const int j = w + kW8 * m;
              bw[s][m][cc][pl] = j < NT ? as_bf16x8(ldg16(q.bpack + pl * nb + ((j * 2 + cc) * KS + s) * 64 + ln.l))
                                        : as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
            }
    }
#pragma unroll
    for (int e = 0; e < ET; ++e)
#pragma unroll
      for (int s = 0; s < K2; ++s)
#pragma unroll
        for (int pl = 0; pl < NP; ++pl) {
          const int ht = w + kW8 * e;
          cw[e][s][pl] = ht < HT ? as_bf16x8(ldg16(q.cpack + pl * nc + (ht * K2 + s) * 64 + ln.l))
                                 : as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
        }
  }

  // the gate's W fragments of the wave's h-tiles, hi plane (rows 16 ht +
  // l%16, inputs 32 s + 8 (l/16) + 0..7, zero past H), and the descriptor of
  // the lo plane
  bf16x8 wg[GATE ? ET : 1][GATE ? KS : 1];
  const __amdgpu_buffer_rsrc_t grsrc = __builtin_amdgcn_make_buffer_rsrc(
      GATE ? q.gpack + HT * KS * 64 : q.bpack, 0, GATE ? HT * KS * kBlock : 0, kBufferWord3);
  if constexpr (GATE) {
#pragma unroll
    for (int e = 0; e < ET; ++e)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int ht = w + kW8 * e;
        wg[e][s] = ht < HT ? as_bf16x8(ldg16(q.gpack + (ht * KS + s) * 64 + ln.l))
                           : as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
      }
    lds_byte* gbias = glds + 4 * gt + 8 * ET * R * kBlock;
    for (int h = threadIdx.x; h < q.Hpad; h += 2 * kThreads)
      reinterpret_cast<S5_LDS float*>(gbias)[h] = q.glu_bias != nullptr && h < q.H ? q.glu_bias[h] : 0.0f;
  }
  bf16x8 wlo[GATE ? ET : 1][GATE ? KS : 1];
  auto load_wlo = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < ET; ++e)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int ht = w + kW8 * e;
        if (ht < HT) {
          const int soff = __builtin_amdgcn_readfirstlane((ht * KS + s) * kBlock);
          const auto v = __builtin_amdgcn_raw_buffer_load_b128(grsrc, ln.l * 16, soff, 0);
          wlo[e][s] = as_bf16x8(make_uint4(v[0], v[1], v[2], v[3]));
        } else {
          wlo[e][s] = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
        }
      }
  };

  constexpr int NB = (KS * R * (BF16 ? 1 : 2) + kW8 - 1) / kW8;
  const __amdgpu_buffer_rsrc_t ursrc = range_rsrc<BF16>(q.u, q, b, qq, rmap.rev);
  const __amdgpu_buffer_rsrc_t yrsrc = y_rsrc<XM, BF16>(q, b, qq, rmap.rev);
  const __amdgpu_buffer_rsrc_t yorsrc = XM == 3 ? range_rsrc<false>(q.yp, q, b, qq, rmap.rev) : yrsrc;
  // the packed B_bar (bf16: one plane of 2 Ppad/16 KS fragments) for the streamed drive
  const __amdgpu_buffer_rsrc_t brsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4*>(q.bpack), 0, (q.Ppad / 16) * 2 * KS * kBlock, kBufferWord3);
  const int HTv = (q.H + 15) >> 4;   // h-tiles holding a feature < H
  const Epi ep = epilogue<XM>(q);

  auto chunks = [&](auto vec_c) {
    constexpr bool VEC = decltype(vec_c)::value;
    {
      UStage<NB> ust;
      fetch_u<R, BF16, NB, kW8, VEC>(q, ursrc, rmap, qq, 0, ust);
      stash8<R, BF16, NB>(q, ust, lds, w, ln.l);
      fetch_u<R, BF16, NB, kW8, VEC>(q, ursrc, rmap, qq, 1, ust);
      stash8<R, BF16, NB>(q, ust, lds + ut, w, ln.l);
    }
    lds_barrier();   // carry, mode table, u tiles 0 and 1
    float4 dk[SB ? 1 : ET];   // D of the wave's h-tiles: features 16 ht + 4 g + 0..3 (streamed form: read at use)
#pragma unroll
    for (int e = 0; e < (SB ? 0 : ET); ++e) {
      const int h0 = 16 * (w + kW8 * e) + 4 * ln.g;
      dk[e] = h0 < q.Hpad ? lds_ld<float4>(reinterpret_cast<const lds_byte*>(mtab.d + h0))
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    cf st[MT][4];
    stream_start8<MT, NT, TV>(q, bq, w, ln, s_c0, st);
    if (EXT && q.xlast != nullptr) {
      const LastTok lt = last_token<R>(q);
      if (qq == lt.qq) write_final_state8<R, MT, NT, TV>(q, b, lt, w, ln, st);
    }
    float4 dl[TV ? MT : 1][TV ? R : 1];
    if constexpr (TV) load_delta8<MT, NT, R>(q, b, qq, 0, w, ln, dl);
    bf16x8 bwin[SB ? kBW : 1][2];   // streamed drive: its first steps of B_bar
    if constexpr (SB) {
      get_bwin8<MT, NT, KS, kBW>(brsrc, w, ln.l, bwin);
      drive_scan8_sb<MT, NT, KS, R, kBW>(w, brsrc, bwin, lds, mtab, ln, st, xlds);
    } else {
      drive_scan8<MT, NT, KS, R, TV, BF16, !GATE>(bil, w, bw, lds, mtab, ln, dl, st, xlds);
    }
    // Delta of chunk i+1 is loaded an iteration ahead (before that
    // iteration's u loads), so that waiting for it never waits for them
    if constexpr (TV) load_delta8<MT, NT, R>(q, b, qq, 1, w, ln, dl);
    lds_barrier();   // x tile 0 (and the carry read before x tile 1 is written)

    // Iteration i: readout of chunk i (x tile i & 1), y of chunk i-1 (its
    // sums from the previous iteration, u tile i-1), drive and scan of chunk
    // i+1 (u tile i+1 -> x tile (i+1) & 1), u tile i+2 staged.
    f32x4 yprev[ET][R];
    YOld<false> yold_prev, yold_cur;
#pragma unroll
    for (int e = 0; e < ET; ++e)
#pragma unroll
      for (int n = 0; n < R; ++n) yprev[e][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    auto epilogue_of = [&](int c, const f32x4 (&ya)[ET][R], const YOld<false>& yo) __attribute__((always_inline)) {
      const lds_byte* ub = lds + (c & 3) * ut;
#pragma unroll
      for (int e = 0; e < ET; ++e) {
        const int ht = w + kW8 * e;
        if (ht >= HTv) continue;   // wave-uniform
        const int h0 = 16 * ht + 4 * ln.g;
#pragma unroll
        for (int n = 0; n < R; ++n) {
          float uv[4];
          u_for_y8<R, BF16>(ub, ht, n, ln.t, ln.g, uv);
          f32x4 a = ya[e][n];
          if constexpr (kAcc) a += y_old_f32<false>(yo.v[e][n]);
          const float4 d = SB ? lds_ld<float4>(reinterpret_cast<const lds_byte*>(mtab.d + h0)) : dk[SB ? 0 : e];
          store_y<y_bf16<XM, BF16>(), VEC>(yrsrc, rmap(rel_row<R>(q, ln.t, c, n)) * q.H, h0, q.H, a, d, uv,
                                           Epi{false, ep.gelu, ep.tanh_form}, yrsrc);
        }
      }
    };
    // the gate: chunk c's y -> g tile (c & 1) and the multiplier (first
    // half), then, a barrier later, W g, the logistic gate and the store
    // (each lane's multipliers wait in LDS for its own gate_out, one block
    // per wave, h-tile and step)
    lds_byte* gml = glds + 4 * gt + (w * ET * R) * kBlock + ln.l * 16;
    const lds_byte* gbias = glds + 4 * gt + 8 * ET * R * kBlock;
    auto gate_in = [&](int c, const f32x4 (&ya)[ET][R]) __attribute__((always_inline)) {
      const lds_byte* ub = lds + (c & 3) * ut;
      lds_byte* gb = glds + (c & 1) * 2 * gt;
#pragma unroll
      for (int e = 0; e < ET; ++e) {
        const int ht = w + kW8 * e;
        if (ht >= HT) continue;   // wave-uniform
        // g fragment position of the lane's 4 features (as u_for_y8 reads a u tile)
        const int sk = ht >> 1;
        const int off = (ln.t + 16 * (2 * (ht & 1) + (ln.g >> 1))) * 16 + 8 * (ln.g & 1);
#pragma unroll
        for (int n = 0; n < R; ++n) {
          f32x4 yv = {0.0f, 0.0f, 0.0f, 0.0f};
          if (ht < HTv) {   // (features past H: g = 0, and W is zero there)
            float uv[4];
            u_for_y8<R, BF16>(ub, ht, n, ln.t, ln.g, uv);
            const float4 d = dk[e];
            yv = f32x4{fmaf(d.x, uv[0], ya[e][n][0]), fmaf(d.y, uv[1], ya[e][n][1]),
                       fmaf(d.z, uv[2], ya[e][n][2]), fmaf(d.w, uv[3], ya[e][n][3])};
            yv = __builtin_convertvector(__builtin_convertvector(yv, bf16x4), f32x4);   // the stored y
          }
          f32x4 g;
#pragma unroll
          for (int r = 0; r < 4; ++r) g[r] = gelu_erf(yv[r]);
          const bf16x4 ghi = __builtin_convertvector(g, bf16x4);
          const bf16x4 glo = __builtin_convertvector(g - __builtin_convertvector(ghi, f32x4), bf16x4);
          lds_st<uint2>(gb + (sk * R + n) * kBlock + off, __builtin_bit_cast(uint2, ghi));
          lds_st<uint2>(gb + gt + (sk * R + n) * kBlock + off, __builtin_bit_cast(uint2, glo));
          const f32x4 mv = q.glu_variant == 1 ? g : yv;
          lds_st<float4>(gml + (e * R + n) * kBlock, make_float4(mv[0], mv[1], mv[2], mv[3]));
        }
      }
    };
    auto gate_out = [&](int c) __attribute__((always_inline)) {
      const lds_byte* gb = glds + (c & 1) * 2 * gt;
      f32x4 z[ET][R];
#pragma unroll
      for (int e = 0; e < ET; ++e)
#pragma unroll
        for (int n = 0; n < R; ++n) z[e][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int sk = 0; sk < KS; ++sk) {
        bf16x8 gh[1][R], gl[1][R];
        get_u8<R, true>(gb, sk, ln.l, gh);
        get_u8<R, true>(gb + gt, sk, ln.l, gl);
#pragma unroll
        for (int e = 0; e < ET; ++e)
#pragma unroll
          for (int n = 0; n < R; ++n) {
            z[e][n] = mfma(wg[e][sk], gl[0][n], z[e][n]);
            z[e][n] = mfma(wlo[e][sk], gh[0][n], z[e][n]);
            z[e][n] = mfma(wg[e][sk], gh[0][n], z[e][n]);
          }
      }
#pragma unroll
      for (int e = 0; e < ET; ++e) {
        const int ht = w + kW8 * e;
        if (ht >= HTv) continue;   // wave-uniform
        const int h0 = 16 * ht + 4 * ln.g;
        const float4 b4 = lds_ld<float4>(gbias + 4 * h0);
        const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int n = 0; n < R; ++n) {
          const float4 m4 = lds_ld<float4>(gml + (e * R + n) * kBlock);
          const float mv[4] = {m4.x, m4.y, m4.z, m4.w};
          f32x4 o;
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = mv[r] * __builtin_amdgcn_rcpf(1.0f + __expf(-(z[e][n][r] + bv[r])));
          const float zero4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
          store_y<BF16, VEC>(yrsrc, rmap(rel_row<R>(q, ln.t, c, n)) * q.H, h0, q.H, o,
                             make_float4(0.0f, 0.0f, 0.0f, 0.0f), zero4, Epi{false, false, false}, yrsrc);
        }
      }
    };
    for (int i = 0; i < q.nck; ++i) {
      float4 dnext[TV ? MT : 1][TV ? R : 1];
      if constexpr (TV) load_delta8<MT, NT, R>(q, b, qq, i + 2, w, ln, dnext);
      UStage<NB> ust;
      fetch_u<R, BF16, NB, kW8, VEC>(q, ursrc, rmap, qq, i + 2, ust);
      if constexpr (kAcc) load_y_old8<R, false, VEC, ET>(q, yorsrc, rmap, i, w, ln, yold_cur);
      if constexpr (SB) {
        if (i + 1 < q.nck) get_bwin8<MT, NT, KS, kBW>(brsrc, w, ln.l, bwin);
      }
      if constexpr (GATE) {
        if (i > 0) gate_out(i - 1);   // g tile (i-1) & 1 is complete (the last barrier)
      }
      // readout of chunk i
      f32x4 yacc[ET][R];
#pragma unroll
      for (int e = 0; e < ET; ++e)
#pragma unroll
        for (int n = 0; n < R; ++n) yacc[e][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      const lds_byte* xr = xlds + (i & 1) * xt;
      if (w < HT) {   // wave-uniform: waves past the h-tiles read nothing out
        // x fragments read kAhead K-steps ahead of their MFMAs (left alone,
        // the scheduler puts each read next to its use and waits there)
        constexpr int kAhead = NP == 2 || SB || GATE ? 1 : 3;
        bf16x8 xf[K2][NP][R];
#pragma unroll
        for (int s = 0; s < kAhead && s < K2; ++s) get_x<R, NP>(xr, K2, s, ln.l, xf[s]);
        __builtin_amdgcn_sched_group_barrier(0x100, (kAhead < K2 ? kAhead : K2) * NP * R, 0);
#pragma unroll
        for (int s = 0; s < K2; ++s) {
          if (s + kAhead < K2) get_x<R, NP>(xr, K2, s + kAhead, ln.l, xf[s + kAhead]);
#pragma unroll
          for (int e = 0; e < ET; ++e) mfma_read<R, NP>(cw[e][s], xf[s], yacc[e]);
          if (s + kAhead < K2) __builtin_amdgcn_sched_group_barrier(0x100, NP * R, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, ET * R * (NP == 2 ? 3 : 1), 0);
        }
      }
      if constexpr (GATE) {
        gate_in(i, yacc);
      } else if constexpr (SB) {
        epilogue_of(i, yacc, yold_cur);   // (no registers to keep the sums for the next iteration)
      } else if (i > 0) {
        epilogue_of(i - 1, yprev, yold_prev);   // y of chunk i-1 beside those MFMAs
      }
      // drive and scan of chunk i+1 (none after the last chunk)
      if (i + 1 < q.nck) {
        if constexpr (SB) {
          drive_scan8_sb<MT, NT, KS, R, kBW>(w, brsrc, bwin, lds + ((i + 1) & 3) * ut, mtab, ln, st,
                                             xlds + ((i + 1) & 1) * xt);
        } else {
          drive_scan8<MT, NT, KS, R, TV, BF16, !GATE>(bil, w, bw, lds + ((i + 1) & 3) * ut, mtab, ln, dl, st,
                                                      xlds + ((i + 1) & 1) * xt);
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // keep the stash (and its wait) after the chunk's work
      stash8<R, BF16, NB>(q, ust, lds + ((i + 2) & 3) * ut, w, ln.l);
      if constexpr (GATE) load_wlo();   // for gate_out of chunk i (next iteration, or after the loop)
      if constexpr (!SB && !GATE) {
#pragma unroll
        for (int e = 0; e < ET; ++e)
#pragma unroll
          for (int n = 0; n < R; ++n) yprev[e][n] = yacc[e][n];
        if constexpr (kAcc) yold_prev = yold_cur;
      }
      if constexpr (TV) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int n = 0; n < R; ++n) dl[m][n] = dnext[m][n];
      }
      lds_barrier();   // x tile i+1, u tile i+2 complete; x tile i, u tile i-2 free
    }
    if constexpr (GATE) {
      gate_out(q.nck - 1);   // (after the loop's last barrier)
    } else if constexpr (!SB) {
      epilogue_of(q.nck - 1, yprev, yold_prev);
    }
  };
  if (u_rows_vectorized(q.H, BF16)) {
    chunks(std::true_type{});
  } else {
    chunks(std::false_type{});
  }
}

}  // namespace fused
}  // namespace s5
