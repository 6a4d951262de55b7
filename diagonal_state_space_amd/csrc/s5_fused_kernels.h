// Fused S5 forward kernels for gfx950 (CDNA4): device templates.
//
// The recurrence x_k = a_k x_{k-1} + b_k (paper eq. 2 after the zero-order
// hold of eq. 6; App. H gives the pair operator (a_j a_i, a_j b_i + b_j)) is
// computed without writing the L x P state to HBM, in two passes over u:
//
//   pass 1 (k_reduce): per stream, the state reached from a zero start and the
//     product of its a_k; per workgroup range, the same for its 16 streams
//     combined (a 16-lane scan of pairs with DPP row shifts).
//   pass 2 (k_scan): the state entering each stream (carry of the earlier
//     ranges, then a 16-lane exclusive scan), then per chunk
//       drive    Bu^T[2P x 16R] = B_bar[2P x H] . u^T[H x 16R]   (MFMA)
//       scan     x_k = a_k x_{k-1} + b_k, sequential in each lane (VALU)
//       readout  y^T[H x 16R] = C'[H x 2P] . x^T[2P x 16R] + D u  (MFMA)
//
// with C'[h, 2p] = Re C~[h,p], C'[h, 2p+1] = -Im C~[h,p], so that
// Re(C~ x) = C' [Re x; Im x] (paper eq. 2 and App. A; output factor 1 for a
// full spectrum). The 16 columns of every MFMA tile are 16 streams of
// consecutive tokens, so lane (t = l%16, g = l/16) of wave w owns stream t
// and, of mode tile j = w + 4jj, the modes 16 j + 4 g + r (r < 4): the
// drive's result tile is already in the lane that scans it, and the lane's
// states (modes 4g..4g+3 of the tile, both parts) are already the readout's
// B operand fragment. Float32 I/O splits every float32 operand v into bf16
// parts hi = bf16(v), lo = bf16(v - hi) and sums hi.hi + hi.lo + lo.hi.
//
// LDS holds 1 KB blocks of 64 lanes x 16 bytes in operand-fragment order, so
// every LDS access is lane-contiguous: u tiles (staged through registers one
// chunk ahead; two buffers in pass 1, three in pass 2, where the readout's D u
// term reads them too) and x tiles (two buffers).
#pragma once

#include <type_traits>

#include "s5_common.h"
#include "s5_fused.h"

namespace s5 {
namespace fused {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeepKS = 4;     // drive K-steps held in registers (H <= 128)
constexpr int kKeepHT = 2;     // readout h-tiles per wave held in registers (H <= 128)

// LDS pointers keep their address space explicitly: a generic pointer picked
// at run time compiles to FLAT accesses, whose waits also wait (in-order
// vmcnt) for the asynchronous global->LDS copies in flight.
#define S5_LDS __attribute__((address_space(3)))
typedef S5_LDS unsigned char lds_byte;

// Workgroup barrier for LDS traffic: waits for this wave's LDS accesses only
// (LDS-scoped fences), so global loads in flight (the next u tile) and stores
// (y) are not waited for. Waves here exchange data only through LDS.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

struct pf2 {   // plain float pair, accessed member by member in LDS
  float x, y;
};
__device__ __forceinline__ void st_pf2(S5_LDS pf2* p, float x, float y) {
  p->x = x;
  p->y = y;
}
__device__ __forceinline__ cf ld_pf2(const S5_LDS pf2* p) { return {p->x, p->y}; }

typedef uint32_t lds_v4 __attribute__((ext_vector_type(4)));
typedef uint32_t lds_v2 __attribute__((ext_vector_type(2)));

// 16- or 8-byte LDS accesses of HIP vector types through native vectors
template <typename T>
__device__ __forceinline__ T lds_ld(const lds_byte* p) {
  static_assert(sizeof(T) == 16 || sizeof(T) == 8, "16- or 8-byte LDS access");
  if constexpr (sizeof(T) == 16) {
    return __builtin_bit_cast(T, *reinterpret_cast<const S5_LDS lds_v4*>(p));
  } else {
    return __builtin_bit_cast(T, *reinterpret_cast<const S5_LDS lds_v2*>(p));
  }
}
template <typename T>
__device__ __forceinline__ void lds_st(lds_byte* p, const T& v) {
  static_assert(sizeof(T) == 16 || sizeof(T) == 8, "16- or 8-byte LDS access");
  if constexpr (sizeof(T) == 16) {
    *reinterpret_cast<S5_LDS lds_v4*>(p) = __builtin_bit_cast(lds_v4, v);
  } else {
    *reinterpret_cast<S5_LDS lds_v2*>(p) = __builtin_bit_cast(lds_v2, v);
  }
}

// ---- 16-lane row scan of (a, x) pairs -----------------------------------------

template <int D>
__device__ __forceinline__ float row_shr(float v, float fill) {
  // DPP row_shr:D; lanes t < D of each 16-lane row get `fill`
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(v), 0x110 + D, 0xF, 0xF, false));
}

template <int D>
__device__ __forceinline__ void row_scan_step(cf& A, cf& X) {
  const cf Ap = {row_shr<D>(A.re, 1.0f), row_shr<D>(A.im, 0.0f)};
  const cf Xp = {row_shr<D>(X.re, 0.0f), row_shr<D>(X.im, 0.0f)};
  X = cfma(A, Xp, X);   // later segment (A, X) after the earlier (Ap, Xp)
  A = cmul(A, Ap);
}

// Inclusive scan over the 16 lanes of each row, lane order = stream order.
__device__ __forceinline__ void row_scan(cf& A, cf& X) {
  row_scan_step<1>(A, X);
  row_scan_step<2>(A, X);
  row_scan_step<4>(A, X);
  row_scan_step<8>(A, X);
}

// the value of lane 15 - t of the lane's 16-lane row (DPP row_mirror)
__device__ __forceinline__ float row_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
}

// ---- geometry ---------------------------------------------------------------------

struct Lane {
  int tid, w, l, t, g;
};

// ids within a group of kWaves waves (the role of a wave-specialized kernel)
__device__ __forceinline__ Lane lane_ids() {
  Lane x;
  x.tid = threadIdx.x & (kThreads - 1);
  // wave-uniform (scalar branches); the mask tells the compiler its range
  x.w = __builtin_amdgcn_readfirstlane(x.tid >> 6) & (kWaves - 1);
  x.l = x.tid & 63;
  x.t = x.l & 15;
  x.g = x.l >> 4;
  return x;
}

// token (within the sequence) of stream t, chunk i, step n
template <int R>
__device__ __forceinline__ int tok_of(const FusedParams& q, int qq, int t, int i, int n) {
  return (qq * kStreams + t) * q.Lseg + i * R + n;
}

// Row (in [B*L]) of the first token of workgroup range (b, qq). Hot global
// accesses use this uniform row's address plus a 32-bit lane offset (the host
// keeps a range below 1 GiB), so that no 64-bit per-lane address stays live.
__device__ __forceinline__ size_t range_row0(const FusedParams& q, int b, int qq) {
  return static_cast<size_t>(b) * q.L + static_cast<size_t>(qq) * kStreams * q.Lseg;
}

// row of (stream t, chunk i, step n) relative to range_row0
template <int R>
__device__ __forceinline__ uint32_t rel_row(const FusedParams& q, int t, int i, int n) {
  return static_cast<uint32_t>(t * q.Lseg + i * R + n);
}

// ---- state before the first step and after the last ---------------------------------
// Token L-1 of every sequence lies in workgroup range `qq`, stream `t`, chunk
// `i`, step `n`. When the caller asks for the final state, pass 1 records that
// stream's state from a zero start through token L-1 (and, time-varying, the
// product of its transitions), and pass 2 applies them to the stream's start
// state: x_{L-1} = A x_start + X. (The scan itself runs on past L-1 over the
// zero input of the padding tokens, which would decay the state.)
struct LastTok {
  int qq, t, i, n;
};
template <int R>
__device__ __forceinline__ LastTok last_token(const FusedParams& q) {
  const int k = q.L - 1;
  const int span = kStreams * q.Lseg;
  LastTok lt;
  lt.qq = k / span;
  const int rem = k - lt.qq * span;
  lt.t = rem / q.Lseg;
  const int r2 = rem - lt.t * q.Lseg;
  lt.i = r2 / R;
  lt.n = r2 - lt.i * R;
  return lt;
}

// pass 1, in the lane of stream lt.t after step lt.n of chunk lt.i
__device__ __forceinline__ void record_partial(const FusedParams& q, int b, int pm, const cf& x, const cf& a) {
  float2* c = q.cap + static_cast<size_t>(b) * 2 * q.Ppad;
  c[pm] = make_float2(x.re, x.im);
  c[q.Ppad + pm] = make_float2(a.re, a.im);
}

// pass 2, in the lanes of stream lt.t of range lt.qq right after their start
// state is known: the state after token L-1 for the lane's modes. The
// time-invariant transition over the m steps is Lambda_bar^m (packed in float64).
template <int R, int MPW, bool TV>
__device__ __forceinline__ void write_final_state(const FusedParams& q, int b, const LastTok& lt, const Lane& ln,
                                                  const cf (&st)[MPW][4]) {
  if (ln.t != lt.t) return;
  const float2* c = q.cap + static_cast<size_t>(b) * 2 * q.Ppad;
#pragma unroll
  for (int jj = 0; jj < MPW; ++jj)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pm = 16 * (ln.w + kWaves * jj) + 4 * ln.g + r;
      if (pm >= q.P) continue;
      const cf X = {c[pm].x, c[pm].y};
      cf A;
      if constexpr (TV) {
        A = {c[q.Ppad + pm].x, c[q.Ppad + pm].y};
      } else {
        const float2 al = q.modes[pm].alast;   // abar^m, from the float64 packing
        A = {al.x, al.y};
      }
      const cf x = cfma(A, st[jj][r], X);
      q.xlast[static_cast<size_t>(b) * q.P + pm] = make_float2(x.re, x.im);
    }
}

// ---- u tile: global -> registers -> LDS in fragment order -----------------------------
// Block (s, n[, half]) holds, in lane (t, g), u[tok(t, i, n)][32 s + 8 g + ...]:
// 8 bf16, or 4 floats per half (halves 0 and 1 = elements 0-3 and 4-7). Wave w
// moves blocks w, w + 4, ...: fetch_u loads them into registers a chunk ahead,
// stash_u writes them to LDS before the barrier that publishes the tile.
// SPLIT (float32 u, pass 1): the same bytes hold instead the two bf16 planes
// of the drive's operands, hi and lo (u = hi + lo to 2^-17), split once when
// the tile is staged rather than by each of the eight waves that read it.
// Pass 2 keeps the floats: its D u feedthrough reads u itself.
// (Copies straight from global memory to LDS were measured slower here: every
// LDS access after one waits for it.)
//
// The loads are buffer loads through a descriptor that spans the rows of the
// workgroup range: an element past the sequence end, past H, or of a chunk
// that does not exist gets an offset beyond the descriptor's size, and the
// hardware returns zeros for it. No branch and no select depends on the data
// being there, so the compiler has no reason to wait for a load before its
// value is stored to LDS.
template <int NB>
struct UStage {
  uint4 v[NB];
};

// registers per thread for the u tile: KS R NPU blocks over NWV waves
template <int R, bool BF16, bool KEEP, int NWV = kWaves>
constexpr int u_stage_blocks() {
  return ((KEEP ? kKeepKS : 16) * R * (BF16 ? 1 : 2) + NWV - 1) / NWV;
}

// Whether every lane block of u is one whole 16-byte vector of a row (H a
// multiple of 8 bf16 / 4 floats): then a block is one 16-byte load, else one
// load per element. Kernels instantiate their chunk loops for both cases.
__host__ __device__ inline bool u_rows_vectorized(int H, bool bf16) { return bf16 ? (H % 8 == 0) : (H % 4 == 0); }

constexpr int kBufferOOB = static_cast<int>(0x80000000u);   // beyond any descriptor size here
constexpr int kBufferWord3 = 0x00020000;                     // raw buffer, 32-bit data format

// descriptor over the rows (of H elements) of workgroup range (b, qq) of u or
// y: rows past the sequence end are outside it (below 1 GiB, host-checked).
// In reverse time (the backward scan) range qq is the mirror of forward range
// Q-1-qq: the same rows, run from the last of the padded range to the first
// (see RowMap), so that both scans cut the sequence at the same tokens.
template <bool BF16>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void* t, const FusedParams& q, int b, int qq,
                                                             bool rev) {
  constexpr int esz = BF16 ? 2 : 4;
  const int qf = rev ? q.Q - 1 - qq : qq;
  const int tok0 = qf * kStreams * q.Lseg;
  const int rows = min(q.L - tok0, kStreams * q.Lseg);
  const size_t row0 = range_row0(q, b, qf);
  // The fields are workgroup-uniform; reading them from the first lane tells
  // the compiler so (where it cannot prove it, every buffer access would be
  // wrapped in a loop over the distinct descriptors of the wave's lanes).
  const uint64_t a = reinterpret_cast<uint64_t>(static_cast<const char*>(t) + row0 * q.H * esz);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  const int nbytes = __builtin_amdgcn_readfirstlane(rows * q.H * esz);
  char* base = reinterpret_cast<char*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, nbytes, kBufferWord3);
}

// Memory row, relative to the range descriptor's base, of relative token row
// r: r in forward time. In reverse time (the backward scan) the range's token
// rows run backward from the last row of the padded range, so row
// 16 Lseg - 1 - r; rows past the sequence end (the padding of the last
// forward range, which the backward scan meets first, from a zero state that
// zero inputs leave zero) go to last + 1, outside the descriptor.
struct RowMap {
  bool rev;
  int last;   // rows of the range - 1
  int full;   // 16 Lseg - 1
  __device__ __forceinline__ int operator()(uint32_t r) const {
    const int ri = static_cast<int>(r);
    const int m = full - ri;
    return !rev ? ri : (m <= last ? m : last + 1);
  }
};

template <bool REV>
__device__ __forceinline__ RowMap row_map(const FusedParams& q, int qq) {
  if (REV && q.rev) {
    const int qf = q.Q - 1 - qq;
    return {true, min(q.L - qf * kStreams * q.Lseg, kStreams * q.Lseg) - 1, kStreams * q.Lseg - 1};
  }
  return {false, 0, 0};
}

// Output epilogue by instance: XM = 2 always GELU (the form from q.gelu:
// 1 exact, 2 tanh); XM = 3 adds to y (the
// backward scan of the bidirectional form), then GELU if asked. The addition
// reads y in the store path; a load there behind a runtime test would make
// the compiler wait for every outstanding load (the prefetched u tiles) at
// the merge, so it is compiled only where every call adds. Runtime tests in
// the store path also split the readout loop's scheduling regions, so the
// plain and state-only instances have none.
struct Epi {
  bool accum;
  bool gelu;
  bool tanh_form;   // GELU in its tanh form (else the exact form)
};

template <int XM>
__device__ __forceinline__ Epi epilogue(const FusedParams& q) {
  return {XM == 3, XM == 2 || (XM == 3 && q.gelu != 0), (XM == 2 || XM == 3) && q.gelu == 2};
}

// Instances of the bidirectional form's two passes 2: XM = 4 (forward half)
// stores y, D u included, as float32 into q.yp; XM = 3 (backward, reverse
// time) adds those float32 values to its readout and stores y in the I/O type
// once (for float32 I/O q.yp is y itself).
template <int XM, bool BF16>
constexpr bool y_bf16() { return BF16 && XM != 4; }

template <int XM, bool BF16>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t y_rsrc(const FusedParams& q, int b, int qq, bool rev) {
  return range_rsrc<y_bf16<XM, BF16>()>(XM == 4 ? static_cast<void*>(q.yp) : q.y, q, b, qq, rev);
}

template <int R, bool BF16, int NB, int NWV, bool VEC>
__device__ __forceinline__ void fetch_u(const FusedParams& q, __amdgpu_buffer_rsrc_t rsrc, const RowMap& rm, int qq,
                                        int i, UStage<NB>& st) {
  constexpr int NPU = BF16 ? 1 : 2;
  constexpr int esz = BF16 ? 2 : 4;
  Lane ln = lane_ids();
  if constexpr (NWV != kWaves) ln.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & (NWV - 1);
  const int nblk = (q.Hpad >> 5) * R * NPU;
  const bool live = i < q.nck;   // chunk i exists (callers fetch unconditionally)
#pragma unroll
  for (int e = 0; e < NB; ++e) {
    const int blk = ln.w + NWV * e;   // wave-uniform; blocks past the tile load zeros (not stored)
    const int half = blk % NPU;
    const int f = blk / NPU;
    const int n = f % R;
    const int s = f / R;
    const int tok = tok_of<R>(q, qq, ln.t, i, n);
    const int h0 = 32 * s + 8 * ln.g + 4 * half;
    // (in reverse time the row map sends the padding outside the descriptor)
    const bool row_ok = live && blk < nblk && (rm.rev || tok < q.L);
    const int roff = rm(rel_row<R>(q, ln.t, i, n)) * q.H;
    if constexpr (VEC) {
      const int off = row_ok && h0 < q.H ? (roff + h0) * esz : kBufferOOB;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
      st.v[e] = make_uint4(v[0], v[1], v[2], v[3]);
    } else if constexpr (BF16) {
      uint32_t v4[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int h = h0 + 2 * m;
        const int olo = row_ok && h < q.H ? (roff + h) * esz : kBufferOOB;
        const int ohi = row_ok && h + 1 < q.H ? (roff + h + 1) * esz : kBufferOOB;
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rsrc, olo, 0, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rsrc, ohi, 0, 0);
        v4[m] = lo | (hi << 16);
      }
      st.v[e] = make_uint4(v4[0], v4[1], v4[2], v4[3]);
    } else {
      uint32_t v4[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int o = row_ok && h0 + m < q.H ? (roff + h0 + m) * esz : kBufferOOB;
        v4[m] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, o, 0, 0);
      }
      st.v[e] = make_uint4(v4[0], v4[1], v4[2], v4[3]);
    }
  }
}

template <int R, bool BF16, int NB, int NWV, bool SPLIT = false>
__device__ __forceinline__ void stash_u(const FusedParams& q, const UStage<NB>& st, lds_byte* ub) {
  Lane ln = lane_ids();
  if constexpr (NWV != kWaves) ln.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & (NWV - 1);
  const int nblk = (q.Hpad >> 5) * R * (BF16 ? 1 : 2);
#pragma unroll
  for (int e = 0; e < NB; ++e) {
    const int blk = ln.w + NWV * e;
    if (blk >= nblk) {
      // This wave loaded nothing into v[e] (fetch_u skipped the same block),
      // but the compiler cannot tell: without this (free) wait it assumes a
      // load may still be writing v[e] at the next fetch and waits there for
      // every outstanding load instead.
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
      continue;
    }
    if constexpr (BF16 || !SPLIT) {
      lds_st<uint4>(ub + blk * kBlock + ln.l * 16, st.v[e]);
    } else {
      // the bf16 hi and lo operand planes of the fragment (blocks 2f and
      // 2f + 1), this half's four elements at bytes 8 half .. 8 half + 7 of
      // the lane's slot
      const int half = blk & 1;
      const int f = blk >> 1;
      const f32x4 v = {__uint_as_float(st.v[e].x), __uint_as_float(st.v[e].y), __uint_as_float(st.v[e].z),
                       __uint_as_float(st.v[e].w)};
      const bf16x4 hi = __builtin_convertvector(v, bf16x4);
      const bf16x4 lo = __builtin_convertvector(v - __builtin_convertvector(hi, f32x4), bf16x4);
      lds_st<uint2>(ub + (2 * f) * kBlock + ln.l * 16 + 8 * half, __builtin_bit_cast(uint2, hi));
      lds_st<uint2>(ub + (2 * f + 1) * kBlock + ln.l * 16 + 8 * half, __builtin_bit_cast(uint2, lo));
    }
  }
}

// drive operand fragments of K-step s from the u tile: [plane][n]
template <int R, bool BF16, bool SPLIT = false>
__device__ __forceinline__ void get_u(const lds_byte* ub, int s, int l, bf16x8 (&uf)[BF16 ? 1 : 2][R]) {
#pragma unroll
  for (int n = 0; n < R; ++n) {
    if constexpr (BF16) {
      uf[0][n] = as_bf16x8(lds_ld<uint4>(ub + (s * R + n) * kBlock + l * 16));
    } else if constexpr (SPLIT) {
      uf[0][n] = as_bf16x8(lds_ld<uint4>(ub + ((s * R + n) * 2) * kBlock + l * 16));
      uf[1][n] = as_bf16x8(lds_ld<uint4>(ub + ((s * R + n) * 2 + 1) * kBlock + l * 16));
    } else {
      const float4 a = lds_ld<float4>(ub + ((s * R + n) * 2) * kBlock + l * 16);
      const float4 c = lds_ld<float4>(ub + ((s * R + n) * 2 + 1) * kBlock + l * 16);
      const f32x8 f = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
      const bf16x8 hi = __builtin_convertvector(f, bf16x8);
      uf[0][n] = hi;
      uf[1][n] = __builtin_convertvector(f - __builtin_convertvector(hi, f32x8), bf16x8);
    }
  }
}

// ---- drive: acc[jj][cc][n] = rows (mode 16 j + 4 g + r, part cc) of B_bar . u^T ----

template <int MPW, int NP>
__device__ __forceinline__ void load_b_step(const FusedParams& q, int w, int l, int s, bf16x8 (&a)[MPW][2][NP]) {
  const int KS = q.Hpad >> 5;
  const int nb = (q.Ppad / 16) * 2 * KS * 64;
#pragma unroll
  for (int jj = 0; jj < MPW; ++jj)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int pl = 0; pl < NP; ++pl)
        a[jj][cc][pl] = as_bf16x8(ldg16(q.bpack + pl * nb + (((w + kWaves * jj) * 2 + cc) * KS + s) * 64 + l));
}

template <int MPW, int R, int NP>
__device__ __forceinline__ void mfma_drive(const bf16x8 (&a)[MPW][2][NP], const bf16x8 (&uf)[NP][R],
                                           f32x4 (&acc)[MPW][2][R]) {
#pragma unroll
  for (int jj = 0; jj < MPW; ++jj)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int n = 0; n < R; ++n) {
        acc[jj][cc][n] = mfma(a[jj][cc][0], uf[0][n], acc[jj][cc][n]);
        if constexpr (NP == 2) {
          acc[jj][cc][n] = mfma(a[jj][cc][0], uf[1][n], acc[jj][cc][n]);
          acc[jj][cc][n] = mfma(a[jj][cc][1], uf[0][n], acc[jj][cc][n]);
        }
      }
}

// B_bar held in registers for all (at most kKeepKS) K-steps
template <int MPW, int NP>
struct BKeep {
  bf16x8 f[kKeepKS][MPW][2][NP];
};

template <int MPW, int NP>
__device__ __forceinline__ void load_b_keep(const FusedParams& q, int w, int l, BKeep<MPW, NP>& bk) {
  const int KS = q.Hpad >> 5;
#pragma unroll
  for (int s = 0; s < kKeepKS; ++s) {
    if (s < KS) {
      load_b_step<MPW, NP>(q, w, l, s, bk.f[s]);
    } else {
#pragma unroll
      for (int jj = 0; jj < MPW; ++jj)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int pl = 0; pl < NP; ++pl) bk.f[s][jj][cc][pl] = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
    }
  }
}

template <int MPW, int R, bool BF16, bool KEEP, bool SPLIT = false>
__device__ __forceinline__ void drive(const FusedParams& q, const BKeep<MPW, BF16 ? 1 : 2>& bk,
                                      const lds_byte* ub, int w, int l, f32x4 (&acc)[MPW][2][R]) {
  constexpr int NP = BF16 ? 1 : 2;
#pragma unroll
  for (int jj = 0; jj < MPW; ++jj)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int n = 0; n < R; ++n) acc[jj][cc][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int KS = q.Hpad >> 5;
  if constexpr (KEEP) {
    // branch-free: weights of K-steps s >= KS are zero, and their u operand is
    // read from the last real K-step (finite data of the same tokens)
#pragma unroll
    for (int s = 0; s < kKeepKS; ++s) {
      bf16x8 uf[NP][R];
      get_u<R, BF16, SPLIT>(ub, s < KS ? s : KS - 1, l, uf);
      mfma_drive<MPW, R, NP>(bk.f[s], uf, acc);
    }
  } else {
    bf16x8 a[MPW][2][NP];
    load_b_step<MPW, NP>(q, w, l, 0, a);
    for (int s = 0; s < KS; ++s) {
      bf16x8 an[MPW][2][NP];
      if (s + 1 < KS) load_b_step<MPW, NP>(q, w, l, s + 1, an);
      bf16x8 uf[NP][R];
      get_u<R, BF16, SPLIT>(ub, s, l, uf);
      mfma_drive<MPW, R, NP>(a, uf, acc);
      if (s + 1 < KS) {
#pragma unroll
        for (int jj = 0; jj < MPW; ++jj)
#pragma unroll
          for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int pl = 0; pl < NP; ++pl) a[jj][cc][pl] = an[jj][cc][pl];
      }
    }
  }
}

// ---- time-varying inputs: Delta for the lane's 4 modes of each tile ------------------

template <int MPW, int R>
__device__ __forceinline__ void load_delta(const FusedParams& q, int b, int qq, int i, const Lane& ln,
                                           float4 (&dl)[MPW][R]) {
  const bool vec = (q.P & 3) == 0;
#pragma unroll
  for (int jj = 0; jj < MPW; ++jj) {
    const int pm0 = 16 * (ln.w + kWaves * jj) + 4 * ln.g;
#pragma unroll
    for (int n = 0; n < R; ++n) {
      const int tok = tok_of<R>(q, qq, ln.t, i, n);
      float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (tok < q.L && pm0 < q.P) {
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
      dl[jj][n] = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

__device__ __forceinline__ float f4_at(const float4& v, int r) {
  return r == 0 ? v.x : (r == 1 ? v.y : (r == 2 ? v.z : v.w));
}

// ---- per-mode constants in LDS --------------------------------------------------------
// Read inside the chunk loops from LDS rather than global memory: a global
// load there would wait (in-order vmcnt) behind the asynchronous u copies.
struct ModeTable {
  S5_LDS pf2* ab;      // abar (time-invariant) or lambda (time-varying)   [Ppad]
  S5_LDS float* hr;    // hrev (time-varying)                              [Ppad]
  S5_LDS float* d;     // D, zero past H (pass 2)                          [Hpad]

  // the per-step discretisation's constants of mode p (time-varying)
  __device__ __forceinline__ StepMode step_mode(int p) const { return {ld_pf2(ab + p), hr[p]}; }
};

template <bool TV>
__device__ __forceinline__ ModeTable fill_mode_table(const FusedParams& q, lds_byte* base, bool with_d) {
  ModeTable mt;
  mt.ab = reinterpret_cast<S5_LDS pf2*>(base);
  mt.hr = reinterpret_cast<S5_LDS float*>(mt.ab + q.Ppad);
  mt.d = TV ? mt.hr + q.Ppad : reinterpret_cast<S5_LDS float*>(mt.ab + q.Ppad);
  for (int p = threadIdx.x; p < q.Ppad; p += kThreads) {
    const ModeParams& mq = q.modes[p];
    if constexpr (TV) {
      st_pf2(mt.ab + p, mq.lam.x, mq.lam.y);
      mt.hr[p] = mq.hrev;
    } else {
      st_pf2(mt.ab + p, mq.abar.x, mq.abar.y);
    }
  }
  if (with_d) {
    for (int h = threadIdx.x; h < q.Hpad; h += kThreads) mt.d[h] = h < q.H && q.d != nullptr ? q.d[h] : 0.0f;
  }
  return mt;   // visible after the caller's next barrier
}

// ---- pass 1 --------------------------------------------------------------------------

// MPW: mode tiles per wave (Ppad = 64 MPW); R: tokens per stream per chunk.
template <int MPW, int R, bool TV, bool BF16, bool KEEP, int XM>
__global__ void __launch_bounds__(kThreads, 1) k_reduce(FusedParams q) {
  constexpr bool EXT = XM != 0;   // options of the extended entry point
  constexpr int NP = BF16 ? 1 : 2;
  extern __shared__ __align__(16) unsigned char smem[];
  if (q.Ppad != 64 * MPW || q.R != R) return;   // dispatch mismatch: do nothing
  const Lane ln = lane_ids();
  const int bq = blockIdx.x;
  const int b = bq / q.Q;
  const int qq = bq - b * q.Q;
  const bool bil = EXT && q.bilinear;        // bilinear per-step discretisation
  const RowMap rmap = row_map<EXT>(q, qq);     // forward or reverse time
  const LastTok lt = last_token<R>(q);
  const int cap_chunk = EXT && q.xlast != nullptr && qq == lt.qq ? lt.i : -1;   // chunk holding token L-1
  const int KS = q.Hpad >> 5;
  lds_byte* lds = (lds_byte*)smem;
  const int ut = static_cast<int>(u_tile_bytes(KS, R, BF16));
  ModeTable mt{};
  if constexpr (TV) mt = fill_mode_table<true>(q, lds + 2 * ut, false);

  BKeep<MPW, NP> bk;
  if constexpr (KEEP) load_b_keep<MPW, NP>(q, ln.w, ln.l, bk);

  cf abar[MPW][4];
  cf z[MPW][4];
  cf A[MPW][4];
#pragma unroll
  for (int jj = 0; jj < MPW; ++jj)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pm = 16 * (ln.w + kWaves * jj) + 4 * ln.g + r;
      const float2 ab = q.modes[pm].abar;
      abar[jj][r] = {ab.x, ab.y};
      z[jj][r] = {0.0f, 0.0f};
      A[jj][r] = {1.0f, 0.0f};
    }

  constexpr int NB = u_stage_blocks<R, BF16, KEEP>();
  const __amdgpu_buffer_rsrc_t ursrc = range_rsrc<BF16>(q.u, q, b, qq, rmap.rev);
  auto chunks = [&](auto vec_c) {
  constexpr bool VEC = decltype(vec_c)::value;
  float4 dl[TV ? MPW : 1][TV ? R : 1];
  if constexpr (TV) load_delta<MPW, R>(q, b, qq, 0, ln, dl);
  {
    UStage<NB> ust;
    fetch_u<R, BF16, NB, kWaves, VEC>(q, ursrc, rmap, qq, 0, ust);
    stash_u<R, BF16, NB, kWaves, !BF16>(q, ust, lds);
  }
  lds_barrier();
  for (int i = 0; i < q.nck; ++i) {
    // Delta of the next chunk is loaded before the next u tile is, so that
    // waiting for it (in-order vmcnt) never waits for the u loads
    float4 dn[TV ? MPW : 1][TV ? R : 1];
    if constexpr (TV) {
      if (i + 1 < q.nck) load_delta<MPW, R>(q, b, qq, i + 1, ln, dn);
    }
    // u tile i+1 into registers now, into LDS before the barrier
    UStage<NB> ust;
    fetch_u<R, BF16, NB, kWaves, VEC>(q, ursrc, rmap, qq, i + 1, ust);
    f32x4 acc[MPW][2][R];
    drive<MPW, R, BF16, KEEP, !BF16>(q, bk, lds + (i & 1) * ut, ln.w, ln.l, acc);
    const bool rec = cap_chunk == i;   // this chunk holds token L-1 (uniform)
#pragma unroll
    for (int jj = 0; jj < MPW; ++jj) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        cf x = z[jj][r];
        const int pmr = 16 * (ln.w + kWaves * jj) + 4 * ln.g + r;
        if constexpr (TV) {
          const StepMode sm = mt.step_mode(pmr);
          cf Ar = A[jj][r];
#pragma unroll
          for (int n = 0; n < R; ++n) {
            const cf am1 = disc_am1(bil, sm, f4_at(dl[jj][n], r));
            x = step_am1(am1, x, {acc[jj][0][n][r], acc[jj][1][n][r]});
            Ar = cfma(am1, Ar, Ar);
            if (rec && n == lt.n && ln.t == lt.t) record_partial(q, b, pmr, x, Ar);
          }
          A[jj][r] = Ar;
        } else {
#pragma unroll
          for (int n = 0; n < R; ++n) {
            x = cfma(abar[jj][r], x, {acc[jj][0][n][r], acc[jj][1][n][r]});
            if (rec && n == lt.n && ln.t == lt.t) record_partial(q, b, pmr, x, cf{1.0f, 0.0f});
          }
        }
        z[jj][r] = x;
      }
    }
    // u tile i+1 into the buffer that drive(i-1) read before the last barrier
    __builtin_amdgcn_sched_barrier(0);   // keep the stash (and its wait) after this chunk's work
    stash_u<R, BF16, NB, kWaves, !BF16>(q, ust, lds + ((i + 1) & 1) * ut);
    lds_barrier();
    if constexpr (TV) {
#pragma unroll
      for (int jj = 0; jj < MPW; ++jj)
#pragma unroll
        for (int n = 0; n < R; ++n) dl[jj][n] = dn[jj][n];
    }
  }
  };
  if (u_rows_vectorized(q.H, BF16)) {
    chunks(std::true_type{});
  } else {
    chunks(std::false_type{});
  }

  // stream aggregates, then the range total over the 16 streams
#pragma unroll
  for (int jj = 0; jj < MPW; ++jj) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pm = 16 * (ln.w + kWaves * jj) + 4 * ln.g + r;
      const size_t si = (static_cast<size_t>(bq) * kStreams + ln.t) * q.Ppad + pm;
      q.sagg[si] = make_float2(z[jj][r].re, z[jj][r].im);
      cf At;
      if constexpr (TV) {
        q.sagg_a[si] = make_float2(A[jj][r].re, A[jj][r].im);
        At = A[jj][r];
      } else {
        const float2 as = q.modes[pm].aseg;
        At = {as.x, as.y};
      }
      cf Xt = z[jj][r];
      row_scan(At, Xt);
      if (ln.t == kStreams - 1) {
        const size_t ti = static_cast<size_t>(bq) * q.Ppad + pm;
        q.tot[ti] = make_float2(Xt.re, Xt.im);
        q.tot_a[ti] = make_float2(At.re, At.im);
      }
    }
  }
}

// ---- pass 1 with eight waves (register-resident B_bar) --------------------------------
// Wave w (0..7) owns mode tiles j = w + 8 jj (j < 4 MPW): half the weights
// and states of a four-wave split, so two waves fit on each SIMD and one
// wave's scan overlaps the other's MFMAs. All waves share each u tile.
// KS: the drive's K-steps (Hpad = 32 KS, at most 4), so that no MFMA multiplies padding.
// XM = 2 (time-invariant, forward time): the bidirectional form's pass 1,
// which also sums each stream's backward-scan aggregate from the same drive:
// the backward scan enters a stream at its last token, so its state at the
// stream's first token, from a zero start, is sum_k abar^k b_k over the
// stream's tokens k = 0, 1, ... (with transition abar^Lseg, as forward).
template <int MPW, int KS, int R, bool TV, bool BF16, int XM>
__global__ void __launch_bounds__(2 * kThreads, 1) k_reduce_ws(FusedParams q) {
  constexpr bool EXT = XM != 0;   // options of the extended entry point
  constexpr bool BOTH = XM == 2;
  static_assert(!BOTH || !TV, "the backward scan is time-invariant");
  constexpr int NP = BF16 ? 1 : 2;
  constexpr int NW8 = 2 * kWaves;
  constexpr int NT = 4 * MPW;                 // mode tiles
  constexpr int M8 = (NT + NW8 - 1) / NW8;    // tiles per wave, at most
  extern __shared__ __align__(16) unsigned char smem[];
  if (q.Ppad != 64 * MPW || q.Hpad != 32 * KS || q.R != R || q.nck % reduce_group(BF16, TV, KS) != 0) return;   // dispatch mismatch
  Lane ln = lane_ids();
  ln.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & (NW8 - 1);   // 0..7
  const int bq = blockIdx.x;
  const int b = bq / q.Q;
  const int qq = bq - b * q.Q;
  const bool bil = EXT && q.bilinear;        // bilinear per-step discretisation
  const RowMap rmap = row_map<EXT>(q, qq);     // forward or reverse time
  const LastTok lt = last_token<R>(q);
  const int cap_chunk = EXT && q.xlast != nullptr && qq == lt.qq ? lt.i : -1;   // chunk holding token L-1
  constexpr int ut = static_cast<int>(u_tile_bytes(KS, R, BF16));
  lds_byte* lds = (lds_byte*)smem;
  const ModeTable mt = fill_mode_table<TV>(q, lds + 2 * reduce_group(BF16, TV, KS) * ut, false);

  // B_bar fragments of the wave's tiles, all K-steps: [s][m][cc][pl]
  bf16x8 bw[KS][M8][2][NP];
  {
    const int nb = (q.Ppad / 16) * 2 * KS * 64;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int m = 0; m < M8; ++m)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int pl = 0; pl < NP; ++pl) {
            const int j = ln.w + NW8 * m;
            bw[s][m][cc][pl] = j < NT
                ? as_bf16x8(ldg16(q.bpack + pl * nb + ((j * 2 + cc) * KS + s) * 64 + ln.l))
                : as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
          }
  }
  cf z[M8][4];
  cf A[TV ? M8 : 1][4];
#pragma unroll
  for (int m = 0; m < M8; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[m][r] = {0.0f, 0.0f};
      if constexpr (TV) A[m][r] = {1.0f, 0.0f};
    }
  // backward aggregates (BOTH): sum of abar^k b_k and the running power abar^k
  cf zb[BOTH ? M8 : 1][4], pw[BOTH ? M8 : 1][4];
  if constexpr (BOTH) {
#pragma unroll
    for (int m = 0; m < M8; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        zb[m][r] = {0.0f, 0.0f};
        pw[m][r] = {1.0f, 0.0f};
      }
  }

  constexpr int NB = (KS * R * (BF16 ? 1 : 2) + NW8 - 1) / NW8;   // u staging blocks per wave
  constexpr int G = reduce_group(BF16, TV, KS);   // chunks per barrier (nck is a multiple of G)
  const __amdgpu_buffer_rsrc_t ursrc = range_rsrc<BF16>(q.u, q, b, qq, rmap.rev);

  // Delta of chunk i (time-varying)
  auto delta = [&](int i, float4 (&dl)[TV ? M8 : 1][TV ? R : 1]) __attribute__((always_inline)) {
    if constexpr (TV) {
#pragma unroll
      for (int m = 0; m < M8; ++m) {
        const int pm0 = 16 * (ln.w + NW8 * m) + 4 * ln.g;
#pragma unroll
        for (int n = 0; n < R; ++n) {
          const int tok = tok_of<R>(q, qq, ln.t, i, n);
          float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
          if (tok < q.L && pm0 < q.P) {
            const float* dp = q.delta + range_row0(q, b, qq) * q.P +
                              (rel_row<R>(q, ln.t, i, n) * static_cast<uint32_t>(q.P) + pm0);
            if ((q.P & 3) == 0) {
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
  };
  // drive (B_bar u) of one chunk from its u tile ub
  auto mma = [&](const lds_byte* ub, f32x4 (&acc)[M8][2][R]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < M8; ++m)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int n = 0; n < R; ++n) acc[m][cc][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8 uf[NP][R];
      get_u<R, BF16, !BF16>(ub, s, ln.l, uf);
#pragma unroll
      for (int m = 0; m < M8; ++m) {
        // waves past the last tile (NT not a multiple of 8) issue no MFMAs
        if ((NT % NW8) != 0 && ln.w + NW8 * m >= NT) continue;   // wave-uniform
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int n = 0; n < R; ++n) {
            acc[m][cc][n] = mfma(bw[s][m][cc][0], uf[0][n], acc[m][cc][n]);
            if constexpr (NP == 2) {
              acc[m][cc][n] = mfma(bw[s][m][cc][0], uf[1][n], acc[m][cc][n]);
              acc[m][cc][n] = mfma(bw[s][m][cc][1], uf[0][n], acc[m][cc][n]);
            }
          }
      }
    }
  };
  // the stream states through one chunk's drive; rec: the chunk holding token
  // L-1. Time-invariant: a separate copy for that chunk (rec_c), so that the
  // others test nothing per step; time-varying: a runtime test (rec_rt), which
  // measured faster there than the second copy.
  auto scan = [&](auto rec_c, bool rec_rt, const f32x4 (&acc)[M8][2][R],
                  const float4 (&dl)[TV ? M8 : 1][TV ? R : 1]) __attribute__((always_inline)) {
    const bool rec = decltype(rec_c)::value || rec_rt;
#pragma unroll
    for (int m = 0; m < M8; ++m) {
      const int j = ln.w + NW8 * m;
      if (j >= NT) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pm = 16 * j + 4 * ln.g + r;
        cf x = z[m][r];
        if constexpr (TV) {
          const StepMode sm = mt.step_mode(pm);
          cf Ar = A[m][r];
#pragma unroll
          for (int n = 0; n < R; ++n) {
            const cf am1 = disc_am1(bil, sm, f4_at(dl[m][n], r));
            x = step_am1(am1, x, {acc[m][0][n][r], acc[m][1][n][r]});
            Ar = cfma(am1, Ar, Ar);
            if (rec && n == lt.n && ln.t == lt.t) record_partial(q, b, pm, x, Ar);
          }
          A[m][r] = Ar;
        } else {
          const cf ab = ld_pf2(mt.ab + pm);
#pragma unroll
          for (int n = 0; n < R; ++n) {
            const cf bu = {acc[m][0][n][r], acc[m][1][n][r]};
            x = cfma(ab, x, bu);
            if constexpr (BOTH) {
              zb[m][r] = cfma(pw[m][r], bu, zb[m][r]);
              pw[m][r] = cmul(pw[m][r], ab);
            }
            if (rec && n == lt.n && ln.t == lt.t) record_partial(q, b, pm, x, cf{1.0f, 0.0f});
          }
        }
        z[m][r] = x;
      }
    }
  };

  // Chunks in groups of G: group gi's u tiles sit in LDS half gi & 1 (G tiles
  // each); the next group's tiles are loaded into registers at the top of a
  // group and stored to the other half after its work, then one barrier.
  // Between barriers the waves drift apart, so one wave's scan overlaps
  // another's MFMAs, and a load has a whole group of work to arrive.
  auto groups = [&](auto vec_c) {
    constexpr bool VEC = decltype(vec_c)::value;
    {
      UStage<NB> ust[G];
#pragma unroll
      for (int c = 0; c < G; ++c) fetch_u<R, BF16, NB, NW8, VEC>(q, ursrc, rmap, qq, c, ust[c]);
#pragma unroll
      for (int c = 0; c < G; ++c) stash_u<R, BF16, NB, NW8, !BF16>(q, ust[c], lds + c * ut);
    }
    lds_barrier();   // mode table, u tiles of group 0
    // Delta of the chunk being scanned (time-varying), loaded a chunk ahead:
    // waiting for a global load issued right before its use exposed its
    // whole latency on every chunk
    float4 dl[TV ? M8 : 1][TV ? R : 1];
    delta(0, dl);
    for (int i0 = 0; i0 < q.nck; i0 += G) {
      const int half = (i0 / G) & 1;
      UStage<NB> ust[G];
#pragma unroll
      for (int c = 0; c < G; ++c) fetch_u<R, BF16, NB, NW8, VEC>(q, ursrc, rmap, qq, i0 + G + c, ust[c]);
      // a real loop: unrolled, the compiler hoists all G chunks' MFMAs ahead
      // of the scans and runs out of registers
#pragma unroll 1
      for (int c = 0; c < G; ++c) {
        f32x4 acc[M8][2][R];
        float4 dnext[TV ? M8 : 1][TV ? R : 1];
        delta(i0 + c + 1, dnext);
        mma(lds + (half * G + c) * ut, acc);
        // the MFMAs as one burst, then the discretisation and scan: the two
        // waves of a SIMD alternate between the matrix core and the vector
        // unit (interleaving them in both waves made each wave's vector work
        // wait behind the other wave's MFMAs)
        if constexpr (TV) __builtin_amdgcn_sched_barrier(0);
        if constexpr (TV) {
          scan(std::false_type{}, EXT && cap_chunk == i0 + c, acc, dl);
        } else if (EXT && cap_chunk == i0 + c) {
          scan(std::true_type{}, false, acc, dl);
        } else {
          scan(std::false_type{}, false, acc, dl);
        }
        if constexpr (TV) {
#pragma unroll
          for (int m = 0; m < M8; ++m)
#pragma unroll
            for (int n = 0; n < R; ++n) dl[m][n] = dnext[m][n];
        }
      }
      // the next group's tiles into the other half (read by the previous group
      // before the last barrier)
      __builtin_amdgcn_sched_barrier(0);   // keep the stash (and its wait) after the group's work
#pragma unroll
      for (int c = 0; c < G; ++c) stash_u<R, BF16, NB, NW8, !BF16>(q, ust[c], lds + ((1 - half) * G + c) * ut);
      lds_barrier();
    }
  };
  if (u_rows_vectorized(q.H, BF16)) {
    groups(std::true_type{});
  } else {
    groups(std::false_type{});
  }

  // stream aggregates, then the range total over the 16 streams
  float2 aseg[TV ? 1 : M8][4];   // loaded together (one round of latency)
  if constexpr (!TV) {
#pragma unroll
    for (int m = 0; m < M8; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = ln.w + NW8 * m;
        aseg[m][r] = j < NT ? q.modes[16 * j + 4 * ln.g + r].aseg : make_float2(0.0f, 0.0f);
      }
  }
#pragma unroll
  for (int m = 0; m < M8; ++m) {
    const int j = ln.w + NW8 * m;
    if (j >= NT) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pm = 16 * j + 4 * ln.g + r;
      const size_t si = (static_cast<size_t>(bq) * kStreams + ln.t) * q.Ppad + pm;
      q.sagg[si] = make_float2(z[m][r].re, z[m][r].im);
      cf At;
      if constexpr (TV) {
        q.sagg_a[si] = make_float2(A[m][r].re, A[m][r].im);
        At = A[m][r];
      } else {
        At = {aseg[m][r].x, aseg[m][r].y};
      }
      cf Xt = z[m][r];
      cf Ab = At;
      row_scan(At, Xt);
      if (ln.t == kStreams - 1) {
        const size_t ti = static_cast<size_t>(bq) * q.Ppad + pm;
        q.tot[ti] = make_float2(Xt.re, Xt.im);
        q.tot_a[ti] = make_float2(At.re, At.im);
      }
      if constexpr (BOTH) {
        // the backward pass's range Q-1-qq, stream 15-t; its range total
        // combines the streams in its own order: lanes mirrored, then the scan
        const size_t bqm = static_cast<size_t>(b) * q.Q + (q.Q - 1 - qq);
        const size_t sib = (bqm * kStreams + (kStreams - 1 - ln.t)) * q.Ppad + pm;
        q.sagg_b[sib] = make_float2(zb[m][r].re, zb[m][r].im);
        cf Xb = {row_mirror(zb[m][r].re), row_mirror(zb[m][r].im)};
        row_scan(Ab, Xb);
        if (ln.t == kStreams - 1) {
          q.tot_b[bqm * q.Ppad + pm] = make_float2(Xb.re, Xb.im);
          q.tot_a_b[bqm * q.Ppad + pm] = make_float2(Ab.re, Ab.im);
        }
      }
    }
  }
}

// ---- pass 2 --------------------------------------------------------------------------

template <int MPW, int NP>
struct CKeep {
  bf16x8 f[kKeepHT][4 * MPW][NP];
};

// D u feedthrough of the readout lane's 4 outputs y[tok(t, i, n)][h0..h0+3],
// h0 = 16 ht + 4 g, taken from u tile i in LDS (zero past H and L): block
// (ht/2, n), lane t + 16 (2 (ht&1) + g/2), elements 4 (g&1)..+3.
template <int R, bool BF16>
__device__ __forceinline__ void u_for_y(const lds_byte* ub, int ht, int n, const Lane& ln, float (&uv)[4]) {
  const int s = ht >> 1;
  const int lp = ln.t + 16 * (2 * (ht & 1) + (ln.g >> 1));
  if constexpr (BF16) {
    const uint2 p = lds_ld<uint2>(ub + (s * R + n) * kBlock + lp * 16 + 8 * (ln.g & 1));
    uv[0] = __uint_as_float(p.x << 16);
    uv[1] = __uint_as_float(p.x & 0xffff0000u);
    uv[2] = __uint_as_float(p.y << 16);
    uv[3] = __uint_as_float(p.y & 0xffff0000u);
  } else {
    const float4 p = lds_ld<float4>(ub + ((s * R + n) * 2 + (ln.g & 1)) * kBlock + lp * 16);
    uv[0] = p.x; uv[1] = p.y; uv[2] = p.z; uv[3] = p.w;
  }
}

// y = acc + D u for 4 consecutive features h0..h0+3 of one row (row offset
// roff, in elements, inside the range descriptor yr; y stored as bf16 when
// BF16, else float32), plus (ep.accum) the float32 values at the same place
// of descriptor yo, then the GELU form the epilogue asks for; bf16 rounding by
// the hardware conversion (round to nearest even). Rows past the sequence end
// fall outside the descriptor and features >= H get an offset beyond it, so
// the hardware drops those writes. VEC: H % 4 == 0, one vector store.
template <bool BF16, bool VEC>
__device__ __forceinline__ void store_y(__amdgpu_buffer_rsrc_t yr, int roff, int h0, int H, const f32x4& acc,
                                        const float4& d4, const float (&uv)[4], const Epi& ep,
                                        __amdgpu_buffer_rsrc_t yo) {
  constexpr int esz = BF16 ? 2 : 4;
  f32x4 yv = {fmaf(d4.x, uv[0], acc[0]), fmaf(d4.y, uv[1], acc[1]), fmaf(d4.z, uv[2], acc[2]),
              fmaf(d4.w, uv[3], acc[3])};
  if constexpr (VEC) {
    const int off = h0 < H ? (roff + h0) * esz : kBufferOOB;
    if (ep.accum) {
      const int offo = h0 < H ? (roff + h0) * 4 : kBufferOOB;
      yv += __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(yo, offo, 0, 0));
    }
    if (ep.gelu) {
      if (ep.tanh_form) {
#pragma unroll
        for (int m = 0; m < 4; ++m) yv[m] = gelu_tanh(yv[m]);
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) yv[m] = gelu_erf(yv[m]);
      }
    }
    if constexpr (BF16) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, __builtin_convertvector(yv, bf16x4)), yr, off,
                                            0, 0);
    } else {
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, yv), yr, off, 0, 0);
    }
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int off = h0 + m < H ? (roff + h0 + m) * esz : kBufferOOB;
      if (ep.accum) {
        const int offo = h0 + m < H ? (roff + h0 + m) * 4 : kBufferOOB;
        yv[m] += __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(yo, offo, 0, 0));
      }
      if (ep.gelu) yv[m] = ep.tanh_form ? gelu_tanh(yv[m]) : gelu_erf(yv[m]);
      if constexpr (BF16) {
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, static_cast<__bf16>(yv[m])), yr, off,
                                              0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv[m]), yr, off, 0, 0);
      }
    }
  }
}

__device__ __forceinline__ void load_d(const FusedParams& q, int h0, float (&dv)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) dv[r] = h0 + r < q.H && q.d != nullptr ? q.d[h0 + r] : 0.0f;
}

// readout operand fragments of K-step s from the x tile: [plane][n]
template <int R, int NP>
__device__ __forceinline__ void get_x(const lds_byte* xb, int K2, int s, int l, bf16x8 (&xf)[NP][R]) {
#pragma unroll
  for (int pl = 0; pl < NP; ++pl)
#pragma unroll
    for (int n = 0; n < R; ++n)
      xf[pl][n] = as_bf16x8(lds_ld<uint4>(xb + ((pl * K2 + s) * R + n) * kBlock + l * 16));
}

template <int R, int NP>
__device__ __forceinline__ void mfma_read(const bf16x8 (&c)[NP], const bf16x8 (&xf)[NP][R], f32x4 (&y)[R]) {
#pragma unroll
  for (int n = 0; n < R; ++n) {
    y[n] = mfma(c[0], xf[0][n], y[n]);
    if constexpr (NP == 2) {
      y[n] = mfma(c[0], xf[1][n], y[n]);
      y[n] = mfma(c[1], xf[0][n], y[n]);
    }
  }
}

template <int MPW, int NP>
__device__ __forceinline__ void load_c_step(const FusedParams& q, int ht, int s, int l, bf16x8 (&c)[NP]) {
  constexpr int K2 = 4 * MPW;
  const int nc = (q.Hpad / 16) * K2 * 64;
#pragma unroll
  for (int pl = 0; pl < NP; ++pl) c[pl] = as_bf16x8(ldg16(q.cpack + pl * nc + (ht * K2 + s) * 64 + l));
}

// y for chunk i of the workgroup's streams from the x tile and u tile in LDS
// (y stored as bf16 when YB, else float32; yo: the float32 values added when
// ep.accum)
template <int MPW, int R, bool BF16, bool KEEP, bool VEC, bool YB>
__device__ __forceinline__ void readout(const FusedParams& q, __amdgpu_buffer_rsrc_t yr, const RowMap& rm,
                                        const Epi& ep,
                                        const CKeep<MPW, BF16 ? 1 : 2>& ck, const S5_LDS float* s_d,
                                        const lds_byte* xb, const lds_byte* ub, int i, const Lane& ln,
                                        __amdgpu_buffer_rsrc_t yo) {
  constexpr int NP = BF16 ? 1 : 2;
  constexpr int K2 = 4 * MPW;
  const int HT = q.Hpad >> 4;
  const int HTv = (q.H + 15) >> 4;   // h-tiles holding a feature < H
  if constexpr (KEEP) {
    f32x4 yacc[kKeepHT][R];
#pragma unroll
    for (int e = 0; e < kKeepHT; ++e)
#pragma unroll
      for (int n = 0; n < R; ++n) yacc[e][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // branch-free: C' fragments of h-tiles >= HT are zero
#pragma unroll
    for (int s = 0; s < K2; ++s) {
      bf16x8 xf[NP][R];
      get_x<R, NP>(xb, K2, s, ln.l, xf);
#pragma unroll
      for (int e = 0; e < kKeepHT; ++e) mfma_read<R, NP>(ck.f[e][s], xf, yacc[e]);
    }
#pragma unroll
    for (int e = 0; e < kKeepHT; ++e) {
      const int ht = ln.w + kWaves * e;
      if (ht >= HTv) continue;   // wave-uniform
      const int h0 = 16 * ht + 4 * ln.g;
      const float4 d4 = lds_ld<float4>(reinterpret_cast<const lds_byte*>(s_d + h0));
#pragma unroll
      for (int n = 0; n < R; ++n) {
        float uv[4];
        u_for_y<R, BF16>(ub, ht, n, ln, uv);
        store_y<YB, VEC>(yr, rm(rel_row<R>(q, ln.t, i, n)) * q.H, h0, q.H, yacc[e][n], d4, uv, ep, yo);
      }
    }
  } else {
    // C' streamed from L2: h-tiles (ht0, ht0 + 4), K-steps in batches of G, one batch ahead
    constexpr int G = BF16 ? 4 : 2;
    static_assert(K2 % G == 0, "readout K-steps must split into whole batches");
    for (int ht0 = ln.w; ht0 < HT; ht0 += 2 * kWaves) {
      const bool has1 = ht0 + kWaves < HT;
      f32x4 yacc[2][R];
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int n = 0; n < R; ++n) yacc[e][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      bf16x8 cb[G][2][NP];
#pragma unroll
      for (int kk = 0; kk < G; ++kk) {
        load_c_step<MPW, NP>(q, ht0, kk, ln.l, cb[kk][0]);
        if (has1) load_c_step<MPW, NP>(q, ht0 + kWaves, kk, ln.l, cb[kk][1]);
      }
#pragma unroll 1
      for (int s0 = 0; s0 < K2; s0 += G) {
        bf16x8 cn[G][2][NP];
        if (s0 + G < K2) {
#pragma unroll
          for (int kk = 0; kk < G; ++kk) {
            load_c_step<MPW, NP>(q, ht0, s0 + G + kk, ln.l, cn[kk][0]);
            if (has1) load_c_step<MPW, NP>(q, ht0 + kWaves, s0 + G + kk, ln.l, cn[kk][1]);
          }
        }
#pragma unroll
        for (int kk = 0; kk < G; ++kk) {
          bf16x8 xf[NP][R];
          get_x<R, NP>(xb, K2, s0 + kk, ln.l, xf);
          mfma_read<R, NP>(cb[kk][0], xf, yacc[0]);
          if (has1) mfma_read<R, NP>(cb[kk][1], xf, yacc[1]);
        }
        if (s0 + G < K2) {
#pragma unroll
          for (int kk = 0; kk < G; ++kk)
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
              for (int pl = 0; pl < NP; ++pl) cb[kk][e][pl] = cn[kk][e][pl];
        }
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int ht = ht0 + kWaves * e;
        if ((e == 1 && !has1) || ht >= HTv) continue;
        const int h0 = 16 * ht + 4 * ln.g;
        float dv[4];
        load_d(q, h0, dv);
#pragma unroll
        for (int n = 0; n < R; ++n) {
          float uv[4];
          u_for_y<R, BF16>(ub, ht, n, ln, uv);
          store_y<YB, VEC>(yr, rm(rel_row<R>(q, ln.t, i, n)) * q.H, h0, q.H, yacc[e][n],
                           make_float4(dv[0], dv[1], dv[2], dv[3]), uv, ep, yo);
        }
      }
    }
  }
}

// y of chunk i from the register-weight readout's accumulators: feedthrough
// from u tile i in LDS and D from the LDS table (h-tiles past H: the stores
// fall outside the descriptor and are dropped)
// y values already in memory for the readout lane's outputs of chunk i (the
// backward scan adds to them), raw: 4 bf16 or 4 floats per (h-tile, step),
// zeros outside the range or past H. Loaded a chunk ahead of their use.
template <bool BF16>
struct YOld {
  std::conditional_t<BF16, uint2, uint4> v[kKeepHT][2];
};

template <int R, bool BF16, bool VEC>
__device__ __forceinline__ void load_y_old(const FusedParams& q, __amdgpu_buffer_rsrc_t yr, const RowMap& rm, int i,
                                           const Lane& ln, YOld<BF16>& o) {
  static_assert(R <= 2, "two steps per chunk at most");
  constexpr int esz = BF16 ? 2 : 4;
#pragma unroll
  for (int e = 0; e < kKeepHT; ++e) {
    const int h0 = 16 * (ln.w + kWaves * e) + 4 * ln.g;
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
        uint32_t w[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int off = h0 + m < q.H ? (roff + h0 + m) * esz : kBufferOOB;
          w[m] = BF16 ? static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(yr, off, 0, 0))
                      : __builtin_amdgcn_raw_buffer_load_b32(yr, off, 0, 0);
        }
        if constexpr (BF16) {
          o.v[e][n] = make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
        } else {
          o.v[e][n] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    }
  }
}

template <bool BF16>
__device__ __forceinline__ f32x4 y_old_f32(const std::conditional_t<BF16, uint2, uint4>& v) {
  if constexpr (BF16) {
    return f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                 __uint_as_float(v.y & 0xffff0000u)};
  } else {
    return f32x4{__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
  }
}

// ACC: add `old` (float32 values already in memory, loaded a chunk ahead) to
// the sums; y stored as bf16 when YB, else float32
template <int R, bool BF16, bool VEC, bool ACC, bool YB>
__device__ __forceinline__ void readout_store(const FusedParams& q, __amdgpu_buffer_rsrc_t yr, const RowMap& rm,
                                              const Epi& ep,
                                              const float4 (&dk)[kKeepHT], const f32x4 (&yacc)[kKeepHT][R],
                                              const lds_byte* ub, int i, const Lane& ln,
                                              const YOld<false>* old) {
  float uv[kKeepHT][R][4];
#pragma unroll
  for (int e = 0; e < kKeepHT; ++e)
#pragma unroll
    for (int n = 0; n < R; ++n) u_for_y<R, BF16>(ub, ln.w + kWaves * e, n, ln, uv[e][n]);
#pragma unroll
  for (int e = 0; e < kKeepHT; ++e) {
    const int h0 = 16 * (ln.w + kWaves * e) + 4 * ln.g;
#pragma unroll
    for (int n = 0; n < R; ++n) {
      f32x4 a = yacc[e][n];
      if constexpr (ACC) a += y_old_f32<false>(old->v[e][n]);
      store_y<YB, VEC>(yr, rm(rel_row<R>(q, ln.t, i, n)) * q.H, h0, q.H, a, dk[e], uv[e][n],
                       Epi{false, ep.gelu, ep.tanh_form}, yr);
    }
  }
}

template <int MPW, int R, bool TV, bool BF16, bool KEEP, int XM>
__global__ void __launch_bounds__(kThreads, 1) k_scan(FusedParams q) {
  constexpr bool EXT = XM != 0;   // options of the extended entry point
  constexpr int NP = BF16 ? 1 : 2;
  constexpr int K2 = 4 * MPW;
  extern __shared__ __align__(16) unsigned char smem[];
  if (q.Ppad != 64 * MPW || q.R != R) return;   // dispatch mismatch: do nothing
  const Lane ln = lane_ids();
  const int bq = blockIdx.x;
  const int b = bq / q.Q;
  const int qq = bq - b * q.Q;
  const bool bil = EXT && q.bilinear;        // bilinear per-step discretisation
  const RowMap rmap = row_map<XM == 3>(q, qq);   // forward or reverse time
  const int KS = q.Hpad >> 5;
  const int ut = static_cast<int>(u_tile_bytes(KS, R, BF16));
  const int xt = static_cast<int>(x_tile_bytes(K2, R, BF16));
  // u tile i lives in u buffer i % 3 from its load (two chunks ahead) to the
  // feedthrough of its readout; x tile i in x buffer i % 2
  lds_byte* lds = (lds_byte*)smem;
  lds_byte* xlds = lds + 3 * ut;
  // register-weight instances read per-mode constants and D from LDS
  ModeTable mt{};
  if constexpr (KEEP) mt = fill_mode_table<TV>(q, lds + 3 * ut + 2 * xt, true);

  BKeep<MPW, NP> bk;
  CKeep<MPW, NP> ck;
  if constexpr (KEEP) {
    load_b_keep<MPW, NP>(q, ln.w, ln.l, bk);
    const int HT = q.Hpad >> 4;
#pragma unroll
    for (int e = 0; e < kKeepHT; ++e) {
      const int ht = ln.w + kWaves * e;
#pragma unroll
      for (int s = 0; s < K2; ++s) {
        if (ht < HT) {
          load_c_step<MPW, NP>(q, ht, s, ln.l, ck.f[e][s]);
        } else {
#pragma unroll
          for (int pl = 0; pl < NP; ++pl) ck.f[e][s][pl] = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
        }
      }
    }
  }

  // ---- state entering each stream ----
  // carry into the range: the totals of the sequence's earlier ranges, folded in
  // order; it waits in LDS (the second x buffer is not written before the loop).
  S5_LDS pf2* s_c0 = reinterpret_cast<S5_LDS pf2*>(xlds + xt);
  if (ln.tid < q.Ppad) {
    cf c = {0.0f, 0.0f};   // the state before step 0: zero, or the caller's
    if (EXT && q.x0 != nullptr && ln.tid < q.P) {
      const float2 v = q.x0[static_cast<size_t>(b) * q.P + ln.tid];
      c = {v.x, v.y};
    }
    const size_t base = static_cast<size_t>(b) * q.Q * q.Ppad + ln.tid;
    // time-invariant: the range power from the float64 packing (as range_carry)
    cf ar = {0.0f, 0.0f};
    if constexpr (!TV) {
      const float2 v = q.modes[ln.tid].arange;
      ar = {v.x, v.y};
    }
    constexpr int kBatch = 8;
    for (int q0 = 0; q0 < qq; q0 += kBatch) {
      cf xs[kBatch], as[kBatch];
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        if (q0 + e < qq) {
          const float2 xv = q.tot[base + static_cast<size_t>(q0 + e) * q.Ppad];
          xs[e] = {xv.x, xv.y};
          if constexpr (TV) {
            const float2 av = q.tot_a[base + static_cast<size_t>(q0 + e) * q.Ppad];
            as[e] = {av.x, av.y};
          } else {
            as[e] = ar;
          }
        }
      }
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        if (q0 + e < qq) c = cfma(as[e], c, xs[e]);
      }
    }
    st_pf2(s_c0 + ln.tid, c.re, c.im);
  }
  lds_barrier();

  cf abar[KEEP ? 1 : MPW][4];   // register copy when the table is not in LDS
  cf st[MPW][4];
#pragma unroll
  for (int jj = 0; jj < MPW; ++jj) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pm = 16 * (ln.w + kWaves * jj) + 4 * ln.g + r;
      const ModeParams& mq = q.modes[pm];
      if constexpr (!KEEP) abar[jj][r] = {mq.abar.x, mq.abar.y};
      const size_t si = (static_cast<size_t>(bq) * kStreams + ln.t) * q.Ppad + pm;
      const float2 xv = q.sagg[si];
      cf X = {xv.x, xv.y};
      cf A;
      if constexpr (TV) {
        const float2 av = q.sagg_a[si];
        A = {av.x, av.y};
      } else {
        A = {mq.aseg.x, mq.aseg.y};
      }
      row_scan(A, X);
      const cf Ae = {row_shr<1>(A.re, 1.0f), row_shr<1>(A.im, 0.0f)};
      const cf Xe = {row_shr<1>(X.re, 0.0f), row_shr<1>(X.im, 0.0f)};
      st[jj][r] = cfma(Ae, ld_pf2(s_c0 + pm), Xe);
    }
  }
  if (EXT && q.xlast != nullptr) {
    const LastTok lt = last_token<R>(q);
    if (qq == lt.qq) write_final_state<R, MPW, TV>(q, b, lt, ln, st);
  }

  // ---- chunk pipeline ----
  constexpr int NB = u_stage_blocks<R, BF16, KEEP>();
  const __amdgpu_buffer_rsrc_t ursrc = range_rsrc<BF16>(q.u, q, b, qq, rmap.rev);
  const __amdgpu_buffer_rsrc_t yrsrc = y_rsrc<XM, BF16>(q, b, qq, rmap.rev);
  const __amdgpu_buffer_rsrc_t yorsrc = XM == 3 ? range_rsrc<false>(q.yp, q, b, qq, rmap.rev) : yrsrc;
  auto chunks = [&](auto vec_c) {
  constexpr bool VEC = decltype(vec_c)::value;
  {
    UStage<NB> ust;
    fetch_u<R, BF16, NB, kWaves, VEC>(q, ursrc, rmap, qq, 0, ust);
    stash_u<R, BF16, NB, kWaves>(q, ust, lds);
    fetch_u<R, BF16, NB, kWaves, VEC>(q, ursrc, rmap, qq, 1, ust);
    stash_u<R, BF16, NB, kWaves>(q, ust, lds + ut);
  }
  lds_barrier();
  float4 dl[TV ? MPW : 1][TV ? R : 1];
  if constexpr (TV) load_delta<MPW, R>(q, b, qq, 0, ln, dl);
  f32x4 acc[MPW][2][R];
  drive<MPW, R, BF16, KEEP>(q, bk, lds, ln.w, ln.l, acc);

  // scan of mode group (jj, r) of the chunk in acc, in place: acc becomes x
  auto scan_group = [&](int jj, int r) {
    cf x = st[jj][r];
    if constexpr (TV) {
      const int pm = 16 * (ln.w + kWaves * jj) + 4 * ln.g + r;
      StepMode sm;
      if constexpr (KEEP) {
        sm = mt.step_mode(pm);
      } else {
        const ModeParams& mq = q.modes[pm];
        sm = {{mq.lam.x, mq.lam.y}, mq.hrev};
      }
#pragma unroll
      for (int n = 0; n < R; ++n) {
        x = step_am1(disc_am1(bil, sm, f4_at(dl[jj][n], r)), x, {acc[jj][0][n][r], acc[jj][1][n][r]});
        acc[jj][0][n][r] = x.re;
        acc[jj][1][n][r] = x.im;
      }
    } else {
      cf ab;
      if constexpr (KEEP) {
        ab = ld_pf2(mt.ab + 16 * (ln.w + kWaves * jj) + 4 * ln.g + r);
      } else {
        ab = abar[jj][r];
      }
#pragma unroll
      for (int n = 0; n < R; ++n) {
        x = cfma(ab, x, {acc[jj][0][n][r], acc[jj][1][n][r]});
        acc[jj][0][n][r] = x.re;
        acc[jj][1][n][r] = x.im;
      }
    }
    st[jj][r] = x;
  };
  // x tile blocks (mode tile j = w + 4 jj, n), lane (t, g): modes 16 j + 4 g + r, parts interleaved
  auto write_x = [&](int jj, lds_byte* xb) {
#pragma unroll
    for (int n = 0; n < R; ++n) {
      float v[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[2 * r] = acc[jj][0][n][r];
        v[2 * r + 1] = acc[jj][1][n][r];
      }
      const int blk = (ln.w + kWaves * jj) * R + n;
      uint4 hi, lo;
      put_frag(v, &hi, BF16 ? nullptr : &lo);
      lds_st<uint4>(xb + blk * kBlock + ln.l * 16, hi);
      if constexpr (!BF16) lds_st<uint4>(xb + (K2 * R + blk) * kBlock + ln.l * 16, lo);
    }
  };

  {
    int ui = 0;   // i % 3
    for (int i = 0; i < q.nck; ++i) {
      const int ui1 = ui == 2 ? 0 : ui + 1;
#pragma unroll
      for (int jj = 0; jj < MPW; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) scan_group(jj, r);
      lds_byte* xb = xlds + (i & 1) * xt;
#pragma unroll
      for (int jj = 0; jj < MPW; ++jj) write_x(jj, xb);
      lds_barrier();   // x tile i and u tile i+1 complete
      // Delta of chunk i+1 is loaded before u tile i+2, so that waiting for it
      // (in-order vmcnt) never waits for the u loads
      if constexpr (TV) {
        if (i + 1 < q.nck) load_delta<MPW, R>(q, b, qq, i + 1, ln, dl);
      }
      // u tile i+2 into registers now, into LDS after the drive: into the
      // buffer of tile i-1, whose last readers (drive(i-1), readout(i-1))
      // finished before the previous barrier
      UStage<NB> ust;
      fetch_u<R, BF16, NB, kWaves, VEC>(q, ursrc, rmap, qq, i + 2, ust);
      drive<MPW, R, BF16, KEEP>(q, bk, lds + ui1 * ut, ln.w, ln.l, acc);
      // (before the readout's y stores, so that waiting for the loads does
      // not wait for them)
      const int ui2 = ui1 == 2 ? 0 : ui1 + 1;
      __builtin_amdgcn_sched_barrier(0);   // keep the stash (and its wait) after the drive
      stash_u<R, BF16, NB, kWaves>(q, ust, lds + ui2 * ut);
      readout<MPW, R, BF16, KEEP, VEC, y_bf16<XM, BF16>()>(q, yrsrc, rmap, epilogue<XM>(q), ck, mt.d, xb,
                                                         lds + ui * ut, i, ln, yorsrc);
      ui = ui1;
    }
  }
  };
  if (u_rows_vectorized(q.H, BF16)) {
    chunks(std::true_type{});
  } else {
    chunks(std::false_type{});
  }
}

// ---- pass 2, wave-specialized (register-resident weights) ------------------------------
// Eight waves: waves 0-3 drive (B_bar in registers: drive MFMA, scan, x tile),
// waves 4-7 read out (C' in registers: readout MFMA, D u feedthrough, y, and
// the staging of the u tiles). Waves are placed on the four SIMDs in turn, so
// every SIMD runs one wave of each kind: the drive wave's scan and the
// readout wave's LDS waits proceed while the other wave's MFMAs run. Chunk
// i+1 is driven and scanned while chunk i is read out; one barrier per chunk.

// carry into the workgroup's range: the totals of the sequence's earlier
// ranges folded in order (one thread per mode)
template <bool EXT, bool TV>
__device__ __forceinline__ void range_carry(const FusedParams& q, int b, int qq, int p, S5_LDS pf2* s_c0) {
  cf c = {0.0f, 0.0f};   // the state before step 0: zero, or the caller's
  if (EXT && q.x0 != nullptr && p < q.P) {
    const float2 v = q.x0[static_cast<size_t>(b) * q.P + p];
    c = {v.x, v.y};
  }
  const size_t base = static_cast<size_t>(b) * q.Q * q.Ppad + p;
  constexpr int kBatch = 16;
  // time-invariant: every range's transition is the same power of abar,
  // taken from the float64 packing (rounded once) rather than the range's
  // product of its 16 stream powers (each rounded), whose rounding a fold
  // over many ranges would compound for modes with |abar| near 1
  cf ar = {0.0f, 0.0f};
  if constexpr (!TV) {
    const float2 v = q.modes[p].arange;
    ar = {v.x, v.y};
  }
  for (int q0 = 0; q0 < qq; q0 += kBatch) {
    cf xs[kBatch], as[kBatch];
#pragma unroll
    for (int e = 0; e < kBatch; ++e) {
      if (q0 + e < qq) {
        const float2 xv = q.tot[base + static_cast<size_t>(q0 + e) * q.Ppad];
        xs[e] = {xv.x, xv.y};
        if constexpr (TV) {
          const float2 av = q.tot_a[base + static_cast<size_t>(q0 + e) * q.Ppad];
          as[e] = {av.x, av.y};
        } else {
          as[e] = ar;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < kBatch; ++e) {
      if (q0 + e < qq) c = cfma(as[e], c, xs[e]);
    }
  }
  st_pf2(s_c0 + p, c.re, c.im);
}

// state entering the lane's stream for its modes: exclusive 16-lane scan of
// the stream aggregates, applied to the range carry
template <int MPW, bool TV>
__device__ __forceinline__ void stream_start(const FusedParams& q, int bq, const Lane& ln, const S5_LDS pf2* s_c0,
                                             cf (&st)[MPW][4]) {
  // all loads first (one round of latency), then the scans
  float2 xv[MPW][4], av[MPW][4];
#pragma unroll
  for (int jj = 0; jj < MPW; ++jj) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pm = 16 * (ln.w + kWaves * jj) + 4 * ln.g + r;
      const size_t si = (static_cast<size_t>(bq) * kStreams + ln.t) * q.Ppad + pm;
      xv[jj][r] = q.sagg[si];
      av[jj][r] = TV ? q.sagg_a[si] : q.modes[pm].aseg;
    }
  }
#pragma unroll
  for (int jj = 0; jj < MPW; ++jj) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pm = 16 * (ln.w + kWaves * jj) + 4 * ln.g + r;
      cf X = {xv[jj][r].x, xv[jj][r].y};
      cf A = {av[jj][r].x, av[jj][r].y};
      row_scan(A, X);
      const cf Ae = {row_shr<1>(A.re, 1.0f), row_shr<1>(A.im, 0.0f)};
      const cf Xe = {row_shr<1>(X.re, 0.0f), row_shr<1>(X.im, 0.0f)};
      st[jj][r] = cfma(Ae, ld_pf2(s_c0 + pm), Xe);
    }
  }
}

// Drive, scan and x tile of the wave's mode tiles j0 .. j0 + JG - 1 (those
// below MPW) for one chunk: the accumulators of JG tiles only are live.
// UA: the u fragments of all K-steps come in `ua` (bf16 I/O); otherwise each
// K-step's fragments are read from the u tile `ub` right before its MFMAs.
template <int MPW, int JG, int R, bool TV, bool BF16, bool UA>
__device__ __forceinline__ void drive_scan_tiles(bool bil, int j0, int KS, const BKeep<MPW, BF16 ? 1 : 2>& bk,
                                                 const bf16x8 (&ua)[UA ? kKeepKS : 1][BF16 ? 1 : 2][R],
                                                 const lds_byte* ub, const ModeTable& mt,
                                                 const Lane& ln, const float4 (&dl)[TV ? MPW : 1][TV ? R : 1],
                                                 cf (&st)[MPW][4], lds_byte* xb) {
  constexpr int NP = BF16 ? 1 : 2;
  constexpr int K2 = 4 * MPW;
  f32x4 acc[JG][2][R];
#pragma unroll
  for (int jj = 0; jj < JG; ++jj)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int n = 0; n < R; ++n) acc[jj][cc][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < kKeepKS; ++s) {
    bf16x8 uk[NP][R];
    if constexpr (UA) {
#pragma unroll
      for (int pl = 0; pl < NP; ++pl)
#pragma unroll
        for (int n = 0; n < R; ++n) uk[pl][n] = ua[s][pl][n];
    } else {
      get_u<R, BF16>(ub, s < KS ? s : KS - 1, ln.l, uk);
    }
#pragma unroll
    for (int jj = 0; jj < JG; ++jj) {
      if (j0 + jj >= MPW) continue;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int n = 0; n < R; ++n) {
          acc[jj][cc][n] = mfma(bk.f[s][j0 + jj][cc][0], uk[0][n], acc[jj][cc][n]);
          if constexpr (NP == 2) {
            acc[jj][cc][n] = mfma(bk.f[s][j0 + jj][cc][0], uk[1][n], acc[jj][cc][n]);
            acc[jj][cc][n] = mfma(bk.f[s][j0 + jj][cc][1], uk[0][n], acc[jj][cc][n]);
          }
        }
    }
  }
#pragma unroll
  for (int jj = 0; jj < JG; ++jj) {
    if (j0 + jj >= MPW) continue;
    const int j = j0 + jj;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pm = 16 * (ln.w + kWaves * j) + 4 * ln.g + r;
      cf x = st[j][r];
      if constexpr (TV) {
        const StepMode sm = mt.step_mode(pm);
#pragma unroll
        for (int n = 0; n < R; ++n) {
          x = step_am1(disc_am1(bil, sm, f4_at(dl[j][n], r)), x, {acc[jj][0][n][r], acc[jj][1][n][r]});
          acc[jj][0][n][r] = x.re;
          acc[jj][1][n][r] = x.im;
        }
      } else {
        const cf ab = ld_pf2(mt.ab + pm);
#pragma unroll
        for (int n = 0; n < R; ++n) {
          x = cfma(ab, x, {acc[jj][0][n][r], acc[jj][1][n][r]});
          acc[jj][0][n][r] = x.re;
          acc[jj][1][n][r] = x.im;
        }
      }
      st[j][r] = x;
    }
#pragma unroll
    for (int n = 0; n < R; ++n) {
      float v[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[2 * r] = acc[jj][0][n][r];
        v[2 * r + 1] = acc[jj][1][n][r];
      }
      const int blk = (ln.w + kWaves * j) * R + n;
      uint4 hi, lo;
      put_frag(v, &hi, BF16 ? nullptr : &lo);
      lds_st<uint4>(xb + blk * kBlock + ln.l * 16, hi);
      if constexpr (!BF16) lds_st<uint4>(xb + (K2 * R + blk) * kBlock + ln.l * 16, lo);
    }
  }
}

// one chunk of a drive wave, JG mode tiles at a time (one with float32 I/O
// and the time-varying step, whose hi/lo weights and per-step registers
// leave no room for a second tile's accumulators)
template <int MPW, int R, bool TV, bool BF16>
__device__ __forceinline__ void drive_scan_chunk(bool bil, int KS, const BKeep<MPW, BF16 ? 1 : 2>& bk, const lds_byte* ub,
                                                 const ModeTable& mt, const Lane& ln,
                                                 const float4 (&dl)[TV ? MPW : 1][TV ? R : 1],
                                                 cf (&st)[MPW][4], lds_byte* xb) {
  constexpr int JG = (MPW >= 4 || (TV && !BF16)) ? 1 : (MPW < 2 ? MPW : 2);
  // the chunk's u fragments (K-steps past KS repeat the last real one against
  // zero weights): read from LDS once for all tile groups where registers
  // allow, else again for each group
  constexpr bool kOnce = BF16;
  bf16x8 ua[kOnce ? kKeepKS : 1][BF16 ? 1 : 2][R];
  if constexpr (kOnce) {
#pragma unroll
    for (int s = 0; s < kKeepKS; ++s) get_u<R, BF16>(ub, s < KS ? s : KS - 1, ln.l, ua[s]);
  }
#pragma unroll
  for (int j0 = 0; j0 < MPW; j0 += JG) drive_scan_tiles<MPW, JG, R, TV, BF16, kOnce>(bil, j0, KS, bk, ua, ub, mt, ln, dl, st, xb);
}

template <int MPW, int R, bool TV, bool BF16, int XM>
__global__ void __launch_bounds__(2 * kThreads, 1) k_scan_ws(FusedParams q) {
  constexpr bool EXT = XM != 0;   // options of the extended entry point
  constexpr int NP = BF16 ? 1 : 2;
  constexpr int K2 = 4 * MPW;
  extern __shared__ __align__(16) unsigned char smem[];
  if (q.Ppad != 64 * MPW || q.R != R) return;   // dispatch mismatch: do nothing
  const bool driver = threadIdx.x < kThreads;    // waves 0-3; waves 4-7 read out
  const Lane ln = lane_ids();                    // ids within the role
  const int bq = blockIdx.x;
  const int b = bq / q.Q;
  const int qq = bq - b * q.Q;
  const bool bil = EXT && q.bilinear;        // bilinear per-step discretisation
  const RowMap rmap = row_map<XM == 3>(q, qq);   // forward or reverse time
  const int KS = q.Hpad >> 5;
  const int HT = q.Hpad >> 4;
  const int ut = static_cast<int>(u_tile_bytes(KS, R, BF16));
  const int xt = static_cast<int>(x_tile_bytes(K2, R, BF16));
  // u tile i in buffer i % 3 (staged by the readout waves two chunks ahead,
  // read by drive(i) and by the feedthrough of readout(i)); x tile i in x
  // buffer i % 2 (written by the drive waves, read by the readout waves)
  lds_byte* lds = (lds_byte*)smem;
  lds_byte* xlds = lds + 3 * ut;
  const ModeTable mt = fill_mode_table<TV>(q, lds + 3 * ut + 2 * xt, true);
  S5_LDS pf2* s_c0 = reinterpret_cast<S5_LDS pf2*>(xlds + xt);   // free until x tile 1
  if (driver && ln.tid < q.Ppad) range_carry<EXT, TV>(q, b, qq, ln.tid, s_c0);

  constexpr int NB = u_stage_blocks<R, BF16, true>();
  const __amdgpu_buffer_rsrc_t ursrc = range_rsrc<BF16>(q.u, q, b, qq, rmap.rev);
  const __amdgpu_buffer_rsrc_t yrsrc = y_rsrc<XM, BF16>(q, b, qq, rmap.rev);
  const __amdgpu_buffer_rsrc_t yorsrc = XM == 3 ? range_rsrc<false>(q.yp, q, b, qq, rmap.rev) : yrsrc;
  // one register array holds the role's weights: B_bar fragments [s][jj][cc][pl]
  // in drive waves, C' fragments [e][s][pl] in readout waves (16 MPW NP each)
  static_assert(sizeof(BKeep<MPW, NP>) == sizeof(CKeep<MPW, NP>), "both roles hold 16 MPW NP fragments");
  union Weights {
    BKeep<MPW, NP> b;
    CKeep<MPW, NP> c;
  };
  Weights wts;
  cf st[MPW][4];
  if (driver) {
    load_b_keep<MPW, NP>(q, ln.w, ln.l, wts.b);
  } else {
#pragma unroll
    for (int e = 0; e < kKeepHT; ++e) {
      const int ht = ln.w + kWaves * e;
#pragma unroll
      for (int s = 0; s < K2; ++s) {
        if (ht < HT) {
          load_c_step<MPW, NP>(q, ht, s, ln.l, wts.c.f[e][s]);
        } else {
#pragma unroll
          for (int pl = 0; pl < NP; ++pl) wts.c.f[e][s][pl] = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
        }
      }
    }
  }
  auto chunks = [&](auto vec_c) {
  constexpr bool VEC = decltype(vec_c)::value;
  if (!driver) {
    UStage<NB> ust;
    fetch_u<R, BF16, NB, kWaves, VEC>(q, ursrc, rmap, qq, 0, ust);
    stash_u<R, BF16, NB, kWaves>(q, ust, lds);
    fetch_u<R, BF16, NB, kWaves, VEC>(q, ursrc, rmap, qq, 1, ust);
    stash_u<R, BF16, NB, kWaves>(q, ust, lds + ut);
  }
  lds_barrier();   // carry, mode table, u tiles 0 and 1
  float4 dk[kKeepHT];   // D of the readout wave's h-tiles: features 16 ht + 4 g + 0..3
#pragma unroll
  for (int e = 0; e < kKeepHT; ++e) {
    const int h0 = 16 * (ln.w + kWaves * e) + 4 * ln.g;
    dk[e] = h0 < q.Hpad ? lds_ld<float4>(reinterpret_cast<const lds_byte*>(mt.d + h0)) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float4 dl[TV ? MPW : 1][TV ? R : 1];
  if (driver) {
    stream_start<MPW, TV>(q, bq, ln, s_c0, st);
    if (EXT && q.xlast != nullptr) {
      const LastTok lt = last_token<R>(q);
      if (qq == lt.qq) write_final_state<R, MPW, TV>(q, b, lt, ln, st);
    }
    if constexpr (TV) load_delta<MPW, R>(q, b, qq, 0, ln, dl);
    drive_scan_chunk<MPW, R, TV, BF16>(EXT && q.bilinear, KS, wts.b, lds, mt, ln, dl, st, xlds);
  }
  lds_barrier();   // x tile 0

  // One loop per role (each ends an iteration at the same barrier), so that
  // neither role's registers are live in the other's code.
  // Iteration i: drive waves scan chunk i+1 into x tile (i+1)&1 from u tile
  // (i+1)%3; readout waves turn x tile i&1 into y and stage u tile i+2.
  if (driver) {
    int ui = 0;   // i % 3
    for (int i = 0; i < q.nck; ++i) {
      const int ui1 = ui == 2 ? 0 : ui + 1;
      if (i + 1 < q.nck) {
        if constexpr (TV) load_delta<MPW, R>(q, b, qq, i + 1, ln, dl);
        drive_scan_chunk<MPW, R, TV, BF16>(EXT && q.bilinear, KS, wts.b, lds + ui1 * ut, mt, ln, dl, st, xlds + ((i + 1) & 1) * xt);
      }
      lds_barrier();   // x tile i+1 and u tile i+2 complete; x tile i and u tile i-1 free
      ui = ui1;
    }
  } else {
    // backward scan (XM = 3): the y being added to, a chunk ahead in registers
    constexpr bool kAcc = XM == 3;
    YOld<false> yold;
    int ui = 0;   // i % 3
    for (int i = 0; i < q.nck; ++i) {
      const int ui1 = ui == 2 ? 0 : ui + 1;
      const int ui2 = ui1 == 2 ? 0 : ui1 + 1;
      // u tile i+2 into registers now, into LDS after this chunk's MFMAs
      // (not carried across iterations: no register shuffles, no early wait)
      UStage<NB> ust2;
      fetch_u<R, BF16, NB, kWaves, VEC>(q, ursrc, rmap, qq, i + 2, ust2);
      // (the values this chunk's readout adds: issued with the u loads, ahead
      // of the readout MFMAs that hide their latency)
      if constexpr (kAcc) load_y_old<R, false, VEC>(q, yorsrc, rmap, i, ln, yold);
      const lds_byte* xr = xlds + (i & 1) * xt;
      f32x4 yacc[kKeepHT][R];
#pragma unroll
      for (int e = 0; e < kKeepHT; ++e)
#pragma unroll
        for (int n = 0; n < R; ++n) yacc[e][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      // x fragments read kAhead K-steps ahead of their MFMAs
      constexpr int kAhead = NP == 2 ? 1 : 3;
      bf16x8 xf[K2][NP][R];
#pragma unroll
      for (int s = 0; s < kAhead && s < K2; ++s) get_x<R, NP>(xr, K2, s, ln.l, xf[s]);
      // the u loads first, then the x reads kAhead K-steps ahead of their
      // MFMAs (left alone, the scheduler puts each load next to its use)
      __builtin_amdgcn_sched_group_barrier(
          0x020, (VEC ? NB : NB * (BF16 ? 8 : 4)) + (kAcc ? kKeepHT * R * (VEC ? 1 : 4) : 0), 0);
      __builtin_amdgcn_sched_group_barrier(0x100, (kAhead < K2 ? kAhead : K2) * NP * R, 0);
#pragma unroll
      for (int s = 0; s < K2; ++s) {
        if (s + kAhead < K2) get_x<R, NP>(xr, K2, s + kAhead, ln.l, xf[s + kAhead]);
#pragma unroll
        for (int e = 0; e < kKeepHT; ++e) mfma_read<R, NP>(wts.c.f[e][s], xf[s], yacc[e]);
        if (s + kAhead < K2) __builtin_amdgcn_sched_group_barrier(0x100, NP * R, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, kKeepHT * R * (NP == 2 ? 3 : 1), 0);
      }
      // u tile i+2 into the buffer of tile i-1 (read by drive(i-1) and
      // readout(i-1), both before the previous barrier); before this chunk's
      // y stores, so that waiting for the loads does not wait for them
      __builtin_amdgcn_sched_barrier(0);   // keep the stash (and its wait) after the MFMAs
      stash_u<R, BF16, NB, kWaves>(q, ust2, lds + ui2 * ut);
      readout_store<R, BF16, VEC, kAcc, y_bf16<XM, BF16>()>(q, yrsrc, rmap, epilogue<XM>(q), dk, yacc,
                                                             lds + ui * ut, i, ln, &yold);
      lds_barrier();   // x tile i+1 and u tile i+2 complete; x tile i and u tile i-1 free
      ui = ui1;
    }
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

#include "s5_scan8.h"

namespace s5 {
namespace fused {

// ---- launch -----------------------------------------------------------------------------

template <auto Kern>
hipError_t launch_one(int blocks, int threads, size_t lds, hipStream_t s, const FusedParams& q) {
  if (q.dry) return hipSuccess;   // the instance exists; nothing is launched
  // the first launch of each instance lifts its dynamic LDS limit
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(Kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(Kern, dim3(blocks), dim3(threads), lds, s, q);
  return hipGetLastError();
}

// XM (pass 2): 0 plain calls (option code compiled out); 1 initial and final
// state, bilinear steps; 2 those and GELU; 3 those and reverse time, adding
// to y and GELU on request (the backward scan of the bidirectional form).
// Pass 1 writes no y: its instance 1 serves every call with options.
template <int MPW, int R, bool TV, bool BF16, bool KEEP>
hipError_t launch_reduce_t(const FusedParams& q, const FusedPlan& p, hipStream_t s) {
  const int blocks = q.B * q.Q;
  const bool xm = q.x0 != nullptr || q.xlast != nullptr || q.rev || (q.bilinear && TV);
  if constexpr (KEEP) {
    constexpr int M8 = (4 * MPW + 2 * kWaves - 1) / (2 * kWaves);   // mode tiles per wave
    auto go = [&](auto ks_c) {
      constexpr int KS = decltype(ks_c)::value;
      if constexpr (!TV && (KS <= 4 || M8 == 1)) {
        if (q.both) return launch_one<k_reduce_ws<MPW, KS, R, TV, BF16, 2>>(blocks, 2 * kThreads, p.lds_reduce_ws, s, q);
      }
      if (q.both) return hipErrorInvalidValue;   // not planned
      if (xm) return launch_one<k_reduce_ws<MPW, KS, R, TV, BF16, 1>>(blocks, 2 * kThreads, p.lds_reduce_ws, s, q);
      return launch_one<k_reduce_ws<MPW, KS, R, TV, BF16, 0>>(blocks, 2 * kThreads, p.lds_reduce_ws, s, q);
    };
    // the drive's K-steps: H <= 128, and time-invariant H <= 256 where the
    // weights fit 128 registers (M8 KS NP <= 16)
    constexpr int kMaxKS = TV ? 4 : 16 / (M8 * (BF16 ? 1 : 2));
    auto big = [&](auto ks_c) {
      if constexpr (decltype(ks_c)::value <= kMaxKS) {
        return go(ks_c);
      } else {
        return hipErrorInvalidValue;
      }
    };
    switch (p.ks) {
      case 1: return go(std::integral_constant<int, 1>{});
      case 2: return go(std::integral_constant<int, 2>{});
      case 3: return go(std::integral_constant<int, 3>{});
      case 4: return go(std::integral_constant<int, 4>{});
      case 5: return big(std::integral_constant<int, 5>{});
      case 6: return big(std::integral_constant<int, 6>{});
      case 7: return big(std::integral_constant<int, 7>{});
      case 8: return big(std::integral_constant<int, 8>{});
      default: return hipErrorInvalidValue;
    }
  } else {
    if (q.both) return hipErrorInvalidValue;   // the host runs the backward pass 1 separately here
    if (xm) return launch_one<k_reduce<MPW, R, TV, BF16, KEEP, 1>>(blocks, kThreads, p.lds_reduce, s, q);
    return launch_one<k_reduce<MPW, R, TV, BF16, KEEP, 0>>(blocks, kThreads, p.lds_reduce, s, q);
  }
}

// pass 2 on the symmetric eight-wave kernel (KS drive K-steps). Instances:
// the time-varying step (plain, state, GELU; the gate with bf16 I/O), the
// streamed drive above four K-steps (time-invariant bf16: plain, state, GELU,
// both bidirectional halves) and, at most four K-steps time-invariant, the
// gate only (the plain call takes the wave-specialized kernel there).
template <int MPW, int KS, bool TV, bool BF16>
hipError_t launch_scan8_t(const FusedParams& q, const FusedPlan& p, hipStream_t s) {
  const int blocks = q.B * q.Q;
  if (q.rev != q.accum) return hipErrorInvalidValue;   // reverse time only for the backward scan
  const int xm = q.glu_w != nullptr ? 5
               : q.ypart ? 4
               : q.accum ? 3
               : q.gelu ? 2
               : (q.x0 != nullptr || q.xlast != nullptr || (q.bilinear && TV)) ? 1 : 0;
  auto go = [&](auto xm_c) {
    return launch_one<k_scan8<MPW, KS, TV, BF16, decltype(xm_c)::value>>(blocks, 2 * kThreads, p.lds_scan, s, q);
  };
  using X0 = std::integral_constant<int, 0>;
  using X1 = std::integral_constant<int, 1>;
  using X2 = std::integral_constant<int, 2>;
  using X3 = std::integral_constant<int, 3>;
  using X4 = std::integral_constant<int, 4>;
  using X5 = std::integral_constant<int, 5>;
  if constexpr (TV) {
    if (xm == 0) return go(X0{});
    if (xm == 1) return go(X1{});
    if (xm == 2) return go(X2{});
    if constexpr (BF16) {
      if (xm == 5) return go(X5{});
    }
    return hipErrorInvalidValue;   // the backward scan is time-invariant only
  } else if constexpr (KS > 4) {
    if constexpr (BF16) {
      if (xm == 0) return go(X0{});
      if (xm == 1) return go(X1{});
      if (xm == 2) return go(X2{});
      if (xm == 3) return go(X3{});
      if (xm == 4) return go(X4{});
    }
    return hipErrorInvalidValue;
  } else {
    if constexpr (BF16) {
      if (xm == 5) return go(X5{});
    }
    return hipErrorInvalidValue;
  }
}

template <int MPW, int R, bool TV, bool BF16, bool KEEP>
hipError_t launch_scan_t(const FusedParams& q, const FusedPlan& p, hipStream_t s) {
  const int blocks = q.B * q.Q;
  if (q.rev != q.accum) return hipErrorInvalidValue;   // reverse time only for the backward scan
  const int xm = q.ypart ? 4 : q.accum ? 3 : q.gelu ? 2 : (q.x0 != nullptr || q.xlast != nullptr || (q.bilinear && TV)) ? 1 : 0;
  if constexpr (TV) {
    if (xm >= 3) return hipErrorInvalidValue;   // the backward scan is time-invariant only
  }
  if (xm == 4 && !BF16) return hipErrorInvalidValue;   // float32 I/O: the forward half is y itself
  if constexpr (KEEP && TV && MPW > 2) {
    return hipErrorInvalidValue;   // not planned: the time-varying step keeps at most two tiles per wave
  } else if constexpr (KEEP) {
    if constexpr (!TV) {
      if (xm == 3) return launch_one<k_scan_ws<MPW, R, TV, BF16, 3>>(blocks, 2 * kThreads, p.lds_scan, s, q);
      if constexpr (BF16) {
        if (xm == 4) return launch_one<k_scan_ws<MPW, R, TV, BF16, 4>>(blocks, 2 * kThreads, p.lds_scan, s, q);
      }
    }
    if (xm == 2) return launch_one<k_scan_ws<MPW, R, TV, BF16, 2>>(blocks, 2 * kThreads, p.lds_scan, s, q);
    if (xm == 1) return launch_one<k_scan_ws<MPW, R, TV, BF16, 1>>(blocks, 2 * kThreads, p.lds_scan, s, q);
    return launch_one<k_scan_ws<MPW, R, TV, BF16, 0>>(blocks, 2 * kThreads, p.lds_scan, s, q);
  } else {
    if constexpr (!TV) {
      if (xm == 3) return launch_one<k_scan<MPW, R, TV, BF16, KEEP, 3>>(blocks, kThreads, p.lds_scan, s, q);
      if constexpr (BF16) {
        if (xm == 4) return launch_one<k_scan<MPW, R, TV, BF16, KEEP, 4>>(blocks, kThreads, p.lds_scan, s, q);
      }
    }
    if (xm == 2) return launch_one<k_scan<MPW, R, TV, BF16, KEEP, 2>>(blocks, kThreads, p.lds_scan, s, q);
    if (xm == 1) return launch_one<k_scan<MPW, R, TV, BF16, KEEP, 1>>(blocks, kThreads, p.lds_scan, s, q);
    return launch_one<k_scan<MPW, R, TV, BF16, KEEP, 0>>(blocks, kThreads, p.lds_scan, s, q);
  }
}

}  // namespace fused
}  // namespace s5
