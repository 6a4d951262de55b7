// Host side of the S5 forward path: launch plan, workspace layout and the
// three launches (parameter packing, aggregate pass, state and output pass),
// all on the caller's stream.
#include <algorithm>

#include "s5_fused.h"
#include "s5_internal.h"

namespace s5 {

using fused::kStreams;

void fused_shape(bool bf16_io, bool time_varying, int Ppad, int Hpad, bool gate, FusedPlan& p) {
  const int MPW = Ppad / 64, KS = Hpad / 32, K2 = Ppad / 16, NP = bf16_io ? 1 : 2;
  const size_t lds_max = 160 * 1024;
  // weights in registers: all drive K-steps (H <= 128) and readout h-tiles,
  // 16 MPW NP fragments of 16 bytes per lane. Pass 1 (eight waves, each with
  // half the mode tiles) keeps them up to MPW NP = 4; pass 2 (two waves per
  // SIMD, 256 registers each) up to MPW NP = 4, and with the time-varying step
  // (its interval registers and discretisation beside the weights) up to two
  // mode tiles per wave
  // pass 1's eight waves hold M8 = ceil(4 MPW / 8) mode tiles each: at most
  // 128 registers of weights (M8 KS NP <= 16), so time-invariant shapes up to
  // H = 256 (KS = 8) keep them; the time-varying step up to H = 128
  const int M8 = (4 * MPW + 7) / 8;
  // (pass 1's register-weight instances are compiled for KS <= 8)
  const bool keep = MPW * NP <= 4 && M8 * KS * NP <= 16 && KS <= 8 && (KS <= 4 || !time_varying);
  const bool keep_scan = KS <= 4 && MPW * NP <= 4 && !(time_varying && MPW > 2);
  p.R = 0;
  // bf16 instances are compiled for R = 2 (which always fits); float32 ones
  // also for R = 1, taken where three u tiles and two x tiles of R = 2
  // exceed the LDS
  const int cand[2] = {2, 1};
  for (int R : cand) {
    if (bf16_io && R != 2) continue;
    bool k = keep && R == 2;
    const bool ks = keep_scan && R == 2;
    const size_t lr = 2 * fused::u_tile_bytes(KS, R, bf16_io) +
                      (time_varying ? fused::mode_table_bytes(Ppad, Hpad, true, false) : 0);
    size_t ls = 3 * fused::u_tile_bytes(KS, R, bf16_io) + 2 * fused::x_tile_bytes(K2, R, bf16_io) +
                      (ks ? fused::mode_table_bytes(Ppad, Hpad, time_varying, true) : 0);
    if (ls > lds_max || lr > lds_max) continue;
    // eight-wave pass 1: two groups of u tiles and the mode table
    const size_t lrw = 2 * fused::reduce_group(bf16_io, time_varying, KS) * fused::u_tile_bytes(KS, R, bf16_io) +
                       fused::mode_table_bytes(Ppad, Hpad, time_varying, false);
    if (k && lrw > lds_max) k = false;   // the four-wave pass 1 instead
    p.R = R;
    p.keep = k;
    p.keep_scan = ks;
    // the symmetric eight-wave pass 2: weights of a wave's share in registers
    // (at most 128 VGPRs of them), four u tiles (three bf16 planes for float32
    // u), two x tiles and the mode table in LDS
    {
      const int NT = 4 * MPW, MT = (NT + 7) / 8, HT = 2 * KS, ET = (HT + 7) / 8;
      // time-invariant bf16 with more than four drive K-steps (H > 128): C'
      // in registers, B_bar streamed from L2
      const bool sb = !time_varying && bf16_io && KS > 4 && KS <= 8;
      const int wregs = 4 * ((sb ? 0 : KS * MT * 2 * NP) + ET * NT * NP);
      const size_t l8 = 4 * static_cast<size_t>(KS) * R * (bf16_io ? 1 : 3) * fused::kBlock +
                        2 * fused::x_tile_bytes(K2, R, bf16_io) + fused::mode_table_bytes(Ppad, Hpad, time_varying, true);
      // taken for the time-varying step, whose per-step vector work the
      // symmetric split spreads over both waves of each SIMD, and where the
      // wave-specialized kernel's weights do not fit (H > 128); the
      // time-invariant pass 2 with H <= 128 is matrix-core bound and runs
      // faster with its roles specialized
      const bool tv8 = ks && time_varying && KS <= 4 && MPW <= (bf16_io ? 4 : 2);
      // the gated activation inside this pass (bf16, H <= 128): a ring of two
      // g tiles of two planes, the multipliers and the bias too
      const bool gate8 = gate && bf16_io && KS <= 4 && (tv8 || (ks && !time_varying));
      const size_t lg = l8 + (gate8 ? (4 * static_cast<size_t>(KS) + 8 * ET) * R * fused::kBlock + 4 * Hpad : 0);
      p.scan8 = (tv8 || sb || gate8) && R == 2 && wregs <= 128 && lg <= lds_max;
      p.ks = KS;
      if (p.scan8) ls = lg;
    }
    p.group = k ? fused::reduce_group(bf16_io, time_varying, KS) : 1;
    // (above four K-steps with two mode tiles per wave, the second sum's
    // registers do not fit beside the weights)
    p.both = k && !time_varying && (KS <= 4 || M8 == 1);
    p.lds_reduce_ws = lrw;
    p.lds_reduce = lr;
    p.lds_scan = ls;
    break;
  }
}

void fused_split(int B, int L, int H, int P, int ncu, FusedPlan& p) {
  const int per = kStreams * p.R;                  // tokens of one chunk of a range
  const int chunks = (L + per - 1) / per;          // chunks with a single range
  int Q = std::max(1, (ncu + B - 1) / B);          // ranges per sequence to fill the CUs
  Q = std::max(1, std::min(Q, chunks));
  const int g = std::max(1, p.group);
  auto chunks_for = [&](int q) { return ((L + q * per - 1) / (q * per) + g - 1) / g * g; };
  p.nck = chunks_for(Q);
  p.Lseg = p.R * p.nck;
  p.Q = (L + kStreams * p.Lseg - 1) / (kStreams * p.Lseg);
  // a range's rows of u, y and Delta stay below 1 GiB (32-bit lane offsets)
  const int64_t row_bytes = static_cast<int64_t>(std::max(H, P)) * 4;
  while (static_cast<int64_t>(kStreams) * p.Lseg * row_bytes >= (int64_t{1} << 30) && p.nck > g) {
    Q = std::min(chunks, 2 * Q);
    p.nck = chunks_for(Q);
    p.Lseg = p.R * p.nck;
    p.Q = (L + kStreams * p.Lseg - 1) / (kStreams * p.Lseg);
  }
}

namespace {

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int device_cus() {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return ncu;
}

}  // namespace

bool forward_layout(const ForwardArgs& a, ForwardLayout& l) {
  l = ForwardLayout{};
  l.Ppad = ((a.P + 63) / 64) * 64;
  l.Hpad = ((a.H + 31) / 32) * 32;
  fused_shape(a.bf16_io, a.time_varying, l.Ppad, l.Hpad, a.glu_w != nullptr, l.plan);
  if (l.plan.R == 0) return false;
  const int ncu = device_cus();
  fused_split(a.B, a.L, a.H, a.P, ncu > 0 ? ncu : 256, l.plan);
  const size_t planes = a.bf16_io ? 1 : 2;
  const size_t nb = static_cast<size_t>(l.Ppad / 16) * 2 * (l.Hpad / 32) * 64;
  const size_t nc = static_cast<size_t>(l.Hpad / 16) * (2 * l.Ppad / 32) * 64;
  const size_t nranges = static_cast<size_t>(a.B) * l.plan.Q;
  size_t off = 0;
  l.bpack = off;  off += align_up(planes * nb * 16);
  l.cpack = off;  off += align_up(planes * nc * 16);
  l.modes = off;  off += align_up(l.Ppad * sizeof(ModeParams));
  l.sagg = off;   off += align_up(nranges * kStreams * l.Ppad * sizeof(float2));
  l.sagg_a = off; off += a.time_varying ? align_up(nranges * kStreams * l.Ppad * sizeof(float2)) : 0;
  l.tot = off;    off += align_up(nranges * l.Ppad * sizeof(float2));
  l.tot_a = off;  off += align_up(nranges * l.Ppad * sizeof(float2));
  l.cap = off;    off += align_up(static_cast<size_t>(a.B) * 2 * l.Ppad * sizeof(float2));
  if (a.bidir) {
    l.sagg_b = off;  off += align_up(nranges * kStreams * l.Ppad * sizeof(float2));
    l.tot_b = off;   off += align_up(nranges * l.Ppad * sizeof(float2));
    l.tot_a_b = off; off += align_up(nranges * l.Ppad * sizeof(float2));
    l.yp = off;      off += a.bf16_io ? align_up(static_cast<size_t>(a.B) * a.L * a.H * sizeof(float)) : 0;
    l.cpack_b = off; off += align_up(planes * nc * 16);
  }
  if (a.glu_w != nullptr) {
    l.gpack = off;   off += align_up(2 * static_cast<size_t>(l.Hpad / 16) * (l.Hpad / 32) * 64 * 16);
  }
  l.total = off;
  return true;
}

namespace {

using Launcher = hipError_t (*)(const FusedParams&, const FusedPlan&, hipStream_t);

hipError_t timed(int k, const hipEvent_t* ev, int nev, hipStream_t s, hipError_t (*fn)(const FusedParams&, const FusedPlan&, hipStream_t),
                 const FusedParams& q, const FusedPlan& p) {
  const bool rec = ev != nullptr && 2 * k + 1 < nev;
  if (rec) (void)hipEventRecord(ev[2 * k], s);
  const hipError_t e = fn(q, p, s);
  if (rec) (void)hipEventRecord(ev[2 * k + 1], s);
  return e;
}

hipError_t pack_launcher(const FusedParams& q, const FusedPlan&, hipStream_t s) { return launch_pack(q, s); }

}  // namespace

hipError_t launch_reduce(const FusedParams& q, const FusedPlan& p, hipStream_t s) {
  if (q.bf16_io) return q.time_varying ? launch_reduce_bf16_tv(q, p, s) : launch_reduce_bf16_ti(q, p, s);
  return q.time_varying ? launch_reduce_f32_tv(q, p, s) : launch_reduce_f32_ti(q, p, s);
}

hipError_t launch_scan(const FusedParams& q, const FusedPlan& p, hipStream_t s) {
  if (q.bf16_io) return q.time_varying ? launch_scan_bf16_tv(q, p, s) : launch_scan_bf16_ti(q, p, s);
  return q.time_varying ? launch_scan_f32_tv(q, p, s) : launch_scan_f32_ti(q, p, s);
}

namespace {
__global__ void __launch_bounds__(256) k_state_passthrough(const float2* x0, float2* xlast, int64_t n) {
  for (int64_t k = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; k < n;
       k += static_cast<int64_t>(gridDim.x) * blockDim.x)
    xlast[k] = x0 != nullptr ? x0[k] : make_float2(0.0f, 0.0f);
}
}  // namespace

namespace {
__global__ void __launch_bounds__(256) k_widen_bf16(const unsigned short* in, float* out, int64_t n) {
  for (int64_t k = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; k < n;
       k += static_cast<int64_t>(gridDim.x) * blockDim.x)
    out[k] = __uint_as_float(static_cast<unsigned>(in[k]) << 16);
}

__global__ void __launch_bounds__(256) k_narrow_bf16(const float* in, __bf16* out, int64_t n) {
  for (int64_t k = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; k < n;
       k += static_cast<int64_t>(gridDim.x) * blockDim.x)
    out[k] = static_cast<__bf16>(in[k]);   // hardware conversion: round to nearest even
}

unsigned copy_blocks(int64_t n) { return static_cast<unsigned>((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024); }
}  // namespace

hipError_t launch_widen_bf16(const void* in, float* out, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_widen_bf16, dim3(copy_blocks(n)), dim3(256), 0, stream, static_cast<const unsigned short*>(in),
                     out, n);
  return hipGetLastError();
}

hipError_t launch_narrow_bf16(const float* in, void* out, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_narrow_bf16, dim3(copy_blocks(n)), dim3(256), 0, stream, in, static_cast<__bf16*>(out), n);
  return hipGetLastError();
}

hipError_t launch_state_passthrough(const float2* x0, float2* xlast, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(k_state_passthrough, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, x0, xlast, n);
  return hipGetLastError();
}

hipError_t launch_forward(const ForwardArgs& a, const ForwardLayout& l, void* ws, hipStream_t stream,
                          const hipEvent_t* ev, int nev, bool dry) {
  if (l.plan.R == 0) return hipErrorInvalidValue;
  if (dry) ev = nullptr;
  // workspace addresses (integer arithmetic: ws is null on a dry walk)
  auto at = [ws](size_t off) { return reinterpret_cast<void*>(reinterpret_cast<uintptr_t>(ws) + off); };
  FusedParams q{};
  q.dry = dry ? 1 : 0;
  q.B = a.B; q.L = a.L; q.H = a.H; q.P = a.P;
  q.Hpad = l.Hpad; q.Ppad = l.Ppad;
  q.R = l.plan.R; q.nck = l.plan.nck; q.Lseg = l.plan.Lseg; q.Q = l.plan.Q;
  q.bf16_io = a.bf16_io;
  q.time_varying = a.time_varying;
  q.u = a.u; q.y = a.y;
  q.lam = a.lam; q.b_tilde = a.b_tilde; q.c_tilde = a.c_tilde;
  q.d = a.d; q.log_delta = a.log_delta; q.delta = a.delta;
  q.x0 = a.x0; q.xlast = a.xlast;
  q.glu_w = a.glu_w; q.glu_bias = a.glu_bias; q.glu_variant = a.glu_variant;
  q.gpack = a.glu_w != nullptr ? static_cast<uint4*>(at(l.gpack)) : nullptr;
  q.c_ld = a.c_ld > 0 ? a.c_ld : a.P;
  q.c_off = a.c_off;
  q.c_scale = a.c_scale;
  q.bilinear = a.bilinear;
  q.rev = a.rev;
  q.accum = a.accum;
  q.gelu = a.gelu;
  q.bpack = static_cast<uint4*>(at(l.bpack));
  q.cpack = static_cast<uint4*>(at(l.cpack));
  q.modes = static_cast<ModeParams*>(at(l.modes));
  q.sagg = static_cast<float2*>(at(l.sagg));
  q.sagg_a = a.time_varying ? static_cast<float2*>(at(l.sagg_a)) : nullptr;
  q.tot = static_cast<float2*>(at(l.tot));
  q.tot_a = static_cast<float2*>(at(l.tot_a));
  q.cap = static_cast<float2*>(at(l.cap));
  if (!a.bidir) {
    hipError_t e = timed(0, ev, nev, stream, pack_launcher, q, l.plan);
    if (e != hipSuccess) return e;
    e = timed(1, ev, nev, stream, launch_reduce, q, l.plan);
    if (e != hipSuccess) return e;
    return timed(2, ev, nev, stream, launch_scan, q, l.plan);
  }
  // Bidirectional form (time-invariant, stateless): the backward scan runs in
  // reverse time over the mirrored ranges (backward range qq = forward range
  // Q-1-qq), so the eight-wave pass 1 sums both scans' aggregates from one
  // drive. The forward pass 2 stores y (D u included) as float32 (into the
  // workspace for bf16 I/O, into y itself for float32 I/O); the backward
  // pass 2 adds its readout (second half of C~) and stores y once, then GELU.
  q.yp = a.bf16_io ? static_cast<float*>(at(l.yp)) : static_cast<float*>(a.y);
  q.sagg_b = static_cast<float2*>(at(l.sagg_b));
  q.tot_b = static_cast<float2*>(at(l.tot_b));
  q.tot_a_b = static_cast<float2*>(at(l.tot_a_b));
  q.rev = 0;
  q.accum = 0;
  q.gelu = 0;
  q.both = l.plan.both ? 1 : 0;
  q.ypart = a.bf16_io ? 1 : 0;
  q.cpack_b = static_cast<uint4*>(at(l.cpack_b));   // both halves' C' in one packing launch
  hipError_t e = timed(0, ev, nev, stream, pack_launcher, q, l.plan);
  if (e != hipSuccess) return e;
  e = timed(1, ev, nev, stream, launch_reduce, q, l.plan);
  if (e != hipSuccess) return e;
  e = timed(2, ev, nev, stream, launch_scan, q, l.plan);
  if (e != hipSuccess) return e;
  FusedParams r = q;
  r.c_off = a.c_off + a.P;
  r.d = nullptr;
  r.rev = 1;
  r.accum = 1;
  r.gelu = a.gelu;
  r.both = 0;
  r.ypart = 0;
  r.sagg = q.sagg_b;
  r.tot = q.tot_b;
  r.tot_a = q.tot_a_b;
  r.cpack = q.cpack_b;
  r.cpack_b = nullptr;
  if (ev != nullptr && 7 < nev) {   // (no second packing launch: an empty pair)
    (void)hipEventRecord(ev[6], stream);
    (void)hipEventRecord(ev[7], stream);
  }
  if (!q.both) {
    e = timed(4, ev, nev, stream, launch_reduce, r, l.plan);
  } else if (ev != nullptr && 9 < nev) {
    (void)hipEventRecord(ev[8], stream);
    (void)hipEventRecord(ev[9], stream);
  }
  if (e != hipSuccess) return e;
  return timed(5, ev, nev, stream, launch_scan, r, l.plan);
}

}  // namespace s5
