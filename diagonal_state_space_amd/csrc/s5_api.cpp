// C ABI of the S5 forward path: host-side validation, stream-ordered scratch
// memory and dispatch to the kernels. See include/s5.h for the contract.
#include "s5.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "s5_internal.h"

// Scratch of the allocation-free entry point: one fixed array per device,
// held until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: its device address is resolved once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[S5_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local hipEvent_t tl_events[S5_PROFILING_MAX_EVENTS] = {};
thread_local int tl_nevents = 0;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + static_cast<uintptr_t>(bytes)};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Test hook: S5_TEST_FAIL_ALLOC=1 makes scratch allocation report failure.
bool alloc_fail_hook() {
  const char* v = std::getenv("S5_TEST_FAIL_ALLOC");
  return v != nullptr && v[0] == '1';
}

// Scratch memory: a cache of device buffers owned by the library, reused
// across calls. (Stream-ordered hipMallocAsync/hipFreeAsync per call would do,
// but hipFreeAsync blocks the host until the stream has caught up, which
// serialises the host's launches with the GPU's work.) A buffer belongs to the
// stream of its last use and is reused only by later calls on that stream,
// where stream order makes it safe; a call on another stream takes a new
// buffer. No event marks a buffer's last use: a marker between two calls on
// one stream cost ~5 us of GPU time between their kernels. When all 64 slots
// hold buffers of other streams, the call waits for the device once (after
// which none of them is in use) and takes one over. Buffers are kept until
// the process ends.
struct Scratch {
  void* ptr = nullptr;
  size_t bytes = 0;
  int dev = -1;
  hipStream_t last = nullptr;   // stream of the last use
  bool busy = false;            // taken by a call that has not enqueued its release yet
};
std::mutex g_scratch_mu;
Scratch* g_scratch[64] = {};
int g_nscratch = 0;

// A buffer of at least `bytes` on the current device for work on `stream`.
hipError_t scratch_acquire(size_t bytes, hipStream_t stream, Scratch** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  Scratch* pick = nullptr;
  for (int i = 0; i < g_nscratch && pick == nullptr; ++i) {
    Scratch* s = g_scratch[i];
    if (!s->busy && s->dev == dev && s->bytes >= bytes && s->last == stream) pick = s;
  }
  if (pick == nullptr && g_nscratch == 64) {
    // full: once the device is idle, no buffer that is not taken is in use
    // (a buffer released before this point had its work enqueued before it)
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return e;
    int victim = -1;
    for (int i = 0; i < g_nscratch && pick == nullptr; ++i) {
      Scratch* s = g_scratch[i];
      if (s->busy || s->dev != dev) continue;
      if (s->bytes >= bytes) {
        pick = s;
      } else if (victim < 0) {
        victim = i;
      }
    }
    if (pick == nullptr) {
      if (victim < 0) return hipErrorOutOfMemory;
      Scratch* v = g_scratch[victim];
      (void)hipFree(v->ptr);
      delete v;
      g_scratch[victim] = g_scratch[--g_nscratch];
    }
  }
  if (pick == nullptr) {
    Scratch* s = new Scratch();
    e = hipMalloc(&s->ptr, bytes);
    if (e != hipSuccess) {
      delete s;
      return e;
    }
    s->bytes = bytes;
    s->dev = dev;
    g_scratch[g_nscratch++] = s;
    pick = s;
  }
  pick->busy = true;
  *out = pick;
  return hipSuccess;
}

// The call's work on `stream` is enqueued: the buffer belongs to `stream` now.
hipError_t scratch_release(Scratch* s, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  s->last = stream;
  s->busy = false;
  return hipSuccess;
}

constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
void* g_noalloc_ptr[kMaxDevices] = {};

// device address of `scratch` on the current device
hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (g_noalloc_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_noalloc_ptr[dev] = p;
  }
  *out = g_noalloc_ptr[dev];
  return hipSuccess;
}

// bf16 I/O with at most this many features runs the float32-operand
// arithmetic (u widened into scratch, y rounded to bf16 once at the end): with
// so few outputs a readout sum over hundreds of modes can cancel to far
// below its terms, and the bf16 rounding of B_bar, C' and the states then
// shows at the percent level of the output's RMS
constexpr int64_t kWidenMaxH = 8;

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

s5_status check_sizes(int64_t P, int64_t H) {
  if (P < 1 || H < 1) return S5_ERR_INVALID_ARGUMENT;
  if (P > S5_MAX_P || H > S5_MAX_H) return S5_ERR_UNSUPPORTED;
  return S5_OK;
}

// Options of the extended entry point (defaults: the plain forward pass).
struct Options {
  float c_scale = 1.0f;    // readout factor: 2 for half-spectrum storage
  bool bilinear = false;   // bilinear discretisation
  int gelu = 0;            // GELU epilogue: 0 no, 1 exact form, 2 tanh form
  bool bidir = false;      // forward and backward scans, C~ with 2P columns
  const float* glu_w = nullptr;      // gated activation of the output (null: none)
  const float* glu_bias = nullptr;
  int glu_variant = 0;
};

s5_status forward_common(int64_t B, int64_t L, int64_t H, int64_t P, s5_dtype io, const void* u,
                         const s5_c64* lambda, const s5_c64* b_tilde, const s5_c64* c_tilde,
                         const float* d, const float* log_delta, const float* delta, void* y,
                         bool time_varying, const s5_c64* x0, s5_c64* x_last, const Options& opt,
                         hipStream_t stream, bool noalloc = false) {
  if (B < 0 || L < 0) return S5_ERR_INVALID_ARGUMENT;
  s5_status st = check_sizes(P, H);
  if (st != S5_OK) return st;
  if (io != S5_F32 && io != S5_BF16) return S5_ERR_UNSUPPORTED;
  const int64_t tokens = B * L;
  if (B > 0 && L > INT32_MAX / B) return S5_ERR_UNSUPPORTED;
  if (!lambda || !b_tilde || !c_tilde || !d) return S5_ERR_INVALID_ARGUMENT;
  if (time_varying ? false : !log_delta) return S5_ERR_INVALID_ARGUMENT;
  if (tokens > 0 && (!u || !y || (time_varying && !delta))) return S5_ERR_INVALID_ARGUMENT;
  // the backward scan is defined for the time-invariant, stateless form only
  if (opt.bidir && (time_varying || x0 || x_last)) return S5_ERR_INVALID_ARGUMENT;
  if (opt.glu_w && H > S5_GLU_MAX_H) return S5_ERR_UNSUPPORTED;
  const int64_t c_cols = opt.bidir ? 2 * P : P;
  const void* ptrs[] = {u, lambda, b_tilde, c_tilde, d, log_delta, delta, y, x0, x_last, opt.glu_w, opt.glu_bias};
  for (const void* p : ptrs) {
    if (p && !aligned16(p)) return S5_ERR_UNSUPPORTED;
  }
  const int64_t es = io == S5_BF16 ? 2 : 4;
  if (tokens > 0) {
    const Range ry = range_of(y, tokens * H * es);
    const Range inputs[] = {range_of(u, tokens * H * es),
                            range_of(lambda, P * 8),
                            range_of(b_tilde, P * H * 8),
                            range_of(c_tilde, H * c_cols * 8),
                            range_of(d, H * 4),
                            log_delta ? range_of(log_delta, P * 4) : Range{0, 0},
                            delta ? range_of(delta, tokens * P * 4) : Range{0, 0},
                            x0 ? range_of(x0, B * P * 8) : Range{0, 0},
                            opt.glu_w ? range_of(opt.glu_w, H * H * 4) : Range{0, 0},
                            opt.glu_bias ? range_of(opt.glu_bias, H * 4) : Range{0, 0}};
    for (const Range& r : inputs) {
      if (overlaps(ry, r)) return S5_ERR_INVALID_ARGUMENT;
    }
  }
  if (x_last && B > 0) {
    // the final state is written while other workgroups still read x0 and the
    // inputs: it may overlap none of them, nor y
    const Range rx = range_of(x_last, B * P * 8);
    const Range others[] = {tokens > 0 ? range_of(u, tokens * H * es) : Range{0, 0},
                            range_of(lambda, P * 8),
                            range_of(b_tilde, P * H * 8),
                            range_of(c_tilde, H * c_cols * 8),
                            range_of(d, H * 4),
                            log_delta ? range_of(log_delta, P * 4) : Range{0, 0},
                            delta && tokens > 0 ? range_of(delta, tokens * P * 4) : Range{0, 0},
                            tokens > 0 ? range_of(y, tokens * H * es) : Range{0, 0},
                            x0 ? range_of(x0, B * P * 8) : Range{0, 0}};
    for (const Range& r : others) {
      if (overlaps(rx, r)) return S5_ERR_INVALID_ARGUMENT;
    }
  }
  if (tokens == 0) {
    if (B > 0 && L == 0 && x_last) {
      const hipError_t e = s5::launch_state_passthrough(reinterpret_cast<const float2*>(x0),
                                                        reinterpret_cast<float2*>(x_last), B * P, stream);
      return e == hipSuccess ? S5_OK : S5_ERR_HIP;
    }
    return S5_OK;
  }

  s5::ForwardArgs a{};
  a.B = static_cast<int>(B);
  a.L = static_cast<int>(L);
  a.H = static_cast<int>(H);
  a.P = static_cast<int>(P);
  const bool io_bf16 = io == S5_BF16;
  const bool widen = io_bf16 && H <= kWidenMaxH;
  a.bf16_io = io_bf16 && !widen;
  a.time_varying = time_varying;
  a.u = u;
  a.lam = reinterpret_cast<const float2*>(lambda);
  a.b_tilde = reinterpret_cast<const float2*>(b_tilde);
  a.c_tilde = reinterpret_cast<const float2*>(c_tilde);
  a.d = d;
  a.log_delta = log_delta;
  a.delta = delta;
  a.y = y;
  a.x0 = reinterpret_cast<const float2*>(x0);
  a.xlast = reinterpret_cast<float2*>(x_last);
  a.c_scale = opt.c_scale;
  a.bilinear = opt.bilinear;
  a.gelu = opt.gelu;
  a.bidir = opt.bidir;
  a.c_ld = static_cast<int>(c_cols);
  // the gate inside the output pass where that pass's symmetric kernel
  // takes it (bf16 io, H <= 128, no backward scan), else after the layer
  bool glu_fused = opt.glu_w != nullptr && a.bf16_io && H <= 128 && !opt.bidir;
  if (glu_fused) {
    a.glu_w = opt.glu_w;
    a.glu_bias = opt.glu_bias;
    a.glu_variant = opt.glu_variant;
  }

  s5::ForwardLayout lay;
  if (!s5::forward_layout(a, lay)) return S5_ERR_UNSUPPORTED;
  if (glu_fused && !lay.plan.scan8) {
    // no symmetric output pass for this shape: the plain plan, gate after it
    glu_fused = false;
    a.glu_w = nullptr;
    a.glu_bias = nullptr;
    a.glu_variant = 0;
    if (!s5::forward_layout(a, lay)) return S5_ERR_UNSUPPORTED;
  }
  // every launch of the plan has a compiled kernel instance (a host-side walk
  // of the dispatch): otherwise refuse the call before anything is enqueued
  if (s5::launch_forward(a, lay, nullptr, stream, nullptr, 0, true) != hipSuccess) return S5_ERR_UNSUPPORTED;
  // widened bf16 I/O: float32 copies of u and y after the plan's scratch
  const size_t wide = widen ? align256(static_cast<size_t>(tokens) * H * sizeof(float)) : 0;
  const size_t total = lay.total + 2 * wide;
  // the float32 pass on the scratch copies, between the two conversions
  auto run = [&](void* base) -> hipError_t {
    if (!widen) return s5::launch_forward(a, lay, base, stream, tl_events, tl_nevents);
    float* u32 = reinterpret_cast<float*>(static_cast<char*>(base) + lay.total);
    float* y32 = reinterpret_cast<float*>(static_cast<char*>(base) + lay.total + wide);
    s5::ForwardArgs w = a;
    w.u = u32;
    w.y = y32;
    hipError_t e = s5::launch_widen_bf16(u, u32, tokens * H, stream);
    if (e == hipSuccess) e = s5::launch_forward(w, lay, base, stream, tl_events, tl_nevents);
    if (e == hipSuccess) e = s5::launch_narrow_bf16(y32, y, tokens * H, stream);
    return e;
  };
  if (noalloc) {
    // the fixed per-device array; the options path (backward scan) never comes here
    if (total > S5_NOALLOC_SCRATCH_BYTES || opt.bidir) return S5_ERR_UNSUPPORTED;
    void* fixed = nullptr;
    if (noalloc_scratch(&fixed) != hipSuccess) return S5_ERR_HIP;
    return run(fixed) == hipSuccess ? S5_OK : S5_ERR_HIP;
  }
  if (alloc_fail_hook()) return S5_ERR_OUT_OF_MEMORY;
  Scratch* ws = nullptr;
  hipError_t e = scratch_acquire(total, stream, &ws);
  if (e == hipErrorOutOfMemory) return S5_ERR_OUT_OF_MEMORY;
  if (e != hipSuccess) return S5_ERR_HIP;
  e = run(ws->ptr);
  if (e == hipSuccess && opt.glu_w != nullptr && !glu_fused) {
    s5::GluArgs g{};
    g.T = static_cast<int>(tokens);
    g.H = static_cast<int>(H);
    g.bf16_io = io_bf16;
    g.variant = opt.glu_variant;
    g.y = y;
    g.w = opt.glu_w;
    g.bias = opt.glu_bias;
    g.out = y;   // in place
    e = s5::launch_glu(g, stream);
  }
  const hipError_t ef = scratch_release(ws, stream);
  if (e != hipSuccess || ef != hipSuccess) return S5_ERR_HIP;
  return S5_OK;
}

}  // namespace

extern "C" {

s5_status s5_discretize(int64_t P, int64_t H, const s5_c64* lambda, const s5_c64* b_tilde,
                        const float* log_delta, s5_c64* lambda_bar, s5_c64* b_bar,
                        hipStream_t stream) {
  s5_status st = check_sizes(P, H);
  if (st != S5_OK) return st;
  if (!lambda || !b_tilde || !log_delta || !lambda_bar || !b_bar) return S5_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {lambda, b_tilde, log_delta, lambda_bar, b_bar};
  for (const void* p : ptrs) {
    if (!aligned16(p)) return S5_ERR_UNSUPPORTED;
  }
  const Range outs[] = {range_of(lambda_bar, P * 8), range_of(b_bar, P * H * 8)};
  const Range ins[] = {range_of(lambda, P * 8), range_of(b_tilde, P * H * 8),
                       range_of(log_delta, P * 4)};
  if (overlaps(outs[0], outs[1])) return S5_ERR_INVALID_ARGUMENT;
  for (const Range& o : outs) {
    for (const Range& i : ins) {
      if (overlaps(o, i)) return S5_ERR_INVALID_ARGUMENT;
    }
  }
  const hipError_t e = s5::launch_discretize(
      static_cast<int>(P), static_cast<int>(H), reinterpret_cast<const float2*>(lambda),
      reinterpret_cast<const float2*>(b_tilde), log_delta, reinterpret_cast<float2*>(lambda_bar),
      reinterpret_cast<float2*>(b_bar), stream);
  return e == hipSuccess ? S5_OK : S5_ERR_HIP;
}

s5_status s5_forward(int64_t B, int64_t L, int64_t H, int64_t P, s5_dtype io, const void* u,
                     const s5_c64* lambda, const s5_c64* b_tilde, const s5_c64* c_tilde,
                     const float* d, const float* log_delta, void* y, hipStream_t stream) {
  return forward_common(B, L, H, P, io, u, lambda, b_tilde, c_tilde, d, log_delta, nullptr, y,
                        false, nullptr, nullptr, Options{}, stream);
}

s5_status s5_forward_noalloc(int64_t B, int64_t L, int64_t H, int64_t P, s5_dtype io, const void* u,
                             const s5_c64* lambda, const s5_c64* b_tilde, const s5_c64* c_tilde,
                             const float* d, const float* log_delta, void* y, hipStream_t stream) {
  return forward_common(B, L, H, P, io, u, lambda, b_tilde, c_tilde, d, log_delta, nullptr, y,
                        false, nullptr, nullptr, Options{}, stream, true);
}

s5_status s5_forward_stateful(int64_t B, int64_t L, int64_t H, int64_t P, s5_dtype io, const void* u,
                              const s5_c64* lambda, const s5_c64* b_tilde, const s5_c64* c_tilde,
                              const float* d, const float* log_delta, const s5_c64* x0, void* y,
                              s5_c64* x_last, hipStream_t stream) {
  return forward_common(B, L, H, P, io, u, lambda, b_tilde, c_tilde, d, log_delta, nullptr, y,
                        false, x0, x_last, Options{}, stream);
}

s5_status s5_forward_timevarying(int64_t B, int64_t L, int64_t H, int64_t P, s5_dtype io,
                                 const void* u, const s5_c64* lambda, const s5_c64* b_tilde,
                                 const s5_c64* c_tilde, const float* d, const float* delta,
                                 void* y, hipStream_t stream) {
  return forward_common(B, L, H, P, io, u, lambda, b_tilde, c_tilde, d, nullptr, delta, y, true,
                        nullptr, nullptr, Options{}, stream);
}

s5_status s5_forward_timevarying_stateful(int64_t B, int64_t L, int64_t H, int64_t P, s5_dtype io,
                                          const void* u, const s5_c64* lambda, const s5_c64* b_tilde,
                                          const s5_c64* c_tilde, const float* d, const float* delta,
                                          const s5_c64* x0, void* y, s5_c64* x_last, hipStream_t stream) {
  return forward_common(B, L, H, P, io, u, lambda, b_tilde, c_tilde, d, nullptr, delta, y, true, x0,
                        x_last, Options{}, stream);
}

s5_status s5_forward_ex(const s5_forward_desc* x, hipStream_t stream) {
  if (x == nullptr) return S5_ERR_INVALID_ARGUMENT;
  const bool v1 = x->size == S5_FORWARD_DESC_SIZE_V1;   // a caller built before the gate fields
  if (!v1 && x->size != sizeof(s5_forward_desc)) return S5_ERR_INVALID_ARGUMENT;
  const uint32_t known = S5_FLAG_HALF_SPECTRUM | S5_FLAG_BILINEAR | S5_FLAG_GELU | S5_FLAG_BIDIRECTIONAL |
                         S5_FLAG_GELU_TANH | (v1 ? 0u : static_cast<uint32_t>(S5_FLAG_GLU));
  if ((x->flags & ~known) != 0) return S5_ERR_INVALID_ARGUMENT;
  if ((x->flags & S5_FLAG_GELU) && (x->flags & S5_FLAG_GELU_TANH)) return S5_ERR_INVALID_ARGUMENT;
  if ((x->log_delta == nullptr) == (x->delta == nullptr)) return S5_ERR_INVALID_ARGUMENT;
  Options o;
  o.c_scale = (x->flags & S5_FLAG_HALF_SPECTRUM) ? 2.0f : 1.0f;
  o.bilinear = (x->flags & S5_FLAG_BILINEAR) != 0;
  o.gelu = (x->flags & S5_FLAG_GELU) ? 1 : (x->flags & S5_FLAG_GELU_TANH) ? 2 : 0;
  o.bidir = (x->flags & S5_FLAG_BIDIRECTIONAL) != 0;
  if (x->flags & S5_FLAG_GLU) {
    // the gate applies its own GELU: no GELU form beside it
    if (o.gelu != 0 || x->glu_w == nullptr || (x->glu_variant != 1 && x->glu_variant != 2))
      return S5_ERR_INVALID_ARGUMENT;
    o.glu_w = x->glu_w;
    o.glu_bias = x->glu_bias;
    o.glu_variant = x->glu_variant;
  }
  return forward_common(x->B, x->L, x->H, x->P, x->io, x->u, x->lambda, x->b_tilde, x->c_tilde, x->d,
                        x->log_delta, x->delta, x->y, x->delta != nullptr, x->x0, x->x_last, o, stream);
}

s5_status s5_step(int64_t B, int64_t H, int64_t P, s5_dtype io, uint32_t flags, const void* u,
                  const s5_c64* lambda, const s5_c64* b_tilde, const s5_c64* c_tilde, const float* d,
                  const float* log_delta, const float* delta, s5_c64* x, void* y, hipStream_t stream) {
  if (B < 0) return S5_ERR_INVALID_ARGUMENT;
  s5_status st = check_sizes(P, H);
  if (st != S5_OK) return st;
  if (io != S5_F32 && io != S5_BF16) return S5_ERR_UNSUPPORTED;
  const uint32_t known = S5_FLAG_HALF_SPECTRUM | S5_FLAG_BILINEAR | S5_FLAG_GELU | S5_FLAG_GELU_TANH;
  if ((flags & ~known) != 0) return S5_ERR_INVALID_ARGUMENT;   // no backward scan in a single step
  if ((flags & S5_FLAG_GELU) && (flags & S5_FLAG_GELU_TANH)) return S5_ERR_INVALID_ARGUMENT;
  if ((log_delta == nullptr) == (delta == nullptr)) return S5_ERR_INVALID_ARGUMENT;
  if (!lambda || !b_tilde || !c_tilde || !d) return S5_ERR_INVALID_ARGUMENT;
  if (B > 0 && (!u || !x || !y)) return S5_ERR_INVALID_ARGUMENT;
  if (B > INT32_MAX / (H > P ? H : P)) return S5_ERR_UNSUPPORTED;
  const void* ptrs[] = {u, lambda, b_tilde, c_tilde, d, log_delta, delta, x, y};
  for (const void* p : ptrs) {
    if (p && !aligned16(p)) return S5_ERR_UNSUPPORTED;
  }
  if (B == 0) return S5_OK;
  const int64_t es = io == S5_BF16 ? 2 : 4;
  // x is read and written in place; y and x may overlap no input and not each other
  const Range rx = range_of(x, B * P * 8), ry = range_of(y, B * H * es);
  const Range inputs[] = {range_of(u, B * H * es), range_of(lambda, P * 8), range_of(b_tilde, P * H * 8),
                          range_of(c_tilde, H * P * 8), range_of(d, H * 4),
                          log_delta ? range_of(log_delta, P * 4) : Range{0, 0},
                          delta ? range_of(delta, B * P * 4) : Range{0, 0}};
  if (overlaps(rx, ry)) return S5_ERR_INVALID_ARGUMENT;
  for (const Range& r : inputs) {
    if (overlaps(rx, r) || overlaps(ry, r)) return S5_ERR_INVALID_ARGUMENT;
  }
  s5::StepArgs a{};
  a.B = static_cast<int>(B);
  a.H = static_cast<int>(H);
  a.P = static_cast<int>(P);
  a.bf16_io = io == S5_BF16;
  a.bilinear = (flags & S5_FLAG_BILINEAR) != 0;
  a.gelu = (flags & S5_FLAG_GELU) ? 1 : (flags & S5_FLAG_GELU_TANH) ? 2 : 0;
  a.c_scale = (flags & S5_FLAG_HALF_SPECTRUM) ? 2.0f : 1.0f;
  a.u = u;
  a.lam = reinterpret_cast<const float2*>(lambda);
  a.b_tilde = reinterpret_cast<const float2*>(b_tilde);
  a.c_tilde = reinterpret_cast<const float2*>(c_tilde);
  a.d = d;
  a.log_delta = log_delta;
  a.delta = delta;
  a.x = reinterpret_cast<float2*>(x);
  a.y = y;
  return s5::launch_step(a, stream) == hipSuccess ? S5_OK : S5_ERR_HIP;
}

s5_status s5_glu(int64_t T, int64_t H, s5_dtype io, int variant, const void* y, const float* w,
                 const float* bias, void* out, hipStream_t stream) {
  if (T < 0 || H < 1) return S5_ERR_INVALID_ARGUMENT;
  if (H > S5_GLU_MAX_H || T > INT32_MAX / H) return S5_ERR_UNSUPPORTED;
  if (io != S5_F32 && io != S5_BF16) return S5_ERR_UNSUPPORTED;
  if (variant != 1 && variant != 2) return S5_ERR_INVALID_ARGUMENT;
  if (!w || (T > 0 && (!y || !out))) return S5_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {y, w, bias, out};
  for (const void* p : ptrs) {
    if (p && !aligned16(p)) return S5_ERR_UNSUPPORTED;
  }
  if (T == 0) return S5_OK;
  const int64_t es = io == S5_BF16 ? 2 : 4;
  const Range ro = range_of(out, T * H * es), ry = range_of(y, T * H * es);
  // out may be y itself (in place); otherwise it overlaps no input
  if (out != y && overlaps(ro, ry)) return S5_ERR_INVALID_ARGUMENT;
  if (overlaps(ro, range_of(w, H * H * 4))) return S5_ERR_INVALID_ARGUMENT;
  if (bias && overlaps(ro, range_of(bias, H * 4))) return S5_ERR_INVALID_ARGUMENT;
  s5::GluArgs a{};
  a.T = static_cast<int>(T);
  a.H = static_cast<int>(H);
  a.bf16_io = io == S5_BF16;
  a.variant = variant;
  a.y = y;
  a.w = w;
  a.bias = bias;
  a.out = out;
  return s5::launch_glu(a, stream) == hipSuccess ? S5_OK : S5_ERR_HIP;
}

const char* s5_status_string(s5_status s) {
  switch (s) {
    case S5_OK: return "S5_OK";
    case S5_ERR_INVALID_ARGUMENT: return "S5_ERR_INVALID_ARGUMENT";
    case S5_ERR_UNSUPPORTED: return "S5_ERR_UNSUPPORTED";
    case S5_ERR_OUT_OF_MEMORY: return "S5_ERR_OUT_OF_MEMORY";
    case S5_ERR_HIP: return "S5_ERR_HIP";
  }
  return "S5_ERR_UNKNOWN";
}

s5_status s5_set_profiling_events(const hipEvent_t* events, int count) {
  if (count < 0 || count > S5_PROFILING_MAX_EVENTS || (count & 1) != 0) return S5_ERR_INVALID_ARGUMENT;
  if (count > 0 && events == nullptr) return S5_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < count; ++i) {
    if (events[i] == nullptr) return S5_ERR_INVALID_ARGUMENT;
  }
  for (int i = 0; i < S5_PROFILING_MAX_EVENTS; ++i) tl_events[i] = i < count ? events[i] : nullptr;
  tl_nevents = count;
  return S5_OK;
}

}  // extern "C"
