// Host side of the S5 forward path: workspace layout and the two launches
// (parameter packing, then the fused chunk kernel), both on the caller's stream.
#include "s5_fused.h"
#include "s5_internal.h"

namespace s5 {

namespace {

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Layout {
  int Ppad, Hpad, T, nch;
  size_t bpack, cpack, modes, flags, ticket, agg, agg_a, incl, total;
};

Layout layout(const ForwardArgs& a) {
  Layout l{};
  l.Ppad = ((a.P + 63) / 64) * 64;
  l.Hpad = ((a.H + 31) / 32) * 32;
  l.T = fused_chunk_tokens(a.bf16_io, a.time_varying, l.Ppad, l.Hpad);
  if (l.T == 0) return l;
  l.nch = (a.L + l.T - 1) / l.T;
  const size_t planes = a.bf16_io ? 1 : 2;
  const size_t nb = static_cast<size_t>(l.Ppad / 16) * 2 * (l.Hpad / 32) * 64;
  const size_t nc = static_cast<size_t>(l.Hpad / 16) * (2 * l.Ppad / 32) * 64;
  const size_t nflags = static_cast<size_t>(a.B) * l.nch;
  const size_t nagg = nflags * l.Ppad;
  size_t off = 0;
  l.bpack = off;  off += align_up(planes * nb * 16);
  l.cpack = off;  off += align_up(planes * nc * 16);
  l.modes = off;  off += align_up(l.Ppad * sizeof(ModeParams));
  l.flags = off;  off += align_up(nflags * sizeof(unsigned));
  l.ticket = off; off += align_up(sizeof(unsigned));
  l.agg = off;    off += align_up(nagg * sizeof(float2));
  l.agg_a = off;  off += a.time_varying ? align_up(nagg * sizeof(float2)) : 0;
  l.incl = off;   off += align_up(nagg * sizeof(float2));
  l.total = off;
  return l;
}

}  // namespace

size_t forward_workspace_bytes(const ForwardArgs& a) {
  const Layout l = layout(a);
  return l.T == 0 ? 0 : l.total;
}

bool forward_supported(const ForwardArgs& a) { return layout(a).T != 0; }

hipError_t launch_forward(const ForwardArgs& a, void* ws, hipStream_t stream, hipEvent_t ev_start,
                          hipEvent_t ev_stop) {
  const Layout l = layout(a);
  if (l.T == 0) return hipErrorInvalidValue;
  char* base = static_cast<char*>(ws);
  FusedParams q{};
  q.B = a.B; q.L = a.L; q.H = a.H; q.P = a.P;
  q.Hpad = l.Hpad; q.Ppad = l.Ppad;
  q.T = l.T; q.R = l.T / 16;
  q.nch = l.nch;
  q.nflags = a.B * l.nch;
  q.bf16_io = a.bf16_io;
  q.time_varying = a.time_varying;
  q.spin_limit = 1u << 24;
  q.u = a.u; q.y = a.y;
  q.lam = a.lam; q.b_tilde = a.b_tilde; q.c_tilde = a.c_tilde;
  q.d = a.d; q.log_delta = a.log_delta; q.delta = a.delta;
  q.bpack = reinterpret_cast<uint4*>(base + l.bpack);
  q.cpack = reinterpret_cast<uint4*>(base + l.cpack);
  q.modes = reinterpret_cast<ModeParams*>(base + l.modes);
  q.flags = reinterpret_cast<unsigned*>(base + l.flags);
  q.ticket = reinterpret_cast<unsigned*>(base + l.ticket);
  q.agg = reinterpret_cast<float2*>(base + l.agg);
  q.agg_a = a.time_varying ? reinterpret_cast<float2*>(base + l.agg_a) : nullptr;
  q.incl = reinterpret_cast<float2*>(base + l.incl);
  hipError_t e = launch_pack(q, stream);
  if (e != hipSuccess) return e;
  return launch_fused(q, stream, ev_start, ev_stop);
}

}  // namespace s5
