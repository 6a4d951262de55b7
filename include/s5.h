/*
 * s5.h - C ABI of the S5 layer forward hot path on AMD Instinct MI355X (gfx950).
 *
 * The S5 layer ("Simplified State Space Layers for Sequence Modeling", Smith,
 * Warrington & Linderman, ICLR 2023) maps an input sequence u_k in R^H to
 * pre-activation outputs y_k in R^H through a diagonal complex linear state
 * x_k in C^P:
 *
 *   zero-order hold (paper eq. 6; App. A `discretize`):
 *       Lambda_bar = exp(Lambda * Delta),
 *       B_bar      = ((Lambda_bar - 1) / Lambda)[:, None] * B~
 *   recurrence (paper eq. 2, evaluated as an associative scan, Sec. 2.2/App. H):
 *       x_k = Lambda_bar * x_{k-1} + B_bar u_k,    x_{-1} = 0
 *   readout with diagonal feedthrough (App. A `apply_ssm`; paper eq. 5):
 *       y_k = Re(C~ x_k) + D * u_k          (full spectrum, factor 1)
 *
 * The time-varying variant (paper Sec. 3.3 and 6.3: a different
 * discretisation for every observation interval) uses one interval per
 * (batch, step, mode): Lambda_bar_k = exp(Lambda * Delta_k) and
 * B_bar_k = ((Lambda_bar_k - 1)/Lambda)[:, None] * B~ with the interval Delta_k
 * that ends at step k.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array pointer is a DEVICE pointer to caller-owned, contiguous,
 *   row-major memory, aligned to at least 16 bytes. The library never frees
 *   or retains a caller pointer after the call returns.
 * - Complex values are interleaved (re, im) float32 pairs: `s5_c64`, the
 *   layout of torch.complex64 and numpy.complex64.
 * - Every call is asynchronous on `stream` (NULL = the null stream) and does
 *   not synchronise the host (except when it allocates scratch, below).
 *   Internal scratch memory comes from buffers the library keeps for reuse:
 *   a buffer belongs to the stream of its last use and later calls on that
 *   stream reuse it; a call on another stream has hipMalloc add one (which
 *   may synchronise). Buffers live until the process ends: one per stream
 *   the library was called on, at most 64, each as large as the largest
 *   scratch asked for on it so far (a few MB at the benchmark sizes); past
 *   64, a call waits for the device once and takes over another stream's
 *   buffer. A stream must not be destroyed while work the library enqueued
 *   on it is still executing (synchronise it first).
 * - Arguments are validated on the host before anything is enqueued; a call
 *   that returns an error has enqueued nothing. Errors of kernels that run
 *   later surface at the caller's next synchronisation with the stream.
 * - Device data is not inspected: intervals must be finite and >= 0 (the
 *   pages reject other intervals); NaN or Inf inputs propagate causally
 *   (a bad u[b,k,:] affects only y[b,k',:] with k' >= k).
 * - The output y must not overlap any input.
 * - Calls are re-entrant and may run concurrently on different streams.
 */
#ifndef S5_H
#define S5_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque HIP handles, declared identically to hip_runtime_api.h. */
typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;

typedef struct {
  float re;
  float im;
} s5_c64;

/* Element type of u and y (both have the same type). */
typedef enum { S5_F32 = 0, S5_BF16 = 1 } s5_dtype;

typedef enum {
  S5_OK = 0,
  S5_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, overlapping output */
  S5_ERR_UNSUPPORTED = 2,      /* dtype, size limit or alignment not supported, or
                                  no compiled kernel for the call (checked on the
                                  host before anything is enqueued; no call within
                                  the size limits meets it) */
  S5_ERR_OUT_OF_MEMORY = 3,    /* scratch allocation failed */
  S5_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed */
} s5_status;

/* Size limits of the compiled kernels. */
#define S5_MAX_P 256  /* complex modes */
#define S5_MAX_H 512  /* input/output features */

/*
 * s5_discretize - zero-order hold of the diagonal system (paper eq. 6;
 * App. A `discretize`; abhik.ai review, row 2 "Integrate a held input
 * exactly").
 *
 *   P, H        number of complex modes (1..S5_MAX_P), features (1..S5_MAX_H)
 *   lambda      [P]    continuous eigenvalues Lambda
 *   b_tilde     [P,H]  input matrix B~
 *   log_delta   [P]    float32 log of the per-mode interval, Delta = exp(.)
 *   lambda_bar  [P]    out: exp(Lambda * Delta)
 *   b_bar       [P,H]  out: ((Lambda_bar - 1)/Lambda) * B~ row-wise; for
 *                      |Lambda*Delta| < 1e-4 the gain is Delta*phi1(Lambda*Delta)
 *                      (the removable singularity at Lambda = 0 gives Delta)
 * Internally float64; outputs rounded to float32.
 * Errors: S5_ERR_INVALID_ARGUMENT for a null pointer or P, H < 1;
 *         S5_ERR_UNSUPPORTED for P > S5_MAX_P or H > S5_MAX_H or misalignment.
 */
s5_status s5_discretize(int64_t P, int64_t H, const s5_c64* lambda, const s5_c64* b_tilde,
                        const float* log_delta, s5_c64* lambda_bar, s5_c64* b_bar,
                        hipStream_t stream);

/*
 * s5_forward - time-invariant S5 forward pass (App. A `apply_ssm` composed
 * with `discretize`; per-mode intervals Delta = exp(log_delta), paper Sec. 3.2).
 *
 *   B, L        batch size and sequence length (>= 0; B*L == 0 is a no-op)
 *   H, P        features (1..S5_MAX_H) and complex modes (1..S5_MAX_P)
 *   io          element type of u and y
 *   u           [B,L,H] input
 *   lambda      [P]     continuous eigenvalues
 *   b_tilde     [P,H]   input matrix B~
 *   c_tilde     [H,P]   output matrix C~
 *   d           [H]     float32 diagonal feedthrough D
 *   log_delta   [P]     float32 log interval per mode
 *   y           [B,L,H] out: pre-activation Re(C~ x_k) + D u_k, rounded to
 *                       `io` (bf16: round to nearest even)
 * Precision: the state and all accumulation are float32. Products with B_bar
 * and C~ run on the matrix cores: bf16 operands for bf16 io; for float32 io
 * each float32 operand is split into a high and a low bf16 part and three
 * products are summed (about 2^-16 relative per product). bf16 io with
 * H <= 8 is computed as float32 io (u widened, y rounded to bf16 once, with
 * 8*B*L*H bytes more scratch): with so few outputs a readout over many modes
 * can cancel far below its terms, where bf16 operands would show.
 * Errors: S5_ERR_INVALID_ARGUMENT (null pointer, negative B or L, P or H < 1,
 * y overlapping an input), S5_ERR_UNSUPPORTED (unknown io, size limits,
 * misalignment), S5_ERR_OUT_OF_MEMORY, S5_ERR_HIP.
 */
s5_status s5_forward(int64_t B, int64_t L, int64_t H, int64_t P, s5_dtype io, const void* u,
                     const s5_c64* lambda, const s5_c64* b_tilde, const s5_c64* c_tilde,
                     const float* d, const float* log_delta, void* y, hipStream_t stream);

/*
 * s5_forward_timevarying - S5 forward pass with one interval per
 * (batch, step, mode), for irregularly sampled sequences (paper Sec. 3.3
 * "provide a different Lambda_bar_k at each step" and Sec. 6.3; abhik.ai
 * review, "Sampling intervals carry physical meaning").
 *
 * Arguments as s5_forward, except
 *   delta       [B,L,P] float32 interval Delta_k for step k and mode p
 *               (precondition: finite and >= 0; a zero interval is the
 *               identity step with zero input gain)
 * Step k uses Delta_k in both Lambda_bar_k and B_bar_k.
 * Errors: as s5_forward.
 */
s5_status s5_forward_timevarying(int64_t B, int64_t L, int64_t H, int64_t P, s5_dtype io,
                                 const void* u, const s5_c64* lambda, const s5_c64* b_tilde,
                                 const s5_c64* c_tilde, const float* d, const float* delta,
                                 void* y, hipStream_t stream);

/*
 * s5_forward_stateful / s5_forward_timevarying_stateful - the forward passes
 * above, started from a given state and reporting the state after the last
 * step, so that a long sequence can be processed in pieces (or step by step)
 * with the state carried between calls: running [0, L1) and then [L1, L) with
 * the first call's x_last as the second call's x0 gives the outputs of one
 * run over [0, L), up to rounding. (abhik.ai review, "Associative scans
 * preserve the recurrence": a nonzero initial state enters every prefix
 * through its transition part; streaming keeps only the current state,
 * paper Sec. 2.2 and 3.4; papercache notes Sec. 3.3, online generation.)
 *
 * Arguments as s5_forward / s5_forward_timevarying, plus
 *   x0          [B,P] state before step 0 (x_{-1}); NULL = zero state
 *   x_last      [B,P] out: the state after step L-1 (x_{L-1}); NULL = not
 *               written. L = 0 copies x0 (or zeros) to it.
 * Both complex64, 16-byte aligned. x_last may overlap no input, not y and
 * not x0 (update a state in place by alternating two buffers); x0 may not
 * overlap y.
 * Precision: as s5_forward; x_last is float32 (time-invariant: the
 * transition over the last stream's steps is evaluated in float64).
 * Errors: as s5_forward.
 */
s5_status s5_forward_stateful(int64_t B, int64_t L, int64_t H, int64_t P, s5_dtype io, const void* u,
                              const s5_c64* lambda, const s5_c64* b_tilde, const s5_c64* c_tilde,
                              const float* d, const float* log_delta, const s5_c64* x0, void* y,
                              s5_c64* x_last, hipStream_t stream);
s5_status s5_forward_timevarying_stateful(int64_t B, int64_t L, int64_t H, int64_t P, s5_dtype io,
                                          const void* u, const s5_c64* lambda, const s5_c64* b_tilde,
                                          const s5_c64* c_tilde, const float* d, const float* delta,
                                          const s5_c64* x0, void* y, s5_c64* x_last, hipStream_t stream);

/*
 * s5_forward_ex - the forward pass with its options, described by one struct
 * (all entry points above are special cases of it).
 *
 * Options (desc->flags, any combination unless noted):
 *   S5_FLAG_HALF_SPECTRUM  the P stored modes are one partner of each
 *       conjugate pair: y_k = 2 Re(C~ x_k) + D u_k, the feedthrough not
 *       doubled (abhik.ai review, row 4 "Reconstruct real outputs and keep
 *       the direct path"; wikillm notes, "Paper vs code", readout factor 2).
 *   S5_FLAG_BILINEAR  bilinear discretisation instead of zero-order hold:
 *       with z = Lambda*Delta, Lambda_bar = (1 + z/2)/(1 - z/2) and
 *       B_bar = Delta/(1 - z/2) * B~ (intuitivepapers S4 notes,
 *       "Discretization and the step size"; abhik.ai review: the official
 *       code offers it as an alternative). Time-invariant or time-varying.
 *   S5_FLAG_GELU  y is GELU of the pre-activation, y * Phi(y) with the
 *       standard normal distribution function Phi (the function's definition;
 *       papercache notes App. A `apply_S5_layer` applies a GELU to the
 *       pre-activations), in float32 with erf from Abramowitz & Stegun
 *       7.1.26 (absolute error < 1.5e-7).
 *   S5_FLAG_GELU_TANH  y is the tanh approximation of GELU,
 *       y/2 (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))), the form the App. A
 *       listing's library call computes by default; within 5e-4 of the exact
 *       form. Exclusive with S5_FLAG_GELU.
 *   S5_FLAG_BIDIRECTIONAL  a second, backward scan over the same Lambda_bar
 *       and B_bar, x'_k = Lambda_bar x'_{k+1} + B_bar u_k from x'_L = 0,
 *       read out by the second half of C~, which then has 2P columns:
 *       y_k = Re(C~[:, :P] x_k) + Re(C~[:, P:] x'_k) + D u_k (wikillm
 *       notes, "Paper vs code", bidirectional scans). Time-invariant only,
 *       without x0/x_last. The forward half is kept in float32 (for bf16
 *       io in library scratch of 4*B*L*H bytes), so y is rounded once.
 *   S5_FLAG_GLU  the gated activation of s5_glu applied to the layer's
 *       output, out = (GELU(y) or y) * sigma(W GELU(y) + bias) with W =
 *       glu_w, bias = glu_bias (NULL: none), variant glu_variant (1 or 2),
 *       written to y. For bf16 io with H <= 128 and without the backward
 *       scan it runs inside the output pass (y is stored once, gated);
 *       otherwise as s5_glu on y in place after the layer. Either way the
 *       gate reads y as the layer stores it (rounded to bf16 for bf16 io)
 *       and gives the bits of s5_glu on that y. H <= S5_GLU_MAX_H.
 *       Scratch: 4*H*H bytes more (W's packed operand planes) when fused.
 *       Exclusive with S5_FLAG_GELU and S5_FLAG_GELU_TANH (the gate applies
 *       its own GELU, the exact form).
 *
 * Fields of s5_forward_desc:
 *   size        sizeof(s5_forward_desc) (for later extension)
 *   flags       S5_FLAG_* bits; unknown bits are rejected
 *   io, B, L, H, P, u, lambda, b_tilde, d, y   as s5_forward
 *   c_tilde     [H,P], or [H,2P] with S5_FLAG_BIDIRECTIONAL
 *   log_delta   [P] per-mode log interval (time-invariant), or NULL
 *   delta       [B,L,P] per-step interval (time-varying), or NULL;
 *               exactly one of log_delta and delta is given
 *   x0, x_last  as s5_forward_stateful (NULL: zero / not written)
 *   glu_w, glu_bias, glu_variant   with S5_FLAG_GLU: W [H,H] float32
 *               (output j reads row j), bias [H] float32 or NULL, 1 or 2;
 *               ignored without it. A caller built before these fields may
 *               pass size = S5_FORWARD_DESC_SIZE_V1 (then no S5_FLAG_GLU).
 * Errors: as s5_forward_stateful; S5_ERR_INVALID_ARGUMENT for a wrong size
 * field, unknown flags, both GELU forms or a GELU form with the gate, both or
 * neither interval arrays, S5_FLAG_BIDIRECTIONAL with delta, x0 or x_last,
 * or S5_FLAG_GLU without glu_w, with another variant or with glu_w or
 * glu_bias overlapping y; S5_ERR_UNSUPPORTED for S5_FLAG_GLU with
 * H > S5_GLU_MAX_H.
 */
enum {
  S5_FLAG_HALF_SPECTRUM = 1u << 0,
  S5_FLAG_BILINEAR = 1u << 1,
  S5_FLAG_GELU = 1u << 2,
  S5_FLAG_BIDIRECTIONAL = 1u << 3,
  S5_FLAG_GELU_TANH = 1u << 4,
  S5_FLAG_GLU = 1u << 5
};

typedef struct {
  uint32_t size;
  uint32_t flags;
  s5_dtype io;
  int64_t B, L, H, P;
  const void* u;
  const s5_c64* lambda;
  const s5_c64* b_tilde;
  const s5_c64* c_tilde;
  const float* d;
  const float* log_delta;
  const float* delta;
  const s5_c64* x0;
  void* y;
  s5_c64* x_last;
  /* fields added after the first version (see S5_FORWARD_DESC_SIZE_V1) */
  const float* glu_w;
  const float* glu_bias;
  int32_t glu_variant;
} s5_forward_desc;

/* size of s5_forward_desc up to x_last, the first version of the struct */
#define S5_FORWARD_DESC_SIZE_V1 ((uint32_t)offsetof(s5_forward_desc, glu_w))

s5_status s5_forward_ex(const s5_forward_desc* desc, hipStream_t stream);

/*
 * s5_step - one recurrent step for B sequences: the online form, which keeps
 * only the current state (abhik.ai review, "Associative scans preserve the
 * recurrence": streaming keeps one state per layer, paper Sec. 2.2/3.4;
 * papercache notes Sec. 3.3, online generation):
 *     x <- Lambda_bar x + B_bar u,    y = Re(C~ x) + D u
 * with the discretisation of s5_forward (log_delta, per-mode) or of
 * s5_forward_timevarying (delta, this step's interval per sequence and mode).
 * Equal, up to rounding, to s5_forward_stateful / s5_forward_ex over L = 1
 * with x0 = x and x_last written back to x.
 *
 *   B, H, P     sequences (>= 0; 0 is a no-op), features, complex modes
 *   io          element type of u and y
 *   flags       S5_FLAG_HALF_SPECTRUM, S5_FLAG_BILINEAR, S5_FLAG_GELU or
 *               S5_FLAG_GELU_TANH (as in s5_forward_ex);
 *               S5_FLAG_BIDIRECTIONAL is rejected
 *   u           [B,H]  this step's input
 *   lambda, b_tilde [P,H], c_tilde [H,P], d [H]   as s5_forward
 *   log_delta   [P] per-mode log interval, or NULL
 *   delta       [B,P] this step's interval, or NULL (exactly one is given)
 *   x           [B,P] complex64 state, read and overwritten in place
 *   y           [B,H]  out
 * Precision: float32 state and sums on the vector units (no bf16 operands);
 * time-invariant discretisation in float64, per-step intervals in float32.
 * x and y may overlap no input and not each other.
 * Errors: S5_ERR_INVALID_ARGUMENT (null pointer, B < 0, P or H < 1, unknown
 * or bidirectional flag, both or neither interval arrays, overlaps),
 * S5_ERR_UNSUPPORTED (io, size limits, misalignment), S5_ERR_HIP.
 */
s5_status s5_step(int64_t B, int64_t H, int64_t P, s5_dtype io, uint32_t flags, const void* u,
                  const s5_c64* lambda, const s5_c64* b_tilde, const s5_c64* c_tilde, const float* d,
                  const float* log_delta, const float* delta, s5_c64* x, void* y, hipStream_t stream);

/*
 * s5_glu - the gated activation that follows the layer in the S5 network
 * (wikillm notes, "Paper vs code": GLU variant and dense gate bias; the
 * pseudocode's half_glu1 step), for T tokens of H features:
 *     g = GELU(y),  gate = sigma(W g + bias)      (sigma: logistic function)
 *     variant 1: out = g * gate     (the paper's gate)
 *     variant 2: out = y * gate     (the un-activated y gated)
 *
 *   T, H        tokens (>= 0; 0 is a no-op) and features (1..S5_GLU_MAX_H)
 *   io          element type of y and out
 *   variant     1 or 2
 *   y           [T,H]  input (e.g. the y of s5_forward with B*L tokens)
 *   w           [H,H]  float32, row-major: output j reads w[j, :]
 *   bias        [H]    float32, or NULL for none
 *   out         [T,H]  out; may be y itself (in place), else overlaps no input
 * Precision: W g on the matrix cores from the bf16 hi/lo split of both
 * float32 operands with three products (relative error below 2^-15 of
 * sum |W||g|, for either io); float32 sums, GELU and gate.
 * Errors: S5_ERR_INVALID_ARGUMENT (null pointer, T < 0, H < 1, variant not
 * 1 or 2, overlaps), S5_ERR_UNSUPPORTED (io, H > S5_GLU_MAX_H,
 * misalignment), S5_ERR_HIP.
 */
#define S5_GLU_MAX_H 256
s5_status s5_glu(int64_t T, int64_t H, s5_dtype io, int variant, const void* y, const float* w,
                 const float* bias, void* out, hipStream_t stream);

/*
 * s5_forward_noalloc - s5_forward for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid hipMalloc. Same arguments, same kernels, same results (bit for
 * bit) as s5_forward; the scratch memory (packed operands and the per-range
 * aggregates) comes from a fixed array of S5_NOALLOC_SCRATCH_BYTES that the
 * library holds on each device it runs on until the process ends, instead
 * of from the library's hipMalloc'd buffers. Nothing is allocated, by this
 * call or by anything it calls.
 *
 * Every call on one device uses that device's one array: calls that overlap
 * on a device (on different streams, or from different host threads without
 * ordering) race and must be serialised by the caller; calls in order on one
 * stream are safe. No part of the array needs to start at zero.
 * The scratch a call needs grows with the number of sequence ranges the
 * kernels split the work into (about max(B, 256) ranges of 16 token streams)
 * times the padded mode count: about 9.6 MB at B = 16, P = 256. Larger needs
 * return S5_ERR_UNSUPPORTED before anything is enqueued.
 * Errors: as s5_forward, plus S5_ERR_UNSUPPORTED when the call needs more
 * than S5_NOALLOC_SCRATCH_BYTES of scratch.
 */
#define S5_NOALLOC_SCRATCH_BYTES (32u << 20)
s5_status s5_forward_noalloc(int64_t B, int64_t L, int64_t H, int64_t P, s5_dtype io, const void* u,
                             const s5_c64* lambda, const s5_c64* b_tilde, const s5_c64* c_tilde,
                             const float* d, const float* log_delta, void* y, hipStream_t stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* s5_status_string(s5_status s);

/*
 * s5_set_profiling_events - measurement hook for benchmarks. `events` holds
 * `count` caller-owned events (count even, 0..S5_PROFILING_MAX_EVENTS). Every
 * later s5_forward / s5_forward_timevarying call made from the calling host
 * thread records events[2k] on its stream right before its k-th kernel launch
 * and events[2k+1] right after it, for k < count/2, so that
 * hipEventElapsedTime gives that kernel's duration alone. The launches of one
 * forward call are, in order: k = 0 parameter packing (discretisation and
 * operand layouts), k = 1 the aggregate pass (state of every token range from
 * a zero start), k = 2 the state and output pass; the bidirectional form of
 * s5_forward_ex adds k = 3..5, the same three for the backward scan. count 0
 * turns the hook off. (Also recorded by s5_forward_stateful,
 * s5_forward_timevarying_stateful and s5_forward_ex.)
 * The handles are copied; the events stay owned by the caller and must
 * outlive the calls that record them. The setting is per host thread.
 * Errors: S5_ERR_INVALID_ARGUMENT for an odd or out-of-range count, a NULL
 * array with count > 0, or a NULL handle among the first count.
 */
#define S5_PROFILING_MAX_EVENTS 12
s5_status s5_set_profiling_events(const hipEvent_t* events, int count);

#ifdef __cplusplus
}
#endif

#endif /* S5_H */
