"""Seeded synthetic inputs for the S5 forward path.

This module is shared by the tests, the benchmark and the oracle checks. It
holds only input generation: the HiPPO-N starting spectrum, parameter draws and
the five S5-shaped workloads. It holds none of the forward computation
(discretisation, projection, scan or readout); those live in the HIP library
and, independently, in the float64 oracle.

Sources for the recipes (cited by page title and section):

* HiPPO-N matrix A_N = A_LegS + p p^T with p_n = sqrt(n + 1/2): diagonal -1/2,
  skew-symmetric off-diagonal entries ("S5: Simplified State Space Layers for
  Sequence Modeling", abhik.ai review, row 5 "Build the normal starting matrix";
  S4 review on intuitivepapers.ai, section on the NPLR decomposition).
* Lambda = -1/2 + i*omega with omega the eigenvalues of -i*S, S = A_N + I/2,
  real part fixed at -1/2 (wikillm notes on arXiv 2208.04933, "Paper vs code",
  eigenvalue initialisation; paper App. B.1.1).
* Block-diagonal initialisation: J copies of an R x R HiPPO-N block
  (paper App. B.1.1, J hyperparameter).
* D ~ N(0, 1) (paper App. B.1.2); log Delta ~ U[log dmin, log dmax) with
  defaults 1e-3..1e-1 and 1e-4..1e-1 for Path-X (paper App. B.1.3).
* B~ and C~ sampled directly as complex normals with E|z|^2 = 1/H (the Path-X
  complex_normal option noted in "Paper vs code"); real and imaginary parts are
  i.i.d. N(0, 1/(2H)).

Draw order for every config with one numpy Generator(PCG64) seeded with
``seed``: B~.re, B~.im, C~.re, C~.im, D, log Delta, then the config-specific
draws in the order listed in ``_draw_inputs``.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "S5Workload",
    "CONFIG_SPECS",
    "hippo_legs",
    "hippo_normal",
    "hippo_n_eigenvalues",
    "block_lambda",
    "bf16_round",
    "bf16_bits",
    "make_config",
    "make_random",
]


# --------------------------------------------------------------------------
# bfloat16 helpers (storage format only: round-to-nearest-even from fp32)
# --------------------------------------------------------------------------

def bf16_bits(x) -> np.ndarray:
    """Round to bfloat16 (round to nearest, ties to even) and return the 16-bit
    patterns as uint16. Input is first rounded to float32."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    nan = np.isnan(f)
    out = r.astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Expand uint16 bfloat16 patterns to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x) -> np.ndarray:
    """Values of ``x`` after rounding to bfloat16, as float32."""
    return bf16_to_f32(bf16_bits(x))


# --------------------------------------------------------------------------
# HiPPO-N starting spectrum
# --------------------------------------------------------------------------

def hippo_legs(n: int) -> np.ndarray:
    """HiPPO-LegS state matrix: -(2i+1)^1/2 (2j+1)^1/2 below the diagonal,
    -(i+1) on it, 0 above it (S4 review, HiPPO section)."""
    if n < 1:
        raise ValueError("state size must be positive")
    idx = np.arange(n, dtype=np.float64)
    q = np.sqrt(2.0 * idx + 1.0)
    a = -np.outer(q, q)
    a = np.tril(a, -1)
    a[np.diag_indices(n)] = -(idx + 1.0)
    return a


def hippo_normal(n: int) -> np.ndarray:
    """HiPPO-N = HiPPO-LegS + p p^T with p_i = sqrt(i + 1/2)."""
    p = np.sqrt(np.arange(n, dtype=np.float64) + 0.5)
    return hippo_legs(n) + np.outer(p, p)


def hippo_n_eigenvalues(n: int) -> np.ndarray:
    """The n eigenvalues -1/2 + i*omega of HiPPO-N, omega ascending.

    S = A_N + I/2 is real skew-symmetric, so -i*S is Hermitian with real
    eigenvalues omega; the real part is set to exactly -1/2."""
    s = hippo_normal(n) + 0.5 * np.eye(n)
    omega = np.linalg.eigvalsh(-1j * s)
    return (-0.5 + 1j * omega).astype(np.complex128)


def block_lambda(block: int, blocks: int) -> np.ndarray:
    """Lambda for the block-diagonal initialisation: ``blocks`` copies of the
    ``block``-size HiPPO-N spectrum, concatenated."""
    return np.tile(hippo_n_eigenvalues(block), blocks)


# --------------------------------------------------------------------------
# Workload container
# --------------------------------------------------------------------------

@dataclasses.dataclass
class S5Workload:
    """Inputs for one S5 forward call, exactly as handed to the library.

    Floating-point arrays hold the values the device sees: float32 for fp32
    configs; for bf16 configs ``u`` holds the bf16-rounded values (as float32)
    and ``u_bf16`` the raw 16-bit patterns."""

    name: str
    B: int
    L: int
    H: int
    P: int
    io: str                       # "f32" or "bf16"
    time_varying: bool
    lam: np.ndarray               # [P] complex64
    b_tilde: np.ndarray           # [P, H] complex64
    c_tilde: np.ndarray           # [H, P] complex64
    d: np.ndarray                 # [H] float32
    log_delta: np.ndarray         # [P] float32
    u: np.ndarray                 # [B, L, H] float32 (bf16-exact for bf16 io)
    delta: Optional[np.ndarray] = None    # [B, L, P] float32 (time-varying)
    u_bf16: Optional[np.ndarray] = None   # [B, L, H] uint16 (bf16 io)
    seed: int = 0
    tol: float = 2e-4             # max|err| / rms(y_oracle) acceptance bound

    @property
    def tokens(self) -> int:
        return self.B * self.L


# Config table: (name, B, L, H, P, io, block, blocks, dmin, dmax, input kind, tv, tol)
CONFIG_SPECS = {
    0: dict(name="tiny", B=1, L=256, H=16, P=8, io="f32", block=8, blocks=1,
            dmin=1e-3, dmax=1e-1, kind="normal", tv=False, tol=2e-4),
    1: dict(name="medium", B=32, L=1024, H=128, P=64, io="f32", block=32, blocks=2,
            dmin=1e-3, dmax=1e-1, kind="normal", tv=False, tol=2e-4),
    2: dict(name="long", B=16, L=4096, H=256, P=192, io="bf16", block=48, blocks=4,
            dmin=1e-3, dmax=1e-1, kind="tokens", tv=False, tol=2e-2),
    3: dict(name="very_long", B=16, L=16384, H=128, P=256, io="bf16", block=32, blocks=8,
            dmin=1e-4, dmax=1e-1, kind="pixels", tv=False, tol=2e-2),
    4: dict(name="irregular", B=16, L=16000, H=96, P=128, io="f32", block=128, blocks=1,
            dmin=1e-3, dmax=1e-1, kind="random_walk", tv=True, tol=2e-4),
}


def _complex_normal(rng: np.random.Generator, shape, var: float) -> np.ndarray:
    sd = math.sqrt(var / 2.0)
    re = rng.normal(0.0, sd, size=shape)
    im = rng.normal(0.0, sd, size=shape)
    return (re + 1j * im).astype(np.complex64)


def _draw_params(rng, H, P, lam, dmin, dmax):
    b_tilde = _complex_normal(rng, (P, H), 1.0 / H)
    c_tilde = _complex_normal(rng, (H, P), 1.0 / H)
    d = rng.normal(0.0, 1.0, size=H).astype(np.float32)
    log_delta = rng.uniform(math.log(dmin), math.log(dmax), size=P).astype(np.float32)
    return lam.astype(np.complex64), b_tilde, c_tilde, d, log_delta


def _draw_inputs(rng, kind, B, L, H, P, log_delta, tv):
    """Config-specific draws, in this order:
    normal:      u ~ N(0,1) [B,L,H]
    tokens:      tok ~ U{0..15} [B,L]; E ~ N(0,1) [16,H]; u = E[tok]
    pixels:      pix ~ Bernoulli(0.1) [B,L]; w ~ N(0,1) [H]; c ~ N(0,1) [H];
                 u = pix*w + c (linear encoder of a flattened binary image)
    random_walk: (tv) dt ~ Exp(1) [B,L]; w ~ N(0,1) [B,L,H]; u = cumsum_t w
    The time-varying step tensor is Delta[b,k,p] = exp(logDelta_p) * dt[b,k],
    evaluated in float64 from the float32 logDelta and rounded to float32."""
    delta = None
    if tv:
        dt = rng.exponential(1.0, size=(B, L))
        delta = (np.exp(log_delta.astype(np.float64))[None, None, :]
                 * dt[:, :, None]).astype(np.float32)
    if kind == "normal":
        u = rng.normal(0.0, 1.0, size=(B, L, H))
    elif kind == "tokens":
        tok = rng.integers(0, 16, size=(B, L))
        emb = rng.normal(0.0, 1.0, size=(16, H))
        u = emb[tok]
    elif kind == "pixels":
        pix = (rng.random(size=(B, L)) < 0.1).astype(np.float64)
        w = rng.normal(0.0, 1.0, size=H)
        c = rng.normal(0.0, 1.0, size=H)
        u = pix[:, :, None] * w[None, None, :] + c[None, None, :]
    elif kind == "random_walk":
        w = rng.normal(0.0, 1.0, size=(B, L, H))
        u = np.cumsum(w, axis=1)
    else:
        raise ValueError(f"unknown input kind {kind!r}")
    return u, delta


def _finish(name, B, L, H, P, io, tv, params, u, delta, seed, tol):
    lam, b_tilde, c_tilde, d, log_delta = params
    u_bits = None
    if io == "bf16":
        u_bits = bf16_bits(u)
        u32 = bf16_to_f32(u_bits)
    elif io == "f32":
        u32 = np.asarray(u, dtype=np.float32)
    else:
        raise ValueError(f"unknown io dtype {io!r}")
    return S5Workload(name=name, B=B, L=L, H=H, P=P, io=io, time_varying=tv,
                      lam=lam, b_tilde=b_tilde, c_tilde=c_tilde, d=d,
                      log_delta=log_delta, u=np.ascontiguousarray(u32),
                      delta=None if delta is None else np.ascontiguousarray(delta),
                      u_bf16=u_bits, seed=seed, tol=tol)


def make_config(i: int, seed: int = 0, B: Optional[int] = None,
                L: Optional[int] = None) -> S5Workload:
    """One of the five S5-shaped workloads (0 tiny, 1 medium, 2 long,
    3 very long / Path-X shaped, 4 irregular sampling). ``B`` and ``L`` may be
    reduced for quick tests; the recipe and draw order stay the same."""
    spec = CONFIG_SPECS[i]
    Bv = spec["B"] if B is None else B
    Lv = spec["L"] if L is None else L
    H, P = spec["H"], spec["P"]
    lam = block_lambda(spec["block"], spec["blocks"])
    assert lam.shape[0] == P
    rng = np.random.default_rng(seed)
    params = _draw_params(rng, H, P, lam, spec["dmin"], spec["dmax"])
    u, delta = _draw_inputs(rng, spec["kind"], Bv, Lv, H, P, params[4], spec["tv"])
    return _finish(f"cfg{i}_{spec['name']}", Bv, Lv, H, P, spec["io"], spec["tv"],
                   params, u, delta, seed, spec["tol"])


def make_random(B: int, L: int, H: int, P: int, io: str = "f32", tv: bool = False,
                seed: int = 0, block: Optional[int] = None, dmin: float = 1e-3,
                dmax: float = 1e-1, kind: str = "normal") -> S5Workload:
    """A workload of arbitrary shape with the same recipe (HiPPO-N blocks of
    size ``block``, default min(P, 32), repeated to cover P; trailing modes
    take the first eigenvalues of one more block when P is not a multiple)."""
    blk = min(P, 32) if block is None else block
    reps = -(-P // blk)
    lam = block_lambda(blk, reps)[:P]
    rng = np.random.default_rng(seed)
    params = _draw_params(rng, H, P, lam, dmin, dmax)
    u, delta = _draw_inputs(rng, kind, B, L, H, P, params[4], tv)
    tol = 2e-2 if io == "bf16" else 2e-4
    return _finish(f"rand_B{B}_L{L}_H{H}_P{P}_{io}{'_tv' if tv else ''}", B, L, H, P,
                   io, tv, params, u, delta, seed, tol)
