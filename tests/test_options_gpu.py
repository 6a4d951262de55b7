"""GPU parity of the forward pass's options (s5_forward_ex) against the
float64 oracle's forward_ex, through the C ABI: half-spectrum readout,
bilinear discretisation, GELU epilogue, bidirectional scans, and their
combinations with each other and with the initial/final state.

Bounds as test_parity_gpu: max |y_gpu - y_oracle| / rms(y_oracle) <= 2e-4
for float32 I/O; for bf16 I/O the excess over the bf16 output rounding
(2^-8 |y|) <= 2e-2 of rms (the bidirectional form included: its forward half
is kept in float32, so y is rounded once). Final states: <= the same
fraction of rms(x), for bf16 I/O beyond 2^-8 |x| (the operands' relative
rounding, as for y).

The gated activation is checked in two parts: the layer's output y_hat (the
same call without the gate) against the oracle's y as above, and the gated
output against the oracle's gate of y_hat, beyond the gate's product
rounding bound (gate_bound.glu_allowance, exact input). The gate applies to
the layer's output as stored in the I/O type (inside the output pass too,
where y is rounded to bf16 before the gate), and it amplifies perturbations
of its input by its slope times |m| times |W| (a few percent of rms for bf16
rounding at |y| ~ 15): comparing with the oracle's gate of the oracle's y
would measure that conditioning, not the kernels."""

import math

import numpy as np
import pytest

import oracle.s5_oracle as orc
import workloads as wl
from gate_bound import glu_allowance

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BF16_UNIT_ROUNDOFF = 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diagonal_state_space_amd  # noqa: F401  (fails loudly if libs5.so is missing)


def _c_tilde2(H, P, seed):
    """[H, 2P] output matrix of the bidirectional form (complex N(0, 1/H)),
    rounded to complex64 as the GPU receives it."""
    rng = np.random.default_rng(seed)
    c = (rng.normal(size=(H, 2 * P)) + 1j * rng.normal(size=(H, 2 * P))) / math.sqrt(2 * H)
    return c.astype(np.complex64)


def _y_err(io, y, yo):
    """max excess / rms(y_oracle); bf16: the excess over the output's own rounding."""
    yg = y.float().cpu().numpy().astype(np.float64)
    rms = math.sqrt(float(np.mean(yo ** 2)))
    excess = np.abs(yg - yo)
    if io == "bf16":
        excess = excess - BF16_UNIT_ROUNDOFF * np.abs(yo)
    return float(np.max(excess)) / rms


def _x_err(xg, xo, io="f32"):
    """max error / rms(x_oracle); bf16 I/O: the excess over 2^-8 |x_oracle|
    (each mode's state carries the bf16 operands' relative rounding)."""
    xg = xg.cpu().numpy().astype(np.complex128)
    rms = math.sqrt(float(np.mean(np.abs(xo) ** 2)))
    excess = np.abs(xg - xo)
    if io == "bf16":
        excess = excess - BF16_UNIT_ROUNDOFF * np.abs(xo)
    return float(np.max(excess)) / rms


def _run(w, opts, c2=None, x0=None):
    import diagonal_state_space_amd as s5
    cuda = torch.device("cuda:0")
    if w.io == "bf16":
        u = torch.from_numpy(w.u_bf16.view(np.int16)).view(torch.bfloat16).to(cuda)
    else:
        u = torch.from_numpy(w.u).to(cuda)
    dev = {k: torch.from_numpy(np.ascontiguousarray(getattr(w, k))).to(cuda)
           for k in ("lam", "b_tilde", "c_tilde", "d", "log_delta")}
    ct = torch.from_numpy(c2).to(cuda) if c2 is not None else dev["c_tilde"]
    kw = {}
    if w.time_varying:
        kw["delta"] = torch.from_numpy(w.delta).to(cuda)
    else:
        kw["log_delta"] = dev["log_delta"]
    x0d = None if x0 is None else torch.from_numpy(x0.astype(np.complex64)).to(cuda)
    if opts.get("glu"):
        gw, gb = _glu_params(w.H, opts)
        kw["glu_w"] = torch.from_numpy(gw).to(cuda)
        kw["glu_bias"] = None if gb is None else torch.from_numpy(gb).to(cuda)
        kw["glu_variant"] = opts["glu"]
    y, xl = s5.forward_ex(u, dev["lam"], dev["b_tilde"], ct, dev["d"], x0=x0d,
                          final_state=opts.get("state", False), half_spectrum=opts.get("half", False),
                          bilinear=opts.get("bilinear", False), gelu=opts.get("gelu", False),
                          gelu_tanh=opts.get("gelu_tanh", False), bidirectional=opts.get("bidir", False), **kw)
    torch.cuda.synchronize()
    return y, xl


def _glu_params(H, opts):
    """The gate's W [H, H] (N(0, 1/H)) and bias (N(0, 1/4), or None), float32."""
    rng = np.random.default_rng(1000 + H)
    gw = (rng.normal(size=(H, H)) / math.sqrt(H)).astype(np.float32)
    gb = (0.5 * rng.normal(size=H)).astype(np.float32) if opts.get("glu_bias") else None
    return gw, gb


def _oracle(w, opts, c2=None, x0=None):
    """The oracle's layer output (without the gate) and final state."""
    kw = {"delta": w.delta} if w.time_varying else {"log_delta": w.log_delta}
    return orc.forward_ex(w.u, w.lam, w.b_tilde, c2 if c2 is not None else w.c_tilde, w.d, x0=x0,
                          conj_sym=opts.get("half", False), method="bilinear" if opts.get("bilinear") else "zoh",
                          activation="gelu" if opts.get("gelu") else "gelu_tanh" if opts.get("gelu_tanh") else None,
                          bidirectional=opts.get("bidir", False), **kw)


def _gate_err(w, opts, y_gated, y_hat):
    """Gated output against the oracle's gate of the layer's own output y_hat,
    beyond the gate's amplification of its product's rounding (and, bf16, the
    output's own rounding), / rms."""
    gw, gb = _glu_params(w.H, opts)
    yh = y_hat.float().cpu().numpy().astype(np.float64)
    ref = orc.glu(yh, gw, gb, opts["glu"])
    got = y_gated.float().cpu().numpy().astype(np.float64)
    excess = np.abs(got - ref) - glu_allowance(yh, gw, gb, opts["glu"], rho=0.0)
    if w.io == "bf16":
        excess = excess - BF16_UNIT_ROUNDOFF * np.abs(ref)
    return float(np.max(excess)) / math.sqrt(float(np.mean(ref ** 2)))


CASES = [
    # (B, L, H, P, io, tv), options
    ((2, 300, 24, 40, "f32", False), {"half": True}),
    ((2, 1000, 128, 256, "bf16", False), {"half": True}),
    ((2, 513, 96, 128, "f32", True), {"half": True}),
    ((2, 700, 64, 64, "f32", False), {"bilinear": True}),
    ((1, 5001, 128, 256, "bf16", False), {"bilinear": True}),
    ((2, 513, 96, 128, "f32", True), {"bilinear": True}),
    ((2, 4097, 128, 256, "bf16", True), {"bilinear": True}),
    ((2, 800, 64, 64, "f32", False), {"bilinear": True, "state": True}),
    ((2, 513, 96, 128, "f32", True), {"bilinear": True, "state": True}),
    ((2, 300, 24, 40, "f32", False), {"gelu": True}),
    ((2, 1000, 128, 256, "bf16", False), {"gelu": True}),
    ((2, 513, 96, 128, "f32", True), {"gelu": True, "state": True}),
    ((2, 300, 24, 40, "f32", False), {"gelu_tanh": True}),
    ((2, 1000, 128, 256, "bf16", False), {"gelu_tanh": True}),
    ((2, 513, 96, 128, "f32", True), {"gelu_tanh": True, "state": True}),
    ((2, 600, 64, 64, "f32", False), {"bidir": True, "gelu_tanh": True}),
    ((1, 1, 5, 3, "f32", False), {"bidir": True}),
    ((2, 97, 24, 40, "f32", False), {"bidir": True}),
    ((2, 97, 24, 40, "bf16", False), {"bidir": True}),
    ((2, 1000, 256, 192, "f32", False), {"bidir": True}),           # four-wave kernels
    ((1, 5001, 128, 256, "bf16", False), {"bidir": True}),          # many ranges, ragged end
    ((2, 3000, 128, 128, "bf16", False), {"bidir": True, "half": True, "gelu": True, "bilinear": True}),
    ((2, 2000, 96, 128, "f32", False), {"bidir": True, "gelu": True}),
    # four-wave kernels (weights streamed from L2) with each option instance
    ((2, 1000, 256, 192, "bf16", False), {"gelu": True}),
    ((1, 700, 512, 256, "bf16", False), {"bidir": True, "half": True}),
    # H > 128 bf16: streamed drive in pass 2; pass 1 sums both scans (P = 128)
    # or runs the backward pass 1 on its own (P = 192)
    ((2, 1000, 256, 128, "bf16", False), {"bidir": True, "gelu": True}),
    ((2, 777, 250, 192, "bf16", False), {"bidir": True}),
    ((2, 600, 200, 256, "f32", False), {"bilinear": True, "state": True}),
    # the gated activation: inside the output pass (bf16, H <= 128, no backward
    # scan), else after the layer
    ((2, 1000, 128, 256, "bf16", False), {"glu": 1, "glu_bias": True}),
    ((2, 777, 96, 128, "bf16", False), {"glu": 2}),
    ((2, 513, 96, 128, "bf16", True), {"glu": 1, "glu_bias": True}),
    ((2, 600, 64, 64, "bf16", False), {"glu": 1, "state": True}),
    ((2, 300, 24, 40, "bf16", False), {"glu": 2, "glu_bias": True, "half": True, "bilinear": True}),
    ((2, 300, 24, 40, "f32", False), {"glu": 1, "glu_bias": True}),
    ((2, 1000, 256, 192, "bf16", False), {"glu": 2}),
    ((2, 97, 24, 40, "bf16", False), {"glu": 1, "bidir": True}),
    ((1, 600, 128, 256, "bf16", True), {"glu": 1}),
    ((2, 513, 160, 96, "f32", True), {"bilinear": True, "gelu": True, "state": True}),
]


def _name(case):
    (B, L, H, P, io, tv), o = case
    return f"B{B}_L{L}_H{H}_P{P}_{io}{'_tv' if tv else ''}_" + "+".join(
        sorted(k if v is True else f"{k}{v}" for k, v in o.items() if v))


@pytest.mark.parametrize("case", CASES, ids=[_name(c) for c in CASES])
def test_option_parity(case):
    (B, L, H, P, io, tv), opts = case
    w = wl.make_random(B, L, H, P, io=io, tv=tv, seed=101 + L + P, kind="random_walk" if tv else "normal")
    c2 = _c_tilde2(H, P, seed=L) if opts.get("bidir") else None
    x0 = None
    if opts.get("state"):
        rng = np.random.default_rng(P)
        x0 = (rng.normal(size=(B, P)) + 1j * rng.normal(size=(B, P))) * 0.5
    print(f"[options] {_name(case)}", flush=True)
    y, xl = _run(w, opts, c2, x0)
    yo, xo = _oracle(w, opts, c2, x0)
    eg = None
    if opts.get("glu"):
        y_gated = y
        y, xl = _run(w, {k: v for k, v in opts.items() if k not in ("glu", "glu_bias")}, c2, x0)
        eg = _gate_err(w, opts, y_gated, y)
    ey = _y_err(io, y, yo)
    msg = f"[options]   y {ey:.3e} (tol {w.tol:.0e})"
    if eg is not None:
        msg += f"  gated {eg:.3e}"
    if opts.get("state"):
        ex = _x_err(xl, xo, io)
        msg += f"  x_last {ex:.3e}"
        assert ex <= w.tol
    print(msg, flush=True)
    assert ey <= w.tol
    assert eg is None or eg <= w.tol


def test_plain_options_match_plain_entry_point():
    """forward_ex with no options gives the bits of s5_forward."""
    import diagonal_state_space_amd as s5
    w = wl.make_random(2, 1000, 128, 256, io="bf16", seed=3)
    cuda = torch.device("cuda:0")
    u = torch.from_numpy(w.u_bf16.view(np.int16)).view(torch.bfloat16).to(cuda)
    t = {k: torch.from_numpy(np.ascontiguousarray(getattr(w, k))).to(cuda)
         for k in ("lam", "b_tilde", "c_tilde", "d", "log_delta")}
    y1 = s5.forward(u, t["lam"], t["b_tilde"], t["c_tilde"], t["d"], t["log_delta"])
    y2, _ = s5.forward_ex(u, t["lam"], t["b_tilde"], t["c_tilde"], t["d"], log_delta=t["log_delta"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
