"""Seeded random sweep over shapes and option combinations of s5_forward_ex
against the float64 oracle (bounds as test_options_gpu: 2e-4 of rms for
float32 I/O; bf16: the excess over the output's rounding <= 2e-2 of rms, the
bidirectional form included, whose y is rounded once). About half of the
cases with H <= 256 and no GELU also apply the gated activation, checked as in
test_options_gpu: the layer's own output against the oracle, the gated
output against the oracle's gate of that output beyond its product's
rounding bound."""

import math

import numpy as np
import pytest

import oracle.s5_oracle as orc
import workloads as wl
from gate_bound import glu_allowance

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diagonal_state_space_amd  # noqa: F401  (fails loudly if libs5.so is missing)


def _cases(n=32, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        B, L = int(rng.integers(1, 4)), int(rng.integers(1, 1500))
        H, P = int(rng.integers(1, 513)), int(rng.integers(1, 257))
        io = "bf16" if rng.random() < 0.5 else "f32"
        tv = bool(rng.random() < 0.3)
        bidir = (not tv) and bool(rng.random() < 0.3)
        opts = {"half": bool(rng.random() < 0.3), "bilinear": bool(rng.random() < 0.3),
                "gelu": bool(rng.random() < 0.3), "bidir": bidir, "state": (not bidir) and bool(rng.random() < 0.5)}
        out.append((k, B, L, H, P, io, tv, opts))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}")
def test_random_options(case):
    import diagonal_state_space_amd as s5
    k, B, L, H, P, io, tv, opts = case
    rng = np.random.default_rng(k)
    w = wl.make_random(B, L, H, P, io=io, tv=tv, seed=500 + k, kind="random_walk" if tv else "normal")
    bidir = opts["bidir"]
    c2 = None
    if bidir:
        c2 = ((rng.normal(size=(H, 2 * P)) + 1j * rng.normal(size=(H, 2 * P))) / math.sqrt(2 * H)).astype(np.complex64)
    x0 = None
    if opts["state"]:
        x0 = ((rng.normal(size=(B, P)) + 1j * rng.normal(size=(B, P))) * 0.5).astype(np.complex64)
    print(f"[random] B{B} L{L} H{H} P{P} {io} tv={tv} " + ",".join(n for n, v in opts.items() if v), flush=True)
    dev = torch.device("cuda:0")
    u = (torch.from_numpy(w.u_bf16.view(np.int16)).view(torch.bfloat16) if io == "bf16"
         else torch.from_numpy(w.u)).to(dev)
    t = {n: torch.from_numpy(np.ascontiguousarray(getattr(w, n))).to(dev)
         for n in ("lam", "b_tilde", "c_tilde", "d", "log_delta")}
    kw = {"delta": torch.from_numpy(w.delta).to(dev)} if tv else {"log_delta": t["log_delta"]}
    # the gated activation (its own draws, so that the cases above stay as they were)
    grng = np.random.default_rng(10000 + k)
    glu = H <= 256 and not opts["gelu"] and bool(grng.random() < 0.6)
    gvar = 1 + int(grng.random() < 0.5)
    gw = (grng.normal(size=(H, H)) / math.sqrt(H)).astype(np.float32)
    gb = (0.5 * grng.normal(size=H)).astype(np.float32) if grng.random() < 0.5 else None

    def call(gate):
        gkw = {}
        if gate:
            gkw = {"glu_w": torch.from_numpy(gw).to(dev), "glu_variant": gvar,
                   "glu_bias": torch.from_numpy(gb).to(dev) if gb is not None else None}
        return s5.forward_ex(u, t["lam"], t["b_tilde"], torch.from_numpy(c2).to(dev) if bidir else t["c_tilde"],
                             t["d"], x0=torch.from_numpy(x0).to(dev) if x0 is not None else None,
                             final_state=opts["state"], half_spectrum=opts["half"], bilinear=opts["bilinear"],
                             gelu=opts["gelu"], bidirectional=bidir, **kw, **gkw)
    y_gated = call(True)[0] if glu else None
    y, xl = call(False)
    torch.cuda.synchronize()
    okw = {"delta": w.delta} if tv else {"log_delta": w.log_delta}
    method = "bilinear" if opts["bilinear"] else "zoh"
    yo, xo = orc.forward_ex(w.u, w.lam, w.b_tilde, c2 if bidir else w.c_tilde, w.d, x0=x0, conj_sym=opts["half"],
                            method=method, activation="gelu" if opts["gelu"] else None, bidirectional=bidir, **okw)
    yg = y.float().cpu().numpy().astype(np.float64)
    rms = math.sqrt(float(np.mean(yo ** 2))) or 1.0
    excess = np.abs(yg - yo)
    if io == "bf16":
        excess = excess - 2.0 ** -8 * np.abs(yo)
    err = float(np.max(excess)) / rms
    msg = f"[random]   y {err:.3e} (tol {w.tol:.0e})"
    if glu:
        ref = orc.glu(yg, gw, gb, gvar)
        gx = np.abs(y_gated.float().cpu().numpy().astype(np.float64) - ref) - glu_allowance(yg, gw, gb, gvar, rho=0.0)
        if io == "bf16":
            gx = gx - 2.0 ** -8 * np.abs(ref)
        gerr = float(np.max(gx)) / (math.sqrt(float(np.mean(ref ** 2))) or 1.0)
        msg += f"  gated (variant {gvar}) {gerr:.3e}"
        assert gerr <= w.tol
    if opts["state"]:
        xex = np.abs(xl.cpu().numpy() - xo)
        if io == "bf16":
            xex = xex - 2.0 ** -8 * np.abs(xo)   # (each mode's state carries the bf16 operands' rounding)
        xerr = float(np.max(xex)) / (math.sqrt(float(np.mean(np.abs(xo) ** 2))) or 1.0)
        msg += f"  x_last {xerr:.3e}"
        assert xerr <= w.tol
    print(msg, flush=True)
    assert np.all(np.isfinite(yg))
    assert err <= w.tol
