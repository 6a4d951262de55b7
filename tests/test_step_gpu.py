"""GPU parity of the single recurrent step (s5_step) against the float64
oracle (one step of the stateful form), and T steps against one stateful
forward call over T tokens, through the C ABI.

Bounds: y as test_parity_gpu (2e-4 of rms for float32 I/O; bf16: the excess
over the output's bf16 rounding <= 2e-2 of rms); the state <= the same
fraction of rms(x). The step runs in float32 on the vector units, so its
error is far below these bounds."""

import math

import numpy as np
import pytest

import oracle.s5_oracle as orc
import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BF16_UNIT_ROUNDOFF = 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diagonal_state_space_amd  # noqa: F401  (fails loudly if libs5.so is missing)


def _y_err(io, y, yo):
    yg = y.float().cpu().numpy().astype(np.float64)
    rms = math.sqrt(float(np.mean(yo ** 2)))
    excess = np.abs(yg - yo)
    if io == "bf16":
        excess = excess - BF16_UNIT_ROUNDOFF * np.abs(yo)
    return float(np.max(excess)) / rms


def _x_err(xg, xo):
    xg = xg.cpu().numpy().astype(np.complex128)
    rms = math.sqrt(float(np.mean(np.abs(xo) ** 2)))
    return float(np.max(np.abs(xg - xo))) / rms


def _params(w):
    cuda = torch.device("cuda:0")
    return {k: torch.from_numpy(np.ascontiguousarray(getattr(w, k))).to(cuda)
            for k in ("lam", "b_tilde", "c_tilde", "d", "log_delta")}


def _u_dev(w, sl):
    cuda = torch.device("cuda:0")
    if w.io == "bf16":
        return torch.from_numpy(np.ascontiguousarray(w.u_bf16[:, sl]).view(np.int16)).view(torch.bfloat16).to(cuda)
    return torch.from_numpy(np.ascontiguousarray(w.u[:, sl])).to(cuda)


CASES = [
    # B, H, P, io, tv, options
    (1, 5, 3, "f32", False, {}),
    (16, 128, 256, "bf16", False, {}),
    (16, 128, 256, "f32", False, {"half_spectrum": True}),
    (7, 96, 128, "f32", True, {}),
    (7, 96, 128, "f32", True, {"bilinear": True}),
    (33, 512, 200, "bf16", False, {"bilinear": True, "gelu": True}),
    (4, 24, 40, "f32", False, {"gelu": True}),
    (4, 24, 40, "f32", False, {"gelu_tanh": True}),
    (7, 96, 128, "f32", True, {"gelu_tanh": True}),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_H{c[1]}_P{c[2]}_{c[3]}{'_tv' if c[4] else ''}_"
                         + "+".join(sorted(c[5])))
def test_step_parity(case):
    import diagonal_state_space_amd as s5
    B, H, P, io, tv, opts = case
    w = wl.make_random(B, 1, H, P, io=io, tv=tv, seed=H + P, kind="random_walk" if tv else "normal")
    t = _params(w)
    rng = np.random.default_rng(B)
    x0 = (rng.normal(size=(B, P)) + 1j * rng.normal(size=(B, P))) * 0.5
    x = torch.from_numpy(x0.astype(np.complex64)).cuda()
    kw = {"delta": torch.from_numpy(np.ascontiguousarray(w.delta[:, 0])).cuda()} if tv else {"log_delta": t["log_delta"]}
    print(f"[step] B{B} H{H} P{P} {io} tv={tv} {opts}", flush=True)
    y = s5.step(_u_dev(w, 0), t["lam"], t["b_tilde"], t["c_tilde"], t["d"], x, **kw, **opts)
    torch.cuda.synchronize()
    okw = {"delta": w.delta} if tv else {"log_delta": w.log_delta}
    yo, xo = orc.forward_ex(w.u, w.lam, w.b_tilde, w.c_tilde, w.d, x0=x0.astype(np.complex64),
                            conj_sym=opts.get("half_spectrum", False),
                            method="bilinear" if opts.get("bilinear") else "zoh",
                            activation="gelu" if opts.get("gelu") else "gelu_tanh" if opts.get("gelu_tanh") else None,
                            **okw)
    ey, ex = _y_err(io, y, yo[:, 0]), _x_err(x, xo)
    print(f"[step]   y {ey:.3e}  x {ex:.3e}  (tol {w.tol:.0e})", flush=True)
    assert ey <= w.tol and ex <= w.tol


@pytest.mark.parametrize("io,tv", [("bf16", False), ("f32", True)])
def test_steps_equal_one_stateful_call(io, tv):
    """T single steps from x0 give the outputs and final state of one stateful
    forward call over the same T tokens (each within its bound of the oracle)."""
    import diagonal_state_space_amd as s5
    B, T, H, P = 4, 40, 128, 128
    w = wl.make_random(B, T, H, P, io=io, tv=tv, seed=9, kind="random_walk" if tv else "normal")
    t = _params(w)
    rng = np.random.default_rng(2)
    x0 = (rng.normal(size=(B, P)) + 1j * rng.normal(size=(B, P))) * 0.5
    x = torch.from_numpy(x0.astype(np.complex64)).cuda()
    ys = []
    for k in range(T):
        kw = ({"delta": torch.from_numpy(np.ascontiguousarray(w.delta[:, k])).cuda()} if tv
              else {"log_delta": t["log_delta"]})
        ys.append(s5.step(_u_dev(w, k), t["lam"], t["b_tilde"], t["c_tilde"], t["d"], x, **kw))
    torch.cuda.synchronize()
    y = torch.stack(ys, dim=1)
    okw = {"delta": w.delta} if tv else {"log_delta": w.log_delta}
    yo, xo = orc.forward_ex(w.u, w.lam, w.b_tilde, w.c_tilde, w.d, x0=x0.astype(np.complex64), **okw)
    ey, ex = _y_err(io, y, yo), _x_err(x, xo)
    print(f"[step] {T} steps {io} tv={tv}: y {ey:.3e}  x {ex:.3e}", flush=True)
    assert ey <= w.tol and ex <= w.tol


def test_per_step_interval_with_a_huge_angle():
    """A per-step interval whose half-angle Im(lambda) dt / 2 is about 2^30
    turns: the float32 product of the interval and Im(lambda)/(4 pi) is then a
    whole number of turns, so the float32 path sees the angle 0 and gives
    Lambda_bar = e^(Re(lambda) dt) (the quadrant count, 2^32, must be reduced
    exactly, not converted with saturation). One step from x0 = 1 with zero
    input leaves x = Lambda_bar x0; checked through s5_step and through the
    time-varying stateful forward pass."""
    import diagonal_state_space_amd as s5
    cuda = torch.device("cuda:0")
    omega = 4.0 * math.pi * 2.0 ** 20
    lam = torch.tensor([complex(-1e-9, omega)], dtype=torch.complex64, device=cuda)
    hrev = np.float32(np.float64(np.complex64(complex(-1e-9, omega)).imag) / (4.0 * math.pi))
    dt = np.float32(1024.0)
    th = np.float32(hrev * dt)
    assert th == np.floor(th) and th >= 2.0 ** 29          # whole turns, beyond 2^29
    expect = math.exp(float(np.float32(-1e-9)) * 1024.0)
    H, P = 4, 1
    bt = torch.zeros(P, H, dtype=torch.complex64, device=cuda)
    ct = torch.ones(H, P, dtype=torch.complex64, device=cuda)
    d = torch.zeros(H, dtype=torch.float32, device=cuda)
    x = torch.ones(1, P, dtype=torch.complex64, device=cuda)
    u = torch.zeros(1, H, dtype=torch.float32, device=cuda)
    delta = torch.full((1, P), float(dt), dtype=torch.float32, device=cuda)
    s5.step(u, lam, bt, ct, d, x, delta=delta)
    x0 = torch.ones(1, P, dtype=torch.complex64, device=cuda)
    _, xl = s5.forward_timevarying_stateful(u.view(1, 1, H), lam, bt, ct, d, delta.view(1, 1, P), x0=x0)
    torch.cuda.synchronize()
    for got in (x.cpu().numpy()[0, 0], xl.cpu().numpy()[0, 0]):
        assert abs(got.real - expect) < 1e-6 and abs(got.imag) < 1e-6, got
