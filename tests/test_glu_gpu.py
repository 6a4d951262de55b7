"""GPU parity of the gated activation (s5_glu) against the float64 oracle's
glu, through the C ABI. The error beyond the product's own rounding bound
(gate_bound.glu_allowance with an exact input: the gate's slope times |m|
times 2^-15 sum |W||GELU(y)|), and for bf16 I/O beyond the output's bf16
rounding (2^-8 |out|), is <= 2e-4 of rms(out_oracle) for float32 I/O and
<= 2e-2 for bf16 I/O. Both I/O types use bf16 hi/lo products; the
large-scale cases (y of rms 15) fail with a single bf16 product."""

import math

import numpy as np
import pytest

import oracle.s5_oracle as orc
from gate_bound import glu_allowance

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diagonal_state_space_amd  # noqa: F401  (fails loudly if libs5.so is missing)


def _bf16_round(a):
    """float32 values rounded to bf16 (nearest, ties to even), as float32."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return b.view(np.float32)


CASES = [
    # T, H, io, variant, bias, in place, scale of y
    (17, 1, "f32", 1, True, False, 1.5),
    (100, 5, "f32", 2, False, False, 1.5),
    (1000, 96, "f32", 1, True, False, 1.5),
    (3001, 128, "f32", 2, True, True, 1.5),
    (2048, 256, "f32", 1, True, False, 1.5),
    (4099, 128, "bf16", 1, True, False, 1.5),
    (999, 256, "bf16", 2, True, True, 1.5),
    (64, 16, "bf16", 1, False, False, 1.5),
    (4099, 128, "bf16", 1, True, False, 15.0),
    (2000, 256, "bf16", 2, True, False, 15.0),
    (1000, 96, "f32", 1, True, False, 15.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"T{c[0]}_H{c[1]}_{c[2]}_v{c[3]}{'_bias' if c[4] else ''}"
                         f"{'_inplace' if c[5] else ''}_s{c[6]:g}")
def test_glu_parity(case):
    import diagonal_state_space_amd as s5
    T, H, io, variant, with_bias, inplace, scale = case
    rng = np.random.default_rng(T + H)
    y = (rng.normal(size=(T, H)) * scale).astype(np.float32)
    w = (rng.normal(size=(H, H)) / math.sqrt(H)).astype(np.float32)
    b = (rng.normal(size=H) * 0.5).astype(np.float32) if with_bias else None
    if io == "bf16":
        y = _bf16_round(y)
        yd = torch.from_numpy(y).to(torch.bfloat16).cuda()
    else:
        yd = torch.from_numpy(y).cuda()
    wd = torch.from_numpy(w).cuda()
    bd = torch.from_numpy(b).cuda() if b is not None else None
    out = s5.glu(yd, wd, bd, variant, out=yd if inplace else None)
    torch.cuda.synchronize()
    ref = orc.glu(y.astype(np.float64), w, b, variant)
    got = out.float().cpu().numpy().astype(np.float64)
    rms = math.sqrt(float(np.mean(ref ** 2)))
    excess = np.abs(got - ref) - glu_allowance(y.astype(np.float64), w, b, variant, rho=0.0)
    tol = 2e-4
    if io == "bf16":
        excess = excess - 2.0 ** -8 * np.abs(ref)
        tol = 2e-2
    err = float(np.max(excess)) / rms
    print(f"[glu] T{T} H{H} {io} v{variant}: {err:.3e} (tol {tol:.0e})", flush=True)
    assert err <= tol
