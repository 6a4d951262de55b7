"""Input-generator checks: shapes, dtypes, the documented draw order,
determinism and bfloat16 rounding. (The generators hold no forward-path
arithmetic; they are shared by both sides of every parity test.)"""

import math

import numpy as np
import pytest

import workloads as wl


def test_bf16_rounding_rne():
    # exact bf16 values pass through unchanged
    x = np.array([1.0, -2.5, 0.0, 2.0 ** 120 * 1.5, 2.0 ** -126], np.float32)
    assert np.array_equal(wl.bf16_round(x), x)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    one = np.float32(1.0)
    half_ulp = np.float32(2.0 ** -8)
    assert wl.bf16_round(np.array([one + half_ulp]))[0] == 1.0
    assert wl.bf16_round(np.array([one + 3 * half_ulp]))[0] == np.float32(1.0 + 2.0 ** -6)
    # just above a tie rounds up
    above = np.nextafter(one + half_ulp, np.float32(2.0))
    assert wl.bf16_round(np.array([above]))[0] == np.float32(1.0 + 2.0 ** -7)
    # relative error bound: unit roundoff 2^-8 (8-bit significand)
    rng = np.random.default_rng(0)
    v = rng.normal(size=10000).astype(np.float32)
    r = wl.bf16_round(v)
    assert np.max(np.abs(r - v) / np.abs(v)) <= 2.0 ** -8
    # every output is a bf16 value (low 16 bits zero)
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)


@pytest.mark.parametrize("i", [0, 1, 2, 3, 4])
def test_config_shapes(i):
    spec = wl.CONFIG_SPECS[i]
    w = wl.make_config(i, B=1, L=64)
    H, P = spec["H"], spec["P"]
    assert w.u.shape == (1, 64, H) and w.u.dtype == np.float32
    assert w.lam.shape == (P,) and w.lam.dtype == np.complex64
    assert w.b_tilde.shape == (P, H) and w.b_tilde.dtype == np.complex64
    assert w.c_tilde.shape == (H, P) and w.c_tilde.dtype == np.complex64
    assert w.d.shape == (H,) and w.log_delta.shape == (P,)
    assert np.all(w.lam.real == -0.5)
    assert np.all(w.log_delta >= np.float32(math.log(spec["dmin"])) - 1e-6)
    assert np.all(w.log_delta <= np.float32(math.log(spec["dmax"])) + 1e-6)
    # block repetition of the HiPPO-N spectrum
    blk = spec["block"]
    for j in range(1, spec["blocks"]):
        assert np.array_equal(w.lam[j * blk:(j + 1) * blk], w.lam[:blk])
    if spec["io"] == "bf16":
        assert w.u_bf16.shape == w.u.shape
        assert np.array_equal(wl.bf16_to_f32(w.u_bf16), w.u)
    if spec["tv"]:
        assert w.delta.shape == (1, 64, P) and w.delta.dtype == np.float32
        assert np.all(w.delta >= 0) and np.all(np.isfinite(w.delta))


def test_draw_order_config0():
    """Re-derive config 0 from the documented draw order."""
    w = wl.make_config(0)
    rng = np.random.default_rng(0)
    H, P = 16, 8
    sd = math.sqrt(1.0 / (2 * H))
    bre = rng.normal(0, sd, (P, H))
    bim = rng.normal(0, sd, (P, H))
    cre = rng.normal(0, sd, (H, P))
    cim = rng.normal(0, sd, (H, P))
    d = rng.normal(0, 1, H)
    logd = rng.uniform(math.log(1e-3), math.log(1e-1), P)
    u = rng.normal(0, 1, (1, 256, H))
    assert np.array_equal(w.b_tilde, (bre + 1j * bim).astype(np.complex64))
    assert np.array_equal(w.c_tilde, (cre + 1j * cim).astype(np.complex64))
    assert np.array_equal(w.d, d.astype(np.float32))
    assert np.array_equal(w.log_delta, logd.astype(np.float32))
    assert np.array_equal(w.u, u.astype(np.float32))


def test_determinism_and_seed():
    a = wl.make_config(3, B=2, L=128)
    b = wl.make_config(3, B=2, L=128)
    c = wl.make_config(3, B=2, L=128, seed=1)
    assert np.array_equal(a.u_bf16, b.u_bf16) and np.array_equal(a.b_tilde, b.b_tilde)
    assert not np.array_equal(a.b_tilde, c.b_tilde)


def test_pixel_and_token_inputs():
    w = wl.make_config(3, B=2, L=4096)
    # u = pix * w + c: every row is either c or w + c (bf16-rounded)
    rows = np.unique(w.u.reshape(-1, w.H), axis=0)
    assert rows.shape[0] == 2
    w2 = wl.make_config(2, B=2, L=512)
    assert np.unique(w2.u.reshape(-1, w2.H), axis=0).shape[0] <= 16


def test_random_walk_and_intervals():
    w = wl.make_config(4, B=2, L=2000)
    # Delta[b,k,p] / exp(logDelta_p) is one gap per (b, k), shared by all modes
    ratio = w.delta.astype(np.float64) / np.exp(w.log_delta.astype(np.float64))
    assert np.max(np.abs(ratio - ratio[:, :, :1]) / ratio[:, :, :1]) < 2e-7
    gaps = ratio[:, :, 0]
    assert 0.9 < gaps.mean() < 1.1
    # a random walk: increments are standard normal
    inc = np.diff(w.u.astype(np.float64), axis=1)
    assert 0.95 < inc.std() < 1.05


def test_make_random_shapes():
    w = wl.make_random(3, 77, 20, 13, io="bf16", tv=True, seed=5)
    assert w.u.shape == (3, 77, 20) and w.lam.shape == (13,) and w.delta.shape == (3, 77, 13)
    assert w.tol == 2e-2
