"""The gated activation's error allowance (tests/gate_bound.py) is a bound:
perturbations of the input within rho, random and adversarial, move the
oracle's gate by no more than it; the three-product bf16 hi/lo evaluation of
W GELU(y) stays within its product term while a single bf16 product does not
(so a dropped lo part fails the GPU tests)."""

import math

import numpy as np
import pytest

import oracle.s5_oracle as orc
from gate_bound import PRODUCT_ROUNDING, glu_allowance


def _bf16(a):
    """float64 -> nearest bf16 (ties to even, via float32), as float64."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return b.view(np.float32).astype(np.float64)


def _case(H, scale, seed):
    rng = np.random.default_rng(seed)
    y = rng.normal(size=(64, H)) * scale
    w = rng.normal(size=(H, H)) / math.sqrt(H)
    b = 0.5 * rng.normal(size=H)
    return rng, y, w, b


@pytest.mark.parametrize("variant", [1, 2])
@pytest.mark.parametrize("scale", [1.5, 15.0])
def test_random_input_perturbation_within_bound(variant, scale):
    rng, y, w, b = _case(96, scale, 7 + variant)
    rho = 2.0 ** -8
    a = glu_allowance(y, w, b, variant, rho)
    rms = math.sqrt(float(np.mean(y ** 2)))
    for _ in range(5):
        dy = rho * (np.abs(y) + rms) * rng.uniform(-1.0, 1.0, size=y.shape)
        d = np.abs(orc.glu(y + dy, w, b, variant) - orc.glu(y, w, b, variant))
        assert np.all(d <= a)


@pytest.mark.parametrize("variant", [1, 2])
def test_adversarial_input_perturbation_within_bound(variant):
    """dy_k = rho (|y_k| + rms) sign(W_jk GELU'(y_k)) for one output j at a
    time: the largest first-order move of z_j the bound allows for."""
    _, y, w, b = _case(48, 15.0, 21)
    y = y[:4]
    rho = 2.0 ** -8
    a = glu_allowance(y, w, b, variant, rho)
    rms = math.sqrt(float(np.mean(y ** 2)))
    h = 1e-6
    gp = (orc.gelu(y + h) - orc.gelu(y - h)) / (2 * h)
    base = orc.glu(y, w, b, variant)
    for j in range(w.shape[0]):
        for sgn in (1.0, -1.0):
            dy = sgn * rho * (np.abs(y) + rms) * np.sign(w[j][None, :] * gp)
            d = np.abs(orc.glu(y + dy, w, b, variant) - base)
            assert np.all(d[:, j] <= a[:, j])


def test_three_product_split_within_product_term():
    _, y, w, b = _case(128, 15.0, 5)
    g = orc.gelu(y)
    z = g @ w.T
    wh, gh = _bf16(w), _bf16(g)
    wl, gl = _bf16(w - wh), _bf16(g - gh)
    z3 = gh @ wh.T + gl @ wh.T + gh @ wl.T
    z1 = gh @ wh.T
    bound = PRODUCT_ROUNDING * (np.abs(g) @ np.abs(w).T)
    assert np.all(np.abs(z3 - z) <= bound)
    assert np.any(np.abs(z1 - z) > bound)       # one bf16 product: outside it
    assert np.all(np.abs(z3 - z) <= bound / 4)  # (the split's own error sits well inside)
