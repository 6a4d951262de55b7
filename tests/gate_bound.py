"""Error allowance of the gated activation (test infrastructure).

The gate o_j = m_j * sigma(z_j), z_j = sum_k W_jk GELU(y_k) + b_j, with
m = GELU(y) (variant 1) or y (variant 2), amplifies a perturbation of its
input: dz_j = sum_k W_jk GELU'(y_k) dy_k and do_j ~ m_j sigma'(z_j) dz_j, so
with |y| of order 10 a relative rounding of y near 2^-9 moves o by several
percent of its RMS. A fixed fraction of RMS cannot bound that; this module
gives the rigorous bound that the arithmetic implies, evaluated from float64
values of the gate at the input the GPU's gate received (or a bound on how far
its input was from it):

  |dy_k| <= rho (|y_k| + rms(y))          input perturbation (0: exact input)
  dm_j    = c_m |dy_j|                     c_m = max |GELU'| (1.13) or 1
  dz_j    = 1.13 sum_k |W_jk| |dy_k| + u_p sum_k |W_jk| |GELU(y_k)|
  A_j     = dm_j s_j + |m_j| (s_j (1 - s_j) dz_j + dz_j^2 / 16) + dm_j dz_j / 4

with s = sigma(z); u_p bounds the matrix product's relative rounding (bf16 hi
and lo parts of both operands, three products, float32 sums: below 2^-15);
dz^2/16 bounds sigma's second-order term (|sigma''| <= 0.097) and dm dz / 4
the cross term (|sigma'| <= 1/4). The GPU output passes where
|o - o_ref| - A <= tol rms(o_ref) (plus its own output rounding)."""

import math

import numpy as np
from scipy.special import erf

GELU_SLOPE_MAX = 1.13   # max |d/dy y Phi(y)| = 1.1289 (at y = sqrt 2)
PRODUCT_ROUNDING = 2.0 ** -15


def _gelu(y):
    return 0.5 * y * (1.0 + erf(y / math.sqrt(2.0)))


def glu_allowance(y, w, bias, variant, rho, u_p=PRODUCT_ROUNDING):
    """A [..., H]: the first- and second-order bound above at input y."""
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    g = _gelu(y)
    z = g @ w.T
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float64)
    s = 1.0 / (1.0 + np.exp(-z))
    m = g if variant == 1 else y
    c_m = GELU_SLOPE_MAX if variant == 1 else 1.0
    dy = rho * (np.abs(y) + math.sqrt(float(np.mean(y ** 2)))) if rho > 0 else np.zeros_like(y)
    aw = np.abs(w)
    dz = GELU_SLOPE_MAX * (dy @ aw.T) + u_p * (np.abs(g) @ aw.T)
    dm = c_m * dy
    return dm * s + np.abs(m) * (s * (1.0 - s) * dz + dz * dz / 16.0) + dm * dz / 4.0
