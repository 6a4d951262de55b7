"""Float64 CPU oracle for the S5 layer forward path.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports, links or runs this
module: only the tests, the package smoke check and the benchmark's CPU
baseline leg may call it. It shares no code with the HIP path.

It is the plain definition of what the forward path computes, written out
step by step in float64 with an explicit sequential loop over time. Sources
(page title and section):

O1  Delta_p = exp(log Delta_p) (time-invariant) or a given Delta[b,k,p]
    (time-varying); a negative or non-finite interval is rejected.
    [paper Sec. 3.2 and App. A `apply_S5_layer`; abhik.ai review, row 2
    "Integrate a held input exactly"]
O2  zero-order hold per mode: z = lambda*Delta, Lambda_bar = exp(z),
    gain = (exp(z) - 1)/lambda = Delta*phi1(z), with phi1(z) = (e^z - 1)/z;
    for |z| < 1e-4 the gain is Delta times the 9-term Taylor series of phi1
    (the review's numerical guard; removable singularity, gain -> Delta as
    lambda -> 0). B_bar = gain[:, None] * B~.
    [paper eq. 6; App. A `discretize`; abhik.ai review, row 2]
O3  drive b_k = B_bar u_k (time-varying: gain_k * (B~ u_k)).
    [abhik.ai review, row 1 "Mix input channels before the recurrence";
    App. A `apply_ssm`]
O4  x_{-1} = 0, x_k = Lambda_bar_k * x_{k-1} + b_k, one step at a time.
    The associative scan of the pages reaches exactly this result up to
    floating-point regrouping. [paper eq. 2 and Sec. 2.2; App. H]
O5  y_k = Re(C~ x_k) + D * u_k, full spectrum (factor 1).
    [App. A `apply_ssm` readout; abhik.ai review, row 4: the factor two applies
    only to half-spectrum storage]
O6  stateful form: the recurrence of O4 started from a given state x0 instead
    of zero (x_{-1} = x0), returning the state after the last step as well, so
    that a sequence can be processed in pieces with the state carried between
    them. A nonzero initial state enters every prefix through its transition
    part. [abhik.ai review, "Associative scans preserve the recurrence" (paper
    Sec. 2.2, App. H) and its note that streaming keeps only the current state
    (Sec. 2.2, 3.4); papercache notes Sec. 3.3, online generation]
O7  half-spectrum storage: when the stored modes are one partner of each
    conjugate pair, y_k = 2 Re(C+ x_k) + D * u_k; the feedthrough is not
    doubled. [abhik.ai review, row 4 "Reconstruct real outputs and keep the
    direct path"; wikillm notes, "Paper vs code", readout factor 2]
O8  bilinear (trapezoid-rule) discretisation as the alternative to O2: with
    z = lambda*Delta, Lambda_bar = (1 + z/2)/(1 - z/2) and gain =
    Delta/(1 - z/2), the diagonal case of the bilinear transform.
    [intuitivepapers S4 notes, "Discretization and the step size" (the
    equation group with the forward and backward half-steps); abhik.ai
    review, "Discretization controls both retention and input gain": the
    official code offers it as an option]
O9  GELU epilogue: y -> y * Phi(y), Phi the standard normal distribution
    function (written with erf), applied to the pre-activation output.
    [papercache notes, App. A `apply_S5_layer`; wikillm notes, gated
    activation step; the plain reading of "GELU" is the exact form]
O9t the tanh form of the GELU epilogue, y/2 (1 + tanh(sqrt(2/pi)(y +
    0.044715 y^3))): the App. A listing ends in the JAX library's gelu, whose
    default is this approximation. [papercache notes, App. A
    `apply_S5_layer`]
O10 bidirectional form: a second, backward scan over the same
    Lambda_bar and B_bar, x'_k = Lambda_bar * x'_{k+1} + B_bar u_k from
    x'_L = 0 (inclusive of step k), read out by the second half of a
    C~ with 2P columns: y_k = Re(C~[:, :P] x_k) + Re(C~[:, P:] x'_k) + D u_k
    (factor 2 on both terms under O7). Time-invariant only; no state in or
    out. [wikillm notes, "Paper vs code", bidirectional scans; abhik.ai
    review, offline bidirectional use]
O11 gated activation after the layer, with a dense H x H matrix W and an
    optional bias b: g = GELU(y); variant 1 returns g * sigma(g W^T + b)
    (the paper's gate), variant 2 returns y * sigma(g W^T + b) (the un-
    activated y gated, GELU only inside the gate); sigma is the logistic
    function. [wikillm notes, "Paper vs code": GLU variant and dense gate
    bias; the pseudocode's half_glu1 step]

Every function is pinned by the checks in tests/test_oracle_pins.py against
closed forms, an ODE solve, the convolution-kernel form, impulse responses,
printed values of the pages and invariants.
"""

from __future__ import annotations

import math

import numpy as np
import scipy.special

__all__ = [
    "SERIES_RADIUS",
    "check_intervals",
    "zoh",
    "discretize",
    "drive",
    "scan_sequential",
    "readout",
    "forward",
    "forward_timevarying",
    "forward_state",
    "forward_timevarying_state",
    "compose",
    "bilinear",
    "readout_half",
    "gelu",
    "gelu_tanh",
    "scan_reverse",
    "forward_ex",
    "sigmoid",
    "glu",
]

# |z| below which the gain uses the Taylor series of phi1 (abhik.ai review, row 2)
SERIES_RADIUS = 1e-4


def check_intervals(delta) -> np.ndarray:
    """O1 precondition: intervals must be finite and non-negative."""
    d = np.asarray(delta, dtype=np.float64)
    if not np.all(np.isfinite(d)) or np.any(d < 0):
        raise ValueError("intervals must be finite and non-negative")
    return d


def zoh(lam, delta):
    """O2: per-element ZOH of a diagonal mode. ``lam`` and ``delta`` broadcast
    against each other. Returns (Lambda_bar, gain), complex128."""
    lam = np.asarray(lam, dtype=np.complex128)
    d = check_intervals(delta)
    lam, d = np.broadcast_arrays(lam, d)
    z = lam * d
    lam_bar = np.exp(z)
    gain = np.empty_like(z)
    small = np.abs(z) < SERIES_RADIUS
    big = ~small
    gain[big] = (lam_bar[big] - 1.0) / lam[big]
    if small.any():
        zs = z[small]
        term = np.ones_like(zs)
        phi = np.ones_like(zs)
        for n in range(1, 9):          # sum_{n=0}^{8} z^n / (n+1)!
            term = term * zs / (n + 1)
            phi = phi + term
        gain[small] = d[small] * phi
    return lam_bar, gain


def discretize(lam, b_tilde, delta):
    """O1-O2 for the time-invariant case: returns (Lambda_bar [P],
    B_bar [P, H]) for per-mode intervals ``delta`` [P]."""
    lam_bar, gain = zoh(lam, delta)
    b_bar = gain[:, None] * np.asarray(b_tilde, dtype=np.complex128)
    return lam_bar, b_bar


def drive(u, b_mat):
    """O3: b_k = B u_k for every (batch, step); u [..., L, H] real,
    ``b_mat`` [P, H] complex -> [..., L, P] complex."""
    return np.asarray(u, dtype=np.float64) @ np.asarray(b_mat, dtype=np.complex128).T


def scan_sequential(lam_bar, bu, x0=None):
    """O4: x_k = a_k * x_{k-1} + b_k from x_{-1} = 0 (O6: from x_{-1} = x0
    when given), explicit loop over k.

    ``bu`` is [B, L, P]; ``lam_bar`` is [P] (time-invariant) or [B, L, P];
    ``x0`` is [B, P] complex or None."""
    bu = np.asarray(bu, dtype=np.complex128)
    lam_bar = np.asarray(lam_bar, dtype=np.complex128)
    Bn, L, P = bu.shape
    tv = lam_bar.ndim == 3
    x = np.zeros((Bn, P), dtype=np.complex128)
    if x0 is not None:
        x[...] = np.asarray(x0, dtype=np.complex128).reshape(Bn, P)
    out = np.empty_like(bu)
    for k in range(L):
        a = lam_bar[:, k, :] if tv else lam_bar
        x = a * x + bu[:, k, :]
        out[:, k, :] = x
    return out


def readout(x, c_tilde, d, u):
    """O5: y_k = Re(C~ x_k) + D * u_k (full spectrum)."""
    cx = np.asarray(x, dtype=np.complex128) @ np.asarray(c_tilde, dtype=np.complex128).T
    return cx.real + np.asarray(d, dtype=np.float64) * np.asarray(u, dtype=np.float64)


def forward(u, lam, b_tilde, c_tilde, d, log_delta):
    """Time-invariant S5 forward (pre-activation output), float64.

    u [B, L, H] real; lam [P]; b_tilde [P, H]; c_tilde [H, P]; d [H];
    log_delta [P]. Returns y [B, L, H] float64."""
    u = np.asarray(u, dtype=np.float64)
    delta = np.exp(np.asarray(log_delta, dtype=np.float64))          # O1
    lam_bar, b_bar = discretize(lam, b_tilde, delta)                  # O2
    bu = drive(u, b_bar)                                              # O3
    x = scan_sequential(lam_bar, bu)                                  # O4
    return readout(x, c_tilde, d, u)                                  # O5


def forward_timevarying(u, lam, b_tilde, c_tilde, d, delta):
    """Time-varying S5 forward: one interval per (batch, step, mode).

    Step k uses Delta_k for both Lambda_bar_k and B_bar_k (the interval that
    ends at step k). u [B, L, H]; delta [B, L, P]. Returns y [B, L, H]."""
    u = np.asarray(u, dtype=np.float64)
    delta = check_intervals(delta)                                    # O1
    lam_bar, gain = zoh(np.asarray(lam)[None, None, :], delta)        # O2
    bu = gain * drive(u, b_tilde)                                     # O3
    x = scan_sequential(lam_bar, bu)                                  # O4
    return readout(x, c_tilde, d, u)                                  # O5


def forward_state(u, lam, b_tilde, c_tilde, d, log_delta, x0=None):
    """O6, time-invariant: y as in ``forward`` with the scan started from x0
    ([B, P] complex, None = zero), and the state after the last step.
    Returns (y [B, L, H], x_last [B, P]); x_last = x0 when L = 0."""
    u = np.asarray(u, dtype=np.float64)
    Bn, L, _ = u.shape
    P = np.asarray(lam).shape[0]
    delta = np.exp(np.asarray(log_delta, dtype=np.float64))          # O1
    lam_bar, b_bar = discretize(lam, b_tilde, delta)                  # O2
    bu = drive(u, b_bar)                                              # O3
    x = scan_sequential(lam_bar, bu, x0)                              # O4, O6
    x_last = x[:, -1, :] if L > 0 else (np.zeros((Bn, P), np.complex128) if x0 is None
                                        else np.asarray(x0, dtype=np.complex128).reshape(Bn, P))
    return readout(x, c_tilde, d, u), x_last                          # O5


def forward_timevarying_state(u, lam, b_tilde, c_tilde, d, delta, x0=None):
    """O6, time-varying: as ``forward_timevarying`` from x0, with the final state."""
    u = np.asarray(u, dtype=np.float64)
    Bn, L, _ = u.shape
    P = np.asarray(lam).shape[0]
    delta = check_intervals(delta)                                    # O1
    lam_bar, gain = zoh(np.asarray(lam)[None, None, :], delta)        # O2
    bu = gain * drive(u, b_tilde)                                     # O3
    x = scan_sequential(lam_bar, bu, x0)                              # O4, O6
    x_last = x[:, -1, :] if L > 0 else (np.zeros((Bn, P), np.complex128) if x0 is None
                                        else np.asarray(x0, dtype=np.complex128).reshape(Bn, P))
    return readout(x, c_tilde, d, u), x_last                          # O5


def compose(earlier, later):
    """The scan's binary operator on affine maps x -> a*x + b: apply
    ``earlier`` then ``later``; result (a_l * a_e, a_l * b_e + b_l).
    [paper App. H; App. A `binary_operator`]"""
    a_e, b_e = earlier
    a_l, b_l = later
    return a_l * a_e, a_l * b_e + b_l


def bilinear(lam, delta):
    """O8: bilinear discretisation of a diagonal mode. ``lam`` and ``delta``
    broadcast against each other. Returns (Lambda_bar, gain), complex128."""
    lam = np.asarray(lam, dtype=np.complex128)
    d = check_intervals(delta)
    lam, d = np.broadcast_arrays(lam, d)
    half = 0.5 * lam * d
    back = 1.0 - half                 # backward half-step (I - Delta/2 A)
    return (1.0 + half) / back, d / back


def readout_half(x, c_tilde, d, u):
    """O7: y_k = 2 Re(C+ x_k) + D * u_k for half-spectrum storage."""
    cx = np.asarray(x, dtype=np.complex128) @ np.asarray(c_tilde, dtype=np.complex128).T
    return 2.0 * cx.real + np.asarray(d, dtype=np.float64) * np.asarray(u, dtype=np.float64)


def gelu(y):
    """O9: GELU(y) = y * Phi(y) with Phi(y) = (1 + erf(y / sqrt 2)) / 2."""
    y = np.asarray(y, dtype=np.float64)
    return y * 0.5 * (1.0 + scipy.special.erf(y / math.sqrt(2.0)))


def gelu_tanh(y):
    """O9t: the tanh approximation y/2 (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3)))."""
    y = np.asarray(y, dtype=np.float64)
    return 0.5 * y * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (y + 0.044715 * y ** 3)))


def scan_reverse(lam_bar, bu):
    """O10: x'_k = a * x'_{k+1} + b_k from x'_L = 0, explicit loop from
    k = L-1 down to 0. ``bu`` [B, L, P]; ``lam_bar`` [P]."""
    bu = np.asarray(bu, dtype=np.complex128)
    lam_bar = np.asarray(lam_bar, dtype=np.complex128)
    Bn, L, P = bu.shape
    x = np.zeros((Bn, P), dtype=np.complex128)
    out = np.empty_like(bu)
    for k in range(L - 1, -1, -1):
        x = lam_bar * x + bu[:, k, :]
        out[:, k, :] = x
    return out


def forward_ex(u, lam, b_tilde, c_tilde, d, log_delta=None, delta=None, x0=None, *,
               conj_sym=False, method="zoh", activation=None, bidirectional=False):
    """The forward path with its options: time-invariant (``log_delta`` [P])
    or time-varying (``delta`` [B, L, P]) intervals, ZOH (O2) or bilinear
    (O8) discretisation, optional initial state (O6), half-spectrum readout
    (O7), bidirectional scans (O10, ``c_tilde`` [H, 2P]) and a GELU epilogue
    (O9, ``activation="gelu"``, or its tanh form O9t, ``"gelu_tanh"``).

    Returns (y [B, L, H] float64, x_last [B, P] complex128, or None for the
    bidirectional form)."""
    u = np.asarray(u, dtype=np.float64)
    Bn, L, H = u.shape
    lam = np.asarray(lam, dtype=np.complex128)
    P = lam.shape[0]
    disc = {"zoh": zoh, "bilinear": bilinear}[method]
    tv = delta is not None
    if tv == (log_delta is not None):
        raise ValueError("give exactly one of log_delta and delta")
    if bidirectional and (tv or x0 is not None):
        raise ValueError("the bidirectional form is time-invariant and stateless")
    if activation not in (None, "gelu", "gelu_tanh"):
        raise ValueError("activation must be None, 'gelu' or 'gelu_tanh'")
    if tv:
        lam_bar, gain = disc(lam[None, None, :], delta)               # O1, O2/O8
        bu = gain * drive(u, b_tilde)                                 # O3
    else:
        lam_bar, gain = disc(lam, np.exp(np.asarray(log_delta, dtype=np.float64)))
        bu = drive(u, gain[:, None] * np.asarray(b_tilde, dtype=np.complex128))
    x = scan_sequential(lam_bar, bu, x0)                              # O4, O6
    c = np.asarray(c_tilde, dtype=np.complex128)
    read = readout_half if conj_sym else readout                      # O7 / O5
    if bidirectional:
        xb = scan_reverse(lam_bar, bu)                                # O10
        y = read(x, c[:, :P], d, u) + read(xb, c[:, P:], np.zeros(H), u)
        x_last = None
    else:
        y = read(x, c, d, u)
        if L > 0:
            x_last = x[:, -1, :]
        elif x0 is None:
            x_last = np.zeros((Bn, P), np.complex128)
        else:
            x_last = np.asarray(x0, dtype=np.complex128).reshape(Bn, P)
    if activation == "gelu":
        y = gelu(y)                                                   # O9
    elif activation == "gelu_tanh":
        y = gelu_tanh(y)                                              # O9t
    return y, x_last


def sigmoid(x):
    """The logistic function 1 / (1 + exp(-x)), float64."""
    return scipy.special.expit(np.asarray(x, dtype=np.float64))


def glu(y, w, bias=None, variant=1):
    """O11: y [..., H] real; w [H, H] (output j reads w[j, :]); bias [H] or
    None. Variant 1: g * sigmoid(g w^T + b), variant 2: y * sigmoid(g w^T + b),
    with g = GELU(y)."""
    y = np.asarray(y, dtype=np.float64)
    g = gelu(y)
    pre = g @ np.asarray(w, dtype=np.float64).T
    if bias is not None:
        pre = pre + np.asarray(bias, dtype=np.float64)
    gate = sigmoid(pre)
    if variant == 1:
        return g * gate
    if variant == 2:
        return y * gate
    raise ValueError("variant must be 1 or 2")
