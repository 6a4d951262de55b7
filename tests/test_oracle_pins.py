"""Pins for the float64 oracle: each check ties the oracle to something other
than itself (a closed form, an ODE solve, the convolution-kernel form, a value
printed on the pages, an algebraic invariant). The `planted` tests at the end
mutate the oracle on the CPU in plausible ways and show that a pin fails.
"""

import itertools
import math
import os

import numpy as np
import pytest
import scipy.integrate
import scipy.special
import scipy.linalg

import oracle.s5_oracle as orc
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _rand_params(rng, H, P, lam=None):
    if lam is None:
        lam = -rng.uniform(0.05, 1.0, P) + 1j * rng.uniform(-20, 20, P)
    b = (rng.normal(size=(P, H)) + 1j * rng.normal(size=(P, H))) / math.sqrt(2 * H)
    c = (rng.normal(size=(H, P)) + 1j * rng.normal(size=(H, P))) / math.sqrt(2 * H)
    d = rng.normal(size=H)
    logd = rng.uniform(math.log(1e-3), math.log(1e-1), P)
    return np.asarray(lam, np.complex128), b, c, d, logd


def _rel(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------------------
# Independent discretisation: Van Loan's augmented-matrix exponential
# ---------------------------------------------------------------------------

def _zoh_expm(lam, delta):
    """expm([[lam*Delta, Delta], [0, 0]]) = [[Lambda_bar, gain], [0, 1]]."""
    lam = np.atleast_1d(np.asarray(lam, np.complex128))
    delta = np.broadcast_to(np.asarray(delta, np.float64), lam.shape)
    lb = np.empty_like(lam)
    g = np.empty_like(lam)
    for i, (l, dt) in enumerate(zip(lam.ravel(), delta.ravel())):
        m = np.array([[l * dt, dt], [0.0, 0.0]], dtype=np.complex128)
        e = scipy.linalg.expm(m)
        lb.ravel()[i] = e[0, 0]
        g.ravel()[i] = e[0, 1]
    return lb, g


# ---- pin functions (reused by the planted-mistake tests) -------------------

def pin_zoh_expm():
    rng = _rng(1)
    lam = np.concatenate([wl.hippo_n_eigenvalues(8), wl.hippo_n_eigenvalues(32)[:6],
                          -rng.uniform(0.01, 3, 10) + 1j * rng.uniform(-400, 400, 10)])
    delta = rng.uniform(1e-4, 0.3, lam.shape)
    lb, g = orc.zoh(lam, delta)
    lb2, g2 = _zoh_expm(lam, delta)
    return max(_rel(lb, lb2), _rel(g, g2))


def pin_constant_input_closed_form():
    """P = 1, H = 2 system whose readout exposes (Re x, Im x); a constant input
    gives x_k = b u (exp(lambda (k+1) Delta) - 1)/lambda (continuous solution
    at t = (k+1) Delta: zero-order hold is exact for held inputs)."""
    lam = np.array([-0.3 + 2.1j])
    logd = np.array([math.log(0.07)])
    bt = np.array([[0.8 - 0.4j, 0.0]])
    ct = np.array([[1.0], [-1j]])
    d = np.zeros(2)
    L = 50
    u = np.zeros((1, L, 2))
    u[0, :, 0] = 1.7
    y = orc.forward(u, lam, bt, ct, d, logd)
    k = np.arange(L)
    x = bt[0, 0] * 1.7 * (np.exp(lam[0] * (k + 1) * 0.07) - 1.0) / lam[0]
    return max(_rel(y[0, :, 0], x.real), _rel(y[0, :, 1], x.imag))


def _ode_reference(u, lam, bt, ct, d, delta_steps):
    """Solve dx_p/dt = lambda_p x_p + (B~ u(t))_p per mode with a
    piecewise-constant input held over each step (mode p's step k lasts
    delta_steps[k, p]), then read y_k = Re(C~ x(end of step k)) + D u_k."""
    L, H = u.shape
    P = lam.shape[0]
    x_end = np.zeros((L, P), np.complex128)
    for p in range(P):
        xp = 0.0 + 0.0j
        for k in range(L):
            drive_k = bt[p] @ u[k]
            dt = delta_steps[k, p]

            def f(t, s, lp=lam[p], dk=drive_k):
                z = s[0] + 1j * s[1]
                dz = lp * z + dk
                return [dz.real, dz.imag]

            sol = scipy.integrate.solve_ivp(f, (0.0, dt), [xp.real, xp.imag],
                                            method="DOP853", rtol=1e-12, atol=1e-14)
            xp = sol.y[0, -1] + 1j * sol.y[1, -1]
            x_end[k, p] = xp
    return (x_end @ ct.T).real + d * u


def pin_ode_time_invariant():
    rng = _rng(2)
    H, P, L = 3, 4, 12
    lam, bt, ct, d, logd = _rand_params(rng, H, P)
    u = rng.normal(size=(1, L, H))
    y = orc.forward(u, lam, bt, ct, d, logd)
    steps = np.broadcast_to(np.exp(logd), (L, P))
    yr = _ode_reference(u[0], lam, bt, ct, d, steps)
    return _rel(y[0], yr)


def pin_ode_time_varying():
    rng = _rng(3)
    H, P, L = 2, 3, 10
    lam, bt, ct, d, logd = _rand_params(rng, H, P)
    u = rng.normal(size=(1, L, H))
    dt = rng.exponential(1.0, size=(1, L))
    delta = np.exp(logd)[None, None, :] * dt[:, :, None]
    delta[0, 4, :] = 0.0   # a zero-length interval inside the sequence
    y = orc.forward_timevarying(u, lam, bt, ct, d, delta)
    yr = _ode_reference(u[0], lam, bt, ct, d, delta[0])
    return _rel(y[0], yr)


def _conv_kernel_forward(u, lam, bt, ct, d, logd):
    """y_k = sum_{j<=k} K_{k-j} u_j + D u_k with K_i = Re(C~ diag(Lb^i) B_bar),
    Lb^i = exp(i*z) evaluated directly (no repeated multiplication) and the
    discretisation taken from the augmented-matrix exponential."""
    delta = np.exp(np.asarray(logd, np.float64))
    lb, g = _zoh_expm(lam, delta)
    z = np.log(lb)  # principal log; exp(i*z) = lb^i for integer i
    bb = g[:, None] * bt
    B, L, H = u.shape
    i = np.arange(L)
    pw = np.exp(np.outer(i, z))                        # [L, P]
    K = np.einsum("hp,ip,pq->ihq", ct, pw, bb).real     # [L, H, H]
    y = np.zeros((B, L, H))
    for k in range(L):
        y[:, k, :] = np.einsum("jhq,bjq->bh", K[k::-1], u[:, :k + 1, :])
    return y + d * u, K


def pin_convolution_form():
    rng = _rng(4)
    errs = []
    H, P, L = 3, 5, 40
    lam, bt, ct, d, logd = _rand_params(rng, H, P)
    u = rng.normal(size=(2, L, H))
    y = orc.forward(u, lam, bt, ct, d, logd)
    yc, _ = _conv_kernel_forward(u, lam, bt, ct, d, logd)
    errs.append(_rel(y, yc))
    w = wl.make_config(0, L=96)
    args = (w.u.astype(np.float64), w.lam, w.b_tilde, w.c_tilde, w.d, w.log_delta)
    y = orc.forward(*args)
    yc, _ = _conv_kernel_forward(*args)
    errs.append(_rel(y, yc))
    return max(errs)


def pin_impulse_response():
    rng = _rng(5)
    H, P, L = 3, 4, 30
    lam, bt, ct, d, logd = _rand_params(rng, H, P)
    _, K = _conv_kernel_forward(np.zeros((1, L, H)), lam, bt, ct, d, logd)
    err = 0.0
    for h in range(H):
        k0 = 7
        u = np.zeros((1, L, H))
        u[0, k0, h] = 1.0
        y = orc.forward(u, lam, bt, ct, d, logd)[0]
        expect = np.zeros((L, H))
        expect[k0:, :] = K[: L - k0, :, h]
        expect[k0, h] += d[h]
        err = max(err, _rel(y, expect))
    return err


def pin_half_spectrum():
    """Conjugate-paired modes: full-spectrum output equals
    2 Re(C+ x+) + D u computed from the stored half (abhik.ai review, row 4)."""
    rng = _rng(6)
    H, Ph, L = 3, 4, 25
    lam_h, bt_h, ct_h, d, logd_h = _rand_params(rng, H, Ph)
    lam = np.concatenate([lam_h, lam_h.conj()])
    bt = np.concatenate([bt_h, bt_h.conj()], axis=0)
    ct = np.concatenate([ct_h, ct_h.conj()], axis=1)
    logd = np.concatenate([logd_h, logd_h])
    u = rng.normal(size=(2, L, H))
    y_full = orc.forward(u, lam, bt, ct, d, logd)
    y_half = 2.0 * orc.forward(u, lam_h, bt_h, ct_h, np.zeros(H), logd_h) + d * u
    return _rel(y_full, y_half)


def pin_scan_bracketings():
    """Every bracketing of the operator over L <= 7 elements gives the state of
    the sequential loop, and two log-depth prefix scans (all prefixes, lengths
    that are not powers of two included) match every step of the loop."""
    rng = _rng(7)
    P = 3
    err = 0.0
    for L in range(1, 8):
        a = np.exp(-rng.uniform(0.01, 0.5, (L, P)) + 1j * rng.uniform(-3, 3, (L, P)))
        b = rng.normal(size=(L, P)) + 1j * rng.normal(size=(L, P))
        xs = orc.scan_sequential(a[None], b[None])[0]

        def all_trees(lo, hi):
            if hi - lo == 1:
                yield (a[lo], b[lo])
                return
            for mid in range(lo + 1, hi):
                for left in all_trees(lo, mid):
                    for right in all_trees(mid, hi):
                        yield orc.compose(left, right)

        for tree in all_trees(0, L):
            err = max(err, _rel(tree[1], xs[-1]))

        # Two log-depth scans of the pairs, each a different bracketing of
        # the same products. Work-efficient form: an up-sweep that combines
        # neighbouring subtrees at strides 1, 2, 4, ..., then a down-sweep
        # that hands every subtree the combination of all pairs before it
        # (the input padded with the identity map (1, 0) to a power of two).
        # Step-doubling form: at each stride d every prefix absorbs the
        # prefix d places before it.
        one = (np.ones(P, np.complex128), np.zeros(P, np.complex128))
        items = [(a[i], b[i]) for i in range(L)]
        n = 1 << (L - 1).bit_length()
        tree = items + [one] * (n - L)
        stride = 1
        while stride < n:
            for right in range(2 * stride - 1, n, 2 * stride):
                tree[right] = orc.compose(tree[right - stride], tree[right])
            stride *= 2
        tree[n - 1] = one
        while stride > 1:
            stride //= 2
            for right in range(2 * stride - 1, n, 2 * stride):
                before, left_total = tree[right], tree[right - stride]
                tree[right - stride] = before
                tree[right] = orc.compose(before, left_total)
        up_down = [orc.compose(tree[i], items[i]) for i in range(L)]
        doubling = list(items)
        stride = 1
        while stride < L:
            doubling = [doubling[i] if i < stride else orc.compose(doubling[i - stride], doubling[i])
                        for i in range(L)]
            stride *= 2
        for pre in (up_down, doubling):
            err = max(err, _rel(np.array([p[1] for p in pre]), xs))
    return err


def pin_tv_equals_ti():
    rng = _rng(8)
    H, P, B, L = 4, 6, 2, 33
    lam, bt, ct, d, logd = _rand_params(rng, H, P)
    u = rng.normal(size=(B, L, H))
    delta = np.broadcast_to(np.exp(logd), (B, L, P)).copy()
    return _rel(orc.forward_timevarying(u, lam, bt, ct, d, delta),
                orc.forward(u, lam, bt, ct, d, logd))


def pin_tv_semigroup():
    """Constant input: cutting one interval into two halves (input held)
    leaves the state at every common physical time unchanged
    (abhik.ai review, "Sampling intervals carry physical meaning")."""
    rng = _rng(9)
    H, P, L = 2, 5, 12
    lam, bt, ct, d, logd = _rand_params(rng, H, P)
    dt = rng.exponential(1.0, size=L)
    uconst = rng.normal(size=H)
    u = np.broadcast_to(uconst, (1, L, H)).copy()
    delta = (np.exp(logd)[None, :] * dt[:, None])[None]
    y = orc.forward_timevarying(u, lam, bt, ct, d, delta)
    s = 5
    dt2 = np.concatenate([dt[:s], [dt[s] / 2, dt[s] / 2], dt[s + 1:]])
    u2 = np.broadcast_to(uconst, (1, L + 1, H)).copy()
    delta2 = (np.exp(logd)[None, :] * dt2[:, None])[None]
    y2 = orc.forward_timevarying(u2, lam, bt, ct, d, delta2)
    keep = np.concatenate([np.arange(s), np.arange(s + 1, L + 1)])
    return _rel(y2[:, keep, :], y)


def pin_tv_zero_interval():
    rng = _rng(10)
    H, P, L = 3, 4, 10
    lam, bt, ct, d, logd = _rand_params(rng, H, P)
    u = rng.normal(size=(1, L, H))
    delta = (np.exp(logd)[None, :] * rng.exponential(1.0, size=(L, 1)))[None]
    delta[0, 6, :] = 0.0
    y = orc.forward_timevarying(u, lam, bt, ct, d, delta)
    # a zero interval is the identity step: C~ x_6 = C~ x_5
    return _rel(y[0, 6] - d * u[0, 6], y[0, 5] - d * u[0, 5])


# ---------------------------------------------------------------------------
# Stateful form (O6): initial state in, final state out
# ---------------------------------------------------------------------------

def pin_state_free_response():
    # u = 0 from a given state: x_k = Lambda_bar^(k+1) x0 in closed form, so
    # y_k = Re(C~ Lambda_bar^(k+1) x0) and the final state Lambda_bar^L x0
    rng = _rng(11)
    H, P, L, B = 3, 5, 9, 2
    lam, bt, ct, d, logd = _rand_params(rng, H, P)
    x0 = rng.normal(size=(B, P)) + 1j * rng.normal(size=(B, P))
    u = np.zeros((B, L, H))
    y, xl = orc.forward_state(u, lam, bt, ct, d, logd, x0)
    lb = np.exp(lam * np.exp(logd))
    powers = lb[None, :] ** np.arange(1, L + 1)[:, None]             # [L, P]
    xk = x0[:, None, :] * powers[None]                               # [B, L, P]
    y_ref = (xk @ ct.T).real
    return max(_rel(y, y_ref), _rel(xl, x0 * lb ** L))


def pin_state_split_run():
    # a sequence processed in two pieces with the state carried between them
    # equals one run, time-invariant and time-varying
    rng = _rng(12)
    H, P, L, B, L1 = 4, 6, 23, 2, 9
    lam, bt, ct, d, logd = _rand_params(rng, H, P)
    u = rng.normal(size=(B, L, H))
    x0 = rng.normal(size=(B, P)) + 1j * rng.normal(size=(B, P))
    y, xl = orc.forward_state(u, lam, bt, ct, d, logd, x0)
    ya, xm = orc.forward_state(u[:, :L1], lam, bt, ct, d, logd, x0)
    yb, xl2 = orc.forward_state(u[:, L1:], lam, bt, ct, d, logd, xm)
    err = max(_rel(np.concatenate([ya, yb], axis=1), y), _rel(xl2, xl))
    delta = np.exp(logd)[None, None, :] * rng.exponential(1.0, size=(B, L, 1))
    y, xl = orc.forward_timevarying_state(u, lam, bt, ct, d, delta, x0)
    ya, xm = orc.forward_timevarying_state(u[:, :L1], lam, bt, ct, d, delta[:, :L1], x0)
    yb, xl2 = orc.forward_timevarying_state(u[:, L1:], lam, bt, ct, d, delta[:, L1:], xm)
    return max(err, _rel(np.concatenate([ya, yb], axis=1), y), _rel(xl2, xl))


def pin_state_superposition():
    # the layer is affine in (u, x0): the output from (u, x0) is the output
    # from (u, 0) plus the free response from x0 with zero input
    rng = _rng(13)
    H, P, L, B = 3, 4, 12, 1
    lam, bt, ct, d, logd = _rand_params(rng, H, P)
    u = rng.normal(size=(B, L, H))
    x0 = rng.normal(size=(B, P)) + 1j * rng.normal(size=(B, P))
    y, xl = orc.forward_state(u, lam, bt, ct, d, logd, x0)
    y_u = orc.forward(u, lam, bt, ct, d, logd)
    y0, xl0 = orc.forward_state(np.zeros_like(u), lam, bt, ct, d, logd, x0)
    _, xl_u = orc.forward_state(u, lam, bt, ct, d, logd, None)
    # (the feedthrough D u is in y_u only: y0 has zero input)
    return max(_rel(y, y_u + y0), _rel(xl, xl_u + xl0))



# ---- options of the forward path (O7-O10) -----------------------------------

def pin_bilinear_trapezoid():
    """O8 is the trapezoid rule: its states satisfy
    x_k - x_{k-1} = (lambda Delta_k / 2)(x_k + x_{k-1}) + Delta_k B~ u_k
    (derivative averaged over both ends of the step, input held at u_k),
    time-invariant and (through forward_ex's final state) time-varying."""
    rng = _rng(40)
    H, P, L = 3, 5, 12
    lam, bt, ct, d, logd = _rand_params(rng, H, P)
    delta = np.exp(logd) * 5.0
    lb, g = orc.bilinear(lam, delta)
    u = rng.normal(size=(2, L, H))
    x = orc.scan_sequential(lb, orc.drive(u, g[:, None] * bt))
    xprev = np.concatenate([np.zeros((2, 1, P)), x[:, :-1]], axis=1)
    res = x - xprev - 0.5 * lam * delta * (x + xprev) - delta * orc.drive(u, bt)
    err = float(np.max(np.abs(res)) / np.max(np.abs(x)))
    # time-varying, through the public form: x_k from prefix runs
    dtv = rng.uniform(0.01, 0.5, size=(2, L, P))
    xs = np.stack([orc.forward_ex(u[:, :k + 1], lam, bt, ct, d, delta=dtv[:, :k + 1],
                                  method="bilinear")[1] for k in range(L)], axis=1)
    xprev = np.concatenate([np.zeros((2, 1, P)), xs[:, :-1]], axis=1)
    res = xs - xprev - 0.5 * lam * dtv * (xs + xprev) - dtv * orc.drive(u, bt)
    return max(err, float(np.max(np.abs(res)) / np.max(np.abs(xs))))


def pin_bilinear_equilibrium():
    """Under a constant input both discretisations settle at the continuous
    system's equilibrium x* = -B~ u / lambda, so y -> Re(C~ x*) + D u."""
    rng = _rng(41)
    H, P, L = 3, 6, 400
    lam = -rng.uniform(1.0, 3.0, P) + 1j * rng.uniform(-5, 5, P)
    _, bt, ct, d, _ = _rand_params(rng, H, P, lam=lam)
    logd = rng.uniform(math.log(0.2), math.log(1.0), P)
    u0 = rng.normal(size=(2, H))
    u = np.repeat(u0[:, None, :], L, axis=1)
    xs = -(u0 @ bt.T) / lam
    y_inf = (xs @ ct.T).real + d * u0
    err = 0.0
    for method in ("bilinear", "zoh"):
        y, _ = orc.forward_ex(u, lam, bt, ct, d, log_delta=logd, method=method)
        err = max(err, _rel(y[:, -1], y_inf))
    return err


def pin_bilinear_map():
    """The bilinear map sends the open left half-plane into the open unit disk
    and the imaginary axis onto the unit circle, for every Delta > 0; against
    ZOH its one-step error is z^3/12 for small z = lambda Delta."""
    rng = _rng(42)
    lam = -rng.uniform(1e-6, 50, 2000) + 1j * rng.uniform(-500, 500, 2000)
    delta = np.exp(rng.uniform(math.log(1e-3), math.log(100.0), 2000))
    lb, _ = orc.bilinear(lam, delta)
    err = max(0.0, float(np.max(np.abs(lb))) - 1.0 + 1e-15)
    lb_axis, _ = orc.bilinear(1j * lam.imag, delta)
    err = max(err, float(np.max(np.abs(np.abs(lb_axis) - 1.0))))
    z = 1e-3 * np.exp(1j * np.linspace(0.3, 2.8, 7))
    lbz, _ = orc.bilinear(z, 1.0)
    ratio = np.abs(lbz - np.exp(z)) / (np.abs(z) ** 3 / 12.0)
    return max(err, float(np.max(np.abs(ratio - 1.0))) * 1e-2)   # ratio within 1 % of 1


def _conjugate_completed(rng, H, Ph):
    lam_h, bt_h, ct_h, d, logd_h = _rand_params(rng, H, Ph)
    full = (np.concatenate([lam_h, lam_h.conj()]), np.concatenate([bt_h, bt_h.conj()], axis=0),
            np.concatenate([ct_h, ct_h.conj()], axis=1), d, np.concatenate([logd_h, logd_h]))
    return (lam_h, bt_h, ct_h, d, logd_h), full


def pin_half_spectrum_ex():
    """O7 through forward_ex: the half-spectrum form equals the full-spectrum
    O5 output of the conjugate-completed system (feedthrough once), for
    time-invariant, time-varying and bidirectional forms."""
    rng = _rng(43)
    H, Ph, L = 3, 4, 25
    (lam_h, bt_h, ct_h, d, logd_h), (lam, bt, ct, _, logd) = _conjugate_completed(rng, H, Ph)
    u = rng.normal(size=(2, L, H))
    err = _rel(orc.forward_ex(u, lam_h, bt_h, ct_h, d, log_delta=logd_h, conj_sym=True)[0],
               orc.forward(u, lam, bt, ct, d, logd))
    dt = rng.uniform(0.0, 0.2, size=(2, L, Ph))
    err = max(err, _rel(orc.forward_ex(u, lam_h, bt_h, ct_h, d, delta=dt, conj_sym=True)[0],
                        orc.forward_timevarying(u, lam, bt, ct, d, np.concatenate([dt, dt], axis=2))))
    ct2_h = (rng.normal(size=(H, 2 * Ph)) + 1j * rng.normal(size=(H, 2 * Ph))) / math.sqrt(2 * H)
    ct2 = np.concatenate([ct2_h[:, :Ph], ct2_h[:, :Ph].conj(), ct2_h[:, Ph:], ct2_h[:, Ph:].conj()], axis=1)
    yh = orc.forward_ex(u, lam_h, bt_h, ct2_h, d, log_delta=logd_h, conj_sym=True, bidirectional=True)[0]
    yf = orc.forward_ex(u, lam, bt, ct2, d, log_delta=logd, bidirectional=True)[0]
    return max(err, _rel(yh, yf))


def pin_gelu_values():
    """O9 against the normal distribution function integrated numerically
    (Phi(x) = 1/2 + int_0^x exp(-t^2/2)/sqrt(2 pi) dt), the table value
    Phi(1) = 0.8413447460685429, and GELU(x) - GELU(-x) = x."""
    xs = np.array([-4.0, -1.7, -1.0, -0.25, 0.0, 0.3, 1.0, 2.5, 6.0])
    phi = np.array([0.5 + scipy.integrate.quad(lambda t: math.exp(-0.5 * t * t), 0.0, x,
                                               epsabs=1e-14, epsrel=1e-13)[0] / math.sqrt(2 * math.pi)
                    for x in xs])
    err = float(np.max(np.abs(orc.gelu(xs) - xs * phi)))
    err = max(err, abs(float(orc.gelu(1.0)) - 0.8413447460685429))
    err = max(err, float(np.max(np.abs(orc.gelu(xs) - orc.gelu(-xs) - xs))))
    return err


def pin_gelu_tanh():
    """O9t, the tanh form: (1 + tanh k)/2 is the logistic function of 2k, so
    the form equals x * expit(2k) evaluated through the exponential; it is odd
    up to the identity f(x) - f(-x) = x; its x^2 Taylor coefficient is
    GELU's, 1/sqrt(2 pi) (from Phi'(0)); and it stays within 5e-4 of
    x Phi(x) with Phi integrated numerically (it approximates GELU)."""
    xs = np.linspace(-6.0, 6.0, 97)
    k = math.sqrt(2.0 / math.pi) * (xs + 0.044715 * xs ** 3)
    f = orc.gelu_tanh(xs)
    err = float(np.max(np.abs(f - xs * scipy.special.expit(2.0 * k))))
    err = max(err, float(np.max(np.abs(f - orc.gelu_tanh(-xs) - xs))))
    h = 1e-4
    c2 = (float(orc.gelu_tanh(h)) + float(orc.gelu_tanh(-h))) / (2.0 * h * h)
    err = max(err, abs(c2 - 1.0 / math.sqrt(2.0 * math.pi)) * 1e-6)
    phi = np.array([0.5 + scipy.integrate.quad(lambda t: math.exp(-0.5 * t * t), 0.0, x,
                                               epsabs=1e-14, epsrel=1e-13)[0] / math.sqrt(2 * math.pi)
                    for x in xs])
    dist = float(np.max(np.abs(f - xs * phi)))
    return err if dist <= 5e-4 else max(err, dist)


def _conv_bidirectional(u, lam, bt, ct2, d, logd):
    """Two-sided convolution: y_k = sum_{j<=k} Kf_{k-j} u_j + sum_{j>=k} Kb_{j-k} u_j
    + D u_k, Kf_i = Re(C_f Lb^i B_bar), Kb_i = Re(C_b Lb^i B_bar), with the
    discretisation from the augmented-matrix exponential and direct powers."""
    P = lam.shape[0]
    lb, g = _zoh_expm(lam, np.exp(logd))
    z = np.log(lb)
    bb = g[:, None] * bt
    B, L, H = u.shape
    pw = np.exp(np.outer(np.arange(L), z))
    kf = np.einsum("hp,ip,pq->ihq", ct2[:, :P], pw, bb).real
    kb = np.einsum("hp,ip,pq->ihq", ct2[:, P:], pw, bb).real
    y = np.zeros((B, L, H))
    for k in range(L):
        y[:, k] = np.einsum("jhq,bjq->bh", kf[k::-1], u[:, :k + 1]) + \
                  np.einsum("jhq,bjq->bh", kb[:L - k], u[:, k:])
    return y + d * u


def pin_bidirectional_convolution():
    rng = _rng(44)
    H, P, L = 3, 5, 30
    lam, bt, _, d, logd = _rand_params(rng, H, P)
    ct2 = (rng.normal(size=(H, 2 * P)) + 1j * rng.normal(size=(H, 2 * P))) / math.sqrt(2 * H)
    u = rng.normal(size=(2, L, H))
    y = orc.forward_ex(u, lam, bt, ct2, d, log_delta=logd, bidirectional=True)[0]
    return _rel(y, _conv_bidirectional(u, lam, bt, ct2, d, logd))


def pin_bidirectional_reversal():
    """Reversing time and swapping the two readout halves reverses the output."""
    rng = _rng(45)
    H, P, L = 4, 6, 33
    lam, bt, _, d, logd = _rand_params(rng, H, P)
    ct2 = (rng.normal(size=(H, 2 * P)) + 1j * rng.normal(size=(H, 2 * P))) / math.sqrt(2 * H)
    u = rng.normal(size=(2, L, H))
    y = orc.forward_ex(u, lam, bt, ct2, d, log_delta=logd, bidirectional=True)[0]
    swapped = np.concatenate([ct2[:, P:], ct2[:, :P]], axis=1)
    yr = orc.forward_ex(u[:, ::-1], lam, bt, swapped, d, log_delta=logd, bidirectional=True)[0]
    return _rel(y, yr[:, ::-1])


def pin_sigmoid_tanh_identity():
    """sigma(x) = (1 + tanh(x / 2)) / 2, and sigma(x) + sigma(-x) = 1."""
    x = np.linspace(-30.0, 30.0, 601)
    err = float(np.max(np.abs(orc.sigmoid(x) - 0.5 * (1.0 + np.tanh(0.5 * x)))))
    return max(err, float(np.max(np.abs(orc.sigmoid(x) + orc.sigmoid(-x) - 1.0))))


def pin_glu_brute_force():
    """O11 against explicit loops over tokens, outputs and inputs on a tiny
    case with a non-symmetric W, for both variants, with and without bias."""
    rng = _rng(47)
    T, H = 3, 5
    y = rng.normal(size=(T, H)) * 2.0
    w = rng.normal(size=(H, H))
    b = rng.normal(size=H)
    err = 0.0
    for variant in (1, 2):
        for bias in (None, b):
            got = orc.glu(y, w, bias, variant)
            for t in range(T):
                g = [y[t, i] * 0.5 * (1.0 + math.erf(y[t, i] / math.sqrt(2.0))) for i in range(H)]
                for j in range(H):
                    pre = sum(w[j, i] * g[i] for i in range(H)) + (0.0 if bias is None else bias[j])
                    gate = 1.0 / (1.0 + math.exp(-pre))
                    want = (g[j] if variant == 1 else y[t, j]) * gate
                    err = max(err, abs(got[t, j] - want))
    return err


def pin_glu_limits():
    """W = 0, b = 0 halves the gated value; a large positive bias opens the
    gate fully (variant 1 gives GELU(y), variant 2 gives y)."""
    rng = _rng(48)
    y = rng.normal(size=(4, 6))
    z = np.zeros((6, 6))
    err = max(float(np.max(np.abs(orc.glu(y, z, None, 1) - 0.5 * orc.gelu(y)))),
              float(np.max(np.abs(orc.glu(y, z, None, 2) - 0.5 * y))))
    big = np.full(6, 60.0)
    err = max(err, float(np.max(np.abs(orc.glu(y, z, big, 1) - orc.gelu(y)))),
              float(np.max(np.abs(orc.glu(y, z, big, 2) - y))))
    return err


ALL_PINS = {
    "zoh_expm": (pin_zoh_expm, 1e-12),
    "constant_input": (pin_constant_input_closed_form, 1e-12),
    "ode_ti": (pin_ode_time_invariant, 1e-8),
    "ode_tv": (pin_ode_time_varying, 1e-8),
    "convolution": (pin_convolution_form, 1e-10),
    "impulse": (pin_impulse_response, 1e-10),
    "half_spectrum": (pin_half_spectrum, 1e-12),
    "bracketings": (pin_scan_bracketings, 1e-12),
    "tv_equals_ti": (pin_tv_equals_ti, 1e-13),
    "tv_semigroup": (pin_tv_semigroup, 1e-12),
    "tv_zero_interval": (pin_tv_zero_interval, 1e-13),
    "state_free_response": (pin_state_free_response, 1e-12),
    "state_split_run": (pin_state_split_run, 1e-12),
    "state_superposition": (pin_state_superposition, 1e-12),
    "bilinear_trapezoid": (pin_bilinear_trapezoid, 1e-12),
    "bilinear_equilibrium": (pin_bilinear_equilibrium, 1e-10),
    "bilinear_map": (pin_bilinear_map, 1e-4),
    "half_spectrum_ex": (pin_half_spectrum_ex, 1e-12),
    "gelu_values": (pin_gelu_values, 1e-13),
    "gelu_tanh": (pin_gelu_tanh, 1e-12),
    "bidirectional_convolution": (pin_bidirectional_convolution, 1e-10),
    "bidirectional_reversal": (pin_bidirectional_reversal, 1e-12),
    "sigmoid_tanh_identity": (pin_sigmoid_tanh_identity, 1e-15),
    "glu_brute_force": (pin_glu_brute_force, 1e-13),
    "glu_limits": (pin_glu_limits, 1e-15),
}


@pytest.mark.parametrize("name", sorted(ALL_PINS))
def test_pin(name):
    fn, tol = ALL_PINS[name]
    err = fn()
    assert err <= tol, f"pin {name}: error {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------------------
# Values printed on the pages
# ---------------------------------------------------------------------------

def _load_golden(name):
    return np.loadtxt(os.path.join(GOLDEN, name), comments="#", ndmin=2)


def test_golden_hippo_n8_eigenvalues():
    ref = _load_golden("hippo_n8_eigenvalues.txt")
    lam = wl.hippo_n_eigenvalues(8)
    assert np.all(lam.real == -0.5)
    assert np.max(np.abs(np.sort(lam.imag) - np.sort(ref[:, 1]))) < 5e-4


def test_golden_bilinear_scalar():
    for lre, lim, dt, expect, dec in _load_golden("bilinear_scalar.txt"):
        lb, _ = orc.bilinear(lre + 1j * lim, dt)
        assert abs(lb.real - expect) <= 0.5 * 10.0 ** (-dec) and abs(lb.imag) < 1e-15


def _s4_two_state_system():
    """The S4 page's two-state example in the form the S5 oracle takes: the
    HiPPO-LegS matrix of size 2 (eigenvalues -1, -2) and its input vector
    B_n = (2n+1)^(1/2), diagonalised numerically (A = V diag(lam) V^-1), so
    that B~ = V^-1 B and C~ = C V with C = [1 0]. The bilinear map is a
    rational function of A, so it commutes with the change of basis."""
    a = wl.hippo_legs(2)
    bvec = np.sqrt(2.0 * np.arange(2) + 1.0)
    lam, v = np.linalg.eig(a)
    bt = np.linalg.solve(v, bvec)[:, None].astype(np.complex128)
    ct = (np.array([[1.0, 0.0]]) @ v).astype(np.complex128)
    return lam.astype(np.complex128), bt, ct


def pin_s4_two_state_pulse():
    """S4 page, section "An LTI system computes a convolution": the bilinear
    two-state system at step size 1 gives the printed kernel (2/3)(1/3)^i as
    its impulse response and the pulse outputs 2/3, 8/9, 26/27, 80/81, then a
    decay by 3 per step (tests/golden/s4_bilinear_n2_pulse.txt)."""
    ref = _load_golden("s4_bilinear_n2_pulse.txt")
    lam, bt, ct = _s4_two_state_system()
    logd = np.zeros(2)                       # Delta = 1
    n = ref.shape[0]
    u = ref[:, 1].reshape(1, n, 1)
    y, _ = orc.forward_ex(u, lam, bt, ct, np.zeros(1), log_delta=logd, method="bilinear")
    imp = np.zeros((1, n, 1))
    imp[0, 0, 0] = 1.0
    k, _ = orc.forward_ex(imp, lam, bt, ct, np.zeros(1), log_delta=logd, method="bilinear")
    return max(float(np.max(np.abs(y[0, :, 0] - ref[:, 2] / ref[:, 3]))),
               float(np.max(np.abs(k[0, :, 0] - ref[:, 4] / ref[:, 5]))))


def test_golden_s4_two_state_pulse():
    assert pin_s4_two_state_pulse() <= 1e-13


def test_golden_zoh_scalar():
    for lre, lim, dt, expect in _load_golden("zoh_scalar.txt"):
        lb, _ = orc.zoh(lre + 1j * lim, dt)
        assert abs(lb.real - expect) < 5e-5 and abs(lb.imag) < 1e-15


# ---------------------------------------------------------------------------
# Generator-side structure (HiPPO-N), stability, validation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [8, 32, 48, 128])
def test_hippo_normal_structure(n):
    a = wl.hippo_normal(n)
    assert np.max(np.abs(np.diag(a) + 0.5)) < 1e-12
    s = a + 0.5 * np.eye(n)
    assert np.max(np.abs(s + s.T)) < 1e-12
    # the Hermitian reading agrees with a general eigen-solver of A_N itself
    lam = wl.hippo_n_eigenvalues(n)
    ev = np.linalg.eigvals(a)
    assert np.max(np.abs(ev.real + 0.5)) < 1e-8 * n
    assert np.max(np.abs(np.sort(ev.imag) - np.sort(lam.imag))) < 1e-8 * n * n
    # conjugate pairs
    assert np.max(np.abs(np.sort(lam.imag) + np.sort(lam.imag)[::-1])) < 1e-9 * n


def test_hippo_legs_plus_rank_one():
    # the S4 page's decomposition: A_N - p p^T is lower triangular with -(n+1)
    n = 6
    p = np.sqrt(np.arange(n) + 0.5)
    legs = wl.hippo_normal(n) - np.outer(p, p)
    assert np.allclose(np.triu(legs, 1), 0, atol=1e-14)
    assert np.allclose(np.diag(legs), -(np.arange(n) + 1.0))


def test_stability_decay():
    lam = wl.hippo_n_eigenvalues(32)
    for dt in [1e-4, 1e-2, 0.1]:
        lb, _ = orc.zoh(lam, dt)
        assert np.all(np.abs(lb) < 1.0)
        assert np.allclose(np.abs(lb), np.exp(-0.5 * dt), rtol=1e-13)
    lb, _ = orc.zoh(lam, 1e-4)
    assert np.allclose(np.abs(lb) ** 16384, math.exp(-0.5 * 1e-4 * 16384), rtol=1e-9)


def test_zero_pole_limit():
    dt = 0.037
    for lam in [0.0 + 0.0j, 1e-9 + 0j, -1e-7 + 3e-7j]:
        _, g = orc.zoh(lam, dt)
        assert abs(g - dt) <= 1e-6 * dt
    # continuity across the series boundary |z| = 1e-4
    lam_dir = np.array([1.0 + 0.0j, -0.6 + 0.8j, 1j])
    for l in lam_dir:
        zs = np.array([1e-4 * (1 - 1e-9), 1e-4 * (1 + 1e-9)])
        _, g = orc.zoh(l * zs / dt, dt)
        assert abs(g[0] - g[1]) <= 1e-11 * abs(g[0])
        # and both sides agree with the augmented-matrix exponential
        _, ge = _zoh_expm(l * zs / dt, dt)
        assert _rel(g, ge) < 1e-11


def test_intervals_rejected():
    for bad in [-1e-3, float("nan"), float("inf")]:
        with pytest.raises(ValueError):
            orc.zoh(np.array([-0.5 + 1j]), np.array([bad]))
    with pytest.raises(ValueError):
        orc.forward_timevarying(np.zeros((1, 2, 1)), np.array([-0.5]), np.ones((1, 1)),
                                np.ones((1, 1)), np.zeros(1), -np.ones((1, 2, 1)))


def test_associativity_exact_and_not_commutative():
    rng = _rng(11)
    for _ in range(200):
        e = [(complex(*rng.integers(-8, 9, 2)), complex(*rng.integers(-8, 9, 2)))
             for _ in range(3)]
        l = orc.compose(orc.compose(e[0], e[1]), e[2])
        r = orc.compose(e[0], orc.compose(e[1], e[2]))
        assert l == r
    # random complex: equal to a few ulps
    a = np.exp(rng.normal(size=(3, 64)) * 0.1 + 1j * rng.normal(size=(3, 64)))
    b = rng.normal(size=(3, 64)) + 1j * rng.normal(size=(3, 64))
    l = orc.compose(orc.compose((a[0], b[0]), (a[1], b[1])), (a[2], b[2]))
    r = orc.compose((a[0], b[0]), orc.compose((a[1], b[1]), (a[2], b[2])))
    assert np.max(np.abs(l[1] - r[1]) / np.abs(r[1])) < 1e-14
    # order matters
    e1, e2 = (2.0 + 0j, 1.0 + 0j), (3.0 + 0j, 5.0 + 0j)
    assert orc.compose(e1, e2) != orc.compose(e2, e1)


def test_lti_properties():
    rng = _rng(12)
    H, P, B, L = 3, 5, 1, 30
    lam, bt, ct, d, logd = _rand_params(rng, H, P)
    u1 = rng.normal(size=(B, L, H))
    u2 = rng.normal(size=(B, L, H))
    f = lambda u: orc.forward(u, lam, bt, ct, d, logd)
    # linearity
    assert _rel(f(2.5 * u1 - 0.75 * u2), 2.5 * f(u1) - 0.75 * f(u2)) < 1e-12
    # time-shift equivariance with zero padding
    s = 7
    us = np.zeros_like(u1)
    us[:, s:, :] = u1[:, :-s, :]
    assert _rel(f(us)[:, s:, :], f(u1)[:, :-s, :]) < 1e-12
    assert np.all(f(us)[:, :s, :] == 0)
    # causality: a change at k0 leaves earlier outputs bit-identical
    k0 = 13
    up = u1.copy()
    up[:, k0, :] += 1.0
    assert np.array_equal(f(up)[:, :k0, :], f(u1)[:, :k0, :])


def test_full_config0_conv_agrees():
    # the tiny config end to end, against the convolution-kernel form
    w = wl.make_config(0)
    args = (w.u.astype(np.float64), w.lam, w.b_tilde, w.c_tilde, w.d, w.log_delta)
    y = orc.forward(*args)
    yc, _ = _conv_kernel_forward(*args)
    assert _rel(y, yc) < 1e-10


# ---------------------------------------------------------------------------
# Planted mistakes (on the CPU, in the oracle): each must trip a pin
# ---------------------------------------------------------------------------

def _fails(pin_name):
    fn, tol = ALL_PINS[pin_name]
    try:
        err = fn()
    except Exception:
        return True
    return not (err <= tol)


def test_planted_readout_factor_two(monkeypatch):
    good = orc.readout
    monkeypatch.setattr(orc, "readout", lambda x, c, d, u: good(2.0 * x, c, d, u))
    # the half-spectrum pin scales both of its sides and cannot see this one
    assert _fails("convolution") and _fails("ode_ti") and _fails("constant_input")


def test_planted_readout_imag_part(monkeypatch):
    monkeypatch.setattr(orc, "readout", lambda x, c, d, u: (np.asarray(x) @ np.asarray(c).T).imag
                        + np.asarray(d) * np.asarray(u))
    assert _fails("half_spectrum") and _fails("convolution") and _fails("ode_ti")


def test_planted_euler_gain(monkeypatch):
    good = orc.zoh

    def euler(lam, delta):
        lb, _ = good(lam, delta)
        return lb, np.broadcast_to(np.asarray(delta, np.float64), lb.shape).astype(np.complex128)

    monkeypatch.setattr(orc, "zoh", euler)
    assert _fails("zoh_expm") and _fails("ode_ti") and _fails("constant_input")


def test_planted_conjugated_transition(monkeypatch):
    good = orc.zoh
    monkeypatch.setattr(orc, "zoh", lambda lam, delta: tuple(
        v.conj() if i == 0 else v for i, v in enumerate(good(lam, delta))))
    assert _fails("zoh_expm") and _fails("convolution") and _fails("ode_tv")


def test_planted_dropped_feedthrough(monkeypatch):
    good = orc.readout
    monkeypatch.setattr(orc, "readout", lambda x, c, d, u: good(x, c, 0.0 * np.asarray(d), u))
    assert _fails("impulse") and _fails("convolution") and _fails("ode_ti")


def test_planted_transposed_readout(monkeypatch):
    monkeypatch.setattr(orc, "readout", lambda x, c, d, u: (np.asarray(x) @ np.asarray(c)).real
                        + np.asarray(d) * np.asarray(u))
    # square case only can even run; shapes differ elsewhere and raise
    assert _fails("convolution") and _fails("impulse")


def test_planted_off_by_one_scan(monkeypatch):
    def shifted(lam_bar, bu):
        bu = np.asarray(bu, np.complex128)
        lam_bar = np.asarray(lam_bar, np.complex128)
        tv = lam_bar.ndim == 3
        x = np.zeros((bu.shape[0], bu.shape[2]), np.complex128)
        out = np.empty_like(bu)
        for k in range(bu.shape[1]):
            out[:, k, :] = x              # state before the update: wrong index
            a = lam_bar[:, k, :] if tv else lam_bar
            x = a * x + bu[:, k, :]
        return out

    monkeypatch.setattr(orc, "scan_sequential", shifted)
    assert _fails("impulse") and _fails("constant_input") and _fails("bracketings")


def test_planted_tv_uses_previous_interval(monkeypatch):
    good = orc.zoh

    def prev_interval(lam, delta):
        d = np.asarray(delta, np.float64)
        if d.ndim == 3:
            d = np.concatenate([d[:, :1], d[:, :-1]], axis=1)
        return good(lam, d)

    monkeypatch.setattr(orc, "zoh", prev_interval)
    assert _fails("ode_tv") and _fails("tv_zero_interval")


def test_planted_series_guard_wrong(monkeypatch):
    # a series with the wrong factorial (z^n / n!) near zero
    good = orc.zoh

    def bad(lam, delta):
        lb, g = good(lam, delta)
        lam_b, d = np.broadcast_arrays(np.asarray(lam, np.complex128),
                                       np.asarray(delta, np.float64))
        z = lam_b * d
        small = np.abs(z) < orc.SERIES_RADIUS
        g = g.copy()
        g[small] = d[small] * np.exp(z[small])
        return lb, g

    monkeypatch.setattr(orc, "zoh", bad)
    with pytest.raises(AssertionError):
        test_zero_pole_limit()


def test_planted_initial_state_not_advanced(monkeypatch):
    # the initial state taken as the state after step 0's transition (x_0 =
    # x0 + b_0 instead of a_0 x0 + b_0)
    def wrong(lam_bar, bu, x0=None):
        bu = np.asarray(bu, np.complex128)
        lam_bar = np.asarray(lam_bar, np.complex128)
        tv = lam_bar.ndim == 3
        x = np.zeros((bu.shape[0], bu.shape[2]), np.complex128)
        out = np.empty_like(bu)
        for k in range(bu.shape[1]):
            a = lam_bar[:, k, :] if tv else lam_bar
            if k == 0 and x0 is not None:
                x = np.asarray(x0, np.complex128) + bu[:, 0, :]
            else:
                x = a * x + bu[:, k, :]
            out[:, k, :] = x
        return out

    monkeypatch.setattr(orc, "scan_sequential", wrong)
    assert _fails("state_free_response") and _fails("state_split_run")


def test_planted_initial_state_ignored(monkeypatch):
    good = orc.scan_sequential
    monkeypatch.setattr(orc, "scan_sequential", lambda lam_bar, bu, x0=None: good(lam_bar, bu))
    # (superposition holds trivially when x0 has no effect)
    assert _fails("state_free_response") and _fails("state_split_run")


def test_planted_bilinear_inverted(monkeypatch):
    good = orc.bilinear
    monkeypatch.setattr(orc, "bilinear", lambda lam, delta: (1.0 / good(lam, delta)[0], good(lam, delta)[1]))
    assert _fails("bilinear_trapezoid") and _fails("bilinear_map") and _fails("bilinear_equilibrium")


def test_planted_bilinear_gain_without_backward_step(monkeypatch):
    good = orc.bilinear
    monkeypatch.setattr(orc, "bilinear", lambda lam, delta: (good(lam, delta)[0],
                                                             np.broadcast_to(orc.check_intervals(delta), np.shape(good(lam, delta)[1])).astype(np.complex128)))
    assert _fails("bilinear_trapezoid") and _fails("bilinear_equilibrium")


def test_planted_bilinear_gain_without_backward_step_trips_s4_example(monkeypatch):
    good = orc.bilinear
    monkeypatch.setattr(orc, "bilinear", lambda lam, delta: (good(lam, delta)[0],
                                                             np.broadcast_to(orc.check_intervals(delta), np.shape(good(lam, delta)[1])).astype(np.complex128)))
    assert pin_s4_two_state_pulse() > 1e-3


def test_planted_bilinear_replaced_by_zoh_trips_s4_example(monkeypatch):
    monkeypatch.setattr(orc, "bilinear", orc.zoh)
    assert pin_s4_two_state_pulse() > 1e-3


def test_planted_bilinear_forward_step_only_trips_s4_example(monkeypatch):
    # Lambda_bar = 1 + z/2 without the backward half-step
    good = orc.bilinear
    monkeypatch.setattr(orc, "bilinear", lambda lam, delta: (1.0 + 0.5 * np.asarray(lam) * orc.check_intervals(delta),
                                                             good(lam, delta)[1]))
    assert pin_s4_two_state_pulse() > 1e-3


def test_planted_compose_order_swapped(monkeypatch):
    monkeypatch.setattr(orc, "compose", lambda earlier, later: (earlier[0] * later[0],
                                                               earlier[0] * later[1] + earlier[1]))
    assert _fails("bracketings")


def test_planted_backward_scan_exclusive(monkeypatch):
    def exclusive(lam_bar, bu):
        bu = np.asarray(bu, np.complex128)
        x = np.zeros((bu.shape[0], bu.shape[2]), np.complex128)
        out = np.empty_like(bu)
        for k in range(bu.shape[1] - 1, -1, -1):
            out[:, k] = x
            x = lam_bar * x + bu[:, k]
        return out
    monkeypatch.setattr(orc, "scan_reverse", exclusive)
    assert _fails("bidirectional_convolution") and _fails("bidirectional_reversal")


def test_planted_half_spectrum_doubles_feedthrough(monkeypatch):
    monkeypatch.setattr(orc, "readout_half", lambda x, c, d, u: 2.0 * orc.readout(x, c, d, u))
    assert _fails("half_spectrum_ex")


def test_planted_gelu_tanh_form(monkeypatch):
    def tanh_gelu(y):
        y = np.asarray(y, np.float64)
        return 0.5 * y * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (y + 0.044715 * y ** 3)))
    monkeypatch.setattr(orc, "gelu", tanh_gelu)
    assert _fails("gelu_values")


def test_planted_gelu_tanh_without_sqrt_two_over_pi(monkeypatch):
    monkeypatch.setattr(orc, "gelu_tanh", lambda y: 0.5 * np.asarray(y, np.float64)
                        * (1.0 + np.tanh(np.asarray(y, np.float64) + 0.044715 * np.asarray(y, np.float64) ** 3)))
    assert _fails("gelu_tanh")


def test_planted_gelu_tanh_cubic_coefficient(monkeypatch):
    monkeypatch.setattr(orc, "gelu_tanh", lambda y: 0.5 * np.asarray(y, np.float64)
                        * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (np.asarray(y, np.float64)
                                                                  + 0.44715 * np.asarray(y, np.float64) ** 3))))
    assert _fails("gelu_tanh")


def test_planted_gelu_tanh_replaced_by_exact_form(monkeypatch):
    monkeypatch.setattr(orc, "gelu_tanh", orc.gelu)
    assert _fails("gelu_tanh")


def test_gelu_forms_differ_through_forward_ex():
    rng = _rng(47)
    lam, bt, ct, d, logd = _rand_params(rng, 4, 6)
    u = 3.0 * rng.normal(size=(1, 40, 4))
    y0 = orc.forward_ex(u, lam, bt, ct, d, log_delta=logd)[0]
    ye = orc.forward_ex(u, lam, bt, ct, d, log_delta=logd, activation="gelu")[0]
    yt = orc.forward_ex(u, lam, bt, ct, d, log_delta=logd, activation="gelu_tanh")[0]
    assert np.array_equal(ye, orc.gelu(y0)) and np.array_equal(yt, orc.gelu_tanh(y0))
    assert 1e-6 < float(np.max(np.abs(ye - yt))) <= 5e-4


def test_forward_ex_reduces_to_the_plain_forms():
    rng = _rng(46)
    H, P, L = 3, 5, 20
    lam, bt, ct, d, logd = _rand_params(rng, H, P)
    u = rng.normal(size=(2, L, H))
    x0 = rng.normal(size=(2, P)) + 1j * rng.normal(size=(2, P))
    y, xl = orc.forward_ex(u, lam, bt, ct, d, log_delta=logd, x0=x0)
    yo, xo = orc.forward_state(u, lam, bt, ct, d, logd, x0)
    assert _rel(y, yo) < 1e-15 and _rel(xl, xo) < 1e-15
    dt = rng.uniform(0, 0.1, size=(2, L, P))
    assert _rel(orc.forward_ex(u, lam, bt, ct, d, delta=dt)[0], orc.forward_timevarying(u, lam, bt, ct, d, dt)) < 1e-15
    ct2 = np.concatenate([ct, np.zeros_like(ct)], axis=1)
    assert _rel(orc.forward_ex(u, lam, bt, ct2, d, log_delta=logd, bidirectional=True)[0],
                orc.forward(u, lam, bt, ct, d, logd)) < 1e-15
    yg = orc.forward_ex(u, lam, bt, ct, d, log_delta=logd, activation="gelu")[0]
    assert _rel(yg, orc.gelu(orc.forward(u, lam, bt, ct, d, logd))) < 1e-15
    with pytest.raises(ValueError):
        orc.forward_ex(u, lam, bt, ct2, d, delta=dt, bidirectional=True)
    with pytest.raises(ValueError):
        orc.forward_ex(u, lam, bt, ct2, d, log_delta=logd, x0=x0, bidirectional=True)


def test_planted_glu_transposed_weight(monkeypatch):
    good = orc.glu
    monkeypatch.setattr(orc, "glu", lambda y, w, bias=None, variant=1: good(y, np.asarray(w).T, bias, variant))
    assert _fails("glu_brute_force")


def test_planted_glu_variant_two_gates_gelu(monkeypatch):
    good = orc.glu
    monkeypatch.setattr(orc, "glu", lambda y, w, bias=None, variant=1: good(y, w, bias, 1))
    assert _fails("glu_brute_force") and _fails("glu_limits")


def test_planted_glu_gate_without_gelu(monkeypatch):
    def raw_gate(y, w, bias=None, variant=1):
        y = np.asarray(y, np.float64)
        pre = y @ np.asarray(w).T + (0.0 if bias is None else bias)
        g = orc.gelu(y)
        return (g if variant == 1 else y) * orc.sigmoid(pre)
    monkeypatch.setattr(orc, "glu", raw_gate)
    assert _fails("glu_brute_force")
