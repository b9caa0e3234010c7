"""Fixed-point solvers for the stacked trajectory, written as plain loops.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The article [PN §1.2] recasts the evaluation of s_t = f_t(s_{t-1}), t = 1..T,
as a root-finding problem F(s) = 0 over the whole trajectory and applies the
update s <- s - J~^{-1}(s) F(s), where the four methods differ only in J~.
With F_t(s) = s_t - f_t(s_{t-1}) (s_0 given), the exact Jacobian of F is the
block lower-bidiagonal matrix with identity blocks on the diagonal and
-A_t = -df_t/ds_{t-1} below it.  Replacing A_t by an approximation A~_t and
solving J~ d = -F by forward substitution gives the update used here:

    p_t  = s_{t-1}                (p_1 = s_0)
    v_t  = f_t(p_t)
    s^_t = v_t + A~_t (s^_{t-1} - p_t),   s^_0 = s_0

with A~_t = 0 (Jacobi, J~ = I), A~_t = I (Picard, identity dynamics
[PN §2.2.3]), A~_t = diag(A_t) (quasi-Newton, diagonal approximation
[PN §2.2.1]), A~_t = band_k(A_t), the entries with |i - j| <= k (banded
approximation for locally coupled systems [PN §2.2.2]), and A~_t = A_t
(Newton).  The forward substitution is a
first-order linear recurrence — the object a parallel scan evaluates
[PN §2.1] — and here it is a deliberately sequential loop.

Readings where the article is silent (documented alongside the build):
  * initial guess s^(0)_t = s_0 for every t;
  * residual r = max over (b, t, d) of |F|, one stop rule per solve;
  * stop when r is not finite (NONFINITE), else when r <= tol (OK), else when
    the number of applied updates reaches max_iter (NOT_CONVERGED);
  * damping is step damping, s <- s + lam (s^ - s) [PN §4.3, §5.3];
  * windows are consecutive, non-overlapping blocks of W steps, each solved
    from its own initial state, which is the last state of the previous
    window [PN §1.3.1, §2.3];
  * residual-driven switching [PN §5.3]: a solve may start with a coarse
    approximation and change to a better one when the residual curve
    stagnates.  Read as: at each check i >= 1 of a window, while still on the
    first mode, r_i > rho * r_{i-1} switches the window to the second mode
    from update i+1 on (update i, which follows check i, keeps the first
    mode); each window starts on the first mode.  The other remedy the
    article names for a stalling curve, more damping, is read the same way:
    with a second damping lam2, the switch also changes the step damping
    from lam to lam2 from update i+1 on (the second mode may equal the first,
    which makes it a pure damping switch);
  * reduced-precision storage [PN §2.3, §4.2] (``storage="f16"``): every
    state the update stores is rounded to nearest-even IEEE binary16 and the
    iteration continues from the stored states; arithmetic is unchanged;
  * the advancing window (``solve_advancing``) is the sliding window of
    [PN §1.3.1] read as: a window of W steps starts at the first step not yet
    accepted; after each check the leading steps of the window whose residual
    is <= tol are accepted and the window slides past them, taking in new
    steps that start from the last state of the current iterate.
"""

from dataclasses import dataclass, field

import numpy as np

from .cells import make_cell

JACOBI, PICARD, QUASI_NEWTON, NEWTON, BANDED = 0, 1, 2, 3, 4
OK, NOT_CONVERGED, NONFINITE = 0, 1, 2


def sequential(cell, x, s0):
    """Ground truth s_t = f_t(s_{t-1}) by the plain time loop [PN §1.1].

    x: [B, T, m], s0: [B, D]  ->  [B, T, D] holding s_1..s_T.
    """
    B, T = x.shape[0], x.shape[1]
    out = np.empty((B, T, cell.D), dtype=cell.dtype)
    prev = np.asarray(s0, dtype=cell.dtype)
    for t in range(T):
        prev = cell.f(prev, x[:, t])
        out[:, t] = prev
    return out


def shift(s, s0):
    """p_t = s_{t-1} with p_1 = s_0: [B, T, D] -> [B, T, D]."""
    return np.concatenate([np.asarray(s0, dtype=s.dtype)[:, None, :], s[:, :-1]], axis=1)


def residual_inf(cell, x, s0, s):
    """max over (b, t, d) of |s_t - f_t(s_{t-1})|; NaN/Inf propagate; 0 if empty."""
    if s.size == 0:
        return 0.0
    v = cell.f(shift(s, s0), x)
    return float(np.max(np.abs(s - v)))


def band(J, k):
    """Entries of J (..., D, D) with |i - j| <= k; the rest set to zero."""
    D = J.shape[-1]
    i = np.arange(D)
    mask = np.abs(i[:, None] - i[None, :]) <= k
    return np.where(mask, J, 0.0).astype(J.dtype)


def jacobian_approx(mode, cell, p, x, bandwidth=1):
    """A~_t for every (b, t): [B, T, D] for the diagonal modes, [B, T, D, D]
    for Newton and the banded mode (half-bandwidth ``bandwidth``)."""
    if mode == JACOBI:
        return np.zeros(p.shape, dtype=cell.dtype)
    if mode == PICARD:
        return np.ones(p.shape, dtype=cell.dtype)
    if mode == QUASI_NEWTON:
        return cell.jac_diag(p, x)
    if mode == NEWTON:
        return cell.jac(p, x)
    if mode == BANDED:
        return band(cell.jac(p, x), bandwidth)
    raise ValueError(f"unknown mode {mode}")


def affine_recurrence(v, p, A, s0):
    """s^_t = v_t + A_t (s^_{t-1} - p_t), s^_0 = s0, by a sequential loop over t.

    A is [B, T, D] (diagonal) or [B, T, D, D] (dense).  This is the forward
    substitution of J~ d = -F; the GPU evaluates the same recurrence with an
    associative scan over the affine maps y -> A_t y + (v_t - A_t p_t).
    """
    B, T, D = v.shape
    out = np.empty_like(v)
    prev = np.asarray(s0, dtype=v.dtype)
    dense = A.ndim == 4
    for t in range(T):
        d = prev - p[:, t]
        if dense:
            step = np.einsum("bij,bj->bi", A[:, t], d)
        else:
            step = A[:, t] * d
        prev = v[:, t] + step
        out[:, t] = prev
    return out


def newton_step(cell, x, s0, s, mode, bandwidth=1):
    """One undamped update s -> s^ of the chosen method [PN §1.2]."""
    p = shift(s, s0)
    v = cell.f(p, x)
    A = jacobian_approx(mode, cell, p, x, bandwidth)
    return affine_recurrence(v, p, A, s0)


@dataclass
class SolveResult:
    s: np.ndarray                 # [B, T, D] final iterate (NaN where never reached)
    iters: int                    # total updates over all windows
    status: int                   # OK / NOT_CONVERGED / NONFINITE
    window_iters: list = field(default_factory=list)   # K per window solved
    window_status: list = field(default_factory=list)
    hist: list = field(default_factory=list)           # per window: [r_0, ..., r_K]
    accepted: list = field(default_factory=list)       # advancing window: steps accepted per check
    window_switch: list = field(default_factory=list)  # per window: check that switched modes, or -1
    round_resid: list = field(default_factory=list)    # advancing window: r_t per check, on request


def _stored(s, storage):
    """The state as a binary16 store would hold it (storage "f16"), else s."""
    if storage == "f16":
        return s.astype(np.float16).astype(s.dtype)
    return s


def _solve_window(cell, x, s0, mode, tol, max_iter, damping, force, bandwidth, switch=None,
                  storage=None):
    """One window.  ``switch`` = (second mode, rho, forced check or None,
    second damping or None)."""
    B, T = x.shape[0], x.shape[1]
    s = np.broadcast_to(np.asarray(s0, dtype=cell.dtype)[:, None, :], (B, T, cell.D)).copy()
    hist = []
    i = 0
    sw = -1                 # check at which the window switched modes
    while True:
        p = shift(s, s0)
        v = cell.f(p, x)
        r = float(np.max(np.abs(s - v))) if s.size else 0.0
        hist.append(r)
        if force is None:
            if not np.isfinite(r):
                return s, i, NONFINITE, hist, sw
            if r <= tol:
                return s, i, OK, hist, sw
            if i == max_iter:
                return s, i, NOT_CONVERGED, hist, sw
        elif i == force:
            status = NONFINITE if not np.isfinite(r) else (OK if r <= tol else NOT_CONVERGED)
            return s, i, status, hist, sw
        if switch is not None and sw < 0 and i >= 1:
            rho, forced = switch[1], switch[2]
            if (forced == i) if forced is not None else (r > rho * hist[-2]):
                sw = i
        switched = switch is not None and 0 <= sw < i
        use = switch[0] if switched else mode
        lam = switch[3] if (switched and switch[3] is not None) else damping
        A = jacobian_approx(use, cell, p, x, bandwidth)
        s_hat = affine_recurrence(v, p, A, s0)
        if lam == 1.0:
            s = s_hat
        else:
            s = s + lam * (s_hat - s)
        s = _stored(s, storage)
        i += 1


def solve(kind, params, x, s0, mode, tol, max_iter, damping=1.0, window=0,
          dtype=np.float64, force_iters=None, bandwidth=1, switch_mode=None, switch_ratio=0.5,
          force_switch=None, storage=None, switch_damping=None):
    """Parallel-in-time fixed-point solve, evaluated sequentially.

    kind/params follow the flat layout of ``make_cell``; x: [B, T, m];
    s0: [B, D].  ``window`` = 0 solves the whole horizon at once; W > 0 solves
    windows of W steps in order (the last may be shorter).  ``force_iters``
    (one count per window) replaces the stop rule by a fixed number of
    updates; it is used to follow a run whose stopping decision landed inside
    the floating-point ambiguity band of the tolerance.  ``bandwidth`` is the
    half-bandwidth k of the banded mode.  ``switch_mode`` (with
    ``switch_ratio`` rho) turns on residual-driven switching; ``force_switch``
    (one check index or -1 per window) replaces its decisions, and
    ``switch_damping`` (in (0, 1], or None to keep ``damping``) is the step
    damping after a switch.  ``storage``
    "f16" stores the iterate in binary16 (x must already hold binary16
    values); the returned trajectory is the stored one.
    """
    x = np.asarray(x)
    s0 = np.asarray(s0)
    B, T = x.shape[0], x.shape[1]
    D = s0.shape[1]
    m = x.shape[2]
    cell = make_cell(kind, params, D, m, dtype)
    xc = x.astype(dtype)
    s_init = s0.astype(dtype)
    out = np.full((B, T, D), np.nan, dtype=dtype)
    W = T if window <= 0 else int(window)
    res = SolveResult(out, 0, OK)
    w0 = 0
    wi = 0
    while w0 < T or (T == 0 and wi == 0):
        w1 = min(T, w0 + W)
        force = None if force_iters is None else int(force_iters[wi])
        switch = None
        if switch_mode is not None:
            fs = None if force_switch is None else int(force_switch[wi])
            switch = (switch_mode, switch_ratio, fs if fs is None or fs >= 0 else 10 ** 9,
                      switch_damping)
        s, K, st, hist, sw = _solve_window(cell, xc[:, w0:w1], s_init, mode, tol, max_iter,
                                           damping, force, bandwidth, switch, storage)
        s = _stored(s, storage)
        res.window_switch.append(sw)
        out[:, w0:w1] = s
        res.iters += K
        res.window_iters.append(K)
        res.window_status.append(st)
        res.hist.append(hist)
        if st == NONFINITE:
            res.status = NONFINITE
            break
        if st == NOT_CONVERGED:
            res.status = NOT_CONVERGED
        if w1 > w0:
            s_init = s[:, -1]
        w0 = w1
        wi += 1
        if T == 0:
            break
    return res


def solve_advancing(cell, x, s0, mode, tol, max_iter, W, damping=1.0, bandwidth=1,
                    force_accept=None, keep_round_resid=False):
    """Advancing-window solve: the window slides past its converged prefix.

    ``cell`` is a cell object (``make_cell``); x: [B, T, m]; s0: [B, D].
    Steps [0, a) are accepted and never change again; the window is [a, e),
    e = min(T, a + W).  Each round:
      1. check: r_t = max over (b, d) of |s_t - f_t(s_{t-1})| for t in [a, e)
         at the current iterate (s_{a-1} accepted, or s0); r = max_t r_t is
         the round's residual.  Non-finite r stops with NONFINITE;
      2. accept: a moves to the first t with r_t > tol (to e if none); a = T
         stops with OK; after max_iter updates the solve stops with
         NOT_CONVERGED;
      3. slide: e = min(T, a + W); steps that enter the window start from the
         last state of the current iterate;
      4. update the window [a, e) once with the chosen method [PN §1.2], from
         the accepted state s_{a-1}, with step damping.
    The count is the number of updates; ``window_iters`` = [count].  On
    exit, steps the window never reached hold its last state.  ``accepted``
    lists the steps accepted at each check with a finite residual.
    ``force_accept`` replaces the acceptance decisions by the given counts (to
    follow a run whose decisions fell inside the floating-point ambiguity band
    of tol); ``keep_round_resid`` keeps each check's r_t.
    """
    x = np.asarray(x, dtype=cell.dtype)
    s0 = np.asarray(s0, dtype=cell.dtype)
    B, T = x.shape[0], x.shape[1]
    D = cell.D
    W = T if W <= 0 else int(W)
    s = np.full((B, T, D), np.nan, dtype=cell.dtype)
    a, e = 0, min(T, W)
    s[:, :e] = s0[:, None, :]
    hist = []
    i = 0
    res = SolveResult(s, 0, OK)
    while T > 0:
        prev = s0 if a == 0 else s[:, a - 1]
        win = s[:, a:e]
        v = cell.f(shift(win, prev), x[:, a:e])
        r_t = np.max(np.abs(win - v), axis=(0, 2))
        r = float(np.max(r_t))
        hist.append(r)
        if keep_round_resid:
            res.round_resid.append(r_t.astype(np.float64))
        if not np.isfinite(r):
            res.status = NONFINITE
            break
        bad = np.nonzero(~(r_t <= tol))[0]
        acc = int(bad[0]) if bad.size else e - a
        if force_accept is not None:
            acc = int(force_accept[len(res.accepted)])
        res.accepted.append(acc)
        a = a + acc
        if a >= T:
            break
        if i == max_iter:
            res.status = NOT_CONVERGED
            break
        e_new = min(T, a + W)
        s[:, e:e_new] = s[:, e - 1:e]
        e = e_new
        prev = s0 if a == 0 else s[:, a - 1]
        win = s[:, a:e]
        s_hat = newton_step(cell, x[:, a:e], prev, win, mode, bandwidth)
        s[:, a:e] = s_hat if damping == 1.0 else win + damping * (s_hat - win)
        i += 1
    if T == 0:
        hist.append(0.0)
    elif e < T:
        s[:, e:] = s[:, e - 1:e]      # steps never reached: the window's last state
    res.iters = i
    res.window_iters = [i]
    res.window_status = [res.status]
    res.hist = [hist]
    return res
