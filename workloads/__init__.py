"""Seeded synthetic workloads shared by the tests, the benchmark and the oracle.

This module only draws random numbers and lays them out; it contains none of
the method's arithmetic.  Both sides (the HIP library and the CPU oracle)
consume the identical float32 arrays it returns.

Every workload is a recurrence s_t = f_t(s_{t-1}) of the kind the article
"并行牛顿方法：加速非线性序列评估的计算革命" treats (RNN forward passes, [PN §1.3.2]),
with the stability regimes of [PN §3.1] (spectral radius well below 1, and
near 1).  The article uses no dataset for this method; these draws stand in
for its unspecified "T=2048 RNN forward" workload.

Generator: numpy.random.Generator(PCG64(seed)), seed = workload number.
Values are drawn in float64 in the order listed, then cast to float32.
Reduced variants (smaller B or T) keep the weights of the full workload and
draw x with the reduced shape from the same stream position.

Parameter layouts are the flat layouts of the C interface:
  diag-tanh: a[D]
  tanh RNN : W[D*D] | U[D*m] | b[D]
  GRU      : W_ih[3D*m] | W_hh[3D*D] | b_ih[3D] | b_hh[3D]  (gates r, z, n)
  Euler    : W[D*D] | U[D*m] | b[D] | h[D]
"""

import json
import os

import numpy as np

CELL_DIAG_TANH, CELL_TANH_RNN, CELL_GRU, CELL_EULER_TANH = 0, 1, 2, 3
JACOBI, PICARD, QUASI_NEWTON, NEWTON, BANDED = 0, 1, 2, 3, 4
MODE_NAMES = {JACOBI: "jacobi", PICARD: "picard", QUASI_NEWTON: "quasi_newton", NEWTON: "newton",
              BANDED: "banded"}

_HERE = os.path.dirname(os.path.abspath(__file__))

# Shapes and solver settings of the five workloads.  ``modes`` lists the
# methods each one is run with; ``tol`` is the residual tolerance; max_iter
# defaults to the window length (the causality bound of [PN §3.1]).
CONFIGS = {
    1: dict(name="tanh_rnn_d4", cell=CELL_TANH_RNN, B=1, T=256, D=4, m=2,
            modes=(NEWTON,), tol=1e-6, damping=1.0, window=0, rho=0.7),
    2: dict(name="gru_d16", cell=CELL_GRU, B=64, T=2048, D=16, m=8,
            modes=(PICARD, QUASI_NEWTON, NEWTON, JACOBI), tol=1e-5, damping=1.0, window=0),
    3: dict(name="diag_tanh_d256", cell=CELL_DIAG_TANH, B=8, T=65536, D=256, m=256,
            modes=(QUASI_NEWTON,), tol=1e-5, damping=1.0, window=0),
    4: dict(name="tanh_rnn_d32", cell=CELL_TANH_RNN, B=32, T=4096, D=32, m=16,
            modes=(NEWTON,), tol=1e-5, damping=1.0, window=0, rho=0.9),
    5: dict(name="gru_d64_near_critical", cell=CELL_GRU, B=4, T=32768, D=64, m=32,
            modes=(QUASI_NEWTON,), tol=1e-5, damping=0.5, window=1024),
    # A locally coupled system, the case the banded Jacobian approximation is
    # meant for [PN §2.2.2]: a tanh RNN on a ring-free 1-D lattice whose
    # recurrent matrix couples each unit to its neighbours within distance
    # ``lattice_band``, plus a weak dense coupling of relative size ``eps``.
    6: dict(name="lattice_tanh_d64", cell=CELL_TANH_RNN, B=16, T=4096, D=64, m=16,
            modes=(BANDED, QUASI_NEWTON, NEWTON), tol=1e-5, damping=1.0, window=0, rho=0.9,
            lattice_band=2, eps=0.05, bandwidth=2),
    # A small-step ODE, the regime of Picard's identity approximation and of
    # the sliding window of [PN §1.3.1]: explicit Euler steps h of the
    # continuous-time RNN ds/dt = -s + tanh(W s + U x(t) + b), solved with a
    # window of W = 256 steps that advances past its converged prefix.
    7: dict(name="ode_ctrnn_d32", cell=CELL_EULER_TANH, B=64, T=8192, D=32, m=8,
            modes=(PICARD, QUASI_NEWTON, NEWTON), tol=1e-5, damping=1.0, window=256,
            window_mode="advancing", rho=0.9, h=0.005),
}


def gru_scale():
    """Scalar applied to W_hh of workload 5 (written by calibrate_gru_scale.py)."""
    path = os.path.join(_HERE, "gru_scale.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        return float(json.load(fh)["c"])


def _rescale_spectral_radius(W, rho):
    ev = np.linalg.eigvals(W)
    return W * (rho / np.max(np.abs(ev)))


def _gru_weights(rng, D, m):
    k = 1.0 / np.sqrt(D)
    W_ih = rng.uniform(-k, k, size=(3 * D, m))
    W_hh = rng.uniform(-k, k, size=(3 * D, D))
    b_ih = rng.uniform(-k, k, size=(3 * D,))
    b_hh = rng.uniform(-k, k, size=(3 * D,))
    return W_ih, W_hh, b_ih, b_hh


def make(cfg, B=None, T=None, scale=None):
    """Return a dict with the float32 arrays and settings of workload ``cfg``.

    Keys: cfg, name, cell, D, m, B, T, params (flat float32), x [B,T,m],
    s0 [B,D] (zeros), modes, tol, damping, window, max_iter, bandwidth (the
    half-bandwidth the banded mode runs with; 1 where unset), window_mode
    ("consecutive" or "advancing").
    """
    c = dict(CONFIGS[cfg])
    B = c["B"] if B is None else int(B)
    T = c["T"] if T is None else int(T)
    D, m = c["D"], c["m"]
    rng = np.random.Generator(np.random.PCG64(cfg))
    if c["cell"] == CELL_TANH_RNN and "lattice_band" in c:
        i = np.arange(D)
        near = np.abs(i[:, None] - i[None, :]) <= c["lattice_band"]
        S = np.where(near, rng.standard_normal((D, D)), 0.0)
        R = rng.standard_normal((D, D)) / np.sqrt(D)
        W = _rescale_spectral_radius(S + c["eps"] * R, c["rho"])
        U = rng.standard_normal((D, m)) / np.sqrt(m)
        b = np.zeros(D)
        x = rng.standard_normal((B, T, m))
        params = np.concatenate([W.ravel(), U.ravel(), b])
    elif c["cell"] == CELL_EULER_TANH:
        W = _rescale_spectral_radius(rng.standard_normal((D, D)), c["rho"])
        U = rng.standard_normal((D, m)) / np.sqrt(m)
        b = rng.standard_normal(D) * 0.1
        h = np.full(D, c["h"])
        x = rng.standard_normal((B, T, m))
        params = np.concatenate([W.ravel(), U.ravel(), b, h])
    elif c["cell"] == CELL_TANH_RNN:
        W = _rescale_spectral_radius(rng.standard_normal((D, D)), c["rho"])
        U = rng.standard_normal((D, m))
        b = np.zeros(D)
        x = rng.standard_normal((B, T, m))
        params = np.concatenate([W.ravel(), U.ravel(), b])
    elif c["cell"] == CELL_GRU:
        W_ih, W_hh, b_ih, b_hh = _gru_weights(rng, D, m)
        if cfg == 5:
            sc = gru_scale() if scale is None else scale
            if sc is None:
                raise RuntimeError("workload 5 needs workloads/gru_scale.json "
                                   "(run workloads/calibrate_gru_scale.py)")
            W_hh = W_hh * sc
            c["scale"] = sc
        x = rng.standard_normal((B, T, m))
        params = np.concatenate([W_ih.ravel(), W_hh.ravel(), b_ih, b_hh])
    elif c["cell"] == CELL_DIAG_TANH:
        a = rng.uniform(0.5, 0.95, size=D)
        # N(0, 0.5) read as variance 0.5.
        x = rng.standard_normal((B, T, m)) * np.sqrt(0.5)
        params = a
    else:
        raise ValueError(cfg)
    c.update(cfg=cfg, B=B, T=T,
             params=np.ascontiguousarray(params, dtype=np.float32),
             x=np.ascontiguousarray(x, dtype=np.float32),
             s0=np.zeros((B, D), dtype=np.float32))
    W = c["window"] if c["window"] else T
    c.setdefault("bandwidth", 1)
    c.setdefault("window_mode", "consecutive")
    # the causality bound of [PN §3.1]: W updates per consecutive window; an
    # advancing window accepts at least one step per undamped update
    c["max_iter"] = int(T if c["window_mode"] == "advancing" else W)
    return c


def lattice_cell_params(kind, D, m, rng, band=2, eps=0.05, rho=0.9):
    """Locally coupled recurrent weights for tests (float32, flat C layout):
    every recurrent matrix couples units within distance ``band``, plus a
    dense part of relative size ``eps``.  tanh RNN: W rescaled to spectral
    radius ``rho``; GRU: each W_hh gate block rescaled likewise; Euler step:
    the tanh RNN's W, U, b and step size 0.1 for every unit."""
    i = np.arange(D)
    near = np.abs(i[:, None] - i[None, :]) <= band

    def lattice():
        S = np.where(near, rng.standard_normal((D, D)), 0.0)
        return _rescale_spectral_radius(S + eps * rng.standard_normal((D, D)) / np.sqrt(D), rho)

    if kind == CELL_TANH_RNN:
        W = lattice()
        U = rng.standard_normal((D, m)) / np.sqrt(m)
        b = rng.standard_normal(D) * 0.1
        return np.concatenate([W.ravel(), U.ravel(), b]).astype(np.float32)
    if kind == CELL_GRU:
        W_ih, _, b_ih, b_hh = _gru_weights(rng, D, m)
        W_hh = np.concatenate([lattice() for _ in range(3)], axis=0)
        return np.concatenate([W_ih.ravel(), W_hh.ravel(), b_ih, b_hh]).astype(np.float32)
    if kind == CELL_EULER_TANH:
        W = lattice()
        U = rng.standard_normal((D, m)) / np.sqrt(m)
        b = rng.standard_normal(D) * 0.1
        h = np.full(D, 0.1)
        return np.concatenate([W.ravel(), U.ravel(), b, h]).astype(np.float32)
    raise ValueError(kind)


def random_cell_params(kind, D, m, rng, scale=1.0):
    """Small random parameter vectors for tests (float32, flat C layout)."""
    if kind == CELL_DIAG_TANH:
        return rng.uniform(-0.95, 0.95, size=D).astype(np.float32) * np.float32(scale)
    if kind == CELL_TANH_RNN:
        W = rng.standard_normal((D, D)) / np.sqrt(D) * scale
        U = rng.standard_normal((D, m)) / np.sqrt(max(m, 1))
        b = rng.standard_normal(D) * 0.1
        return np.concatenate([W.ravel(), U.ravel(), b]).astype(np.float32)
    if kind == CELL_GRU:
        W_ih, W_hh, b_ih, b_hh = _gru_weights(rng, D, m)
        return np.concatenate([W_ih.ravel(), (W_hh * scale).ravel(), b_ih, b_hh]).astype(np.float32)
    if kind == CELL_EULER_TANH:
        W = rng.standard_normal((D, D)) / np.sqrt(D) * scale
        U = rng.standard_normal((D, m)) / np.sqrt(max(m, 1))
        b = rng.standard_normal(D) * 0.1
        h = rng.uniform(0.01, 0.1, D)
        return np.concatenate([W.ravel(), U.ravel(), b, h]).astype(np.float32)
    raise ValueError(kind)
