"""Find the recurrent-weight scale of the near-critical GRU workload (number 5).

The workload asks for a GRU whose state Jacobian has norm close to 0.99, the
critical regime of [PN §3.1] where fixed-point iterations slow down.  Reading
used: draw the default GRU weights of workload 5, multiply all three recurrent
matrices W_hh by one scalar c, and choose c by bisection so that the mean of
the spectral norm ||df_t/ds_{t-1}||_2 over all batch rows and t = 0, 64,
128, ... along the float64 sequential trajectory is 0.990 (+-0.002).

Uses only the CPU oracle; writes workloads/gru_scale.json.  Run:
    python workloads/calibrate_gru_scale.py
"""

import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
import workloads  # noqa: E402

TARGET = 0.990


def mean_jacobian_norm(c):
    wl = workloads.make(5, scale=c)
    D, m = wl["D"], wl["m"]
    cell = oracle.make_cell(wl["cell"], wl["params"], D, m)
    x = wl["x"].astype(np.float64)
    s0 = wl["s0"].astype(np.float64)
    s = oracle.sequential(cell, x, s0)
    ts = np.arange(0, x.shape[1], 64)
    p = np.where(ts[None, :, None] == 0, s0[:, None, :], s[:, np.maximum(ts - 1, 0)])
    J = cell.jac(p, x[:, ts])
    norms = np.linalg.norm(J, ord=2, axis=(-2, -1))
    return float(norms.mean()), float(np.median(norms)), float(norms.max())


def main():
    lo, hi = 1.0, 3.0
    best = None
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        mean, med, mx = mean_jacobian_norm(mid)
        print(f"c={mid:.6f} mean={mean:.5f} median={med:.5f} max={mx:.5f}", flush=True)
        best = (mid, mean, med, mx)
        if abs(mean - TARGET) < 5e-4:
            break
        if mean < TARGET:
            lo = mid
        else:
            hi = mid
    c, mean, med, mx = best
    out = dict(c=c, mean_norm=mean, median_norm=med, max_norm=mx, target=TARGET,
               sample="all batch rows, t = 0, 64, 128, ... of the float64 sequential trajectory")
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gru_scale.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
