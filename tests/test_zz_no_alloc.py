"""pn_eval_noalloc (the entry point that allocates nothing) against pn_eval_ex:
two calls in a row on the shared static scratch, the second with a smaller
input, on each kernel family; both held to the oracle's bar and to each other."""

import ctypes

import numpy as np
import pytest
import torch

import workloads
import newton_evaluation_nonlinear_amd as pn
from _parity import advancing, check_parity, check_parity_advancing, run_gpu, run_oracle, to_dev

J, P, Q, N = pn.JACOBI, pn.PICARD, pn.QUASI_NEWTON, pn.NEWTON


def _run_noalloc(wl, mode):
    params, x, s0 = to_dev(wl)
    res = pn.eval(wl["cell"], params, x, s0, mode=mode, tol=wl["tol"], max_iter=wl["max_iter"],
                  damping=wl["damping"], window=wl["window"], history=True, noalloc=True,
                  window_mode=pn.WINDOW_ADVANCING if advancing(wl) else pn.WINDOW_CONSECUTIVE)
    torch.cuda.synchronize()
    res.out_np = res.out.cpu().numpy()
    return res


# (first call, second smaller call, mode): the channel-wise kernels, the
# matrix-cell tile kernel with the in-sweep check over windows, the
# matrix-core Newton kernels with the carry launch
PAIRS = [((3, 2, 6000), (3, 1, 1500), Q),
         ((5, 2, 3072), (5, 1, 1100), Q),
         ((4, 3, 700), (1, None, None), N),
         ((2, 4, 400), (2, 2, 100), J)]


@pytest.mark.gpu
@pytest.mark.parametrize("first, second, mode", PAIRS)
def test_noalloc_matches_pn_eval_ex_on_two_calls_in_a_row(first, second, mode):
    for cfg, B, T in (first, second):
        wl = workloads.make(cfg, B=B, T=T)
        print(f"[noalloc] cfg{cfg} B={wl['B']} T={wl['T']} mode={mode}", flush=True)
        a = _run_noalloc(wl, mode)
        b = run_gpu(wl, mode)
        assert a.status == b.status and a.iters == b.iters and a.window_iters == b.window_iters
        assert a.resid_hist == b.resid_hist
        np.testing.assert_array_equal(a.out_np, b.out_np)
        check_parity(wl, mode, a, run_oracle(wl, mode), label=f"noalloc cfg{cfg}")


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [P, N])
def test_noalloc_advancing_window_on_two_calls_in_a_row(mode):
    # the advancing window: one resident launch (Picard; its records come back
    # from the static scratch after the launch) or a launch per round (Newton)
    for B, T in ((4, 1500), (2, 600)):
        wl = workloads.make(7, B=B, T=T)
        print(f"[noalloc] cfg7 B={B} T={T} mode={mode}", flush=True)
        a = _run_noalloc(wl, mode)
        b = run_gpu(wl, mode)
        assert a.status == b.status and a.iters == b.iters and a.accepted == b.accepted
        assert a.resid_hist == b.resid_hist
        np.testing.assert_array_equal(a.out_np, b.out_np)
        check_parity_advancing(wl, mode, a, run_oracle(wl, mode), label=f"noalloc cfg7 B={B}")


@pytest.mark.gpu
def test_noalloc_nonfinite_and_not_converged_outcomes():
    wl = workloads.make(2, B=2, T=200)
    wl["x"] = wl["x"].copy()
    wl["x"][1, 150, 3] = np.nan
    a = _run_noalloc(wl, Q)
    assert a.status == pn.NONFINITE and a.iters == 0
    wl = workloads.make(2, B=2, T=200)
    params, x, s0 = to_dev(wl)
    r = pn.eval(wl["cell"], params, x, s0, mode=Q, tol=0.0, max_iter=2, noalloc=True)
    torch.cuda.synchronize()
    ref = run_oracle(wl, Q, tol=0.0, max_iter=2)
    assert r.status == ref.status == pn.NOT_CONVERGED and r.iters == 2
    assert np.max(np.abs(r.out.cpu().numpy() - ref.s)) <= 1e-4


def _raw(B, T, D, opts=None, kind=pn.CELL_DIAG_TANH, m=None, mode=Q):
    c = pn.Cell(kind, D if m is None else m)
    it = ctypes.c_int32(-1)
    a = [ctypes.c_void_p(k << 32) for k in (1, 2, 3, 4)]     # placeholders, never dereferenced
    rc = pn.lib().pn_eval_noalloc(ctypes.byref(c), a[0], a[1], a[2], B, T, D, mode, 1e-5, 5, a[3],
                                  ctypes.byref(it), ctypes.byref(opts) if opts is not None else None)
    return rc


def test_noalloc_rejects_what_it_cannot_serve_before_device_work():
    # past the static scratch: a clear error, no device call
    need = pn.workspace_bytes(pn.CELL_TANH_RNN, 16, 64, 4096, 64, N)
    assert need > 32 << 20
    assert _raw(64, 4096, 64, kind=pn.CELL_TANH_RNN, m=16, mode=N) == pn.EWORKSPACE
    assert "pn_eval_noalloc has" in pn.last_error() and str(need) in pn.last_error()
    o = pn.make_opts()
    o.workspace = 1 << 20
    o.workspace_bytes = 1 << 20
    assert _raw(2, 10, 4, o) == pn.EINVAL and "workspace" in pn.last_error()
    o = pn.make_opts()
    prof = pn.Profile()
    o.profile = ctypes.pointer(prof)
    assert _raw(2, 10, 4, o) == pn.EINVAL and "profil" in pn.last_error()
    assert _raw(0, 10, 4) == pn.OK
