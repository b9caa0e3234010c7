"""The boundary as the C interface states it, on the GPU: pn_eval itself (no
options: library-allocated workspace, null stream), the torch.nn.GRU / RNN
parameter layout fed straight in, and the binding's argument checks raising
before any launch."""

import ctypes
import types

import numpy as np
import pytest
import torch

import oracle
import workloads
import newton_evaluation_nonlinear_amd as pn
from _parity import check_parity, run_oracle

pytestmark = pytest.mark.gpu


def _pn_eval_raw(wl, mode):
    """pn_eval through ctypes: no pn_opts, so the library allocates its own
    workspace and runs on the null stream."""
    dev = torch.device("cuda:0")
    params = torch.from_numpy(wl["params"]).to(dev)
    x = torch.from_numpy(wl["x"]).to(dev)
    s0 = torch.from_numpy(wl["s0"]).to(dev)
    out = torch.full((wl["B"], wl["T"], wl["D"]), float("nan"), device=dev)
    torch.cuda.synchronize()
    c = pn.Cell(wl["cell"], wl["m"])
    it = ctypes.c_int32(-1)
    print(f"[pn_eval] cfg{wl['cfg']} B={wl['B']} T={wl['T']} mode={mode}", flush=True)
    rc = pn.lib().pn_eval(ctypes.byref(c), params.data_ptr(), x.data_ptr(), s0.data_ptr(),
                          wl["B"], wl["T"], wl["D"], mode, wl["tol"], wl["max_iter"],
                          out.data_ptr(), ctypes.byref(it))
    torch.cuda.synchronize()
    assert rc >= 0, pn.last_error()
    return types.SimpleNamespace(status=rc, iters=it.value, window_iters=[it.value], resid_hist=None,
                                 out_np=out.cpu().numpy())


@pytest.mark.parametrize("cfg, B, T, mode", [(1, None, None, pn.NEWTON), (3, 2, 6000, pn.QUASI_NEWTON),
                                            (2, 4, 500, pn.QUASI_NEWTON)])
def test_pn_eval_without_options_matches_the_oracle(cfg, B, T, mode):
    wl = workloads.make(cfg, B=B, T=T)
    assert wl["window"] == 0
    gpu = _pn_eval_raw(wl, mode)
    ref = run_oracle(wl, mode)
    check_parity(wl, mode, gpu, ref, label=f"pn_eval cfg{cfg}")


def _torch_gru_case(D, m, seed):
    torch.manual_seed(seed)
    mod = torch.nn.GRU(m, D, batch_first=True).double()
    with torch.no_grad():
        mod.bias_ih_l0.uniform_(-0.5, 0.5)
        mod.bias_hh_l0.uniform_(-0.5, 0.5)
    flat = np.concatenate([t.detach().numpy().ravel() for t in
                           (mod.weight_ih_l0, mod.weight_hh_l0, mod.bias_ih_l0, mod.bias_hh_l0)])
    return mod, flat.astype(np.float32)


@pytest.mark.parametrize("D, m, mode", [(16, 8, pn.NEWTON), (16, 8, pn.QUASI_NEWTON), (5, 3, pn.NEWTON),
                                        (64, 12, pn.QUASI_NEWTON)])
def test_torch_gru_parameters_pass_straight_in(D, m, mode):
    # the flat vector is torch's own tensors in storage order; the converged
    # solve must reproduce torch.nn.GRU's forward pass (float64, CPU) to the
    # trajectory bar
    mod, flat = _torch_gru_case(D, m, 40 + D)
    # float32-rounded weights back into the reference module, so both see the same numbers
    with torch.no_grad():
        off = 0
        for t in (mod.weight_ih_l0, mod.weight_hh_l0, mod.bias_ih_l0, mod.bias_hh_l0):
            n = t.numel()
            t.copy_(torch.from_numpy(flat[off:off + n].astype(np.float64)).view_as(t))
            off += n
    rng = np.random.default_rng(50 + D)
    B, T = 3, 700
    x = rng.standard_normal((B, T, m)).astype(np.float32)
    s0 = (0.3 * rng.standard_normal((B, D))).astype(np.float32)
    with torch.no_grad():
        ref, _ = mod(torch.from_numpy(x.astype(np.float64)), torch.from_numpy(s0.astype(np.float64))[None])
    dev = torch.device("cuda:0")
    print(f"[torch-gru] D={D} m={m} mode={mode}", flush=True)
    res = pn.eval(pn.CELL_GRU, torch.from_numpy(flat).to(dev), torch.from_numpy(x).to(dev),
                  torch.from_numpy(s0).to(dev), mode=mode, tol=1e-6)
    torch.cuda.synchronize()
    assert res.status == pn.OK
    err = float(np.max(np.abs(res.out.cpu().numpy().astype(np.float64) - ref.numpy())))
    assert err <= 1e-4, err


def test_torch_rnn_parameters_pass_straight_in():
    D, m = 32, 16
    torch.manual_seed(7)
    mod = torch.nn.RNN(m, D, nonlinearity="tanh", batch_first=True).double()
    flat = np.concatenate([mod.weight_hh_l0.detach().numpy().ravel(), mod.weight_ih_l0.detach().numpy().ravel(),
                           (mod.bias_ih_l0 + mod.bias_hh_l0).detach().numpy()]).astype(np.float32)
    cell = oracle.make_cell(pn.CELL_TANH_RNN, flat, D, m)
    rng = np.random.default_rng(8)
    B, T = 2, 900
    x = rng.standard_normal((B, T, m)).astype(np.float32)
    s0 = np.zeros((B, D), np.float32)
    seq = oracle.sequential(cell, x.astype(np.float64), s0.astype(np.float64))
    with torch.no_grad():
        ref, _ = mod(torch.from_numpy(x.astype(np.float64)), torch.from_numpy(s0.astype(np.float64))[None])
    # the torch module's float64 biases differ from the float32 flat vector by rounding only
    assert np.max(np.abs(seq - ref.numpy())) < 1e-5
    dev = torch.device("cuda:0")
    res = pn.eval(pn.CELL_TANH_RNN, torch.from_numpy(flat).to(dev), torch.from_numpy(x).to(dev),
                  torch.from_numpy(s0).to(dev), mode=pn.NEWTON, tol=1e-6)
    torch.cuda.synchronize()
    assert res.status == pn.OK
    assert float(np.max(np.abs(res.out.cpu().numpy() - seq))) <= 1e-4


def test_binding_rejects_bad_arguments_before_any_launch():
    dev = torch.device("cuda:0")
    D, m, B, T = 16, 8, 2, 64
    x = torch.zeros(B, T, m, device=dev)
    s0 = torch.zeros(B, D, device=dev)
    params = torch.zeros(pn.param_count(pn.CELL_GRU, D, m), device=dev)
    with pytest.raises(ValueError, match="params holds"):
        pn.eval(pn.CELL_GRU, params[:-3], x, s0)
    with pytest.raises(ValueError, match="out must have shape"):
        pn.eval(pn.CELL_GRU, params, x, s0, out=torch.zeros(B, T - 1, D, device=dev))
    with pytest.raises(ValueError, match="one device"):
        pn.eval(pn.CELL_GRU, params.cpu(), x, s0)
    # out aliasing an input is caught on the host by the library
    xd = torch.zeros(B, T, D, device=dev)
    with pytest.raises(pn.PnError) as e:
        pn.eval(pn.CELL_DIAG_TANH, torch.full((D,), 0.5, device=dev), xd, s0, out=xd)
    assert e.value.code == pn.EINVAL and "overlaps x" in str(e.value)
    torch.cuda.synchronize()


def test_sequential_gpu_loop_matches_the_oracle_time_loop():
    # The GPU baseline the bench sets beside the solve (pnc_sequential_tanh in
    # libpn_ceiling.so): the plain time loop of the channel-wise cell, against
    # the oracle's float64 time loop; D = 70 leaves a ragged channel block and
    # T = 1000 a ragged prefetch group.
    import os
    wl = workloads.make(3, B=2, T=1000)
    wl["params"] = wl["params"][:70].copy()
    wl["x"] = np.ascontiguousarray(wl["x"][:, :, :70])
    wl["s0"] = (0.3 * np.random.default_rng(7).standard_normal((2, 70))).astype(np.float32)
    B, T, D = 2, 1000, 70
    dev = torch.device("cuda:0")
    a, x, s0 = (torch.from_numpy(wl[k]).to(dev) for k in ("params", "x", "s0"))
    out = torch.full((B, T, D), float("nan"), device=dev)
    lib = ctypes.CDLL(os.path.join(os.path.dirname(pn.__file__), "libpn_ceiling.so"))
    vp, dbl = ctypes.c_void_p, ctypes.c_double
    lib.pnc_sequential_tanh.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.POINTER(dbl), ctypes.POINTER(dbl)]
    best, med = dbl(0.0), dbl(0.0)
    print(f"[pnc_sequential_tanh] B={B} T={T} D={D}", flush=True)
    assert lib.pnc_sequential_tanh(x.data_ptr(), a.data_ptr(), s0.data_ptr(), out.data_ptr(), B, T, D, 2,
                                   ctypes.byref(best), ctypes.byref(med)) == 0
    torch.cuda.synchronize()
    cell = oracle.make_cell(oracle.CELL_DIAG_TANH, wl["params"].astype(np.float64), D, D)
    ref = oracle.sequential(cell, wl["x"].astype(np.float64), wl["s0"].astype(np.float64))
    err = float(np.max(np.abs(out.cpu().numpy().astype(np.float64) - ref)))
    assert err <= 1e-5, err
    assert 0.0 < best.value <= med.value
