"""The C-ABI library: it loads, exports every function include/pn.h declares,
and rejects bad arguments on the host before touching a device."""

import ctypes
import os
import re

import pytest
import torch

import newton_evaluation_nonlinear_amd as pn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "pn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    assert _declared_functions() == sorted(pn.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = pn.lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_and_last_error():
    assert pn.version().startswith("pn ")
    assert "gfx950" in pn.version()
    assert pn.last_error() == ""


# Placeholder device addresses, 4 GiB apart so that no two arrays overlap
# (nothing is dereferenced: every call below fails or returns before device work).
FAKE = {"params": 1 << 32, "x": 2 << 32, "s0": 3 << 32, "out": 4 << 32}


def _eval_raw(kind=pn.CELL_TANH_RNN, m=3, B=2, T=5, D=4, mode=pn.NEWTON, tol=1e-5, max_iter=5,
              ptr=1, opts=None, iters=True, addrs=None, entry="pn_eval_ex"):
    c = pn.Cell(kind, m)
    it = ctypes.c_int32(-7)
    a = dict(FAKE, **(addrs or {}))
    p = {k: (ctypes.c_void_p(v) if ptr else None) for k, v in a.items()}
    rc = getattr(pn.lib(), entry)(ctypes.byref(c), p["params"], p["x"], p["s0"], B, T, D, mode, tol,
                                  max_iter, p["out"], ctypes.byref(it) if iters else None,
                                  ctypes.byref(opts) if opts is not None else None)
    return rc, it.value


@pytest.mark.parametrize("kw, code", [
    (dict(B=-1), pn.EINVAL),
    (dict(T=-3), pn.EINVAL),
    (dict(D=-2), pn.EINVAL),
    (dict(mode=7), pn.EINVAL),
    (dict(mode=5), pn.EINVAL),
    (dict(kind=9), pn.EINVAL),
    (dict(m=0), pn.EINVAL),
    (dict(tol=float("nan")), pn.EINVAL),
    (dict(tol=-1.0), pn.EINVAL),
    (dict(tol=float("inf")), pn.EINVAL),
    (dict(max_iter=-1), pn.EINVAL),
    (dict(ptr=0), pn.EINVAL),
    (dict(iters=False), pn.EINVAL),
    (dict(kind=pn.CELL_DIAG_TANH, m=3, D=4), pn.EINVAL),
    (dict(kind=pn.CELL_GRU, D=65), pn.EUNSUPPORTED),
    (dict(kind=pn.CELL_TANH_RNN, D=100), pn.EUNSUPPORTED),
    (dict(B=70000), pn.EUNSUPPORTED),
])
def test_invalid_arguments_are_rejected_on_the_host(kw, code):
    rc, _ = _eval_raw(**kw)
    assert rc == code
    assert pn.last_error() != ""


def test_invalid_options():
    for field, value in [("damping", 0.0), ("damping", 1.5), ("window", -1), ("chunk", -4)]:
        o = pn.make_opts()
        setattr(o, field, value)
        rc, _ = _eval_raw(opts=o)
        assert rc == pn.EINVAL, field
    o = pn.make_opts()
    o.workspace = 0x1001            # misaligned
    o.workspace_bytes = 1 << 20
    rc, _ = _eval_raw(opts=o)
    assert rc == pn.EWORKSPACE
    o = pn.make_opts()
    o.resid_hist_len = 4            # length without a buffer
    rc, _ = _eval_raw(opts=o)
    assert rc == pn.EINVAL
    o = pn.make_opts(bandwidth=-1)  # the banded mode needs k >= 0
    rc, _ = _eval_raw(mode=pn.BANDED, opts=o)
    assert rc == pn.EINVAL and "bandwidth" in pn.last_error()
    rc, _ = _eval_raw(mode=pn.NEWTON, opts=o)   # ignored by the other modes
    assert rc != pn.EINVAL or "bandwidth" not in pn.last_error()


def test_window_mode_checks():
    o = pn.make_opts(window_mode=2)
    rc, _ = _eval_raw(opts=o)
    assert rc == pn.EINVAL and "window_mode" in pn.last_error()
    # every cell takes the advancing window (an empty batch passes the checks
    # and returns before any device work)
    o = pn.make_opts(window_mode=pn.WINDOW_ADVANCING)
    for kind, m in ((pn.CELL_DIAG_TANH, 4), (pn.CELL_TANH_RNN, 3), (pn.CELL_GRU, 3), (pn.CELL_EULER_TANH, 3)):
        rc, it = _eval_raw(kind=kind, m=m, D=4, B=0, opts=o)
        assert rc == pn.OK and it == 0, kind


def test_switch_options():
    for kw, code in [(dict(switch_mode=7), pn.EINVAL), (dict(switch_mode=pn.NEWTON, switch_ratio=-1.0), pn.EINVAL),
                     (dict(switch_mode=pn.NEWTON, window_mode=pn.WINDOW_ADVANCING), pn.EUNSUPPORTED)]:
        rc, _ = _eval_raw(opts=pn.make_opts(**kw))
        assert rc == code, kw
    for lam2 in (-0.5, 1.5, float("nan"), float("inf")):
        rc, _ = _eval_raw(opts=pn.make_opts(switch_mode=pn.NEWTON, switch_damping=lam2))
        assert rc == pn.EINVAL, lam2
    # every cell accepts switching, the damping switch included (B = 0: no
    # device work)
    for kind, m in ((pn.CELL_DIAG_TANH, 4), (pn.CELL_TANH_RNN, 3), (pn.CELL_GRU, 3), (pn.CELL_EULER_TANH, 3)):
        o = pn.make_opts(switch_mode=pn.QUASI_NEWTON, switch_damping=0.5)
        rc, it = _eval_raw(kind=kind, m=m, D=4, B=0, opts=o)
        assert rc == pn.OK and it == 0, kind
    # one workspace holds the regions of both modes
    nq = pn.workspace_bytes(pn.CELL_GRU, 8, 64, 2048, 16, pn.QUASI_NEWTON)
    nn = pn.workspace_bytes(pn.CELL_GRU, 8, 64, 2048, 16, pn.NEWTON)
    ns = pn.workspace_bytes(pn.CELL_GRU, 8, 64, 2048, 16, pn.QUASI_NEWTON, switch_mode=pn.NEWTON)
    assert ns >= max(nq, nn)
    o = pn.make_opts()
    assert o.switch_mode == -1 and abs(o.switch_ratio - 0.5) < 1e-7 and o.switch_damping == 0.0


def test_f16_entry_checks():
    c = pn.Cell(pn.CELL_TANH_RNN, 3)
    it = ctypes.c_int32(0)
    pp, px, ps, po = (ctypes.c_void_p(FAKE[k]) for k in ("params", "x", "s0", "out"))
    L = pn.lib()

    def call(cell, x=px, B=2, opts=None):
        return L.pn_eval_f16(ctypes.byref(cell), pp, x, ps, B, 5, 4, pn.QUASI_NEWTON, 1e-3, 5, po,
                             ctypes.byref(it), ctypes.byref(opts) if opts is not None else None)

    assert call(c) == pn.EUNSUPPORTED
    c = pn.Cell(pn.CELL_DIAG_TANH, 4)
    assert call(c, opts=pn.make_opts(window=2)) == pn.EUNSUPPORTED
    assert call(c, opts=pn.make_opts(window_mode=pn.WINDOW_ADVANCING)) == pn.EUNSUPPORTED
    assert call(c, opts=pn.make_opts(switch_mode=pn.QUASI_NEWTON, switch_damping=0.5)) == pn.EUNSUPPORTED
    assert call(c, B=-2) == pn.EINVAL
    # pairs of binary16 values need 4-byte alignment
    assert call(c, x=ctypes.c_void_p(FAKE["x"] + 2)) == pn.EINVAL
    # out in binary16 covers 2 bytes per state: [2,5,4] -> 80 bytes
    assert L.pn_eval_f16(ctypes.byref(c), pp, px, ps, 2, 5, 4, pn.QUASI_NEWTON, 1e-3, 5,
                         ctypes.c_void_p(FAKE["x"] + 76), ctypes.byref(it), None) == pn.EINVAL
    assert "overlaps x" in pn.last_error()


def test_euler_cell_sizes():
    c = pn.Cell(pn.CELL_EULER_TANH, 3)
    assert pn.lib().pn_workspace_bytes(ctypes.byref(c), 2, 100, 64, pn.NEWTON, None) > 0
    assert pn.lib().pn_workspace_bytes(ctypes.byref(c), 2, 100, 65, pn.NEWTON, None) == 0
    rc, _ = _eval_raw(kind=4)
    assert rc == pn.EINVAL


def test_options_defaults():
    o = pn.make_opts()
    assert o.damping == 1.0 and o.chunk == 0 and o.window == 0 and o.flags == 0
    assert o.bandwidth == 1 and o.window_mode == pn.WINDOW_CONSECUTIVE and o.profile_stride == 1
    o.profile_stride = -1
    rc, _ = _eval_raw(opts=o)
    assert rc == pn.EINVAL and "profile_stride" in pn.last_error()


def test_empty_problems_succeed_without_work():
    for B, T, D in [(0, 5, 4), (2, 0, 4), (2, 5, 0)]:
        rc, it = _eval_raw(B=B, T=T, D=D, ptr=0)
        assert rc == pn.OK and it == 0


def test_workspace_bytes_is_host_only_and_monotone():
    n1 = pn.workspace_bytes(pn.CELL_DIAG_TANH, 256, 8, 65536, 256, pn.QUASI_NEWTON, chunk=128)
    n2 = pn.workspace_bytes(pn.CELL_DIAG_TANH, 256, 8, 131072, 256, pn.QUASI_NEWTON, chunk=128)
    assert 0 < n1 < n2 and n1 % 256 == 0
    g = pn.Cell(pn.CELL_GRU, 8)
    nq = pn.workspace_bytes(pn.CELL_GRU, 8, 64, 2048, 16, pn.QUASI_NEWTON)
    nn = pn.workspace_bytes(pn.CELL_GRU, 8, 64, 2048, 16, pn.NEWTON)
    assert nn > nq > 0          # dense chunk maps hold D x D per chunk
    assert pn.lib().pn_workspace_bytes(ctypes.byref(g), 1, 10, 65, pn.NEWTON, None) == 0
    # the banded mode keeps dense chunk maps, except where it reduces to the
    # diagonal (k = 0) or the full Jacobian (k >= D - 1)
    nb = pn.workspace_bytes(pn.CELL_GRU, 8, 64, 2048, 16, pn.BANDED, bandwidth=2)
    nb0 = pn.workspace_bytes(pn.CELL_GRU, 8, 64, 2048, 16, pn.BANDED, bandwidth=0)
    nbf = pn.workspace_bytes(pn.CELL_GRU, 8, 64, 2048, 16, pn.BANDED, bandwidth=40)
    assert nb == nn and nb0 == nq and nbf == nn
    assert pn.workspace_bytes(pn.CELL_DIAG_TANH, 256, 8, 4096, 256, pn.BANDED, bandwidth=3) == \
        pn.workspace_bytes(pn.CELL_DIAG_TANH, 256, 8, 4096, 256, pn.QUASI_NEWTON)
    # a window bounds the workspace
    nw = pn.workspace_bytes(pn.CELL_GRU, 32, 4, 32768, 64, pn.QUASI_NEWTON, window=1024)
    nf = pn.workspace_bytes(pn.CELL_GRU, 32, 4, 32768, 64, pn.QUASI_NEWTON)
    assert nw < nf


def test_affine_scan_argument_checks():
    L = pn.lib()
    p = ctypes.c_void_p(1)
    assert L.pn_affine_scan(p, p, p, -1, 4, 4, 0, p, None) == pn.EINVAL
    assert L.pn_affine_scan(p, p, p, 1, 4, 4, 2, p, None) == pn.EINVAL
    assert L.pn_affine_scan(p, p, p, 1, 4, 65, 1, p, None) == pn.EUNSUPPORTED
    assert L.pn_affine_scan(None, p, p, 1, 4, 4, 0, p, None) == pn.EINVAL
    assert L.pn_affine_scan(None, None, None, 0, 4, 4, 0, None, None) == pn.OK
    assert L.pn_affine_scan_workspace_bytes(2, 100, 3, 1, None) > 0


def test_undersized_workspace_is_rejected_before_any_device_work():
    o = pn.make_opts()
    o.workspace = 0x10000
    o.workspace_bytes = 1024
    rc, _ = _eval_raw(kind=pn.CELL_GRU, m=8, B=64, T=2048, D=16, mode=pn.QUASI_NEWTON, opts=o)
    assert rc == pn.EWORKSPACE
    assert "smaller" in pn.last_error()


@pytest.mark.parametrize("inp", ["x", "s0", "params"])
def test_out_overlapping_an_input_is_rejected(inp):
    # out [B,T,D] = [2,5,4] floats: starting inside the input, at its first
    # byte, or ending on its first byte all overlap; one byte past does not
    for delta, bad in ((0, True), (-(2 * 5 * 4 * 4) + 1, True), (-(2 * 5 * 4 * 4), False), (8, True)):
        rc, _ = _eval_raw(addrs={"out": FAKE[inp] + delta})
        if bad:
            assert rc == pn.EINVAL and "overlaps " + inp in pn.last_error(), (inp, delta)
        else:
            assert not (rc == pn.EINVAL and "overlaps" in pn.last_error()), (inp, delta)


def test_python_binding_checks_shapes_before_any_launch():
    # CPU tensors: the shape, length and device checks come first, so these
    # raise ValueError without a GPU
    D, m, B, T = 4, 3, 2, 5
    x = torch.zeros(B, T, m)
    s0 = torch.zeros(B, D)
    good = torch.zeros(pn.param_count(pn.CELL_GRU, D, m))
    assert pn.param_count(pn.CELL_GRU, D, m) == 3 * D * m + 3 * D * D + 6 * D
    assert pn.param_count(pn.CELL_TANH_RNN, D, m) == D * D + D * m + D
    assert pn.param_count(pn.CELL_EULER_TANH, D, m) == D * D + D * m + 2 * D
    assert pn.param_count(pn.CELL_DIAG_TANH, D, D) == D
    with pytest.raises(ValueError, match="params holds"):
        pn.eval(pn.CELL_GRU, good[:-1], x, s0)
    with pytest.raises(ValueError, match="out must have shape"):
        pn.eval(pn.CELL_GRU, good, x, s0, out=torch.zeros(B, T, D + 1))
    with pytest.raises(ValueError, match="disagree on B"):
        pn.eval(pn.CELL_GRU, good, x, torch.zeros(B + 1, D))
    with pytest.raises(ValueError, match="x must be"):
        pn.eval(pn.CELL_GRU, good, x[0], s0)
    with pytest.raises(ValueError, match="unknown cell kind"):
        pn.eval(9, good, x, s0)
    with pytest.raises(ValueError, match="A must have shape"):
        pn.affine_scan(torch.zeros(B, T, D), torch.zeros(B, T, D), s0, dense=True)
    with pytest.raises(ValueError, match="s0 must have shape"):
        pn.affine_scan(torch.zeros(B, T, D), torch.zeros(B, T, D), torch.zeros(B, D + 1))


def test_ceiling_tool_exports_every_declared_symbol():
    text = open(os.path.join(ROOT, "include", "pn_ceiling.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(pnc_[a-z0-9_]+)\s*\(", text)))
    assert names == ["pnc_hbm", "pnc_last_error", "pnc_mfma_f32", "pnc_sequential_tanh"]
    lib = ctypes.CDLL(os.path.join(ROOT, "newton_evaluation_nonlinear_amd", "libpn_ceiling.so"))
    for name in names:
        assert hasattr(lib, name), name
    # argument checks come before any device call
    d = ctypes.c_double(0.0)
    lib.pnc_hbm.argtypes = [ctypes.c_int, ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                            ctypes.POINTER(ctypes.c_double)]
    lib.pnc_last_error.restype = ctypes.c_char_p
    assert lib.pnc_hbm(9, 1 << 20, 1, ctypes.byref(d), ctypes.byref(d)) == -1
    assert lib.pnc_last_error().decode() == "bad argument"
    vp = ctypes.c_void_p
    lib.pnc_sequential_tanh.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    assert lib.pnc_sequential_tanh(None, None, None, None, 1, 1, 1, 1, ctypes.byref(d), ctypes.byref(d)) == -1
    assert lib.pnc_last_error().decode() == "bad argument"
