"""Python binding of libpn (parallel-in-time evaluation of nonlinear recurrences).

Argument marshalling only: every step of the solve runs in the HIP kernels of
``libpn.so``; torch is used for device memory and the current stream.  The
library must have been built (``python -m newton_evaluation_nonlinear_amd._build``);
there is no fallback of any kind.

    out, iters, status = pn.eval(cell, params, x, s0, mode=pn.QUASI_NEWTON, tol=1e-5)

The method, the stop rule and all layouts are documented in include/pn.h.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpn.so")

CELL_DIAG_TANH, CELL_TANH_RNN, CELL_GRU, CELL_EULER_TANH = 0, 1, 2, 3
JACOBI, PICARD, QUASI_NEWTON, NEWTON, BANDED = 0, 1, 2, 3, 4
OK, NOT_CONVERGED, NONFINITE = 0, 1, 2
EINVAL, EUNSUPPORTED, EHIP, EWORKSPACE = -1, -2, -3, -4
FLAG_PERSISTENT, FLAG_MULTI_LAUNCH = 1, 2
WINDOW_CONSECUTIVE, WINDOW_ADVANCING = 0, 1

EXPORTED = ("pn_opts_init", "pn_eval", "pn_eval_ex", "pn_eval_f16", "pn_eval_noalloc",
            "pn_workspace_bytes", "pn_affine_scan", "pn_affine_scan_workspace_bytes", "pn_last_error",
            "pn_version")


class PnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libpn error {code}: {msg}")
        self.code = code


class Cell(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("input_dim", ctypes.c_int32)]


class Profile(ctypes.Structure):
    _fields_ = [("apply_ms", ctypes.c_double), ("apply_launches", ctypes.c_int32),
                ("apply_bytes", ctypes.c_double), ("apply_flops", ctypes.c_double),
                ("total_ms", ctypes.c_double)]


class Opts(ctypes.Structure):
    _fields_ = [("damping", ctypes.c_float), ("chunk", ctypes.c_int32), ("window", ctypes.c_int64),
                ("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t),
                ("resid_hist", ctypes.POINTER(ctypes.c_float)), ("resid_hist_len", ctypes.c_int32),
                ("window_iters", ctypes.POINTER(ctypes.c_int32)),
                ("window_iters_len", ctypes.c_int64),
                ("profile", ctypes.POINTER(Profile)),
                ("flags", ctypes.c_int32), ("bandwidth", ctypes.c_int32),
                ("window_mode", ctypes.c_int32),
                ("accepted", ctypes.POINTER(ctypes.c_int32)), ("accepted_len", ctypes.c_int64),
                ("switch_mode", ctypes.c_int32), ("switch_ratio", ctypes.c_float),
                ("window_switch", ctypes.POINTER(ctypes.c_int32)),
                ("window_switch_len", ctypes.c_int64),
                ("switch_damping", ctypes.c_float),
                ("profile_stride", ctypes.c_int32)]


_lib = None


def lib():
    """Load libpn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m newton_evaluation_nonlinear_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        f = ctypes.c_float
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.pn_opts_init.argtypes = [ctypes.POINTER(Opts)]
        L.pn_opts_init.restype = None
        sig = [ctypes.POINTER(Cell), vp, vp, vp, i64, i64, i64, i32, f, i32, vp,
               ctypes.POINTER(i32)]
        L.pn_eval.argtypes = sig
        L.pn_eval.restype = ctypes.c_int
        L.pn_eval_ex.argtypes = sig + [ctypes.POINTER(Opts)]
        L.pn_eval_ex.restype = ctypes.c_int
        L.pn_eval_f16.argtypes = sig + [ctypes.POINTER(Opts)]
        L.pn_eval_f16.restype = ctypes.c_int
        L.pn_eval_noalloc.argtypes = sig + [ctypes.POINTER(Opts)]
        L.pn_eval_noalloc.restype = ctypes.c_int
        L.pn_workspace_bytes.argtypes = [ctypes.POINTER(Cell), i64, i64, i64, i32, ctypes.POINTER(Opts)]
        L.pn_workspace_bytes.restype = ctypes.c_size_t
        L.pn_affine_scan.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp, ctypes.POINTER(Opts)]
        L.pn_affine_scan.restype = ctypes.c_int
        L.pn_affine_scan_workspace_bytes.argtypes = [i64, i64, i64, i32, ctypes.POINTER(Opts)]
        L.pn_affine_scan_workspace_bytes.restype = ctypes.c_size_t
        L.pn_last_error.argtypes = []
        L.pn_last_error.restype = ctypes.c_char_p
        L.pn_version.argtypes = []
        L.pn_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def version():
    return lib().pn_version().decode()


def last_error():
    return lib().pn_last_error().decode()


def _dev_f32(t, name, dtype=torch.float32):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) torch tensor")
    if t.dtype != dtype or not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous {dtype}")
    return t.data_ptr()


def param_count(cell_kind, D, m):
    """Length of the flat parameter vector of a cell (layouts in include/pn.h)."""
    k = int(cell_kind)
    if k == CELL_DIAG_TANH:
        return D
    if k == CELL_TANH_RNN:
        return D * D + D * m + D
    if k == CELL_GRU:
        return 3 * D * m + 3 * D * D + 6 * D
    if k == CELL_EULER_TANH:
        return D * D + D * m + 2 * D
    raise ValueError(f"unknown cell kind {cell_kind}")


def _check_shapes(cell_kind, params, x, s0, out, sdt):
    """Shapes, lengths and devices the C side cannot see; raises ValueError
    before any launch."""
    for name, t in (("params", params), ("x", x), ("s0", s0)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
    if x.dim() != 3:
        raise ValueError(f"x must be [B, T, m], got shape {tuple(x.shape)}")
    if s0.dim() != 2:
        raise ValueError(f"s0 must be [B, D], got shape {tuple(s0.shape)}")
    B, T, m = x.shape
    D = s0.shape[1]
    if s0.shape[0] != B:
        raise ValueError("x and s0 disagree on B")
    need = param_count(cell_kind, D, m)
    if params.numel() != need:
        raise ValueError(f"params holds {params.numel()} values; cell kind {int(cell_kind)} with "
                         f"D={D}, m={m} needs {need}")
    if out is not None:
        if not isinstance(out, torch.Tensor):
            raise TypeError("out must be a torch tensor")
        if tuple(out.shape) != (B, T, D):
            raise ValueError(f"out must have shape {(B, T, D)}, got {tuple(out.shape)}")
        if out.dtype != sdt:
            raise ValueError(f"out must be {sdt}")
    devs = {t.device for t in (params, x, s0) + ((out,) if out is not None else ())}
    if len(devs) != 1:
        raise ValueError(f"params, x, s0 and out must live on one device, got {sorted(map(str, devs))}")


def _stream_ptr(device):
    return torch.cuda.current_stream(device).cuda_stream


def make_opts(damping=1.0, window=0, chunk=0, stream=None, flags=0, bandwidth=1,
              window_mode=WINDOW_CONSECUTIVE, switch_mode=-1, switch_ratio=0.5, switch_damping=0.0):
    o = Opts()
    lib().pn_opts_init(ctypes.byref(o))
    o.damping = float(damping)
    o.window = int(window)
    o.chunk = int(chunk)
    o.stream = stream
    o.flags = int(flags)
    o.bandwidth = int(bandwidth)
    o.window_mode = int(window_mode)
    o.switch_mode = int(switch_mode)
    o.switch_ratio = float(switch_ratio)
    o.switch_damping = float(switch_damping)
    return o


def workspace_bytes(cell_kind, input_dim, B, T, D, mode, damping=1.0, window=0, chunk=0,
                    bandwidth=1, window_mode=WINDOW_CONSECUTIVE, switch_mode=-1):
    o = make_opts(damping, window, chunk, bandwidth=bandwidth, window_mode=window_mode,
                  switch_mode=switch_mode)
    c = Cell(cell_kind, input_dim)
    n = lib().pn_workspace_bytes(ctypes.byref(c), B, T, D, mode, ctypes.byref(o))
    if n == 0:
        raise PnError(EINVAL, last_error())
    return n


class Result:
    """Outcome of one solve: trajectory, total updates, status and diagnostics."""

    def __init__(self, out, iters, status, window_iters, resid_hist, profile, accepted=None,
                 window_switch=None):
        self.out, self.iters, self.status = out, iters, status
        self.window_iters, self.resid_hist, self.profile = window_iters, resid_hist, profile
        self.accepted = accepted     # advancing window: steps accepted per check
        self.window_switch = window_switch   # switching: per window, the check that switched

    def __iter__(self):
        return iter((self.out, self.iters, self.status))


def eval(cell_kind, params, x, s0, mode=QUASI_NEWTON, tol=1e-5, max_iter=None, damping=1.0,
         window=0, chunk=0, out=None, history=False, profile=False, workspace=None, flags=0,
         bandwidth=1, window_mode=WINDOW_CONSECUTIVE, switch_mode=-1, switch_ratio=0.5,
         switch_damping=0.0, noalloc=False):
    """Solve s_t = f(s_{t-1}, x_t) for t = 1..T over the batch; see include/pn.h.

    params, x [B,T,m], s0 [B,D] are float32 tensors on one HIP device; with
    x in float16 the solve stores x and the iterate in binary16 (pn_eval_f16,
    channel-wise cell; ``out`` float16).
    ``bandwidth`` is the half-bandwidth k of the BANDED mode; ``window_mode``
    WINDOW_ADVANCING slides one window past its converged prefix (max_iter
    then defaults to T and caps the updates of the whole solve); ``switch_mode``
    >= 0 moves each window to that mode when its residual stalls
    (r_i > switch_ratio * r_{i-1}), and to the step damping
    ``switch_damping`` if that is > 0 (``switch_mode`` == ``mode`` switches
    the damping alone).
    ``profile`` True times every steady apply launch with HIP events, an
    integer n > 1 every n-th (Result.profile).
    ``noalloc`` runs pn_eval_noalloc: no workspace is allocated, the library
    uses its static device scratch (float storage; no profile, no workspace).
    Returns a ``Result`` (unpacks as ``out, iters, status``).  Negative
    library statuses raise ``PnError``.
    """
    half = isinstance(x, torch.Tensor) and x.dtype == torch.float16
    sdt = torch.float16 if half else torch.float32
    _check_shapes(cell_kind, params, x, s0, out, sdt)
    B, T, m = x.shape
    D = s0.shape[1]
    W = T if window in (0, None) else int(window)
    advancing = int(window_mode) == WINDOW_ADVANCING
    if max_iter is None:
        max_iter = T if advancing else W
    dev = x.device
    if out is None:
        out = torch.empty((B, T, D), dtype=sdt, device=dev)
    c = Cell(int(cell_kind), int(m))
    o = make_opts(damping, window or 0, chunk, _stream_ptr(dev), flags, bandwidth, window_mode,
                  switch_mode, switch_ratio, switch_damping)
    if noalloc:
        if half or workspace is not None or profile:
            raise ValueError("noalloc takes float storage and neither a workspace nor profiling")
    else:
        nbytes = lib().pn_workspace_bytes(ctypes.byref(c), B, T, D, int(mode), ctypes.byref(o))
        if nbytes == 0:
            raise PnError(EINVAL, last_error())
        if workspace is None or workspace.numel() < nbytes:
            workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
        base = workspace.data_ptr()
        aligned = (base + 255) // 256 * 256
        o.workspace = aligned
        o.workspace_bytes = workspace.numel() - (aligned - base)
    nwin = 1 if advancing else (max(1, -(-T // W)) if T > 0 else 1)
    wit = (ctypes.c_int32 * nwin)()
    o.window_iters = wit
    o.window_iters_len = nwin
    wsw = (ctypes.c_int32 * nwin)(*([-1] * nwin))
    o.window_switch = wsw
    o.window_switch_len = nwin
    hist = None
    if history:
        hlen = min(nwin * (int(max_iter) + 1), 1 << 22)
        hist = (ctypes.c_float * hlen)()
        o.resid_hist = hist
        o.resid_hist_len = hlen
    acc = None
    if advancing and history:
        alen = int(max_iter) + 1
        acc = (ctypes.c_int32 * alen)()
        o.accepted = acc
        o.accepted_len = alen
    prof = Profile() if profile else None
    if prof is not None:
        o.profile = ctypes.pointer(prof)
        o.profile_stride = int(profile)     # True: every steady launch; n: every n-th
    iters = ctypes.c_int32(0)
    entry = lib().pn_eval_noalloc if noalloc else (lib().pn_eval_f16 if half else lib().pn_eval_ex)
    rc = entry(ctypes.byref(c), _dev_f32(params, "params"), _dev_f32(x, "x", sdt),
               _dev_f32(s0, "s0"), B, T, D, int(mode), float(tol), int(max_iter),
               _dev_f32(out, "out", sdt), ctypes.byref(iters), ctypes.byref(o))
    if rc < 0:
        raise PnError(rc, last_error())
    witer = list(wit)
    rh = None
    if history:
        n = sum(k + 1 for k in witer[:nwin])
        rh = list(hist[:min(n, len(hist))])
    pd = None
    if prof is not None:
        pd = {k: getattr(prof, k) for k, _ in Profile._fields_}
    accepted = None
    if acc is not None:
        accepted = list(acc[:min(len(rh or []), len(acc))])
        if rc == NONFINITE:
            accepted = accepted[:-1]
    wswitch = list(wsw)[:len(witer)] if int(switch_mode) >= 0 else None
    return Result(out, int(iters.value), int(rc), witer, rh, pd, accepted, wswitch)


def affine_scan(A, b, s0, dense=False, chunk=0, out=None):
    """out_t = A_t out_{t-1} + b_t (A diagonal [B,T,D] or dense [B,T,D,D])."""
    if b.dim() != 3:
        raise ValueError(f"b must be [B, T, D], got shape {tuple(b.shape)}")
    B, T, D = b.shape
    want = (B, T, D, D) if dense else (B, T, D)
    if tuple(A.shape) != want:
        raise ValueError(f"A must have shape {want}, got {tuple(A.shape)}")
    if tuple(s0.shape) != (B, D):
        raise ValueError(f"s0 must have shape {(B, D)}, got {tuple(s0.shape)}")
    if out is not None and tuple(out.shape) != (B, T, D):
        raise ValueError(f"out must have shape {(B, T, D)}, got {tuple(out.shape)}")
    if len({t.device for t in (A, b, s0) + ((out,) if out is not None else ())}) != 1:
        raise ValueError("A, b, s0 and out must live on one device")
    if out is None:
        out = torch.empty_like(b)
    o = make_opts(chunk=chunk, stream=_stream_ptr(b.device))
    nbytes = lib().pn_affine_scan_workspace_bytes(B, T, D, int(dense), ctypes.byref(o))
    if nbytes == 0:
        raise PnError(EINVAL, last_error())
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=b.device)
    base = ws.data_ptr()
    aligned = (base + 255) // 256 * 256
    o.workspace = aligned
    o.workspace_bytes = ws.numel() - (aligned - base)
    rc = lib().pn_affine_scan(_dev_f32(A, "A"), _dev_f32(b, "b"), _dev_f32(s0, "s0"), B, T, D,
                              int(dense), _dev_f32(out, "out"), ctypes.byref(o))
    if rc < 0:
        raise PnError(rc, last_error())
    return out
