"""Transition maps f_t(p) = f(p, x_t) and their state Jacobians, plain numpy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The article [PN §1.1] states the problem for arbitrary maps f_1..f_T; its
applications section [PN §1.3.2] names RNNs.  Three concrete cells are used:

* ``DiagTanh``  f(p, x) = tanh(a * p + x), one independent channel per state
  entry (params: a[D]; the input has m = D channels).
* ``TanhRNN``   f(p, x) = tanh(W p + U x + b)  (params: W[D,D] | U[D,m] | b[D]).
* ``GRU``       the gated recurrent unit in the convention of torch.nn.GRU,
  gate order (r, z, n), with the hidden bias of the candidate inside the reset
  product (params: W_ih[3D,m] | W_hh[3D,D] | b_ih[3D] | b_hh[3D]).
* ``EulerTanh`` f(p, x) = p + h * (tanh(W p + U x + b) - p): one explicit
  Euler step, per-channel step sizes h, of the continuous-time RNN
  ds/dt = -s + tanh(W s + U x(t) + b).  For small h the dynamics Jacobian is
  close to the identity, the regime of Picard's identity approximation
  [PN §1.3.1, §2.2.3] (params: W[D,D] | U[D,m] | b[D] | h[D]).

Every method is vectorised over any leading axes: ``p`` has shape [..., D] and
``x`` shape [..., m].  Jacobians are with respect to the previous state p,
i.e. A_t = df_t/ds_{t-1} evaluated at p = s_{t-1}.

The derivative formulas below are derived by hand from the cell definitions;
they are pinned against torch.autograd and central finite differences in the
oracle pin tests.
"""

import numpy as np

CELL_DIAG_TANH = 0
CELL_TANH_RNN = 1
CELL_GRU = 2
CELL_EULER_TANH = 3


def _sigmoid(u):
    return 1.0 / (1.0 + np.exp(-u))


def _diag_embed(d):
    """[..., D] -> [..., D, D] with d on the diagonal."""
    D = d.shape[-1]
    out = np.zeros(d.shape + (D,), dtype=d.dtype)
    idx = np.arange(D)
    out[..., idx, idx] = d
    return out


class DiagTanh:
    """s_t = tanh(a * s_{t-1} + x_t), channel by channel."""

    kind = CELL_DIAG_TANH

    def __init__(self, a, dtype=np.float64):
        self.a = np.asarray(a, dtype=dtype)
        self.D = self.a.shape[0]
        self.m = self.D
        self.dtype = dtype

    def f(self, p, x):
        return np.tanh(self.a * p + x)

    def jac_diag(self, p, x):
        v = self.f(p, x)
        return self.a * (1.0 - v * v)

    def jac(self, p, x):
        # The map is channel-wise, so the Jacobian is diagonal.
        return _diag_embed(self.jac_diag(p, x))


class TanhRNN:
    """s_t = tanh(W s_{t-1} + U x_t + b)."""

    kind = CELL_TANH_RNN

    def __init__(self, W, U, b, dtype=np.float64):
        self.W = np.asarray(W, dtype=dtype)
        self.U = np.asarray(U, dtype=dtype)
        self.b = np.asarray(b, dtype=dtype)
        self.D = self.W.shape[0]
        self.m = self.U.shape[1]
        self.dtype = dtype

    def f(self, p, x):
        return np.tanh(p @ self.W.T + x @ self.U.T + self.b)

    def jac(self, p, x):
        # d tanh(u)/du = 1 - tanh(u)^2, chain rule through u = W p + ...:
        # A[i, k] = (1 - v_i^2) W[i, k].
        v = self.f(p, x)
        return (1.0 - v * v)[..., :, None] * self.W

    def jac_diag(self, p, x):
        v = self.f(p, x)
        return (1.0 - v * v) * np.diagonal(self.W)


class GRU:
    """torch.nn.GRU single-layer cell.

    r = sigma(W_ir x + b_ir + W_hr p + b_hr)
    z = sigma(W_iz x + b_iz + W_hz p + b_hz)
    g = W_hn p + b_hn
    n = tanh(W_in x + b_in + r * g)
    f = (1 - z) * n + z * p
    """

    kind = CELL_GRU

    def __init__(self, W_ih, W_hh, b_ih, b_hh, dtype=np.float64):
        self.W_ih = np.asarray(W_ih, dtype=dtype)
        self.W_hh = np.asarray(W_hh, dtype=dtype)
        self.b_ih = np.asarray(b_ih, dtype=dtype)
        self.b_hh = np.asarray(b_hh, dtype=dtype)
        self.D = self.W_hh.shape[1]
        self.m = self.W_ih.shape[1]
        self.dtype = dtype
        D = self.D
        self.W_hr, self.W_hz, self.W_hn = self.W_hh[:D], self.W_hh[D:2 * D], self.W_hh[2 * D:]

    def _gates(self, p, x):
        D = self.D
        gi = x @ self.W_ih.T + self.b_ih
        gh = p @ self.W_hh.T + self.b_hh
        r = _sigmoid(gi[..., :D] + gh[..., :D])
        z = _sigmoid(gi[..., D:2 * D] + gh[..., D:2 * D])
        g = gh[..., 2 * D:]
        n = np.tanh(gi[..., 2 * D:] + r * g)
        return r, z, g, n

    def f(self, p, x):
        r, z, g, n = self._gates(p, x)
        return (1.0 - z) * n + z * p

    def _row_scales(self, p, x):
        """Coefficients of df/dp = diag(z) + diag(cz) W_hz + diag(cn) W_hn + diag(cr) W_hr.

        df_i/dp_k = z_i [i == k]
                    + (p_i - n_i) z_i (1 - z_i) W_hz[i, k]            (through z)
                    + (1 - z_i)(1 - n_i^2) r_i W_hn[i, k]             (through g)
                    + (1 - z_i)(1 - n_i^2) g_i r_i (1 - r_i) W_hr[i, k] (through r)
        """
        r, z, g, n = self._gates(p, x)
        dn = (1.0 - z) * (1.0 - n * n)
        cz = (p - n) * z * (1.0 - z)
        cn = dn * r
        cr = dn * g * r * (1.0 - r)
        return z, cz, cn, cr

    def jac(self, p, x):
        z, cz, cn, cr = self._row_scales(p, x)
        return (_diag_embed(z)
                + cz[..., :, None] * self.W_hz
                + cn[..., :, None] * self.W_hn
                + cr[..., :, None] * self.W_hr)

    def jac_diag(self, p, x):
        z, cz, cn, cr = self._row_scales(p, x)
        return (z + cz * np.diagonal(self.W_hz) + cn * np.diagonal(self.W_hn)
                + cr * np.diagonal(self.W_hr))


class EulerTanh:
    """s_t = s_{t-1} + h * (tanh(W s_{t-1} + U x_t + b) - s_{t-1})."""

    kind = CELL_EULER_TANH

    def __init__(self, W, U, b, h, dtype=np.float64):
        self.W = np.asarray(W, dtype=dtype)
        self.U = np.asarray(U, dtype=dtype)
        self.b = np.asarray(b, dtype=dtype)
        self.h = np.asarray(h, dtype=dtype)
        self.D = self.W.shape[0]
        self.m = self.U.shape[1]
        self.dtype = dtype

    def _g(self, p, x):
        return np.tanh(p @ self.W.T + x @ self.U.T + self.b)

    def f(self, p, x):
        return p + self.h * (self._g(p, x) - p)

    def jac(self, p, x):
        # A[i, k] = (1 - h_i) [i == k] + h_i (1 - g_i^2) W[i, k]
        g = self._g(p, x)
        return (_diag_embed(np.broadcast_to(1.0 - self.h, g.shape))
                + (self.h * (1.0 - g * g))[..., :, None] * self.W)

    def jac_diag(self, p, x):
        g = self._g(p, x)
        return 1.0 - self.h + self.h * (1.0 - g * g) * np.diagonal(self.W)


def make_cell(kind, params, D, m, dtype=np.float64):
    """Build a cell from the flat parameter vector of the C interface.

    Layouts (row-major, concatenated in this order):
      diag-tanh: a[D]                                   (m must equal D)
      tanh RNN : W[D*D] | U[D*m] | b[D]
      GRU      : W_ih[3D*m] | W_hh[3D*D] | b_ih[3D] | b_hh[3D]
      Euler    : W[D*D] | U[D*m] | b[D] | h[D]
    """
    w = np.asarray(params, dtype=np.float64).ravel()
    if kind == CELL_DIAG_TANH:
        if m != D:
            raise ValueError("diag-tanh cell needs input_dim == D")
        if w.size != D:
            raise ValueError("diag-tanh params must hold D values")
        return DiagTanh(w, dtype)
    if kind == CELL_TANH_RNN:
        if w.size != D * D + D * m + D:
            raise ValueError("tanh-RNN params must hold D*D + D*m + D values")
        W = w[:D * D].reshape(D, D)
        U = w[D * D:D * D + D * m].reshape(D, m)
        b = w[D * D + D * m:]
        return TanhRNN(W, U, b, dtype)
    if kind == CELL_GRU:
        n_ih, n_hh = 3 * D * m, 3 * D * D
        if w.size != n_ih + n_hh + 6 * D:
            raise ValueError("GRU params must hold 3D*m + 3D*D + 6D values")
        W_ih = w[:n_ih].reshape(3 * D, m)
        W_hh = w[n_ih:n_ih + n_hh].reshape(3 * D, D)
        b_ih = w[n_ih + n_hh:n_ih + n_hh + 3 * D]
        b_hh = w[n_ih + n_hh + 3 * D:]
        return GRU(W_ih, W_hh, b_ih, b_hh, dtype)
    if kind == CELL_EULER_TANH:
        if w.size != D * D + D * m + 2 * D:
            raise ValueError("Euler params must hold D*D + D*m + 2D values")
        W = w[:D * D].reshape(D, D)
        U = w[D * D:D * D + D * m].reshape(D, m)
        b = w[D * D + D * m:D * D + D * m + D]
        h = w[D * D + D * m + D:]
        return EulerTanh(W, U, b, h, dtype)
    raise ValueError(f"unknown cell kind {kind}")
