"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to a library routine, a closed form, an
invariant stated in the article "并行牛顿方法：加速非线性序列评估的计算革命" [PN], or
brute force on tiny inputs, chosen so that a dropped term, a wrong sign, a
shifted index or a transposed operand in the oracle fails at least one.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import cells as oc
from oracle import solver as osv
import workloads

RNG = np.random.default_rng(1234)


def _rnn_params(D, m, rng, scale=1.0):
    return workloads.random_cell_params(oracle.CELL_TANH_RNN, D, m, rng, scale).astype(np.float64)


def _gru_params(D, m, rng, scale=1.0):
    return workloads.random_cell_params(oracle.CELL_GRU, D, m, rng, scale).astype(np.float64)


# ---------------------------------------------------------------- sequential

def test_sequential_tanh_rnn_matches_torch_rnn():
    D, m, B, T = 5, 3, 3, 17
    rng = np.random.default_rng(1)
    params = _rnn_params(D, m, rng, 1.5)
    cell = oracle.make_cell(oracle.CELL_TANH_RNN, params, D, m)
    x = rng.standard_normal((B, T, m))
    s0 = rng.standard_normal((B, D))
    ref = torch.nn.RNN(m, D, nonlinearity="tanh", batch_first=True).double()
    with torch.no_grad():
        ref.weight_hh_l0.copy_(torch.from_numpy(cell.W))
        ref.weight_ih_l0.copy_(torch.from_numpy(cell.U))
        ref.bias_ih_l0.copy_(torch.from_numpy(cell.b))
        ref.bias_hh_l0.zero_()
        out, _ = ref(torch.from_numpy(x), torch.from_numpy(s0)[None])
    got = oracle.sequential(cell, x, s0)
    np.testing.assert_allclose(got, out.numpy(), rtol=0, atol=1e-12)


def test_sequential_gru_matches_torch_gru():
    D, m, B, T = 6, 4, 3, 19
    rng = np.random.default_rng(2)
    params = _gru_params(D, m, rng, 2.0)
    cell = oracle.make_cell(oracle.CELL_GRU, params, D, m)
    x = rng.standard_normal((B, T, m))
    s0 = rng.standard_normal((B, D)) * 0.5
    ref = torch.nn.GRU(m, D, batch_first=True).double()
    with torch.no_grad():
        ref.weight_ih_l0.copy_(torch.from_numpy(cell.W_ih))
        ref.weight_hh_l0.copy_(torch.from_numpy(cell.W_hh))
        ref.bias_ih_l0.copy_(torch.from_numpy(cell.b_ih))
        ref.bias_hh_l0.copy_(torch.from_numpy(cell.b_hh))
        out, _ = ref(torch.from_numpy(x), torch.from_numpy(s0)[None])
    got = oracle.sequential(cell, x, s0)
    np.testing.assert_allclose(got, out.numpy(), rtol=0, atol=1e-12)


def _flat_from_torch_gru(mod):
    """The flat parameter vector of the C interface, W_ih | W_hh | b_ih | b_hh,
    taken from a torch.nn.GRU's own tensors in their storage order."""
    return np.concatenate([t.detach().numpy().ravel() for t in
                           (mod.weight_ih_l0, mod.weight_hh_l0, mod.bias_ih_l0, mod.bias_hh_l0)])


def _flat_from_torch_rnn(mod):
    """W | U | b for a torch.nn.RNN(tanh): W is weight_hh, U weight_ih, and the
    two torch biases act as one sum."""
    return np.concatenate([mod.weight_hh_l0.detach().numpy().ravel(),
                           mod.weight_ih_l0.detach().numpy().ravel(),
                           (mod.bias_ih_l0 + mod.bias_hh_l0).detach().numpy()])


@pytest.mark.parametrize("D, m", [(6, 4), (5, 9)])
def test_flat_gru_layout_parses_torch_parameters(D, m):
    # The flat layout itself, not cell fields copied back into torch: a
    # freshly initialised torch.nn.GRU (its own weights, every bias nonzero
    # and different) is flattened in the documented order and parsed by
    # make_cell; a swap of b_ih and b_hh (which only matters for the
    # candidate's b_hn inside the reset product), of two gates, or of the
    # input and hidden blocks fails this.
    torch.manual_seed(10 + D)
    mod = torch.nn.GRU(m, D, batch_first=True).double()
    with torch.no_grad():
        mod.bias_ih_l0.uniform_(-1.0, 1.0)
        mod.bias_hh_l0.uniform_(-1.0, 1.0)
        mod.weight_hh_l0.mul_(2.0)
    flat = _flat_from_torch_gru(mod)
    cell = oracle.make_cell(oracle.CELL_GRU, flat, D, m)
    rng = np.random.default_rng(20 + D)
    B, T = 3, 13
    x = rng.standard_normal((B, T, m))
    s0 = 0.5 * rng.standard_normal((B, D))
    with torch.no_grad():
        ref, _ = mod(torch.from_numpy(x), torch.from_numpy(s0)[None])
    np.testing.assert_allclose(oracle.sequential(cell, x, s0), ref.numpy(), rtol=0, atol=1e-12)
    # the same holds for the swapped-bias vector only if b_hn does not matter,
    # which it does here
    n_ih, n_hh = 3 * D * m, 3 * D * D
    swapped = flat.copy()
    swapped[n_ih + n_hh:n_ih + n_hh + 3 * D] = flat[n_ih + n_hh + 3 * D:]
    swapped[n_ih + n_hh + 3 * D:] = flat[n_ih + n_hh:n_ih + n_hh + 3 * D]
    bad = oracle.sequential(oracle.make_cell(oracle.CELL_GRU, swapped, D, m), x, s0)
    assert np.max(np.abs(bad - ref.numpy())) > 1e-3


def test_flat_rnn_layout_parses_torch_parameters():
    D, m = 5, 3
    torch.manual_seed(31)
    mod = torch.nn.RNN(m, D, nonlinearity="tanh", batch_first=True).double()
    with torch.no_grad():
        mod.weight_hh_l0.mul_(2.0)
    cell = oracle.make_cell(oracle.CELL_TANH_RNN, _flat_from_torch_rnn(mod), D, m)
    rng = np.random.default_rng(32)
    x = rng.standard_normal((2, 11, m))
    s0 = rng.standard_normal((2, D))
    with torch.no_grad():
        ref, _ = mod(torch.from_numpy(x), torch.from_numpy(s0)[None])
    np.testing.assert_allclose(oracle.sequential(cell, x, s0), ref.numpy(), rtol=0, atol=1e-12)


def test_sequential_diag_tanh_is_an_rnn_with_diagonal_weights():
    # tanh(a*s + x) is torch's Elman RNN with W_hh = diag(a), W_ih = I, no bias.
    D, B, T = 7, 2, 23
    rng = np.random.default_rng(3)
    a = rng.uniform(-0.95, 0.95, D)
    cell = oracle.make_cell(oracle.CELL_DIAG_TANH, a, D, D)
    x = rng.standard_normal((B, T, D))
    s0 = rng.standard_normal((B, D))
    ref = torch.nn.RNN(D, D, nonlinearity="tanh", batch_first=True).double()
    with torch.no_grad():
        ref.weight_hh_l0.copy_(torch.diag(torch.from_numpy(a)))
        ref.weight_ih_l0.copy_(torch.eye(D, dtype=torch.float64))
        ref.bias_ih_l0.zero_()
        ref.bias_hh_l0.zero_()
        out, _ = ref(torch.from_numpy(x), torch.from_numpy(s0)[None])
    np.testing.assert_allclose(oracle.sequential(cell, x, s0), out.numpy(), rtol=0, atol=1e-12)


def test_sequential_scalar_closed_form():
    # Two hand-evaluated steps of the scalar cell: s1 = tanh(x1), s2 = tanh(a s1 + x2).
    cell = oracle.make_cell(oracle.CELL_DIAG_TANH, np.array([0.5]), 1, 1)
    x = np.array([[[0.25], [-1.0]]])
    s = oracle.sequential(cell, x, np.zeros((1, 1)))
    s1 = np.tanh(0.25)
    assert s[0, 0, 0] == pytest.approx(s1, abs=1e-15)
    assert s[0, 1, 0] == pytest.approx(np.tanh(0.5 * s1 - 1.0), abs=1e-15)


# ---------------------------------------------------------------- Jacobians

def _torch_cell_jacobian(torch_cell, p, x):
    """Per-row Jacobian of a torch RNNCell/GRUCell w.r.t. its hidden state."""
    out = []
    for b in range(p.shape[0]):
        xb = torch.from_numpy(x[b:b + 1])
        J = torch.autograd.functional.jacobian(
            lambda h: torch_cell(xb, h[None])[0], torch.from_numpy(p[b]))
        out.append(J.numpy())
    return np.stack(out)


def test_gru_jacobian_matches_autograd_and_fd():
    D, m, B = 6, 3, 4
    rng = np.random.default_rng(4)
    params = _gru_params(D, m, rng, 2.5)
    cell = oracle.make_cell(oracle.CELL_GRU, params, D, m)
    p = rng.standard_normal((B, D))
    x = rng.standard_normal((B, m))
    tc = torch.nn.GRUCell(m, D).double()
    with torch.no_grad():
        tc.weight_ih.copy_(torch.from_numpy(cell.W_ih))
        tc.weight_hh.copy_(torch.from_numpy(cell.W_hh))
        tc.bias_ih.copy_(torch.from_numpy(cell.b_ih))
        tc.bias_hh.copy_(torch.from_numpy(cell.b_hh))
    ref = _torch_cell_jacobian(tc, p, x)
    J = cell.jac(p, x)
    np.testing.assert_allclose(J, ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(cell.jac_diag(p, x), np.diagonal(ref, axis1=-2, axis2=-1),
                               rtol=0, atol=1e-13)
    # central finite differences, column by column
    h = 1e-6
    fd = np.empty_like(J)
    for k in range(D):
        e = np.zeros(D)
        e[k] = h
        fd[..., k] = (cell.f(p + e, x) - cell.f(p - e, x)) / (2 * h)
    np.testing.assert_allclose(J, fd, rtol=0, atol=1e-8)


def test_tanh_rnn_jacobian_matches_autograd():
    D, m, B = 5, 2, 3
    rng = np.random.default_rng(5)
    params = _rnn_params(D, m, rng, 1.3)
    cell = oracle.make_cell(oracle.CELL_TANH_RNN, params, D, m)
    p = rng.standard_normal((B, D))
    x = rng.standard_normal((B, m))
    tc = torch.nn.RNNCell(m, D, nonlinearity="tanh").double()
    with torch.no_grad():
        tc.weight_hh.copy_(torch.from_numpy(cell.W))
        tc.weight_ih.copy_(torch.from_numpy(cell.U))
        tc.bias_ih.copy_(torch.from_numpy(cell.b))
        tc.bias_hh.zero_()
    ref = _torch_cell_jacobian(tc, p, x)
    np.testing.assert_allclose(cell.jac(p, x), ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(cell.jac_diag(p, x), np.diagonal(ref, axis1=-2, axis2=-1),
                               rtol=0, atol=1e-13)


def test_euler_cell_jacobian_matches_autograd_and_fd():
    D, m, B = 6, 3, 4
    rng = np.random.default_rng(15)
    params = workloads.random_cell_params(oracle.CELL_EULER_TANH, D, m, rng, 1.5).astype(np.float64)
    cell = oracle.make_cell(oracle.CELL_EULER_TANH, params, D, m)
    p = rng.standard_normal((B, D))
    x = rng.standard_normal((B, m))
    W, U, b, h = (torch.from_numpy(a) for a in (cell.W, cell.U, cell.b, cell.h))

    def step(pb, xb):   # one explicit Euler step of ds/dt = -s + tanh(W s + U x + b)
        return pb + h * (torch.tanh(W @ pb + U @ xb + b) - pb)

    ref = np.stack([torch.autograd.functional.jacobian(
        lambda q: step(q, torch.from_numpy(x[i])), torch.from_numpy(p[i])).numpy() for i in range(B)])
    np.testing.assert_allclose(cell.jac(p, x), ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(cell.jac_diag(p, x), np.diagonal(ref, axis1=-2, axis2=-1),
                               rtol=0, atol=1e-13)
    np.testing.assert_allclose(cell.f(p, x),
                               np.stack([step(torch.from_numpy(p[i]), torch.from_numpy(x[i])).numpy()
                                         for i in range(B)]), rtol=0, atol=1e-14)
    eps = 1e-6
    for k in range(D):
        e = np.zeros(D)
        e[k] = eps
        fd = (cell.f(p + e, x) - cell.f(p - e, x)) / (2 * eps)
        np.testing.assert_allclose(cell.jac(p, x)[..., k], fd, rtol=0, atol=1e-8)


def test_euler_cell_sequential_leaky_integrator_closed_form():
    # W = 0 and a constant input: s_t = g + (1 - h)^t (s_0 - g), g = tanh(U x + b)
    D, m, B, T = 4, 2, 2, 50
    rng = np.random.default_rng(16)
    U = rng.standard_normal((D, m))
    b = rng.standard_normal(D) * 0.3
    h = rng.uniform(0.01, 0.2, D)
    params = np.concatenate([np.zeros(D * D), U.ravel(), b, h])
    cell = oracle.make_cell(oracle.CELL_EULER_TANH, params, D, m)
    xc = rng.standard_normal((B, m))
    x = np.broadcast_to(xc[:, None], (B, T, m)).copy()
    s0 = rng.standard_normal((B, D))
    g = np.tanh(xc @ U.T + b)
    t = np.arange(1, T + 1)[None, :, None]
    ref = g[:, None] + (1.0 - h) ** t * (s0 - g)[:, None]
    np.testing.assert_allclose(oracle.sequential(cell, x, s0), ref, rtol=0, atol=1e-13)


def test_diag_tanh_jacobian_fd():
    D, B = 9, 3
    rng = np.random.default_rng(6)
    cell = oracle.make_cell(oracle.CELL_DIAG_TANH, rng.uniform(-1, 1, D), D, D)
    p = rng.standard_normal((B, D))
    x = rng.standard_normal((B, D))
    h = 1e-6
    fd = (cell.f(p + h, x) - cell.f(p - h, x)) / (2 * h)   # channels are independent
    np.testing.assert_allclose(cell.jac_diag(p, x), fd, rtol=0, atol=1e-9)
    J = cell.jac(p, x)
    assert np.all(J - np.einsum("bi,ij->bij", cell.jac_diag(p, x), np.eye(D)) == 0)


# ---------------------------------------------------------------- linear recurrence

def _brute_force_affine(v, p, A, s0):
    """s^_t = sum_{tau<=t} (A_t..A_{tau+1}) c_tau + (A_t..A_1) s0, c = v - A p."""
    B, T, D = v.shape
    dense = A.ndim == 4
    Am = A if dense else np.einsum("btd,de->btde", A, np.eye(D))
    c = v - np.einsum("btij,btj->bti", Am, p)
    out = np.zeros_like(v)
    for b in range(B):
        for t in range(T):
            acc = np.zeros(D)
            for tau in range(-1, t + 1):
                M = np.eye(D)
                for u in range(tau + 1, t + 1):
                    M = Am[b, u] @ M
                acc += M @ (s0[b] if tau == -1 else c[b, tau])
            out[b, t] = acc
    return out


@pytest.mark.parametrize("dense", [False, True])
def test_affine_recurrence_brute_force(dense):
    B, T, D = 2, 7, 3
    rng = np.random.default_rng(7)
    v = rng.standard_normal((B, T, D))
    p = rng.standard_normal((B, T, D))
    A = rng.standard_normal((B, T, D, D) if dense else (B, T, D)) * 0.8
    s0 = rng.standard_normal((B, D))
    np.testing.assert_allclose(oracle.affine_recurrence(v, p, A, s0),
                               _brute_force_affine(v, p, A, s0), rtol=0, atol=1e-12)


def test_affine_combine_is_associative():
    # The scan element is the affine map y -> A y + c; composing "later after
    # earlier" is (A_l A_e, A_l c_e + c_l) [PN §2.1].  Check associativity and
    # that folding the elements reproduces the recurrence.
    rng = np.random.default_rng(8)
    D = 4

    def comb(e, l):
        return (l[0] @ e[0], l[0] @ e[1] + l[1])

    els = [(rng.standard_normal((D, D)), rng.standard_normal(D)) for _ in range(3)]
    a = comb(comb(els[0], els[1]), els[2])
    b = comb(els[0], comb(els[1], els[2]))
    np.testing.assert_allclose(a[0], b[0], atol=1e-13)
    np.testing.assert_allclose(a[1], b[1], atol=1e-13)
    y0 = rng.standard_normal(D)
    y = y0
    for A, c in els:
        y = A @ y + c
    np.testing.assert_allclose(a[0] @ y0 + a[1], y, atol=1e-13)


def test_picard_recurrence_is_a_cumulative_sum():
    # A~ = I turns the recurrence into s0 + cumsum(v - p) [PN §2.2.3, §4.1].
    B, T, D = 3, 50, 4
    rng = np.random.default_rng(9)
    v, p = rng.standard_normal((2, B, T, D))
    s0 = rng.standard_normal((B, D))
    ref = s0[:, None] + torch.cumsum(torch.from_numpy(v - p), dim=1).numpy()
    np.testing.assert_allclose(oracle.affine_recurrence(v, p, np.ones((B, T, D)), s0), ref,
                               rtol=0, atol=1e-12)


# ---------------------------------------------------------------- the update itself

def _dense_update(cell, x, s0, s, mode, bandwidth=1):
    """s - J~^{-1} F(s) with J~ assembled as a (T*D)x(T*D) matrix per batch row
    and solved by numpy.linalg.solve, straight from the update equation [PN §1.2]."""
    B, T, D = s.shape
    p = osv.shift(s, s0)
    F = s - cell.f(p, x)
    A = osv.jacobian_approx(mode, cell, p, x, bandwidth)
    if A.ndim == 3:
        A = np.einsum("btd,de->btde", A, np.eye(D))
    out = np.empty_like(s)
    for b in range(B):
        J = np.eye(T * D)
        for t in range(1, T):
            J[t * D:(t + 1) * D, (t - 1) * D:t * D] = -A[b, t]
        out[b] = (s[b].ravel() - np.linalg.solve(J, F[b].ravel())).reshape(T, D)
    return out


@pytest.mark.parametrize("kind", [oracle.CELL_TANH_RNN, oracle.CELL_GRU, oracle.CELL_DIAG_TANH])
@pytest.mark.parametrize("mode", [oracle.JACOBI, oracle.PICARD, oracle.QUASI_NEWTON, oracle.NEWTON])
def test_update_equals_linear_solve_of_the_stacked_system(kind, mode):
    D, m, B, T = 4, 3, 2, 9
    if kind == oracle.CELL_DIAG_TANH:
        m = D
    rng = np.random.default_rng(10 + kind * 4 + mode)
    params = workloads.random_cell_params(kind, D, m, rng, 1.5).astype(np.float64)
    cell = oracle.make_cell(kind, params, D, m)
    x = rng.standard_normal((B, T, m))
    s0 = rng.standard_normal((B, D)) * 0.3
    s = rng.standard_normal((B, T, D)) * 0.5
    np.testing.assert_allclose(oracle.newton_step(cell, x, s0, s, mode),
                               _dense_update(cell, x, s0, s, mode), rtol=0, atol=1e-11)


@pytest.mark.parametrize("kind", [oracle.CELL_TANH_RNN, oracle.CELL_GRU])
@pytest.mark.parametrize("k", [0, 1, 2])
def test_banded_update_equals_linear_solve(kind, k):
    D, m, B, T = 5, 3, 2, 8
    rng = np.random.default_rng(50 + kind * 3 + k)
    params = workloads.random_cell_params(kind, D, m, rng, 1.5).astype(np.float64)
    cell = oracle.make_cell(kind, params, D, m)
    x = rng.standard_normal((B, T, m))
    s0 = rng.standard_normal((B, D)) * 0.3
    s = rng.standard_normal((B, T, D)) * 0.5
    np.testing.assert_allclose(oracle.newton_step(cell, x, s0, s, oracle.BANDED, k),
                               _dense_update(cell, x, s0, s, oracle.BANDED, k), rtol=0, atol=1e-11)


def test_band_limits_reduce_to_quasi_newton_and_newton():
    # [PN §2.2.2] sits between the diagonal approximation and the full Jacobian
    D, m, B, T = 6, 3, 2, 30
    rng = np.random.default_rng(60)
    params = workloads.random_cell_params(oracle.CELL_GRU, D, m, rng, 2.0).astype(np.float64)
    cell = oracle.make_cell(oracle.CELL_GRU, params, D, m)
    x = rng.standard_normal((B, T, m))
    s0 = np.zeros((B, D))
    s = rng.standard_normal((B, T, D)) * 0.4
    np.testing.assert_array_equal(oracle.newton_step(cell, x, s0, s, oracle.BANDED, 0),
                                  oracle.newton_step(cell, x, s0, s, oracle.QUASI_NEWTON))
    np.testing.assert_array_equal(oracle.newton_step(cell, x, s0, s, oracle.BANDED, D - 1),
                                  oracle.newton_step(cell, x, s0, s, oracle.NEWTON))
    J = rng.standard_normal((3, D, D))
    Bk = oracle.band(J, 1)
    for i in range(D):
        for j in range(D):
            assert Bk[0, i, j] == (J[0, i, j] if abs(i - j) <= 1 else 0.0)
    # more band, fewer updates (on this locally coupled example)
    its = [oracle.solve(oracle.CELL_GRU, params, x, s0, oracle.BANDED, 1e-9, T, bandwidth=k).iters
           for k in (0, 2, D - 1)]
    assert its[0] >= its[1] >= its[2]


def test_banded_is_exact_newton_on_a_banded_lattice():
    # A tanh RNN whose W couples only units within distance k has a Jacobian
    # diag(c) W inside the band, so the banded update is the Newton update and
    # converges as fast.
    D, m, B, T, k = 7, 2, 2, 40, 2
    rng = np.random.default_rng(70)
    i = np.arange(D)
    W = np.where(np.abs(i[:, None] - i[None, :]) <= k, rng.standard_normal((D, D)), 0.0) * 0.4
    U = rng.standard_normal((D, m))
    params = np.concatenate([W.ravel(), U.ravel(), np.zeros(D)])
    cell = oracle.make_cell(oracle.CELL_TANH_RNN, params, D, m)
    x = rng.standard_normal((B, T, m))
    s0 = np.zeros((B, D))
    s = rng.standard_normal((B, T, D)) * 0.3
    np.testing.assert_array_equal(oracle.newton_step(cell, x, s0, s, oracle.BANDED, k),
                                  oracle.newton_step(cell, x, s0, s, oracle.NEWTON))
    nb = oracle.solve(oracle.CELL_TANH_RNN, params, x, s0, oracle.BANDED, 1e-10, T, bandwidth=k)
    nn = oracle.solve(oracle.CELL_TANH_RNN, params, x, s0, oracle.NEWTON, 1e-10, T)
    assert nb.iters == nn.iters
    np.testing.assert_allclose(nb.s, oracle.sequential(cell, x, s0), rtol=0, atol=1e-10)


# ---------------------------------------------------------------- invariants from [PN §3.1]

@pytest.mark.parametrize("kind", [oracle.CELL_TANH_RNN, oracle.CELL_GRU, oracle.CELL_DIAG_TANH])
@pytest.mark.parametrize("mode", [oracle.JACOBI, oracle.PICARD, oracle.QUASI_NEWTON, oracle.NEWTON,
                                  oracle.BANDED])
def test_causality_prefix_exact_and_T_step_convergence(kind, mode):
    # After i undamped updates the first i states equal the sequential ones,
    # so every method has converged after at most T updates.
    D, m, B, T = 3, 2, 2, 8
    if kind == oracle.CELL_DIAG_TANH:
        m = D
    rng = np.random.default_rng(30 + kind * 4 + mode)
    params = workloads.random_cell_params(kind, D, m, rng, 2.0).astype(np.float64)
    cell = oracle.make_cell(kind, params, D, m)
    x = rng.standard_normal((B, T, m))
    s0 = rng.standard_normal((B, D)) * 0.3
    seq = oracle.sequential(cell, x, s0)
    s = np.broadcast_to(s0[:, None], (B, T, D)).copy()
    for i in range(1, T + 1):
        s = oracle.newton_step(cell, x, s0, s, mode)
        if mode == oracle.JACOBI:
            assert np.array_equal(s[:, :i], seq[:, :i])
        else:
            np.testing.assert_allclose(s[:, :i], seq[:, :i], rtol=0, atol=1e-12)
    res = oracle.solve(kind, params, x, s0, mode, 1e-12, T)
    assert res.status == oracle.OK and res.iters <= T
    assert oracle.residual_inf(cell, x, s0, res.s) <= 1e-12


def test_picard_exact_jacobian_case():
    # f_t(s) = s + c_t has A_t = I exactly, so one Picard update is exact.
    class Shift:
        D, m, dtype = 3, 3, np.float64

        def f(self, p, x):
            return p + x

        def jac_diag(self, p, x):
            return np.ones_like(p)

        def jac(self, p, x):
            return np.broadcast_to(np.eye(3), p.shape + (3,)).copy()

    cell = Shift()
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2, 12, 3))
    s0 = rng.standard_normal((2, 3))
    s = np.broadcast_to(s0[:, None], (2, 12, 3)).copy()
    s1 = oracle.newton_step(cell, x, s0, s, oracle.PICARD)
    np.testing.assert_allclose(s1, oracle.sequential(cell, x, s0), atol=1e-13)


def test_newton_on_affine_maps_converges_in_one_update_and_jacobi_on_constants():
    D, T, B = 3, 10, 2
    rng = np.random.default_rng(12)
    A = rng.standard_normal((D, D)) * 0.9

    class Affine:
        dtype = np.float64

        def __init__(self, A):
            self.A, self.D, self.m = A, A.shape[0], A.shape[0]

        def f(self, p, x):
            return p @ self.A.T + x

        def jac(self, p, x):
            return np.broadcast_to(self.A, p.shape + (self.D,)).copy()

        def jac_diag(self, p, x):
            return np.broadcast_to(np.diagonal(self.A), p.shape).copy()

    x = rng.standard_normal((B, T, D))
    s0 = rng.standard_normal((B, D))
    s = np.broadcast_to(s0[:, None], (B, T, D)).copy()
    cell = Affine(A)
    seq = oracle.sequential(cell, x, s0)
    np.testing.assert_allclose(oracle.newton_step(cell, x, s0, s, oracle.NEWTON), seq, atol=1e-12)
    const = Affine(np.zeros((D, D)))     # f_t = c_t
    np.testing.assert_array_equal(oracle.newton_step(const, x, s0, s, oracle.JACOBI),
                                  oracle.sequential(const, x, s0))


def test_quasi_newton_equals_newton_for_channelwise_cell():
    wl = workloads.make(3, B=2, T=512)
    a = [oracle.solve(wl["cell"], wl["params"], wl["x"], wl["s0"], md, 1e-10, 512)
         for md in (oracle.QUASI_NEWTON, oracle.NEWTON)]
    assert a[0].iters == a[1].iters and a[0].status == a[1].status == oracle.OK
    np.testing.assert_array_equal(a[0].s, a[1].s)


def test_newton_converges_quadratically_quasi_newton_linearly():
    wl = workloads.make(2, B=4, T=256)
    rn = oracle.solve(wl["cell"], wl["params"], wl["x"], wl["s0"], oracle.NEWTON, 1e-13, 256)
    rq = oracle.solve(wl["cell"], wl["params"], wl["x"], wl["s0"], oracle.QUASI_NEWTON, 1e-11, 256)
    h = rn.hist[0]
    # consecutive residuals above the float64 floor
    pairs = [(h[i], h[i + 1]) for i in range(len(h) - 1) if h[i + 1] > 1e-13 and h[i] < 0.5]
    assert pairs, h
    for r0, r1 in pairs:
        assert r1 <= 5.0 * r0 * r0, h
    hq = np.array(rq.hist[0])
    ratios = hq[3:-1][1:] / hq[3:-1][:-1]
    assert ratios.max() < 0.9 and ratios.min() > 1e-3, hq   # linear, not quadratic
    assert len(hq) > len(h)


def test_damping_scales_the_step_and_keeps_the_fixed_point():
    D, m, B, T = 4, 3, 2, 12
    rng = np.random.default_rng(13)
    params = workloads.random_cell_params(oracle.CELL_GRU, D, m, rng, 1.5).astype(np.float64)
    cell = oracle.make_cell(oracle.CELL_GRU, params, D, m)
    x = rng.standard_normal((B, T, m))
    s0 = np.zeros((B, D))
    lam = 0.5
    r1 = oracle.solve(oracle.CELL_GRU, params, x, s0, oracle.QUASI_NEWTON, 0, 1, damping=lam)
    s_init = np.zeros((B, T, D))
    step = oracle.newton_step(cell, x, s0, s_init, oracle.QUASI_NEWTON) - s_init
    np.testing.assert_allclose(r1.s - s_init, lam * step, rtol=0, atol=1e-15)
    r = oracle.solve(oracle.CELL_GRU, params, x, s0, oracle.QUASI_NEWTON, 1e-12, 400, damping=lam)
    assert r.status == oracle.OK
    np.testing.assert_allclose(r.s, oracle.sequential(cell, x, s0), atol=1e-11)


def test_windows_chain_and_full_window_is_identical():
    wl = workloads.make(2, B=3, T=300)
    args = (wl["cell"], wl["params"], wl["x"], wl["s0"], oracle.QUASI_NEWTON, 1e-7, 300)
    full = oracle.solve(*args)
    same = oracle.solve(*args, window=300)
    np.testing.assert_array_equal(full.s, same.s)
    assert full.iters == same.iters
    win = oracle.solve(*args, window=64)
    assert len(win.window_iters) == 5 and win.iters == sum(win.window_iters)
    cell = oracle.make_cell(wl["cell"], wl["params"], wl["D"], wl["m"])
    assert oracle.residual_inf(cell, wl["x"].astype(np.float64), wl["s0"].astype(np.float64),
                               win.s) <= 1e-7


# ---------------------------------------------------------------- binary16 storage [PN §2.3]

def test_f16_storage_jacobi_reaches_the_stored_sequential_trajectory():
    # T Jacobi updates (causality) reach the fixed point of the stored map: the
    # sequence s_t = f16(f(s_{t-1})), evaluated here step by step, bit for bit.
    # The residual |s_t - f(s_{t-1})| keeps the rounding error, so tol 0 is
    # never met and the cap stops the solve.
    wl = workloads.make(3, B=2, T=200)
    x16 = wl["x"].astype(np.float16).astype(np.float32)
    cell = oracle.make_cell(wl["cell"], wl["params"], wl["D"], wl["m"])
    prev = wl["s0"].astype(np.float64)
    ref = np.empty((2, 200, wl["D"]))
    for t in range(200):
        prev = cell.f(prev, x16[:, t].astype(np.float64)).astype(np.float16).astype(np.float64)
        ref[:, t] = prev
    r = oracle.solve(wl["cell"], wl["params"], x16, wl["s0"], oracle.JACOBI, 0.0, 200,
                     storage="f16")
    assert r.status == oracle.NOT_CONVERGED and r.iters == 200
    np.testing.assert_array_equal(r.s, ref)
    assert 0 < r.hist[0][-1] <= 2.0 ** -12      # half a binary16 ulp below 1


def test_f16_storage_stores_binary16_and_stays_near_the_float_solution():
    wl = workloads.make(3, B=2, T=2000)
    x16 = wl["x"].astype(np.float16).astype(np.float32)
    h = oracle.solve(wl["cell"], wl["params"], x16, wl["s0"], oracle.QUASI_NEWTON, 1e-3, 2000,
                     storage="f16")
    f = oracle.solve(wl["cell"], wl["params"], x16, wl["s0"], oracle.QUASI_NEWTON, 1e-9, 2000)
    assert h.status == oracle.OK
    np.testing.assert_array_equal(h.s, h.s.astype(np.float16).astype(np.float64))
    # the stored fixed point differs from the float one by rounding, damped by
    # the contraction |a| < 1: a few binary16 ulps (2^-11 below 1)
    assert np.max(np.abs(h.s - f.s)) <= 8 * 2.0 ** -11
    # K = 0 returns s0 as stored
    z = oracle.solve(wl["cell"], wl["params"], x16, wl["s0"] + 0.1, oracle.QUASI_NEWTON, 10.0, 2000,
                     storage="f16")
    assert z.iters == 0
    np.testing.assert_array_equal(z.s[0, 0], (wl["s0"][0] + 0.1).astype(np.float16).astype(np.float64))


# ---------------------------------------------------------------- switching [PN §5.3]

def test_switching_replays_the_mode_sequence_by_hand():
    # rho = 0 switches at check 1: updates 0 and 1 use the first mode, the rest
    # the second; the run equals those updates applied one by one
    wl = workloads.make(2, B=2, T=64)
    cell = oracle.make_cell(wl["cell"], wl["params"], wl["D"], wl["m"])
    x, s0 = wl["x"].astype(np.float64), wl["s0"].astype(np.float64)
    r = oracle.solve(wl["cell"], wl["params"], wl["x"], wl["s0"], oracle.QUASI_NEWTON, 1e-9, 64,
                     switch_mode=oracle.NEWTON, switch_ratio=0.0)
    assert r.status == oracle.OK and r.window_switch == [1]
    s = np.broadcast_to(s0[:, None], x.shape[:2] + (wl["D"],)).copy()
    for k in range(r.iters):
        s = oracle.newton_step(cell, x, s0, s, oracle.QUASI_NEWTON if k <= 1 else oracle.NEWTON)
    np.testing.assert_array_equal(r.s, s)
    # rho = inf never switches: the plain first-mode solve
    q = oracle.solve(wl["cell"], wl["params"], wl["x"], wl["s0"], oracle.QUASI_NEWTON, 1e-9, 64)
    n = oracle.solve(wl["cell"], wl["params"], wl["x"], wl["s0"], oracle.QUASI_NEWTON, 1e-9, 64,
                     switch_mode=oracle.NEWTON, switch_ratio=np.inf)
    assert n.window_switch == [-1] and n.iters == q.iters
    np.testing.assert_array_equal(n.s, q.s)
    # forcing the decision reproduces it; forcing "never" is the plain solve
    f = oracle.solve(wl["cell"], wl["params"], wl["x"], wl["s0"], oracle.QUASI_NEWTON, 1e-9, 64,
                     switch_mode=oracle.NEWTON, switch_ratio=0.0, force_switch=[1])
    np.testing.assert_array_equal(f.s, r.s)
    g = oracle.solve(wl["cell"], wl["params"], wl["x"], wl["s0"], oracle.QUASI_NEWTON, 1e-9, 64,
                     switch_mode=oracle.NEWTON, switch_ratio=0.0, force_switch=[-1])
    np.testing.assert_array_equal(g.s, q.s)


def test_switching_on_stagnation_saves_fine_updates():
    # the lattice workload: the first diagonal updates stall (r grows), the
    # switch moves to the band, which then converges like the band alone
    wl = workloads.make(6, B=2, T=512)
    args = (wl["cell"], wl["params"], wl["x"], wl["s0"])
    b = oracle.solve(*args, oracle.BANDED, 1e-6, 512, bandwidth=2)
    a = oracle.solve(*args, oracle.QUASI_NEWTON, 1e-6, 512, bandwidth=2,
                     switch_mode=oracle.BANDED, switch_ratio=0.5)
    assert a.status == b.status == oracle.OK
    sw = a.window_switch[0]
    assert sw >= 1 and a.hist[0][sw] > 0.5 * a.hist[0][sw - 1]
    assert all(a.hist[0][k] <= 0.5 * a.hist[0][k - 1] for k in range(1, sw))
    assert a.iters - (sw + 1) < b.iters          # fewer updates in the costly mode
    cell = oracle.make_cell(wl["cell"], wl["params"], wl["D"], wl["m"])
    np.testing.assert_allclose(a.s, oracle.sequential(cell, wl["x"].astype(np.float64),
                                                      wl["s0"].astype(np.float64)), atol=1e-5)
    # every window starts on the first mode
    w = oracle.solve(*args, oracle.QUASI_NEWTON, 1e-6, 128, window=128, bandwidth=2,
                     switch_mode=oracle.BANDED, switch_ratio=0.5)
    assert len(w.window_switch) == 4 and all(k >= 1 for k in w.window_switch)


def _error_operators(A, T):
    """Error maps of one undamped update on the affine cell f(p) = A p + x,
    acting on the stacked trajectory error e = s - s* (T blocks of D; s0 is
    exact): Jacobi e -> S_A e, quasi-Newton e -> (I - S_dg)^-1 (S_A - S_dg) e,
    where S_M puts M e_{t-1} in block t and dg is diag(A)."""
    D = A.shape[0]

    def shift(M):
        S = np.zeros((T * D, T * D))
        for t in range(1, T):
            S[t * D:(t + 1) * D, (t - 1) * D:t * D] = M
        return S

    SA, Sd = shift(A), shift(np.diag(np.diagonal(A)))
    I = np.eye(T * D)
    return SA, np.linalg.solve(I - Sd, SA - Sd)


def test_damping_switch_closed_form_on_an_affine_cell():
    # Jacobi with damping lam1 until the switch, then quasi-Newton with lam2:
    # the error after K updates is N2^(K-sw-1) N1^(sw+1) e0 with
    # N = (1 - lam) I + lam G for the mode's error map G
    rng = np.random.default_rng(41)
    D, T = 3, 6
    A = 0.6 * rng.standard_normal((D, D))
    cell = _Affine(A)
    x = rng.standard_normal((1, T, D))
    s0 = rng.standard_normal((1, D))
    star = np.empty((T, D))
    prev = s0[0]
    for t in range(T):
        prev = A @ prev + x[0, t]
        star[t] = prev
    e0 = (np.broadcast_to(s0[0], (T, D)) - star).reshape(-1)
    GJ, GQ = _error_operators(A, T)
    I = np.eye(T * D)
    lam1, lam2 = 0.8, 0.45
    N1, N2 = (1 - lam1) * I + lam1 * GJ, (1 - lam2) * I + lam2 * GQ
    for forced, K in [(None, 7), (3, 9), (1, 2)]:
        # rho = 0 switches at check 1 (r_1 > 0); forced replaces the decision
        s, k, _, hist, sw = osv._solve_window(cell, x, s0, oracle.JACOBI, 0.0, 100, lam1, K, 1,
                                              (oracle.QUASI_NEWTON, 0.0, forced, lam2))
        assert k == K and sw == (1 if forced is None else forced)
        n1 = min(K, sw + 1)
        want = np.linalg.matrix_power(N2, K - n1) @ np.linalg.matrix_power(N1, n1) @ e0
        np.testing.assert_allclose((s[0] - star).reshape(-1), want, rtol=0, atol=1e-12)
    # no second damping: the switch keeps lam1
    s, _, _, _, sw = osv._solve_window(cell, x, s0, oracle.JACOBI, 0.0, 100, lam1, 5, 1,
                                       (oracle.QUASI_NEWTON, 0.0, None, None))
    N2k = (1 - lam1) * I + lam1 * GQ
    want = np.linalg.matrix_power(N2k, 3) @ np.linalg.matrix_power(N1, 2) @ e0
    np.testing.assert_allclose((s[0] - star).reshape(-1), want, rtol=0, atol=1e-12)


def test_damping_switch_replays_by_hand():
    # rho = 0: updates 0 and 1 are undamped quasi-Newton, the rest damped Newton
    wl = workloads.make(2, B=2, T=48)
    cell = oracle.make_cell(wl["cell"], wl["params"], wl["D"], wl["m"])
    x, s0 = wl["x"].astype(np.float64), wl["s0"].astype(np.float64)
    r = oracle.solve(wl["cell"], wl["params"], wl["x"], wl["s0"], oracle.QUASI_NEWTON, 1e-9, 64,
                     switch_mode=oracle.NEWTON, switch_ratio=0.0, switch_damping=0.5)
    assert r.status == oracle.OK and r.window_switch == [1] and r.iters > 3
    s = np.broadcast_to(s0[:, None], x.shape[:2] + (wl["D"],)).copy()
    for k in range(r.iters):
        if k <= 1:
            s = oracle.newton_step(cell, x, s0, s, oracle.QUASI_NEWTON)
        else:
            s = 0.5 * s + 0.5 * oracle.newton_step(cell, x, s0, s, oracle.NEWTON)
    np.testing.assert_allclose(r.s, s, rtol=0, atol=1e-13)


def test_damping_switch_identities_and_fixed_point():
    wl = workloads.make(2, B=2, T=96)
    args = (wl["cell"], wl["params"], wl["x"], wl["s0"], oracle.QUASI_NEWTON, 1e-7, 96)
    q = oracle.solve(*args)
    # the same mode and no second damping (or the same one): the plain solve
    for lam2 in (None, 1.0):
        r = oracle.solve(*args, switch_mode=oracle.QUASI_NEWTON, switch_ratio=0.0,
                         switch_damping=lam2)
        assert r.window_switch == [1] and r.iters == q.iters
        np.testing.assert_array_equal(r.s, q.s)
    # a damping switch moves no fixed point: still the sequential trajectory
    cell = oracle.make_cell(wl["cell"], wl["params"], wl["D"], wl["m"])
    seq = oracle.sequential(cell, wl["x"].astype(np.float64), wl["s0"].astype(np.float64))
    d = oracle.solve(*args, switch_mode=oracle.QUASI_NEWTON, switch_ratio=0.0, switch_damping=0.6)
    assert d.status == oracle.OK and d.iters > q.iters
    np.testing.assert_allclose(d.s, seq, rtol=0, atol=1e-6)
    # the step after the switch is 0.6 of the undamped one (the damping identity)
    f2 = oracle.solve(*args, force_iters=[2])
    f3 = oracle.solve(*args, switch_mode=oracle.QUASI_NEWTON, switch_ratio=0.0,
                      switch_damping=0.6, force_iters=[3])
    full = oracle.newton_step(cell, wl["x"].astype(np.float64), wl["s0"].astype(np.float64),
                              f2.s, oracle.QUASI_NEWTON)
    np.testing.assert_allclose(f3.s - f2.s, 0.6 * (full - f2.s), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- advancing window [PN §1.3.1]

class _Affine:
    """f_t(p) = A p + x_t (m = D)."""
    dtype = np.float64

    def __init__(self, A):
        self.A, self.D, self.m = A, A.shape[0], A.shape[0]

    def f(self, p, x):
        return p @ self.A.T + x

    def jac(self, p, x):
        return np.broadcast_to(self.A, p.shape + (self.D,)).copy()

    def jac_diag(self, p, x):
        return np.broadcast_to(np.diagonal(self.A), p.shape).copy()


def test_advancing_window_hand_traced_jacobi_case():
    # f_t(p) = p/2 + 1, s0 = 0, T = 3, W = 2, tol = 0, traced by hand:
    #   round 0: window [0,2) = (0, 0), r_t = (1, 1), nothing accepted; Jacobi -> (1, 1)
    #   round 1: r = (0, 0.5): accept t=0; window [1,3), new step 2 starts at 1;
    #            update from s_0 = 1 -> (1.5, 1.5)
    #   round 2: r = (0, 0.25): accept t=1; window [2,3); update from 1.5 -> 1.75
    #   round 3: r = (0,): accept t=2 -> done after 3 updates
    cell = _Affine(np.array([[0.5]]))
    x = np.ones((1, 3, 1))
    r = oracle.solve_advancing(cell, x, np.zeros((1, 1)), oracle.JACOBI, 0.0, 100, 2)
    assert r.status == oracle.OK and r.iters == 3 and r.window_iters == [3]
    np.testing.assert_array_equal(r.s[0, :, 0], [1.0, 1.5, 1.75])
    np.testing.assert_array_equal(r.hist[0], [1.0, 0.5, 0.25, 0.0])
    assert r.accepted == [0, 1, 1, 1]
    # forcing the same decisions reproduces the run; forcing fewer acceptances
    # costs updates but reaches the same trajectory
    f = oracle.solve_advancing(cell, x, np.zeros((1, 1)), oracle.JACOBI, 0.0, 100, 2,
                               force_accept=[0, 1, 1, 1], keep_round_resid=True)
    np.testing.assert_array_equal(f.s, r.s)
    assert [list(v) for v in f.round_resid] == [[1.0, 1.0], [0.0, 0.5], [0.0, 0.25], [0.0]]
    g = oracle.solve_advancing(cell, x, np.zeros((1, 1)), oracle.JACOBI, 0.0, 100, 2,
                               force_accept=[0, 0, 1, 1, 1])
    assert g.iters == 4 and g.accepted == [0, 0, 1, 1, 1]
    np.testing.assert_array_equal(g.s, r.s)


@pytest.mark.parametrize("T, W", [(10, 3), (12, 4), (7, 7), (5, 9)])
def test_advancing_window_exact_methods_take_one_update_per_window(T, W):
    # Newton on affine maps and Picard on s + c_t solve a whole window per
    # update, so the window jumps by W every round: ceil(T / W) updates.
    rng = np.random.default_rng(17)
    D = 3
    x = rng.standard_normal((2, T, D))
    s0 = rng.standard_normal((2, D))
    for cell, mode in ((_Affine(rng.standard_normal((D, D)) * 0.5), oracle.NEWTON),
                       (_Affine(np.eye(D)), oracle.PICARD)):
        r = oracle.solve_advancing(cell, x, s0, mode, 1e-10, 100, W)
        assert r.status == oracle.OK and r.iters == -(-T // W), (mode, r.iters)
        np.testing.assert_allclose(r.s, oracle.sequential(cell, x, s0), rtol=0, atol=1e-10)


def test_advancing_window_accepts_only_converged_steps():
    wl = workloads.make(2, B=2, T=200)
    cell = oracle.make_cell(wl["cell"], wl["params"], wl["D"], wl["m"])
    x, s0 = wl["x"].astype(np.float64), wl["s0"].astype(np.float64)
    tol = 1e-7
    for mode in (oracle.QUASI_NEWTON, oracle.JACOBI, oracle.NEWTON):
        r = oracle.solve_advancing(cell, x, s0, mode, tol, 1000, 48)
        assert r.status == oracle.OK
        # every step of the result meets the tolerance, checked step by step
        prev = s0
        for t in range(x.shape[1]):
            assert np.max(np.abs(r.s[:, t] - cell.f(prev, x[:, t]))) <= tol
            prev = r.s[:, t]
        np.testing.assert_allclose(r.s, oracle.sequential(cell, x, s0), rtol=0, atol=1e-5)
    # Jacobi accepts at least one exact step per update: at most T updates
    rj = oracle.solve_advancing(cell, x, s0, oracle.JACOBI, 0.0, 1000, 48)
    assert rj.status == oracle.OK and rj.iters <= 200
    np.testing.assert_allclose(rj.s, oracle.sequential(cell, x, s0), rtol=0, atol=1e-12)


def test_advancing_window_cap_and_nonfinite():
    cell = _Affine(np.array([[0.5]]))
    x = np.ones((1, 6, 1))
    r = oracle.solve_advancing(cell, x, np.zeros((1, 1)), oracle.JACOBI, 0.0, 2, 4)
    assert r.status == oracle.NOT_CONVERGED and r.iters == 2 and len(r.hist[0]) == 3
    assert np.all(np.isfinite(r.s))          # steps never reached hold the window's last state
    x[0, 2, 0] = np.nan
    r = oracle.solve_advancing(cell, x, np.zeros((1, 1)), oracle.JACOBI, 1e-6, 10, 4)
    assert r.status == oracle.NONFINITE and r.iters == 0


def test_residual_of_a_perturbed_trajectory():
    D, m, B, T = 3, 2, 2, 6
    rng = np.random.default_rng(14)
    params = _rnn_params(D, m, rng)
    cell = oracle.make_cell(oracle.CELL_TANH_RNN, params, D, m)
    x = rng.standard_normal((B, T, m))
    s0 = rng.standard_normal((B, D))
    seq = oracle.sequential(cell, x, s0)
    assert oracle.residual_inf(cell, x, s0, seq) <= 1e-15
    pert = seq.copy()
    pert[1, T - 1, 2] += 0.125        # last step: no downstream effect
    assert oracle.residual_inf(cell, x, s0, pert) == pytest.approx(0.125, abs=1e-15)


def test_infinite_parameters_saturate_or_poison_the_newton_jacobian():
    # IEEE arithmetic fixes the outcome: an infinite bias gives tanh = 1
    # exactly with derivative 1 - 1 = 0, so every mode reaches the sequential
    # trajectory; an infinite weight W[2][3] also gives |tanh| = 1 on channel
    # 2, but the Newton Jacobian's entry (1 - 1) x inf is NaN and poisons the
    # first update, while the diagonal Jacobian (1 - 1) x W[2][2] stays 0.
    D, m, B, T = 4, 2, 2, 30
    rng = np.random.default_rng(77)
    params = _rnn_params(D, m, rng)
    x = rng.standard_normal((B, T, m))
    s0 = 0.3 * rng.standard_normal((B, D))
    pb = params.copy()
    pb[D * D + D * m + 1] = np.inf
    cell = oracle.make_cell(oracle.CELL_TANH_RNN, pb, D, m)
    seq = oracle.sequential(cell, x, s0)
    assert np.all(seq[:, :, 1] == 1.0) and np.all(np.isfinite(seq))
    for mode in (oracle.NEWTON, oracle.QUASI_NEWTON, oracle.JACOBI):
        r = oracle.solve(oracle.CELL_TANH_RNN, pb, x, s0, mode, 1e-12, T)
        assert r.status == oracle.OK and np.max(np.abs(r.s - seq)) <= 1e-12
    pw = params.copy()
    pw[2 * D + 3] = np.inf
    with np.errstate(invalid="ignore"):
        seq = oracle.sequential(oracle.make_cell(oracle.CELL_TANH_RNN, pw, D, m), x, s0)
        assert np.all(np.abs(seq[:, :, 2]) == 1.0) and np.all(np.isfinite(seq))
        rn = oracle.solve(oracle.CELL_TANH_RNN, pw, x, s0, oracle.NEWTON, 1e-12, T)
        assert rn.status == oracle.NONFINITE and rn.iters == 1 and np.isfinite(rn.hist[0][0])
        rq = oracle.solve(oracle.CELL_TANH_RNN, pw, x, s0, oracle.QUASI_NEWTON, 1e-12, T)
    assert rq.status == oracle.OK and np.max(np.abs(rq.s - seq)) <= 1e-12


def test_stop_rule_edges():
    wl = workloads.make(2, B=2, T=40)
    a = (wl["cell"], wl["params"], wl["x"], wl["s0"], oracle.QUASI_NEWTON)
    r0 = oracle.solve(*a, 1e-5, 0)
    assert r0.status == oracle.NOT_CONVERGED and r0.iters == 0
    assert np.all(r0.s == 0)
    rbig = oracle.solve(*a, 1e9, 10)
    assert rbig.status == oracle.OK and rbig.iters == 0
    r1 = oracle.solve(*a, 0.0, 3)
    assert r1.status == oracle.NOT_CONVERGED and r1.iters == 3
    x = wl["x"].copy()
    x[1, 7, 0] = np.nan
    rn = oracle.solve(wl["cell"], wl["params"], x, wl["s0"], oracle.QUASI_NEWTON, 1e-5, 10)
    assert rn.status == oracle.NONFINITE and rn.iters == 0
    empty = oracle.solve(wl["cell"], wl["params"], wl["x"][:, :0], wl["s0"], oracle.NEWTON, 1e-5, 5)
    assert empty.status == oracle.OK and empty.iters == 0 and empty.s.shape == (2, 0, 16)
