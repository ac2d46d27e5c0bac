"""Pins of the oracle's dot-product loss and Muon (Newton-Schulz) update.

These are the pages' own inner recipe ([GRAPH] section 3.4, "The dot product
loss", "Muon optimizer for inner loop"). Each pin checks the oracle against
something other than itself: finite differences, autograd, closed forms, an SVD
construction of the Newton-Schulz map, and invariants.
"""
import numpy as np
import pytest
import torch

from oracle import (NS_COEFFS, join_theta, muon_apply, newton_schulz, split_theta, ttt_grad, ttt_loss,
                    ttt_write)


def _rng(seed):
    return np.random.default_rng(seed)


def _problem(n=40, d=4, m=8, H=1, seed=0, wscale=0.3):
    r = _rng(seed)
    K = r.standard_normal((n, H * d))
    V = r.standard_normal((n, H * d))
    theta = r.standard_normal((H, 3 * d * m)) * wscale
    return K, V, theta


# --------------------------------------------------------------------------
# dot-product loss
# --------------------------------------------------------------------------


def test_dot_gradient_matches_central_differences():
    n, d, m = 12, 4, 8
    K, V, theta = _problem(n, d, m, seed=11)
    g, L = ttt_grad(K, V, theta, 1, d, m, loss="dot")
    eps = 1e-6
    num = np.zeros(theta.size)
    for i in range(theta.size):
        tp = theta.copy().reshape(-1)
        tm = theta.copy().reshape(-1)
        tp[i] += eps
        tm[i] -= eps
        num[i] = (ttt_loss(K, V, tp, 1, d, m, loss="dot")[0] - ttt_loss(K, V, tm, 1, d, m, loss="dot")[0]) / (2 * eps)
    err = np.abs(num - g.reshape(-1)).max() / np.abs(g).max()
    assert err < 1e-7, err
    assert L[0] == pytest.approx(ttt_loss(K, V, theta, 1, d, m, loss="dot")[0], rel=1e-13)


def test_dot_gradient_matches_torch_autograd():
    n, d, m = 30, 6, 10
    K, V, theta = _problem(n, d, m, seed=12)
    g, L = ttt_grad(K, V, theta, 1, d, m, loss="dot", chunk=7)
    Wg, Wu, Wd = (torch.tensor(x, requires_grad=True) for x in split_theta(theta[0], d, m))
    Kt, Vt = torch.from_numpy(K), torch.from_numpy(V)
    Y = (torch.nn.functional.silu(Kt @ Wg) * (Kt @ Wu)) @ Wd
    loss = -(Y * Vt).sum()
    loss.backward()
    ref = join_theta(Wg.grad.numpy(), Wu.grad.numpy(), Wd.grad.numpy())
    np.testing.assert_allclose(g[0], ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())
    assert L[0] == pytest.approx(loss.item(), rel=1e-12)


def test_dot_gradient_closed_form_with_unit_gate():
    # gate fixed to 1: T(x) = x W_u W_d, L = -sum_i (k_i W_u W_d) . v_i, so
    # dL/dW_d = -(K W_u)^T V, dL/dW_u = -K^T (V W_d^T), dL/dW_g = 0.
    n, d, m = 25, 5, 7
    K, V, theta = _problem(n, d, m, seed=13)
    g, _ = ttt_grad(K, V, theta, 1, d, m, act="one", loss="dot")
    Wg, Wu, Wd = split_theta(theta[0], d, m)
    gg, gu, gd = split_theta(g[0], d, m)
    np.testing.assert_allclose(gd, -(K @ Wu).T @ V, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gu, -K.T @ (V @ Wd.T), rtol=1e-12, atol=1e-12)
    assert np.all(gg == 0.0)


def test_dot_loss_and_gradient_are_linear_in_values():
    # dL/dY = -V' carries no Y, so loss and gradient are linear in V'.
    n, d, m = 20, 4, 8
    K, V1, theta = _problem(n, d, m, seed=14)
    V2 = _rng(15).standard_normal(V1.shape)
    g1, L1 = ttt_grad(K, V1, theta, 1, d, m, loss="dot")
    g2, L2 = ttt_grad(K, V2, theta, 1, d, m, loss="dot")
    g3, L3 = ttt_grad(K, 2.0 * V1 - 3.0 * V2, theta, 1, d, m, loss="dot")
    np.testing.assert_allclose(g3, 2.0 * g1 - 3.0 * g2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(L3, 2.0 * L1 - 3.0 * L2, rtol=1e-11)


def test_dot_gradient_splits_over_chunks():
    # Eq. 5: the full gradient is the sum of per-minibatch gradients.
    n, d, m = 33, 4, 8
    K, V, theta = _problem(n, d, m, seed=16)
    g, L = ttt_grad(K, V, theta, 1, d, m, loss="dot")
    g1, L1 = ttt_grad(K[:10], V[:10], theta, 1, d, m, loss="dot")
    g2, L2 = ttt_grad(K[10:], V[10:], theta, 1, d, m, loss="dot")
    np.testing.assert_allclose(g, g1 + g2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L, L1 + L2, rtol=1e-12)


# --------------------------------------------------------------------------
# Newton-Schulz / Muon
# --------------------------------------------------------------------------


def _quintic_iterate(x, steps):
    a, b, c = NS_COEFFS
    for _ in range(steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


@pytest.mark.parametrize("shape", [(16, 32), (64, 128), (128, 64), (5, 5)])
def test_newton_schulz_equals_quintic_on_singular_values(shape):
    # In the singular basis of G = U diag(s) V^T every step maps each singular
    # value by the same odd quintic, so NS(G) = U diag(phi(s / ||G||_F)) V^T.
    G = _rng(20).standard_normal(shape)
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    x0 = s / (np.sqrt(np.sum(s * s)) + 1e-7)
    ref = U @ np.diag(_quintic_iterate(x0, 5)) @ Vt
    np.testing.assert_allclose(newton_schulz(G, 5), ref, rtol=1e-10, atol=1e-12)
    # other step counts use the same map
    ref3 = U @ np.diag(_quintic_iterate(x0, 3)) @ Vt
    np.testing.assert_allclose(newton_schulz(G, 3), ref3, rtol=1e-10, atol=1e-12)


def test_newton_schulz_transpose_and_scale():
    G = _rng(21).standard_normal((64, 128))
    np.testing.assert_allclose(newton_schulz(G.T), newton_schulz(G).T, rtol=1e-12, atol=1e-14)
    # the Frobenius normalisation makes the result independent of a positive scale
    np.testing.assert_allclose(newton_schulz(1e3 * G), newton_schulz(G), rtol=1e-6, atol=1e-9)
    assert np.all(newton_schulz(np.zeros((4, 8))) == 0.0)


def test_newton_schulz_output_band():
    # Published behaviour of these coefficients: five steps send every singular
    # value of a normalised matrix that is not tiny (here down to 1e-2 of the
    # largest) into roughly [0.7, 1.2] rather than exactly to 1.
    r = _rng(22)
    U, _ = np.linalg.qr(r.standard_normal((64, 64)))
    Vq, _ = np.linalg.qr(r.standard_normal((128, 64)))
    s = np.geomspace(1.0, 1e-2, 64)
    G = U @ np.diag(s) @ Vq.T
    sv = np.linalg.svd(newton_schulz(G, 5), compute_uv=False)
    assert sv.min() > 0.65 and sv.max() < 1.25, (sv.min(), sv.max())


def test_muon_step_is_a_descent_step_to_first_order():
    # <g, NS(g)> = sum_i s_i phi(s_i) > 0 for each matrix, so a small Muon step
    # lowers the loss, at the first-order rate lr * <g, update>.
    n, d, m = 40, 4, 8
    for loss in ("dot", "mse"):
        K, V, theta = _problem(n, d, m, seed=23)
        g, L0 = ttt_grad(K, V, theta, 1, d, m, loss=loss)
        upd = (theta - muon_apply(theta, g, 1.0, 1, d, m)).reshape(-1)
        slope = float(g.reshape(-1) @ upd)
        assert slope > 0
        ratios = []
        for lr in (1e-3, 1e-4, 1e-5):
            L1 = ttt_loss(K, V, muon_apply(theta, g, lr, 1, d, m), 1, d, m, loss=loss)
            ratios.append((L0[0] - L1[0]) / (lr * slope))
        assert abs(ratios[-1] - 1.0) < 1e-3, ratios
        assert abs(ratios[-1] - 1.0) < abs(ratios[0] - 1.0) + 1e-12


def test_muon_orthogonalises_each_matrix_of_each_head():
    d, m, H = 8, 16, 3
    r = _rng(24)
    theta = r.standard_normal((H, 3 * d * m))
    g = r.standard_normal((H, 3 * d * m))
    out = muon_apply(theta, g, 0.5, H, d, m)
    for h in range(H):
        for G, O in zip(split_theta(g[h], d, m), split_theta((theta[h] - out[h]) / 0.5, d, m)):
            U, s, Vt = np.linalg.svd(G, full_matrices=False)
            x0 = s / (np.sqrt(np.sum(s * s)) + 1e-7)
            np.testing.assert_allclose(O, U @ np.diag(_quintic_iterate(x0, 5)) @ Vt, rtol=1e-9, atol=1e-12)


def test_write_with_muon_composes_steps():
    n, d, m, H = 30, 4, 8, 2
    K, V, theta = _problem(n, d, m, H=H, seed=25)
    th2, losses, grads = ttt_write(K, V, theta, H, d, m, lr=0.1, steps=2, loss="dot", opt="muon")
    th1, _, _ = ttt_write(K, V, theta, H, d, m, lr=0.1, steps=1, loss="dot", opt="muon")
    th11, _, _ = ttt_write(K, V, th1, H, d, m, lr=0.1, steps=1, loss="dot", opt="muon")
    np.testing.assert_allclose(th2, th11, rtol=1e-13, atol=1e-15)
    # the dot loss falls over the two steps
    assert losses[1].sum() < losses[0].sum()
