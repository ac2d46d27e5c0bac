"""Pins of the oracle's TTT write/read (CPU only).

Write objective and read: paper-graph summary "VGG-T3: Offline Feed-Forward 3D
Reconstruction at Scale", section 3.4, Eq. 3 (argmin over theta of a sum of
per-token losses) and Eq. 4 (o_i = T_theta(q_i)); SwiGLU fast-weight MLP from
"TTT MLP Architecture and Inner Optimization"; Eq. 5 minibatch gradient sum from
"Large-Scale Inference Strategies".
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (head_grad, join_theta, split_theta, swiglu_forward, ttt_grad, ttt_loss,
                    ttt_read, ttt_write)


def _rng(seed):
    return np.random.default_rng(seed)


def _problem(n=40, d=4, m=8, H=1, seed=0, wscale=0.3):
    r = _rng(seed)
    K = r.standard_normal((n, H * d))
    V = r.standard_normal((n, H * d))
    theta = r.standard_normal((H, 3 * d * m)) * wscale
    return K, V, theta


def test_handworked_scalar_swiglu(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "swiglu_scalar_handworked.json")))
    env = {"log": math.log}
    Wg = np.array([[eval(g["W_g_expr"], env)]])
    Wu = np.array([[g["W_u"]]])
    Wd = np.array([[g["W_d"]]])
    K = np.array([[g["k"]]])
    V = np.array([[g["v"]]])
    f = swiglu_forward(K, Wg, Wu, Wd)
    exp = {k: eval(v, env) for k, v in g["expected_expr"].items()}
    assert f["Y"][0, 0] == pytest.approx(exp["Y"], rel=1e-14)
    L, gg, gu, gd = head_grad(K, V, Wg, Wu, Wd)
    assert L == pytest.approx(exp["loss"], rel=1e-13)
    assert gd[0, 0] == pytest.approx(exp["g_Wd"], rel=1e-13)
    assert gu[0, 0] == pytest.approx(exp["g_Wu"], rel=1e-13)
    assert gg[0, 0] == pytest.approx(exp["g_Wg"], rel=1e-13)


def test_swiglu_special_values_and_torch_silu():
    r = _rng(1)
    X = r.standard_normal((30, 5))
    Wg, Wu, Wd = r.standard_normal((5, 7)), r.standard_normal((5, 7)), r.standard_normal((7, 5))
    # W_g = 0 -> silu(0) = 0 -> T = 0
    assert np.all(swiglu_forward(X, np.zeros_like(Wg), Wu, Wd)["Y"] == 0.0)
    # sigmoid(0) = 1/2
    assert np.all(swiglu_forward(X, np.zeros_like(Wg), Wu, Wd)["S"] == 0.5)
    # library cross-check: torch silu in float64
    f = swiglu_forward(X, Wg, Wu, Wd)
    Xt = torch.from_numpy(X)
    ref = (torch.nn.functional.silu(Xt @ torch.from_numpy(Wg)) * (Xt @ torch.from_numpy(Wu))) \
        @ torch.from_numpy(Wd)
    np.testing.assert_allclose(f["Y"], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_gradient_matches_central_differences():
    n, d, m = 10, 4, 8
    K, V, theta = _problem(n, d, m, seed=2)
    g, L = ttt_grad(K, V, theta, 1, d, m)
    eps = 1e-6
    num = np.zeros_like(theta)
    for i in range(theta.size):
        tp = theta.copy().reshape(-1)
        tm = theta.copy().reshape(-1)
        tp[i] += eps
        tm[i] -= eps
        num.reshape(-1)[i] = (ttt_loss(K, V, tp, 1, d, m)[0] - ttt_loss(K, V, tm, 1, d, m)[0]) / (2 * eps)
    err = np.abs(num - g).max() / np.abs(g).max()
    assert err < 1e-7, err
    assert L[0] == pytest.approx(ttt_loss(K, V, theta, 1, d, m)[0], rel=1e-14)


def test_gradient_matches_torch_autograd():
    n, d, m = 50, 6, 12
    K, V, theta = _problem(n, d, m, seed=3)
    g, L = ttt_grad(K, V, theta, 1, d, m)
    t = torch.tensor(theta[0], requires_grad=True)
    Wg, Wu, Wd = t[:d * m].view(d, m), t[d * m:2 * d * m].view(d, m), t[2 * d * m:].view(m, d)
    Kt, Vt = torch.from_numpy(K), torch.from_numpy(V)
    Y = (torch.nn.functional.silu(Kt @ Wg) * (Kt @ Wu)) @ Wd
    loss = ((Y - Vt) ** 2).sum() / d
    loss.backward()
    np.testing.assert_allclose(g[0], t.grad.numpy(), rtol=1e-11, atol=1e-13)
    assert L[0] == pytest.approx(loss.item(), rel=1e-13)


def test_one_step_closed_form_gate_one():
    """Gate fixed to 1: T(x) = x W_u W_d, so the step has a closed form."""
    n, d, m, lr = 30, 4, 6, 0.05
    K, V, theta = _problem(n, d, m, seed=4)
    Wg, Wu, Wd = split_theta(theta[0], d, m)
    R = K @ Wu @ Wd - V
    gWd = (K @ Wu).T @ ((2 / d) * R)
    gWu = K.T @ ((2 / d) * R) @ Wd.T
    exp = join_theta(Wg, Wu - lr * gWu, Wd - lr * gWd)
    th1, losses, _ = ttt_write(K, V, theta, 1, d, m, lr, 1, act="one")
    np.testing.assert_allclose(th1[0], exp, rtol=1e-12, atol=1e-14)
    assert losses[0, 0] == pytest.approx(np.sum(R * R) / d, rel=1e-13)


def test_one_step_closed_form_zero_gate_weights():
    """W_g = 0: sigmoid = 1/2 and H = 0, so only W_g moves, by
    -lr * K^T ((dY W_d^T) * U * 1/2) with dY = -(2/d) V'."""
    n, d, m, lr = 25, 5, 7, 0.1
    K, V, theta = _problem(n, d, m, seed=5)
    Wg, Wu, Wd = split_theta(theta[0], d, m)
    Wg = np.zeros_like(Wg)
    theta = join_theta(Wg, Wu, Wd)[None]
    dY = -(2 / d) * V
    exp_gWg = K.T @ ((dY @ Wd.T) * (K @ Wu) * 0.5)
    th1, _, grads = ttt_write(K, V, theta, 1, d, m, lr, 1)
    g = grads[0, 0]
    np.testing.assert_array_equal(g[d * m:], 0.0)
    np.testing.assert_allclose(g[:d * m].reshape(d, m), exp_gWg, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(th1[0], theta[0] - lr * g, rtol=0, atol=0)


def test_gate_one_descends_to_least_squares():
    """Many small steps with gate 1 approach the least-squares fit of V' on K
    (m >= d, so W_u W_d can express any d x d map)."""
    n, d, m = 60, 3, 6
    r = _rng(6)
    K = r.standard_normal((n, d))
    V = K @ r.standard_normal((d, d)) + 0.3 * r.standard_normal((n, d))
    theta = r.standard_normal((1, 3 * d * m)) * 0.3
    X, *_ = np.linalg.lstsq(K, V, rcond=None)
    Lmin = np.sum((K @ X - V) ** 2) / d
    th, losses, _ = ttt_write(K, V, theta, 1, d, m, lr=2e-3, steps=4000, act="one")
    Lend = ttt_loss(K, V, th, 1, d, m, act="one")[0]
    assert losses[0, 0] > 1.5 * Lmin
    assert Lend == pytest.approx(Lmin, rel=1e-3)
    _, Wu, Wd = split_theta(th[0], d, m)
    np.testing.assert_allclose(Wu @ Wd, X, atol=2e-2)


@pytest.mark.parametrize("lr", [1e-1, 1e-2, 1e-3])
def test_monotone_decrease(lr):
    n, d, m = 128, 16, 32
    K, V, theta = _problem(n, d, m, seed=7, wscale=0.02)
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    th1, losses, _ = ttt_write(K, V, theta, 1, d, m, lr, 1)
    assert ttt_loss(K, V, th1, 1, d, m)[0] < losses[0, 0]


def test_first_order_decrease_ratio():
    """(L(theta0) - L(theta1)) / (lr ||g||^2) -> 1 as lr -> 0."""
    n, d, m = 64, 8, 16
    K, V, theta = _problem(n, d, m, seed=8, wscale=0.1)
    g, L0 = ttt_grad(K, V, theta, 1, d, m)
    ratios = []
    for lr in (1e-3, 1e-4, 1e-5):
        L1 = ttt_loss(K, V, theta - lr * g, 1, d, m)[0]
        ratios.append((L0[0] - L1) / (lr * np.sum(g * g)))
    assert abs(ratios[-1] - 1) < 1e-3
    assert abs(ratios[-1] - 1) < abs(ratios[0] - 1)


def test_minibatch_decomposition_eq5():
    n, d, m, H = 97, 4, 8, 2
    K, V, theta = _problem(n, d, m, H, seed=9)
    full, Lf = ttt_grad(K, V, theta, H, d, m, chunk=n)
    for chunk in (1, 7, 32):
        g, L = ttt_grad(K, V, theta, H, d, m, chunk=chunk)
        np.testing.assert_allclose(g, full, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(L, Lf, rtol=1e-12)
    # and by hand: the gradient of the union equals the sum over a split
    a, _ = ttt_grad(K[:40], V[:40], theta, H, d, m)
    b, _ = ttt_grad(K[40:], V[40:], theta, H, d, m)
    np.testing.assert_allclose(a + b, full, rtol=1e-12, atol=1e-13)


def test_view_permutation_invariance():
    """The objective is a sum over tokens, so reordering whole views leaves theta* unchanged."""
    views, tpv, d, m = 5, 12, 4, 8
    K, V, theta = _problem(views * tpv, d, m, seed=10)
    perm = _rng(11).permutation(views)
    idx = np.concatenate([np.arange(p * tpv, (p + 1) * tpv) for p in perm])
    a, _, _ = ttt_write(K, V, theta, 1, d, m, 0.1, 2)
    b, _, _ = ttt_write(K[idx], V[idx], theta, 1, d, m, 0.1, 2)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_heads_are_independent():
    n, d, m, H = 30, 4, 8, 3
    K, V, theta = _problem(n, d, m, H, seed=12)
    g, _ = ttt_grad(K, V, theta, H, d, m)
    K2 = K.copy()
    K2[:, d:2 * d] += 1.0  # perturb head 1 only
    g2, _ = ttt_grad(K2, V, theta, H, d, m)
    np.testing.assert_array_equal(g[0], g2[0])
    np.testing.assert_array_equal(g[2], g2[2])
    assert not np.allclose(g[1], g2[1])
    # single-head call on the slice equals the multi-head call's row
    g1, _ = ttt_grad(K[:, d:2 * d], V[:, d:2 * d], theta[1:2], 1, d, m)
    np.testing.assert_array_equal(g1[0], g[1])


def test_read_is_per_token():
    n, d, m, H = 40, 4, 8, 2
    Q, _, theta = _problem(n, d, m, H, seed=13)
    O = ttt_read(Q, theta, H, d, m)
    rows = np.array([3, 17, 39])
    np.testing.assert_array_equal(ttt_read(Q[rows], theta, H, d, m), O[rows])
    # read equals the forward pass used by the write
    Wg, Wu, Wd = split_theta(theta[1], d, m)
    np.testing.assert_array_equal(O[:, d:2 * d], swiglu_forward(Q[:, d:2 * d], Wg, Wu, Wd)["Y"])


def test_mean_reduction_is_scaled_sum():
    n, d, m = 20, 4, 8
    K, V, theta = _problem(n, d, m, seed=14)
    _, Ls, gs = ttt_write(K, V, theta, 1, d, m, 0.1, 1, reduction="sum")
    _, Lm, gm = ttt_write(K, V, theta, 1, d, m, 0.1, 1, reduction="mean")
    np.testing.assert_allclose(gm, gs / n, rtol=1e-14)
    np.testing.assert_allclose(Lm, Ls / n, rtol=1e-14)


def test_steps_compose():
    """Two steps equal one step applied twice (each step restarts from the updated theta)."""
    n, d, m = 25, 4, 8
    K, V, theta = _problem(n, d, m, seed=15)
    a, La, _ = ttt_write(K, V, theta, 1, d, m, 0.1, 2)
    b1, Lb1, _ = ttt_write(K, V, theta, 1, d, m, 0.1, 1)
    b2, Lb2, _ = ttt_write(K, V, b1, 1, d, m, 0.1, 1)
    np.testing.assert_array_equal(a, b2)
    np.testing.assert_array_equal(La, np.concatenate([Lb1, Lb2]))
