"""Pins of the oracle's offload schedule ([GRAPH] "Large-Scale Inference
Strategies", Eq. 5): streaming the tokens through in minibatches, summing the
per-minibatch gradients and applying once per step gives the full-batch write.
ttt_write is itself pinned (finite differences, autograd, closed forms)."""
import numpy as np
import pytest

from oracle import ttt_grad, ttt_write, ttt_write_offload


def _problem(n, d, m, H, seed):
    r = np.random.default_rng(seed)
    K = r.standard_normal((n, H * d))
    V = r.standard_normal((n, H * d))
    theta = r.standard_normal((H, 3 * d * m)) * 0.3
    return K, V, theta


@pytest.mark.parametrize("minibatch", [1, 7, 16, 53, 200])
@pytest.mark.parametrize("recipe", [("mse", "gd"), ("dot", "muon")])
def test_offload_schedule_equals_full_batch_write(minibatch, recipe):
    loss, opt = recipe
    n, d, m, H = 53, 4, 8, 2
    K, V, theta = _problem(n, d, m, H, seed=40 + minibatch)
    lr = 0.01 if loss == "mse" else 0.05
    ref, ref_losses, _ = ttt_write(K, V, theta, H, d, m, lr=lr, steps=2, loss=loss, opt=opt)
    got, losses = ttt_write_offload(K, V, theta, H, d, m, lr=lr, steps=2, minibatch=minibatch, loss=loss, opt=opt)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(losses, ref_losses, rtol=1e-11, atol=1e-12)


def test_offload_first_step_uses_the_summed_minibatch_gradient():
    # one GD step from theta0 moves theta by exactly -lr * (g_1 + g_2 + g_3)
    n, d, m, H = 30, 4, 8, 1
    K, V, theta = _problem(n, d, m, H, seed=50)
    got, _ = ttt_write_offload(K, V, theta, H, d, m, lr=0.1, steps=1, minibatch=10)
    g = sum(ttt_grad(K[i:i + 10], V[i:i + 10], theta, H, d, m)[0] for i in (0, 10, 20))
    np.testing.assert_allclose((theta - got) / 0.1, g, rtol=1e-10, atol=1e-12)


def test_offload_rejects_empty_minibatch():
    K, V, theta = _problem(4, 4, 8, 1, seed=51)
    with pytest.raises(ValueError):
        ttt_write_offload(K, V, theta, 1, 4, 8, lr=0.1, steps=1, minibatch=0)
