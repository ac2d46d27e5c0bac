"""Parity of the pages' inner recipe on the GPU: dot-product loss and the Muon update.

The oracle side is oracle.ttt_grad / ttt_write with loss="dot", opt="muon"
(pinned in tests/test_oracle_recipe.py); it computes its own V' and theta*.

Bar (per head, normwise max error):
  * dot-loss gradient and loss: 2e-2 (bf16 compute), 1e-4 (fp32 compute);
  * the Muon map theta - lr NS(g) on a given fp32 gradient: 1e-4 (fp32 kernel);
  * a whole Muon write: the fp32 path at 1e-4, the bf16 path at 2e-2.
    NS is not a contraction near the origin: it raises small singular values
    steeply, so a relative gradient error e can turn into an output error of
    up to kappa*e. kappa is measured on the oracle's own gradient, by finite
    perturbation of the oracle's NS (no GPU value enters that measurement),
    and printed beside the error as a diagnostic; it does not widen the bar.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import test_layer_amd as tla
from synth import CONFIGS, make_inputs
from tests.gpu_util import bits, dtheta_ok, rel_err, rel_err_per_head, to64

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 1e-4
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tla.lib()


def _small_vggt(views=3, steps=2, heads=16, dtype="bf16"):
    from dataclasses import replace
    return replace(CONFIGS["views24"], n_views=views, steps=steps, n_heads=heads, dtype=dtype,
                   name=f"vggt{views}v{heads}h")


def _conv(inp):
    c = inp.cfg
    return tla.shortconv(inp.V, inp.conv_w, c.n_views, c.grid_h, c.grid_w, c.n_special)


def _oracle_conv(inp, out):
    c = inp.cfg
    return oracle.shortconv(to64(inp.V).astype(np.float32), inp.conv_w.cpu().numpy(), c.n_views, c.grid_h,
                            c.grid_w, c.n_special, out=out).astype(np.float64)


def _dot_loss_err(L, L_ref, K, Vp, theta, n_heads, d, m):
    """|L - L_ref| / sum_i |Y_i * V'_i| per head: the dot loss is a sum of
    terms of either sign that can cancel to near zero, so its rounding error is
    measured against the sum of the terms' magnitudes (from the oracle)."""
    theta = np.asarray(theta, dtype=np.float64).reshape(n_heads, -1)
    out = np.zeros(n_heads)
    for h in range(n_heads):
        cols = slice(h * d, (h + 1) * d)
        Wg, Wu, Wd = oracle.split_theta(theta[h], d, m)
        Y = oracle.swiglu_forward(K[:, cols], Wg, Wu, Wd)["Y"]
        out[h] = abs(float(L[h]) - float(L_ref[h])) / float(np.sum(np.abs(Y * Vp[:, cols])))
    return out


def _ns_gain(g, n_heads, d, m, trials=4, eps=1e-3, seed=0):
    """Largest observed ratio (relative change of NS(G)) / (relative change of G)
    over random perturbations of each per-head weight-matrix gradient."""
    r = np.random.default_rng(seed)
    worst = 1.0
    for h in range(n_heads):
        for G in oracle.split_theta(g[h], d, m):
            O = oracle.newton_schulz(G)
            for _ in range(trials):
                E = r.standard_normal(G.shape)
                E *= eps * np.abs(G).max() / np.abs(E).max()
                dO = oracle.newton_schulz(G + E) - O
                worst = max(worst, (np.abs(dO).max() / np.abs(O).max()) / eps)
    return worst


# ----------------------------------------------------------------------------
# dot-product loss gradient
# ----------------------------------------------------------------------------


def test_dot_gradient_bf16_parity():
    cfg = _small_vggt(views=3)
    print("[recipe] dot gradient bf16", flush=True)
    inp = make_inputs(cfg, DEV, with_q=False)
    Vp = _conv(inp)
    loss = torch.empty(cfg.n_heads, device=DEV)
    g = tla.ttt_grad(inp.K, Vp, inp.theta0, cfg.n_heads, loss_out=loss, loss="dot")
    torch.cuda.synchronize()
    K64, Vp_ref, th0 = to64(inp.K), _oracle_conv(inp, "bf16"), inp.theta0.cpu().numpy()
    g_ref, L_ref = oracle.ttt_grad(K64, Vp_ref, th0, cfg.n_heads, cfg.d_head, cfg.d_hidden, loss="dot")
    e = rel_err_per_head(to64(g), g_ref, cfg.n_heads, axis_cols=False)
    lerr = _dot_loss_err(loss.cpu().numpy(), L_ref, K64, Vp_ref, th0, cfg.n_heads, cfg.d_head, cfg.d_hidden)
    print(f"  dot gradient rel err max {e.max():.3e}, loss {lerr.max():.3e}", flush=True)
    assert e.max() <= TOL_BF16, e
    assert lerr.max() <= TOL_BF16, lerr


def test_dot_partials_reduce_equal_grad_bitwise():
    cfg = _small_vggt(views=2, heads=4)
    inp = make_inputs(cfg, DEV, with_q=False)
    Vp = _conv(inp)
    g = tla.ttt_grad(inp.K, Vp, inp.theta0, cfg.n_heads, loss="dot")
    ws = tla.make_workspace(cfg.n_tokens, cfg.n_heads, cfg.d_head, cfg.d_hidden, tla.BF16)
    tla.ttt_grad_partials(inp.K, Vp, inp.theta0, cfg.n_heads, ws, loss="dot")
    g2 = torch.empty_like(g)
    tla.ttt_reduce(ws, cfg.n_tokens, cfg.n_heads, cfg.d_head, cfg.d_hidden, tla.BF16, tla.REDUCE_STORE, g2)
    np.testing.assert_array_equal(bits(g), bits(g2))
    # the MSE gradient is a different quantity
    g_mse = tla.ttt_grad(inp.K, Vp, inp.theta0, cfg.n_heads)
    assert not torch.equal(g, g_mse)


def test_dot_gradient_eq5_split_on_gpu():
    cfg = _small_vggt(views=2, heads=4)
    inp = make_inputs(cfg, DEV, with_q=False)
    Vp = _conv(inp)
    n = cfg.n_tokens
    cut = 1000
    g = tla.ttt_grad(inp.K, Vp, inp.theta0, cfg.n_heads, loss="dot")
    acc = tla.ttt_grad(inp.K[:cut], Vp[:cut], inp.theta0, cfg.n_heads, loss="dot")
    tla.ttt_grad(inp.K[cut:n], Vp[cut:n], inp.theta0, cfg.n_heads, grad=acc, accumulate=True, loss="dot")
    e = rel_err_per_head(to64(acc), to64(g), cfg.n_heads, axis_cols=False)
    assert e.max() <= 1e-5, e


def test_dot_gradient_f32_parity():
    cfg = CONFIGS["tiny_f32"]
    inp = make_inputs(cfg, DEV, with_q=False)
    Vp = _conv(inp)
    loss = torch.empty(1, device=DEV)
    g = tla.ttt_grad(inp.K, Vp, inp.theta0, 1, loss_out=loss, loss="dot")
    K64, Vp_ref, th0 = to64(inp.K), _oracle_conv(inp, "f32"), inp.theta0.cpu().numpy()
    g_ref, L_ref = oracle.ttt_grad(K64, Vp_ref, th0, 1, 16, 32, loss="dot")
    assert rel_err(to64(g), g_ref) <= TOL_F32
    assert _dot_loss_err(loss.cpu().numpy(), L_ref, K64, Vp_ref, th0, 1, 16, 32).max() <= TOL_F32


# ----------------------------------------------------------------------------
# Muon update
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("shape", [(64, 128, 16), (16, 32, 3)], ids=lambda s: f"d{s[0]}m{s[1]}h{s[2]}")
@pytest.mark.parametrize("ns_steps", [5, 0, 3])
def test_muon_apply_parity(shape, ns_steps):
    d, m, H = shape
    print(f"[recipe] muon apply d{d} m{m} H{H} ns{ns_steps}", flush=True)
    gen = torch.Generator(device="cpu").manual_seed(100 + d + ns_steps)
    theta = (0.02 * torch.randn((H, 3 * d * m), generator=gen)).to(DEV)
    grad = torch.randn((H, 3 * d * m), generator=gen)
    grad[1 % H, :d * m] *= 1e-3  # a small-norm matrix as well
    grad = grad.to(DEV)
    th0 = theta.cpu().numpy().astype(np.float64)
    tla.ttt_muon_apply(theta, grad, 0.1, H, d, m, ns_steps)
    ref = oracle.muon_apply(th0, grad.cpu().numpy().astype(np.float64), 0.1, H, d, m, ns_steps)
    upd, upd_ref = th0 - theta.cpu().numpy(), th0 - ref
    e = rel_err_per_head(upd, upd_ref, H, axis_cols=False)
    print(f"  update rel err max {e.max():.3e}", flush=True)
    assert e.max() <= TOL_F32, e


def test_muon_apply_zero_gradient_is_identity():
    H, d, m = 2, 64, 128
    theta = torch.randn((H, 3 * d * m), device=DEV)
    before = theta.clone()
    tla.ttt_muon_apply(theta, torch.zeros_like(theta), 0.1, H, d, m, 5)
    np.testing.assert_array_equal(bits(theta), bits(before))


# ----------------------------------------------------------------------------
# whole writes with the pages' recipe
# ----------------------------------------------------------------------------


def test_write_dot_muon_f32_tiny_parity():
    cfg = CONFIGS["tiny_f32"]
    from dataclasses import replace
    cfg = replace(cfg, steps=2)
    inp = make_inputs(cfg, DEV, with_q=True)
    Vp = _conv(inp)
    theta = inp.theta0.clone()
    loss = torch.empty((cfg.steps, 1), device=DEV)
    tla.ttt_write(inp.K, Vp, theta, cfg.lr, cfg.steps, 1, loss_out=loss, loss="dot", optimizer="muon")
    O = tla.ttt_read(inp.Q, theta, 1)
    th0 = inp.theta0.cpu().numpy()
    K64, Vp_ref = to64(inp.K), _oracle_conv(inp, "f32")
    th_ref, L_ref, _ = oracle.ttt_write(K64, Vp_ref, th0, 1, 16, 32, cfg.lr, cfg.steps, loss="dot", opt="muon")
    th = theta.cpu().numpy().astype(np.float64)
    ok, worst = dtheta_ok(th, th_ref, th0, 1, TOL_F32, cfg.steps)
    assert ok, worst
    L = loss.cpu().numpy()
    # step 1 starts from theta0 on both sides; compare its loss at the loss bar
    assert _dot_loss_err(L[0], L_ref[0], K64, Vp_ref, th0, 1, 16, 32).max() <= TOL_F32
    O_ref = oracle.ttt_read(to64(inp.Q), th_ref, 1, 16, 32)
    assert rel_err(to64(O), O_ref) <= TOL_F32


def test_write_dot_muon_bf16_parity():
    cfg = _small_vggt(views=3, steps=2)
    print("[recipe] dot + muon write bf16", flush=True)
    inp = make_inputs(cfg, DEV, with_q=True)
    Vp = _conv(inp)
    theta = inp.theta0.clone()
    loss = torch.empty((cfg.steps, cfg.n_heads), device=DEV)
    tla.ttt_write(inp.K, Vp, theta, cfg.lr, cfg.steps, cfg.n_heads, loss_out=loss, loss="dot", optimizer="muon")
    O = tla.ttt_read(inp.Q, theta, cfg.n_heads)
    th0 = inp.theta0.cpu().numpy()
    K64, Vp_ref = to64(inp.K), _oracle_conv(inp, "bf16")
    th_ref, L_ref, g_ref = oracle.ttt_write(K64, Vp_ref, th0, cfg.n_heads, cfg.d_head, cfg.d_hidden, cfg.lr,
                                            cfg.steps, loss="dot", opt="muon")
    kappa = max(_ns_gain(g_ref[s], cfg.n_heads, cfg.d_head, cfg.d_hidden) for s in range(cfg.steps))
    tol = TOL_BF16
    th = theta.cpu().numpy().astype(np.float64)
    dth = rel_err_per_head(th - th0, th_ref - th0, cfg.n_heads, axis_cols=False)
    lerr = _dot_loss_err(loss.cpu().numpy()[0], L_ref[0], K64, Vp_ref, th0, cfg.n_heads, cfg.d_head, cfg.d_hidden)
    O_ref = oracle.ttt_read(to64(inp.Q), th_ref, cfg.n_heads, cfg.d_head, cfg.d_hidden)
    oerr = rel_err_per_head(to64(O), O_ref, cfg.n_heads)
    print(f"  NS gain {kappa:.2f} (diagnostic), tol {tol:.3e}; delta-theta {dth.max():.3e}, loss {lerr.max():.3e}, "
          f"read {oerr.max():.3e}", flush=True)
    assert dth.max() <= tol, dth
    assert lerr.max() <= tol, lerr
    assert oerr.max() <= tol, oerr


def test_write_dot_muon_deterministic_and_split_equivalent():
    cfg = _small_vggt(views=2, steps=2, heads=4)
    inp = make_inputs(cfg, DEV, with_q=False)
    Vp = _conv(inp)
    a = inp.theta0.clone()
    tla.ttt_write(inp.K, Vp, a, cfg.lr, cfg.steps, cfg.n_heads, loss="dot", optimizer="muon")
    b = inp.theta0.clone()
    tla.ttt_write(inp.K, Vp, b, cfg.lr, cfg.steps, cfg.n_heads, loss="dot", optimizer="muon")
    np.testing.assert_array_equal(bits(a), bits(b))
    # the fused write equals gradient (dot) + Muon apply, step by step
    c = inp.theta0.clone()
    for _ in range(cfg.steps):
        g = tla.ttt_grad(inp.K, Vp, c, cfg.n_heads, loss="dot")
        tla.ttt_muon_apply(c, g, cfg.lr, cfg.n_heads, cfg.d_head, cfg.d_hidden, 5)
    np.testing.assert_array_equal(bits(a), bits(c))


def test_write_dot_gd_bf16_parity():
    cfg = _small_vggt(views=2, steps=2, heads=4)
    inp = make_inputs(cfg, DEV, with_q=False)
    Vp = _conv(inp)
    theta = inp.theta0.clone()
    tla.ttt_write(inp.K, Vp, theta, 1e-4, cfg.steps, cfg.n_heads, loss="dot", optimizer="gd")
    th0 = inp.theta0.cpu().numpy()
    th_ref, _, _ = oracle.ttt_write(to64(inp.K), _oracle_conv(inp, "bf16"), th0, cfg.n_heads, cfg.d_head,
                                    cfg.d_hidden, 1e-4, cfg.steps, loss="dot", opt="gd")
    th = theta.cpu().numpy().astype(np.float64)
    dth = rel_err_per_head(th - th0, th_ref - th0, cfg.n_heads, axis_cols=False)
    assert dth.max() <= TOL_BF16, dth
