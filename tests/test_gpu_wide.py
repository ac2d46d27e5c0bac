"""Parity of the full-width fast-weight MLP on the GPU: one 1024 -> 4096 -> 1024
SwiGLU over the whole token ([GRAPH] "TTT MLP Architecture and Inner
Optimization"), written with gradient descent under the squared-error or the
dot-product loss, then read.

The oracle is the same per-head oracle with one head of d = 1024, m = 4096
(its pins are shape-generic). Bars: 2e-2 normwise per weight matrix and on the
read (bf16 compute), Eq. 5 chunk splits to fp32 rounding (1e-5).
"""
from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import test_layer_amd as tla
from synth import CONFIGS, make_inputs
from tests.gpu_util import bits, dtheta_ok, rel_err, rel_err_per_head, to64

pytestmark = pytest.mark.gpu

TOL = 2e-2
DEV = "cuda"
D, M = 1024, 4096


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tla.lib()


def _cfg(views=1, grid=37, special=5, steps=1):
    return replace(CONFIGS["views24"], name=f"wide{views}v", n_views=views, grid_h=grid, grid_w=grid,
                   n_special=special, n_heads=1, d_head=D, d_hidden=M, steps=steps)


def _scene(cfg, with_q=False):
    inp = make_inputs(cfg, DEV, with_q=with_q)
    Vp = tla.shortconv(inp.V, inp.conv_w, cfg.n_views, cfg.grid_h, cfg.grid_w, cfg.n_special)
    torch.cuda.synchronize()
    return inp, Vp


def _oracle_vp(inp):
    c = inp.cfg
    return oracle.shortconv(to64(inp.V).astype(np.float32), inp.conv_w.cpu().numpy(), c.n_views, c.grid_h,
                            c.grid_w, c.n_special, out="bf16").astype(np.float64)


def _per_matrix_err(g, ref):
    out = []
    for a, b in zip(oracle.split_theta(g.reshape(-1), D, M), oracle.split_theta(ref.reshape(-1), D, M)):
        out.append(rel_err(a, b))
    return np.array(out)


@pytest.mark.parametrize("loss", ["mse", "dot"])
def test_wide_gradient_parity(loss):
    # one view of 37x37 + 5 tokens: 1,374 tokens = 5 full 256-token tiles + a ragged one
    cfg = _cfg()
    print(f"[wide] gradient {loss}", flush=True)
    inp, Vp = _scene(cfg)
    L = torch.empty(1, device=DEV)
    g = tla.ttt_grad(inp.K, Vp, inp.theta0, 1, loss_out=L, loss=loss)
    torch.cuda.synchronize()
    th0 = inp.theta0.cpu().numpy()
    g_ref, L_ref = oracle.ttt_grad(to64(inp.K), _oracle_vp(inp), th0, 1, D, M, loss=loss)
    e = _per_matrix_err(to64(g), g_ref)
    le = abs(L.item() - L_ref[0]) / abs(L_ref[0])
    print(f"  per-matrix rel err {e}, loss {le:.3e}", flush=True)
    assert e.max() <= TOL, e
    if loss == "mse":
        assert le <= TOL, le
    else:
        # the dot loss is a sum of terms of either sign: its error is measured
        # against the sum of the terms' magnitudes (oracle forward)
        Wg, Wu, Wd = oracle.split_theta(th0.reshape(-1), D, M)
        Y = oracle.swiglu_forward(to64(inp.K), Wg, Wu, Wd)["Y"]
        scale = float(np.sum(np.abs(Y * _oracle_vp(inp))))
        ld = abs(L.item() - L_ref[0]) / scale
        print(f"  dot loss error / sum |Y V'| = {ld:.3e}", flush=True)
        assert ld <= TOL, ld


def test_wide_write_two_steps_parity():
    cfg = _cfg(steps=2)
    inp, Vp = _scene(cfg)
    theta = inp.theta0.clone()
    L = torch.empty((2, 1), device=DEV)
    tla.ttt_write(inp.K, Vp, theta, cfg.lr, 2, 1, loss_out=L)
    torch.cuda.synchronize()
    th0 = inp.theta0.cpu().numpy()
    th_ref, L_ref, _ = oracle.ttt_write(to64(inp.K), _oracle_vp(inp), th0, 1, D, M, cfg.lr, 2)
    ok, worst = dtheta_ok(theta.cpu().numpy().astype(np.float64), th_ref, th0, 1, TOL, 2)
    print(f"  wide write dtheta worst/allowance {worst:.3f}", flush=True)
    assert ok, worst
    np.testing.assert_allclose(L.cpu().numpy(), L_ref, rtol=TOL)


def test_wide_read_parity():
    cfg = _cfg()
    inp = make_inputs(cfg, DEV, with_q=True)
    theta = inp.theta0 * 10.0
    O = tla.ttt_read(inp.Q, theta, 1)
    torch.cuda.synchronize()
    O_ref = oracle.ttt_read(to64(inp.Q), theta.cpu().numpy(), 1, D, M)
    e = rel_err(to64(O), O_ref)
    print(f"  wide read rel err {e:.3e}", flush=True)
    assert e <= TOL, e


def test_wide_gradient_eq5_split_and_determinism():
    cfg = _cfg(views=2)
    inp, Vp = _scene(cfg)
    n = cfg.n_tokens
    g = tla.ttt_grad(inp.K, Vp, inp.theta0, 1)
    g2 = tla.ttt_grad(inp.K, Vp, inp.theta0, 1)
    cut = 1000
    acc = tla.ttt_grad(inp.K[:cut], Vp[:cut], inp.theta0, 1)
    tla.ttt_grad(inp.K[cut:n], Vp[cut:n], inp.theta0, 1, grad=acc, accumulate=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(g), bits(g2))
    e = _per_matrix_err(to64(acc), to64(g))
    assert e.max() <= 1e-5, e


def test_wide_two_chunk_scene_against_oracle():
    """102 views = 140,148 tokens: one full 131,072-token chunk of the GEMM
    sequence and a ragged second one, so the in-HBM write accumulates two
    chunks. Against the oracle: the gradient at theta0 and both steps' losses,
    theta* and delta-theta of a 2-step write, and the read with theta* on rows
    on both sides of the chunk boundary and at the tail."""
    cfg = _cfg(views=102, steps=2)
    n = cfg.n_tokens
    assert 131_072 < n < 2 * 131_072
    print(f"[wide] two-chunk scene n={n}", flush=True)
    inp, Vp = _scene(cfg, with_q=True)
    L0 = torch.empty(1, device=DEV)
    g0 = tla.ttt_grad(inp.K, Vp, inp.theta0, 1, loss_out=L0)
    theta = inp.theta0.clone()
    L = torch.empty((2, 1), device=DEV)
    tla.ttt_write(inp.K, Vp, theta, cfg.lr, 2, 1, loss_out=L)
    rows = np.unique(np.concatenate([np.linspace(0, n - 1, 120).astype(np.int64), 131_072 + np.arange(-6, 6),
                                     np.arange(n - 20, n)]))
    O = tla.ttt_read(inp.Q, theta, 1)
    torch.cuda.synchronize()
    print("  gpu done", flush=True)
    th0 = inp.theta0.cpu().numpy().astype(np.float64)
    th_ref, L_ref, g_ref = oracle.ttt_write(to64(inp.K), _oracle_vp(inp), th0, 1, D, M, cfg.lr, 2)
    e = _per_matrix_err(to64(g0), g_ref[0])
    le = [abs(float(L[s, 0]) - L_ref[s, 0]) / abs(L_ref[s, 0]) for s in range(2)]
    print(f"  gradient at theta0 per-matrix rel err {e}; loss rel err {le}", flush=True)
    assert e.max() <= TOL, e
    assert max(le) <= TOL
    assert abs(L0.item() - L_ref[0, 0]) <= TOL * abs(L_ref[0, 0])
    ok, worst = dtheta_ok(theta.cpu().numpy().astype(np.float64), th_ref, th0, 1, TOL, 2)
    print(f"  delta-theta worst/allowance {worst:.3f}", flush=True)
    assert ok, worst
    O_ref = oracle.ttt_read(to64(inp.Q[torch.from_numpy(rows).to(DEV)]), th_ref, 1, D, M)
    er = rel_err(to64(O[torch.from_numpy(rows).to(DEV)]), O_ref)
    print(f"  read with theta* on {rows.size} rows: rel err {er:.3e}", flush=True)
    assert er <= TOL, er


def test_wide_views1000_chunked_gradient_and_sampled_read():
    """The 1000-view scene (1,374,000 tokens: ten full 131,072-token chunks and a
    ragged one). The gradient cannot be checked against the oracle at this
    size; Eq. 5 fixes it instead: it must equal the sum of the gradients of two
    halves cut off chunk boundaries (same per-token products, other fp32
    summation order). The read is per token, so sampled rows are checked
    against the oracle."""
    cfg = _cfg(views=1000, steps=2)
    print("[wide] views1000 gradient halves + sampled read", flush=True)
    inp, Vp = _scene(cfg, with_q=True)
    n = cfg.n_tokens
    L = torch.empty(1, device=DEV)
    g = tla.ttt_grad(inp.K, Vp, inp.theta0, 1, loss_out=L)
    cut = 700_001
    L2 = torch.empty(1, device=DEV)
    acc = tla.ttt_grad(inp.K[:cut], Vp[:cut], inp.theta0, 1, loss_out=L2)
    tla.ttt_grad(inp.K[cut:n], Vp[cut:n], inp.theta0, 1, grad=acc, accumulate=True, loss_out=L2)
    torch.cuda.synchronize()
    e = _per_matrix_err(to64(acc), to64(g))
    print(f"  halves vs whole: per-matrix rel diff {e}", flush=True)
    assert e.max() <= 1e-5, e
    assert abs(L.item() - L2.item()) <= 1e-5 * abs(L.item())
    assert torch.isfinite(g).all()
    # read with a fitted theta: sampled tokens in several chunks, incl. the ragged tail
    theta = inp.theta0.clone()
    tla.ttt_write(inp.K, Vp, theta, cfg.lr, 2, 1)
    O = tla.ttt_read(inp.Q, theta, 1)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.linspace(0, n - 1, 200).astype(np.int64), np.arange(n - 40, n),
                                     131_070 + np.arange(6)]))
    O_ref = oracle.ttt_read(to64(inp.Q[rows]), theta.cpu().numpy(), 1, D, M)
    er = rel_err(to64(O[rows]), O_ref)
    print(f"  sampled read rel err {er:.3e}", flush=True)
    assert er <= TOL, er


def _ns_gain(g, trials=2, eps=1e-3, seed=0):
    """Largest observed ratio (relative change of NS(G)) / (relative change of
    G) over random perturbations of the oracle's own gradient matrices (no GPU
    value enters this)."""
    r = np.random.default_rng(seed)
    worst = 1.0
    for G in oracle.split_theta(g.reshape(-1), D, M):
        O = oracle.newton_schulz(G)
        for _ in range(trials):
            E = r.standard_normal(G.shape)
            E *= eps * np.abs(G).max() / np.abs(E).max()
            dO = oracle.newton_schulz(G + E) - O
            worst = max(worst, (np.abs(dO).max() / np.abs(O).max()) / eps)
    return worst


def test_wide_write_dot_muon_parity():
    """The pages' recipe at the pages' width: dot-product loss, Muon with 5
    Newton-Schulz steps, 2 steps. Bar 2e-2, as for the per-head Muon write;
    the oracle-measured NS error gain is printed as a diagnostic."""
    cfg = _cfg(steps=2)
    print("[wide] dot + muon write", flush=True)
    inp, Vp = _scene(cfg)
    theta = inp.theta0.clone()
    L = torch.empty((2, 1), device=DEV)
    tla.ttt_write(inp.K, Vp, theta, cfg.lr, 2, 1, loss_out=L, loss="dot", optimizer="muon")
    torch.cuda.synchronize()
    th0 = inp.theta0.cpu().numpy()
    K64, Vp_ref = to64(inp.K), _oracle_vp(inp)
    th_ref, L_ref, grads = oracle.ttt_write(K64, Vp_ref, th0, 1, D, M, cfg.lr, 2, loss="dot", opt="muon")
    kappa = _ns_gain(grads[0])
    tol = TOL
    ok, worst = dtheta_ok(theta.cpu().numpy().astype(np.float64), th_ref, th0, 1, tol, 2)
    print(f"  NS gain {kappa:.2f} (diagnostic), dtheta worst/allowance {worst:.3f} (tol {tol:.3g})", flush=True)
    assert ok, worst


@pytest.mark.parametrize("ns_steps", [5, 2])
def test_wide_muon_apply_parity(ns_steps):
    """The Muon map alone on a seeded random gradient (fp32 GEMMs) against the
    oracle's fp64 Newton-Schulz: 1e-4 normwise per matrix, as the per-head
    Muon. One matrix gets a small norm, one a large one."""
    gen = torch.Generator(device="cpu").manual_seed(300 + ns_steps)
    theta = 0.02 * torch.randn((1, 3 * D * M), generator=gen)
    grad = torch.randn((1, 3 * D * M), generator=gen)
    grad[0, :D * M] *= 1e-3
    grad[0, 2 * D * M:] *= 50.0
    th_dev, g_dev = theta.to(DEV), grad.to(DEV)
    ws = torch.empty(tla.muon_workspace_bytes(1, D, M), dtype=torch.uint8, device=DEV)
    tla.ttt_muon_apply(th_dev, g_dev, 0.1, 1, D, M, ns_steps, workspace=ws)
    torch.cuda.synchronize()
    th0 = theta.numpy().astype(np.float64)
    ref = oracle.muon_apply(th0, grad.numpy().astype(np.float64), 0.1, 1, D, M, ns_steps)
    upd, upd_ref = th0 - th_dev.cpu().numpy().astype(np.float64), th0 - ref
    e = _per_matrix_err(upd, upd_ref)
    print(f"  wide muon apply ns{ns_steps} per-matrix rel err {e}", flush=True)
    assert e.max() <= 1e-4, e


@pytest.mark.parametrize("n", [1, 7, 255, 257])
def test_wide_tiny_and_ragged_token_counts(n):
    """Token counts below one tile, and one either side of a 256-row tile
    boundary: gradient, loss and read against the oracle."""
    cfg = _cfg()
    inp, Vp = _scene(cfg, with_q=True)
    K, V, Q = inp.K[:n].contiguous(), Vp[:n].contiguous(), inp.Q[:n].contiguous()
    L = torch.empty(1, device=DEV)
    g = tla.ttt_grad(K, V, inp.theta0, 1, loss_out=L)
    theta = inp.theta0 * 10.0
    O = tla.ttt_read(Q, theta, 1)
    torch.cuda.synchronize()
    th0 = inp.theta0.cpu().numpy()
    Vp_ref = _oracle_vp(inp)[:n]
    g_ref, L_ref = oracle.ttt_grad(to64(K), Vp_ref, th0, 1, D, M)
    e = _per_matrix_err(to64(g), g_ref)
    assert e.max() <= TOL, (n, e)
    assert abs(L.item() - L_ref[0]) <= TOL * abs(L_ref[0])
    O_ref = oracle.ttt_read(to64(Q), theta.cpu().numpy(), 1, D, M)
    assert rel_err(to64(O), O_ref) <= TOL


def test_wide_empty_scene():
    theta = (0.02 * torch.randn((1, 3 * D * M))).to(DEV)
    before = theta.clone()
    empty = torch.empty((0, D), dtype=torch.bfloat16, device=DEV)
    L = torch.full((2, 1), 5.0, device=DEV)
    tla.ttt_write(empty, empty, theta, 0.1, 2, 1, loss_out=L, loss="dot", optimizer="muon")
    g = tla.ttt_grad(empty, empty, theta, 1)
    O = tla.ttt_read(empty, theta, 1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(theta), bits(before))
    assert torch.all(L == 0) and torch.all(g == 0) and O.shape == (0, D)
