"""Parity of the HIP path against the CPU oracle on identical seeded inputs.

Bar (per head, normwise max error max|x - x_ref| / max|x_ref|):
  * ShortConv2D: bit-exact (the fp32 conv contract, bf16 round to nearest even);
  * bf16 compute: theta*, delta-theta = theta* - theta0, gradients and read
    outputs within 2e-2;
  * fp32 compute: within 1e-4.
The oracle always computes its own V' from V and its own theta* from theta0;
nothing it consumes comes from the HIP path.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import test_layer_amd as tla
from synth import CONFIGS, make_inputs
from tests.gpu_util import bits, dtheta_ok, f32_to_bits, rel_err, rel_err_per_head, to64

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 1e-4

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tla.lib()


def _small_vggt(views=3, steps=2, heads=16, dtype="bf16", **kw):
    from dataclasses import replace
    return replace(CONFIGS["views24"], n_views=views, steps=steps, n_heads=heads, dtype=dtype,
                   name=f"vggt{views}v{heads}h", **kw)


def _conv(inp):
    c = inp.cfg
    return tla.shortconv(inp.V, inp.conv_w, c.n_views, c.grid_h, c.grid_w, c.n_special)


def _oracle_conv(inp, out):
    c = inp.cfg
    return oracle.shortconv(to64(inp.V).astype(np.float32), inp.conv_w.cpu().numpy(), c.n_views, c.grid_h,
                            c.grid_w, c.n_special, out=out)


# ----------------------------------------------------------------------------
# ShortConv2D
# ----------------------------------------------------------------------------

CONV_CASES = [
    # (views, grid_h, grid_w, n_special, heads, d_head, dtype)
    (2, 8, 8, 0, 1, 16, "f32"),
    (3, 37, 37, 5, 16, 64, "bf16"),
    (2, 5, 7, 2, 1, 64, "bf16"),
    (1, 1, 1, 1, 1, 8, "bf16"),
    (4, 3, 2, 0, 2, 4, "f32"),
    (2, 37, 37, 5, 4, 64, "f32"),
    # bf16, 64-channel multiples, rows up to 126 columns: the LDS ring kernel,
    # 64-channel strips of 3-row blocks
    (2, 9, 126, 1, 1, 64, "bf16"),  # widest grid row that fits LDS (160 KB)
    (2, 7, 40, 3, 3, 64, "bf16"),   # three channel blocks
    (5, 4, 4, 2, 1, 64, "bf16"),    # a ragged last block of rows
    (3, 1, 9, 0, 1, 64, "bf16"),    # a single grid row
    (2, 9, 79, 1, 2, 64, "bf16"),   # C = 128, but the 128-channel ring would exceed 160 KB
    # with C a multiple of 128 (and rows up to 78 columns): 128-channel strips
    # of 2-row blocks
    (2, 9, 78, 1, 2, 64, "bf16"),   # widest grid row for that ring (160 KB)
    (5, 5, 4, 2, 2, 64, "bf16"),    # a ragged last block of rows
    (3, 1, 9, 0, 2, 64, "bf16"),    # a single grid row
    (2, 2, 3, 0, 4, 64, "bf16"),    # two channel blocks, a tiny grid
    # bf16 outside it: the register-window kernel
    (1, 4, 127, 0, 1, 64, "bf16"),  # grid row too wide for the LDS ring
    (1, 2, 3, 0, 3, 32, "bf16"),    # 96 channels
]


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: "x".join(map(str, c)))
def test_shortconv_bitexact(case):
    from dataclasses import replace
    views, gh, gw, ns, H, d, dt = case
    cfg = replace(CONFIGS["tiny_f32"], n_views=views, grid_h=gh, grid_w=gw, n_special=ns, n_heads=H, d_head=d,
                  d_hidden=2 * d, dtype=dt, normalize=(dt == "bf16"), name="conv")
    print(f"[conv] {case}", flush=True)
    inp = make_inputs(cfg, DEV, with_q=False)
    Vp = _conv(inp)
    torch.cuda.synchronize()
    ref = _oracle_conv(inp, "bf16" if dt == "bf16" else "f32")
    np.testing.assert_array_equal(bits(Vp), f32_to_bits(ref, dt == "bf16"))


def test_shortconv_special_tokens_and_edges_bitexact():
    """Extreme values: subnormal products, signed zeros and large magnitudes follow the contract."""
    from dataclasses import replace
    cfg = replace(CONFIGS["tiny_f32"], n_views=2, grid_h=6, grid_w=5, n_special=3, n_heads=2, d_head=16,
                  dtype="f32", name="conv-edge")
    inp = make_inputs(cfg, DEV, with_q=False)
    V = inp.V.clone()
    V[::3] *= 1e-38  # products land in the subnormal range
    V[1::7] = -0.0
    V[2::5] *= 1e30
    inp.V.copy_(V)
    Vp = _conv(inp)
    ref = _oracle_conv(inp, "f32")
    np.testing.assert_array_equal(bits(Vp), f32_to_bits(ref, False))


def test_shortconv_bf16_extreme_values_bitexact():
    """The LDS ring kernel on signed zeros, subnormal products and large magnitudes (bf16 range)."""
    from dataclasses import replace
    cfg = replace(CONFIGS["tiny_f32"], n_views=3, grid_h=7, grid_w=5, n_special=2, n_heads=2, d_head=64,
                  d_hidden=128, dtype="bf16", normalize=True, name="conv-edge-bf16")
    inp = make_inputs(cfg, DEV, with_q=False)
    V = inp.V.float()
    V[::3] *= 1e-38  # subnormal inputs and products
    V[1::7] = -0.0
    V[2::5] *= 1e30
    inp.V.copy_(V.to(torch.bfloat16))
    Vp = _conv(inp)
    torch.cuda.synchronize()
    ref = _oracle_conv(inp, "bf16")
    np.testing.assert_array_equal(bits(Vp), f32_to_bits(ref, True))


# ----------------------------------------------------------------------------
# Read
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("n_tokens", [1, 16, 17, 31, 48, 1000, 4122])
def test_read_bf16_parity(n_tokens):
    """Token counts around the kernel's 32-token tile and its two 16-token
    halves (a last tile with an empty, a one-token and a full second half)."""
    cfg = _small_vggt(views=3)
    print(f"[read bf16] n={n_tokens}", flush=True)
    inp = make_inputs(cfg, DEV)
    Q = inp.Q[:n_tokens].contiguous()
    O = tla.ttt_read(Q, inp.theta0, cfg.n_heads)
    ref = oracle.ttt_read(to64(Q), inp.theta0.cpu().numpy(), cfg.n_heads, cfg.d_head, cfg.d_hidden)
    err = rel_err_per_head(to64(O), ref, cfg.n_heads)
    assert err.max() <= TOL_BF16, err
    # Per token and head as well, so that one wrong token among thousands
    # cannot hide in a per-head norm. A screen for gross errors (a token left
    # at zero, read from the wrong row or with permuted outputs gives about
    # 1): each token's error relative to the head's mean token norm.
    d = cfg.d_head
    o = to64(O).reshape(n_tokens, cfg.n_heads, d)
    r = ref.reshape(n_tokens, cfg.n_heads, d)
    tok_err = np.linalg.norm(o - r, axis=2) / np.linalg.norm(r, axis=2).mean(axis=0)
    print(f"[read bf16] per-token max {tok_err.max():.2e}", flush=True)
    assert tok_err.max() <= 5 * TOL_BF16, tok_err.max()


def test_read_bf16_trained_weights_parity():
    """A theta far from init (large weights) still matches: exercises the whole sigmoid range."""
    cfg = _small_vggt(views=2, heads=4)
    inp = make_inputs(cfg, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    theta = torch.randn(inp.theta0.shape, generator=g, device=DEV) * 0.5
    O = tla.ttt_read(inp.Q, theta, cfg.n_heads)
    ref = oracle.ttt_read(to64(inp.Q), theta.cpu().numpy(), cfg.n_heads, cfg.d_head, cfg.d_hidden)
    err = rel_err_per_head(to64(O), ref, cfg.n_heads)
    assert err.max() <= TOL_BF16, err


# ----------------------------------------------------------------------------
# Write (gradient, steps) in bf16
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("n_tokens", [1, 64, 100, 4122])
def test_grad_bf16_parity(n_tokens):
    cfg = _small_vggt(views=3)
    print(f"[grad bf16] n={n_tokens}", flush=True)
    inp = make_inputs(cfg, DEV, with_q=False)
    Vp = _conv(inp)
    K = inp.K[:n_tokens].contiguous()
    Vs = Vp[:n_tokens].contiguous()
    loss = torch.empty(cfg.n_heads, device=DEV)
    g = tla.ttt_grad(K, Vs, inp.theta0, cfg.n_heads, loss_out=loss)
    Vp_ref = _oracle_conv(inp, "bf16")[:n_tokens]
    g_ref, L_ref = oracle.ttt_grad(to64(K), Vp_ref.astype(np.float64), inp.theta0.cpu().numpy(), cfg.n_heads,
                                   cfg.d_head, cfg.d_hidden)
    err = rel_err_per_head(to64(g), g_ref, cfg.n_heads, axis_cols=False)
    assert err.max() <= TOL_BF16, err
    lerr = np.abs(loss.cpu().numpy() - L_ref) / np.abs(L_ref)
    assert lerr.max() <= TOL_BF16, lerr


def test_write_bf16_parity_two_steps():
    cfg = _small_vggt(views=3, steps=2)
    inp = make_inputs(cfg, DEV, with_q=True)
    Vp = _conv(inp)
    theta = inp.theta0.clone()
    loss = torch.empty((cfg.steps, cfg.n_heads), device=DEV)
    tla.ttt_write(inp.K, Vp, theta, cfg.lr, cfg.steps, cfg.n_heads, loss_out=loss)
    O = tla.ttt_read(inp.Q, theta, cfg.n_heads)
    th0 = inp.theta0.cpu().numpy()
    Vp_ref = _oracle_conv(inp, "bf16").astype(np.float64)
    th_ref, L_ref, _ = oracle.ttt_write(to64(inp.K), Vp_ref, th0, cfg.n_heads, cfg.d_head, cfg.d_hidden, cfg.lr,
                                        cfg.steps)
    th = theta.cpu().numpy().astype(np.float64)
    assert rel_err_per_head(th, th_ref, cfg.n_heads, axis_cols=False).max() <= TOL_BF16
    dth = rel_err_per_head(th - th0, th_ref - th0, cfg.n_heads, axis_cols=False)
    assert dth.max() <= TOL_BF16, dth
    lerr = np.abs(loss.cpu().numpy() - L_ref) / np.abs(L_ref)
    assert lerr.max() <= TOL_BF16, lerr
    O_ref = oracle.ttt_read(to64(inp.Q), th_ref, cfg.n_heads, cfg.d_head, cfg.d_hidden)
    assert rel_err_per_head(to64(O), O_ref, cfg.n_heads).max() <= TOL_BF16


def test_write_equals_partials_then_reduce_bitwise():
    cfg = _small_vggt(views=2, steps=2, heads=4)
    inp = make_inputs(cfg, DEV, with_q=False)
    Vp = _conv(inp)
    a = inp.theta0.clone()
    tla.ttt_write(inp.K, Vp, a, cfg.lr, cfg.steps, cfg.n_heads)
    b = inp.theta0.clone()
    ws = tla.make_workspace(cfg.n_tokens, cfg.n_heads, cfg.d_head, cfg.d_hidden, tla.BF16)
    for _ in range(cfg.steps):
        tla.ttt_grad_partials(inp.K, Vp, b, cfg.n_heads, ws)
        tla.ttt_reduce(ws, cfg.n_tokens, cfg.n_heads, cfg.d_head, cfg.d_hidden, tla.BF16, tla.REDUCE_APPLY, b,
                       cfg.lr)
    np.testing.assert_array_equal(bits(a), bits(b))
    # grad + apply reproduces the fused step as well (same tree, then theta - lr*g)
    c = inp.theta0.clone()
    for _ in range(cfg.steps):
        g = tla.ttt_grad(inp.K, Vp, c, cfg.n_heads)
        tla.ttt_apply(c, g, cfg.lr, cfg.n_heads, cfg.d_head, cfg.d_hidden)
    np.testing.assert_array_equal(bits(a), bits(c))


@pytest.mark.parametrize("loss", ["mse", "dot"])
def test_loss_value_is_optional_and_leaves_the_gradient_unchanged(loss):
    """Without a loss output the gradient kernel skips the loss value: the
    gradient and theta* are the same bits, and a loss asked of such partials is NaN."""
    cfg = _small_vggt(views=2, steps=2, heads=4)
    inp = make_inputs(cfg, DEV, with_q=False)
    Vp = _conv(inp)
    n, H, d, m = cfg.n_tokens, cfg.n_heads, cfg.d_head, cfg.d_hidden
    ws = tla.make_workspace(n, H, d, m, tla.BF16)
    out = {}
    for want in (True, False):
        g = torch.empty_like(inp.theta0)
        lo = torch.zeros(H, device=DEV)
        tla.ttt_grad_partials(inp.K, Vp, inp.theta0, H, ws, loss=loss, want_loss=want)
        tla.ttt_reduce(ws, n, H, d, m, tla.BF16, tla.REDUCE_STORE, g, 0.0, lo)
        out[want] = (g, lo)
    np.testing.assert_array_equal(bits(out[True][0]), bits(out[False][0]))
    assert torch.isfinite(out[True][1]).all() and torch.isnan(out[False][1]).all()
    a = inp.theta0.clone()
    b = inp.theta0.clone()
    lw = torch.zeros((cfg.steps, H), device=DEV)
    tla.ttt_write(inp.K, Vp, a, cfg.lr, cfg.steps, H, loss_out=lw, loss=loss)
    tla.ttt_write(inp.K, Vp, b, cfg.lr, cfg.steps, H, loss=loss)
    np.testing.assert_array_equal(bits(a), bits(b))
    assert torch.isfinite(lw).all()


def test_eq5_chunked_gradient_on_gpu():
    """Gradient over all tokens == sum of gradients over two token ranges (accumulate)."""
    cfg = _small_vggt(views=3, heads=4)
    inp = make_inputs(cfg, DEV, with_q=False)
    Vp = _conv(inp)
    full = tla.ttt_grad(inp.K, Vp, inp.theta0, cfg.n_heads)
    cut = 1500
    part = tla.ttt_grad(inp.K[:cut].contiguous(), Vp[:cut].contiguous(), inp.theta0, cfg.n_heads)
    tla.ttt_grad(inp.K[cut:].contiguous(), Vp[cut:].contiguous(), inp.theta0, cfg.n_heads, grad=part,
                 accumulate=True)
    err = rel_err_per_head(to64(part), to64(full), cfg.n_heads, axis_cols=False)
    assert err.max() <= 1e-5, err


def test_determinism_bitwise():
    cfg = _small_vggt(views=3, steps=2)
    inp = make_inputs(cfg, DEV)
    outs = []
    for _ in range(2):
        Vp = _conv(inp)
        th = inp.theta0.clone()
        tla.ttt_write(inp.K, Vp, th, cfg.lr, cfg.steps, cfg.n_heads)
        O = tla.ttt_read(inp.Q, th, cfg.n_heads)
        outs.append((bits(Vp), bits(th), bits(O)))
    for x, y in zip(*outs):
        np.testing.assert_array_equal(x, y)


def test_empty_scene_and_single_token():
    cfg = _small_vggt(views=1, heads=2)
    inp = make_inputs(cfg, DEV)
    th = inp.theta0.clone()
    loss = torch.full((2, cfg.n_heads), 7.0, device=DEV)
    tla.ttt_write(inp.K[:0], inp.V[:0], th, 0.1, 2, cfg.n_heads, loss_out=loss)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(th), bits(inp.theta0))
    assert torch.all(loss == 0)
    O = tla.ttt_read(inp.Q[:0], th, cfg.n_heads)
    assert O.shape[0] == 0
    g = tla.ttt_grad(inp.K[:0], inp.V[:0], th, cfg.n_heads)
    assert torch.all(g == 0)
    # one token
    Vp = _conv(inp)
    K1, V1 = inp.K[:1].contiguous(), Vp[:1].contiguous()
    tla.ttt_write(K1, V1, th, 0.1, 1, cfg.n_heads)
    ref, _, _ = oracle.ttt_write(to64(K1), to64(V1), inp.theta0.cpu().numpy(), cfg.n_heads, cfg.d_head,
                                 cfg.d_hidden, 0.1, 1)
    th0 = inp.theta0.cpu().numpy()
    d = rel_err_per_head(th.cpu().numpy() - th0, ref - th0, cfg.n_heads, axis_cols=False)
    assert d.max() <= TOL_BF16, d


# ----------------------------------------------------------------------------
# fp32 mode
# ----------------------------------------------------------------------------

def test_tiny_f32_layer_parity():
    """2 views of 8x8 patches, 1 head, d 16, hidden 32, fp32, 1 step, then the read."""
    cfg = CONFIGS["tiny_f32"]
    inp = make_inputs(cfg, DEV)
    Vp = _conv(inp)
    theta = inp.theta0.clone()
    loss = torch.empty((cfg.steps, cfg.n_heads), device=DEV)
    tla.ttt_write(inp.K, Vp, theta, cfg.lr, cfg.steps, cfg.n_heads, loss_out=loss)
    O = tla.ttt_read(inp.Q, theta, cfg.n_heads)
    th0 = inp.theta0.cpu().numpy()
    Vp_ref = _oracle_conv(inp, "f32")
    np.testing.assert_array_equal(bits(Vp), f32_to_bits(Vp_ref, False))
    th_ref, L_ref, _ = oracle.ttt_write(to64(inp.K), Vp_ref.astype(np.float64), th0, 1, 16, 32, cfg.lr, cfg.steps)
    th = theta.cpu().numpy().astype(np.float64)
    assert rel_err(th, th_ref) <= TOL_F32
    ok, worst = dtheta_ok(th, th_ref, th0, 1, TOL_F32, cfg.steps)
    assert ok, worst
    assert abs(loss.item() - L_ref[0, 0]) / L_ref[0, 0] <= TOL_F32
    g = tla.ttt_grad(inp.K, Vp, inp.theta0, 1)
    g_ref, _ = oracle.ttt_grad(to64(inp.K), Vp_ref.astype(np.float64), th0, 1, 16, 32)
    assert rel_err(to64(g), g_ref) <= TOL_F32
    O_ref = oracle.ttt_read(to64(inp.Q), th_ref, 1, 16, 32)
    assert rel_err(to64(O), O_ref) <= TOL_F32


@pytest.mark.parametrize("recipe", [("mse", "gd"), ("dot", "muon")], ids=lambda r: "_".join(r))
def test_tiny_bf16_layer_parity(recipe):
    """The (16, 32) head shape with bf16 token tensors: 2 views of 8x8 patches, 3
    heads, 2 steps, then the read. The fp32 kernels serve it (exact widening of
    the bf16 inputs, fp32 arithmetic), so the write meets the fp32 bar; the read's
    output is rounded to bf16."""
    from dataclasses import replace
    cfg = replace(CONFIGS["tiny_f32"], dtype="bf16", n_heads=3, steps=2, normalize=True, name="tiny_bf16")
    inp = make_inputs(cfg, DEV)
    assert inp.K.dtype == torch.bfloat16
    Vp = _conv(inp)
    theta = inp.theta0.clone()
    loss = torch.empty((cfg.steps, cfg.n_heads), device=DEV)
    tla.ttt_write(inp.K, Vp, theta, cfg.lr, cfg.steps, cfg.n_heads, loss_out=loss, loss=recipe[0],
                  optimizer=recipe[1])
    O = tla.ttt_read(inp.Q, theta, cfg.n_heads)
    th0 = inp.theta0.cpu().numpy()
    Vp_ref = _oracle_conv(inp, "bf16").astype(np.float64)
    np.testing.assert_array_equal(bits(Vp), f32_to_bits(Vp_ref.astype(np.float32), True))
    th_ref, L_ref, _ = oracle.ttt_write(to64(inp.K), Vp_ref, th0, cfg.n_heads, 16, 32, cfg.lr, cfg.steps,
                                        loss=recipe[0], opt=recipe[1])
    th = theta.cpu().numpy().astype(np.float64)
    err = rel_err_per_head(th, th_ref, cfg.n_heads, axis_cols=False).max()
    ok, worst = dtheta_ok(th, th_ref, th0, cfg.n_heads, TOL_F32 if recipe[1] == "gd" else 1e-3, cfg.steps)
    print(f"[bf16 16x32 {recipe}] theta {err:.2e}, delta-theta worst/allowance {worst:.2f}", flush=True)
    assert err <= TOL_F32
    assert ok, worst
    if recipe[0] == "mse":
        lerr = np.abs(loss.cpu().numpy() - L_ref) / np.abs(L_ref)
        assert lerr.max() <= TOL_F32, lerr
    O_ref = oracle.ttt_read(to64(inp.Q), th_ref, cfg.n_heads, 16, 32)
    oerr = rel_err_per_head(to64(O), O_ref, cfg.n_heads).max()
    print(f"[bf16 16x32 {recipe}] read {oerr:.2e}", flush=True)
    assert oerr <= 4e-3  # one bf16 rounding of each output
    g = tla.ttt_grad(inp.K, Vp, inp.theta0, cfg.n_heads, loss=recipe[0])
    g_ref, _ = oracle.ttt_grad(to64(inp.K), Vp_ref, th0, cfg.n_heads, 16, 32, loss=recipe[0])
    assert rel_err_per_head(to64(g).reshape(cfg.n_heads, -1), g_ref.reshape(cfg.n_heads, -1), cfg.n_heads,
                            axis_cols=False).max() <= TOL_F32


def test_f32_vggt_shape_parity():
    cfg = _small_vggt(views=2, heads=2, dtype="f32", steps=2)
    inp = make_inputs(cfg, DEV)
    Vp = _conv(inp)
    theta = inp.theta0.clone()
    tla.ttt_write(inp.K, Vp, theta, cfg.lr, cfg.steps, cfg.n_heads)
    O = tla.ttt_read(inp.Q, theta, cfg.n_heads)
    th0 = inp.theta0.cpu().numpy()
    Vp_ref = _oracle_conv(inp, "f32").astype(np.float64)
    th_ref, _, _ = oracle.ttt_write(to64(inp.K), Vp_ref, th0, cfg.n_heads, 64, 128, cfg.lr, cfg.steps)
    th = theta.cpu().numpy().astype(np.float64)
    assert rel_err_per_head(th, th_ref, cfg.n_heads, axis_cols=False).max() <= TOL_F32
    ok, worst = dtheta_ok(th, th_ref, th0, cfg.n_heads, TOL_F32, cfg.steps)
    assert ok, worst
    g = tla.ttt_grad(inp.K, Vp, inp.theta0, cfg.n_heads)
    g_ref, _ = oracle.ttt_grad(to64(inp.K), Vp_ref, th0, cfg.n_heads, 64, 128)
    assert rel_err_per_head(to64(g), g_ref, cfg.n_heads, axis_cols=False).max() <= TOL_F32
    O_ref = oracle.ttt_read(to64(inp.Q), th_ref, cfg.n_heads, 64, 128)
    assert rel_err_per_head(to64(O), O_ref, cfg.n_heads).max() <= TOL_F32
