"""The ShortConv2D fused into the write (vggt3_ttt_write_conv): V' is formed
inside each gradient pass from a ring of V rows in LDS ([GRAPH] section 3.4,
"Non-Linear Spatial Mixing via ShortConv2D" feeding the write of "The
Test-Time Training (TTT) Framework").

  * bitwise equal to vggt3_shortconv followed by vggt3_ttt_write_ex (both
    losses, both updates, with and without the V' output and the loss
    values), on grids from 1 x 3 to the widest the ring takes (47 columns),
    with special tokens, ragged last tiles and 1 to 64 chunks per head;
  * the V' it emits is bitwise vggt3_shortconv's;
  * against the oracle (its conv, then its 2-step write) at the small VGGT shape;
  * reads no V row past the scene and writes nothing past its outputs;
  * at 1000 views, bitwise equal to the split path.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import test_layer_amd as tla
from synth import CONFIGS, make_inputs
from tests.gpu_util import bits, rel_err_per_head, to64

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL_BF16 = 2e-2
PH = 3 * 64 * 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tla.lib()


def _scene(nv, gh, gw, ns, H, seed):
    n = nv * (ns + gh * gw)
    C = 64 * H
    g = torch.Generator(device=DEV).manual_seed(seed)
    K = (torch.randn((n, C), generator=g, device=DEV) / 8).to(torch.bfloat16)
    V = (torch.randn((n, C), generator=g, device=DEV) / 8).to(torch.bfloat16)
    w = torch.randn((C, 3, 3), generator=g, device=DEV) / 3
    th0 = torch.randn((H, PH), generator=g, device=DEV) * 0.02
    return K, V, w, th0


GEOMS = [
    # (views, grid_h, grid_w, n_special, heads)
    (3, 37, 37, 5, 16),  # the pages' grid, 32 chunks per head
    (2, 5, 7, 2, 2),
    (3, 4, 1, 1, 1),     # one-column grid, one chunk
    (2, 47, 47, 5, 4),   # the widest grid the ring holds, 64 chunks
    (5, 1, 3, 0, 3),     # one-row grid
    (2, 3, 3, 30, 2),    # more special than patch tokens
    (7, 9, 11, 0, 5),    # no special tokens, ragged last tile
]
RECIPES = [("mse", "gd"), ("dot", "muon")]


def _split_write(K, V, w, geom, th0, recipe, with_loss, lr=0.1, steps=2):
    nv, gh, gw, ns, H = geom
    Vp = tla.shortconv(V, w, nv, gh, gw, ns)
    th = th0.clone()
    loss = torch.empty((steps, H), device=DEV) if with_loss else None
    tla.ttt_write(K, Vp, th, lr, steps, H, loss_out=loss, loss=recipe[0], optimizer=recipe[1])
    return Vp, th, loss


@pytest.mark.parametrize("vout", [False, True], ids=["no_vp", "vp_out"])
@pytest.mark.parametrize("with_loss", [False, True], ids=["noloss", "loss"])
@pytest.mark.parametrize("recipe", RECIPES, ids=lambda r: "_".join(r))
@pytest.mark.parametrize("geom", GEOMS, ids=lambda g: "v{}_{}x{}_s{}_h{}".format(*g))
def test_fused_write_equals_conv_then_write_bitwise(geom, recipe, with_loss, vout):
    nv, gh, gw, ns, H = geom
    print(f"[fused conv] {geom} {recipe} loss={with_loss} vout={vout}", flush=True)
    K, V, w, th0 = _scene(nv, gh, gw, ns, H, seed=sum(geom))
    Vp, th_ref, L_ref = _split_write(K, V, w, geom, th0, recipe, with_loss)
    th = th0.clone()
    loss = torch.empty((2, H), device=DEV) if with_loss else None
    Vo = torch.full_like(V, 7.0) if vout else None
    tla.ttt_write_conv(K, V, w, nv, gh, gw, ns, th, 0.1, 2, H, Vp_out=Vo, loss_out=loss, loss=recipe[0],
                       optimizer=recipe[1])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(th), bits(th_ref))
    if with_loss:
        np.testing.assert_array_equal(bits(loss), bits(L_ref))
    if vout:
        np.testing.assert_array_equal(bits(Vo), bits(Vp))


@pytest.mark.parametrize("recipe", [("dot", "gd"), ("mse", "muon")], ids=lambda r: "_".join(r))
def test_fused_write_other_recipes_bitwise(recipe):
    geom = (3, 37, 37, 5, 16)
    nv, gh, gw, ns, H = geom
    K, V, w, th0 = _scene(nv, gh, gw, ns, H, seed=5)
    _, th_ref, L_ref = _split_write(K, V, w, geom, th0, recipe, True)
    th = th0.clone()
    loss = torch.empty((2, H), device=DEV)
    tla.ttt_write_conv(K, V, w, nv, gh, gw, ns, th, 0.1, 2, H, loss_out=loss, loss=recipe[0], optimizer=recipe[1])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(th), bits(th_ref))
    np.testing.assert_array_equal(bits(loss), bits(L_ref))


def test_fused_write_against_oracle():
    """The oracle's own conv and 2-step write at 3 views, 16 heads."""
    from dataclasses import replace
    cfg = replace(CONFIGS["views24"], n_views=3, steps=2, name="vggt3v16h")
    inp = make_inputs(cfg, DEV, with_q=False)
    theta = inp.theta0.clone()
    loss = torch.empty((cfg.steps, cfg.n_heads), device=DEV)
    tla.ttt_write_conv(inp.K, inp.V, inp.conv_w, cfg.n_views, cfg.grid_h, cfg.grid_w, cfg.n_special, theta, cfg.lr,
                       cfg.steps, cfg.n_heads, loss_out=loss)
    th0 = inp.theta0.cpu().numpy()
    Vp_ref = oracle.shortconv(to64(inp.V).astype(np.float32), inp.conv_w.cpu().numpy(), cfg.n_views, cfg.grid_h,
                              cfg.grid_w, cfg.n_special, out="bf16").astype(np.float64)
    th_ref, L_ref, _ = oracle.ttt_write(to64(inp.K), Vp_ref, th0, cfg.n_heads, cfg.d_head, cfg.d_hidden, cfg.lr,
                                        cfg.steps)
    th = theta.cpu().numpy().astype(np.float64)
    assert rel_err_per_head(th, th_ref, cfg.n_heads, axis_cols=False).max() <= TOL_BF16
    dth = rel_err_per_head(th - th0, th_ref - th0, cfg.n_heads, axis_cols=False)
    print(f"[fused conv vs oracle] delta-theta {dth.max():.2e}", flush=True)
    assert dth.max() <= TOL_BF16, dth
    lerr = np.abs(loss.cpu().numpy() - L_ref) / np.abs(L_ref)
    assert lerr.max() <= TOL_BF16, lerr


def test_fused_write_stays_within_its_rows():
    """V and K views of the first n rows of larger buffers whose remaining rows
    are NaN: same bits as exact-size tensors; nothing written past V', the
    workspace or the loss output."""
    nv, gh, gw, ns, H = 2, 9, 11, 3, 4
    n = nv * (ns + gh * gw)
    C = 64 * H
    PAD, TAIL = 64, 4096
    K, V, w, th0 = _scene(nv, gh, gw, ns, H, seed=77)
    Vp, th_ref, L_ref = _split_write(K, V, w, (nv, gh, gw, ns, H), th0, ("mse", "gd"), True)

    def padded(src):
        big = torch.empty((n + PAD, C), dtype=torch.bfloat16, device=DEV)
        big.view(torch.int16).fill_(0x7FA5)  # a bf16 NaN
        if src is not None:
            big[:n].copy_(src)
        return big
    kb, vb, ob = padded(K), padded(V), padded(None)
    need = tla.workspace_bytes(n, H, 64, 128, tla.BF16)
    wbuf = torch.full((need + TAIL,), 0xA5, dtype=torch.uint8, device=DEV)
    lbuf = torch.full((2 * H + 8,), float("nan"), device=DEV)
    th = th0.clone()
    tla.ttt_write_conv(kb[:n], vb[:n], w, nv, gh, gw, ns, th, 0.1, 2, H, Vp_out=ob[:n], workspace=wbuf[:need],
                       loss_out=lbuf[:2 * H])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(th), bits(th_ref))
    np.testing.assert_array_equal(bits(lbuf[:2 * H].view(2, H)), bits(L_ref))
    np.testing.assert_array_equal(bits(ob[:n]), bits(Vp))
    assert bool((ob[n:].view(torch.int16) == 0x7FA5).all()), "V' rows past the scene were written"
    assert bool((wbuf[need:] == 0xA5).all()), "workspace overrun"
    assert bool(torch.isnan(lbuf[2 * H:]).all()), "loss output overrun"


def test_fused_write_empty_scene():
    H = 2
    th0 = torch.randn((H, PH), device=DEV)
    th = th0.clone()
    loss = torch.full((3, H), 5.0, device=DEV)
    e = torch.empty((0, 64 * H), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((64 * H, 3, 3), device=DEV)
    tla.ttt_write_conv(e, e.clone(), w, 0, 37, 37, 5, th, 0.1, 3, H, loss_out=loss)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(th), bits(th0))
    assert bool((loss == 0).all())


def test_fused_write_views1000_bitwise():
    cfg = CONFIGS["views1000"]
    print(f"[fused conv] views1000 n={cfg.n_tokens}", flush=True)
    inp = make_inputs(cfg, DEV, with_q=False)
    geom = (cfg.n_views, cfg.grid_h, cfg.grid_w, cfg.n_special, cfg.n_heads)
    Vp, th_ref, L_ref = _split_write(inp.K, inp.V, inp.conv_w, geom, inp.theta0, ("mse", "gd"), True, lr=cfg.lr,
                                     steps=cfg.steps)
    for vout in (False, True):
        th = inp.theta0.clone()
        loss = torch.empty((cfg.steps, cfg.n_heads), device=DEV)
        Vo = torch.empty_like(inp.V) if vout else None
        tla.ttt_write_conv(inp.K, inp.V, inp.conv_w, *geom[:4], th, cfg.lr, cfg.steps, cfg.n_heads, Vp_out=Vo,
                           loss_out=loss)
        torch.cuda.synchronize()
        assert torch.equal(th.view(torch.int32), th_ref.view(torch.int32))
        assert torch.equal(loss.view(torch.int32), L_ref.view(torch.int32))
        if vout:
            assert torch.equal(Vo.view(torch.int16), Vp.view(torch.int16))
        del Vo
