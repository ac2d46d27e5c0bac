"""Streamed (offloaded) write and read over host-resident token tensors.

[GRAPH] "Large-Scale Inference Strategies": a single GPU processes a scene
larger than its memory by loading one minibatch at a time, computing its
gradient, accumulating, and applying the summed update (exact by Eq. 5); query
mode reads a frozen theta* the same way.

Bars:
  * the streamed write equals, bit for bit, the device-resident sequence it
    pipelines: ttt_grad on each chunk with accumulate, then one ttt_apply or
    ttt_muon_apply per step (a race between the copy and compute streams, a
    stale staging slot or a wrong chunk offset breaks this);
  * the streamed read equals ttt_read bit for bit;
  * against the oracle's offload schedule (oracle.ttt_write_offload, pinned to
    the full-batch write): 2e-2 on the bf16 path, 1e-4 on the fp32 path.
"""
from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import test_layer_amd as tla
from synth import CONFIGS, make_inputs
from tests.gpu_util import bits, dtheta_ok, rel_err_per_head, to64

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 1e-4
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tla.lib()


def _pinned(t: torch.Tensor) -> torch.Tensor:
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


def _cfg(views=3, heads=16, steps=2):
    return replace(CONFIGS["views24"], n_views=views, n_heads=heads, steps=steps, name=f"stream{views}v{heads}h")


def _scene(cfg):
    inp = make_inputs(cfg, DEV, with_q=True)
    Vp = tla.shortconv(inp.V, inp.conv_w, cfg.n_views, cfg.grid_h, cfg.grid_w, cfg.n_special)
    torch.cuda.synchronize()
    return inp, Vp


def _oracle_vp(inp, out):
    """V' computed by the oracle from the same V (its conv is bit-exact)."""
    c = inp.cfg
    return oracle.shortconv(to64(inp.V).astype(np.float32), inp.conv_w.cpu().numpy(), c.n_views, c.grid_h,
                            c.grid_w, c.n_special, out=out).astype(np.float64)


def _chunked_reference(K, Vp, theta0, cfg, chunk, loss, opt, ns_steps=5):
    """The device-resident sequence the streamed write pipelines."""
    theta = theta0.clone()
    n = K.shape[0]
    # one 16-byte aligned loss row per step (rows of [steps][heads] are not,
    # for a single head)
    rows = [torch.zeros(cfg.n_heads, device=DEV) for _ in range(cfg.steps)]
    g = torch.empty_like(theta)
    for st in range(cfg.steps):
        for c, t0 in enumerate(range(0, n, chunk)):
            tla.ttt_grad(K[t0:t0 + chunk], Vp[t0:t0 + chunk], theta, cfg.n_heads, grad=g, accumulate=c > 0,
                         loss_out=rows[st], loss=loss)
        if opt == "gd":
            tla.ttt_apply(theta, g, cfg.lr, cfg.n_heads, cfg.d_head, cfg.d_hidden)
        else:
            tla.ttt_muon_apply(theta, g, cfg.lr, cfg.n_heads, cfg.d_head, cfg.d_hidden, ns_steps)
    torch.cuda.synchronize()
    return theta, torch.stack(rows)


# chunk sizes for a 3-view scene of 4,122 tokens: many ragged chunks through
# the two slots, two chunks (the resident case), one chunk, a chunk larger
# than the scene, and a chunk shorter than one kernel tile
CHUNKS = [1000, 2500, 2061, 4122, 100_000, 37]


@pytest.mark.parametrize("chunk", CHUNKS)
@pytest.mark.parametrize("recipe", [("mse", "gd"), ("dot", "muon")], ids=["mse_gd", "dot_muon"])
def test_write_streamed_equals_chunked_grad_bitwise(chunk, recipe):
    loss, opt = recipe
    cfg = _cfg()
    print(f"[stream] write bitwise chunk {chunk} {loss}/{opt}", flush=True)
    inp, Vp = _scene(cfg)
    ref_theta, ref_losses = _chunked_reference(inp.K, Vp, inp.theta0, cfg, chunk, loss, opt)
    Kh, Vh = _pinned(inp.K), _pinned(Vp)
    theta = inp.theta0.clone()
    losses = torch.full((cfg.steps, cfg.n_heads), float("nan"), device=DEV)
    tla.ttt_write_streamed(Kh, Vh, theta, cfg.lr, cfg.steps, cfg.n_heads, chunk, loss_out=losses, loss=loss,
                           optimizer=opt)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(theta), bits(ref_theta))
    np.testing.assert_array_equal(bits(losses), bits(ref_losses))


def test_write_streamed_copy_stream_choice_does_not_change_bits():
    cfg = _cfg(views=2, heads=4)
    inp, Vp = _scene(cfg)
    Kh, Vh = _pinned(inp.K), _pinned(Vp)
    outs = []
    for cs in (None, torch.cuda.current_stream(), torch.cuda.Stream()):
        theta = inp.theta0.clone()
        tla.ttt_write_streamed(Kh, Vh, theta, cfg.lr, cfg.steps, cfg.n_heads, 700, copy_stream=cs)
        torch.cuda.synchronize()
        outs.append(bits(theta))
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], outs[2])


def test_write_streamed_bf16_oracle_parity():
    cfg = _cfg(views=3, heads=16)
    print("[stream] write bf16 vs oracle offload schedule", flush=True)
    inp, Vp = _scene(cfg)
    theta = inp.theta0.clone()
    losses = torch.empty((cfg.steps, cfg.n_heads), device=DEV)
    tla.ttt_write_streamed(_pinned(inp.K), _pinned(Vp), theta, cfg.lr, cfg.steps, cfg.n_heads, 1000,
                           loss_out=losses)
    torch.cuda.synchronize()
    th0 = inp.theta0.cpu().numpy()
    th_ref, L_ref = oracle.ttt_write_offload(to64(inp.K), _oracle_vp(inp, "bf16"), th0, cfg.n_heads, cfg.d_head,
                                             cfg.d_hidden, cfg.lr, cfg.steps, minibatch=1000)
    ok, worst = dtheta_ok(theta.cpu().numpy().astype(np.float64), th_ref, th0, cfg.n_heads, TOL_BF16, cfg.steps)
    print(f"  dtheta worst/allowance {worst:.3f}", flush=True)
    assert ok, worst
    e = np.abs(losses.cpu().numpy() - L_ref) / np.abs(L_ref)
    assert e.max() <= TOL_BF16, e


def test_write_streamed_f32_oracle_parity():
    cfg = replace(CONFIGS["tiny_f32"], steps=2)
    inp = make_inputs(cfg, DEV, with_q=False)
    Vp = tla.shortconv(inp.V, inp.conv_w, cfg.n_views, cfg.grid_h, cfg.grid_w, cfg.n_special)
    torch.cuda.synchronize()
    for loss, opt in (("mse", "gd"), ("dot", "muon")):
        theta = inp.theta0.clone()
        tla.ttt_write_streamed(_pinned(inp.K), _pinned(Vp), theta, cfg.lr, cfg.steps, 1, 48, loss=loss,
                               optimizer=opt)
        ref_theta, _ = _chunked_reference(inp.K, Vp, inp.theta0, cfg, 48, loss, opt)
        np.testing.assert_array_equal(bits(theta), bits(ref_theta))
        th0 = inp.theta0.cpu().numpy()
        th_ref, _ = oracle.ttt_write_offload(to64(inp.K), _oracle_vp(inp, "f32"), th0, 1, 16, 32, cfg.lr, cfg.steps,
                                             minibatch=48, loss=loss, opt=opt)
        ok, worst = dtheta_ok(theta.cpu().numpy().astype(np.float64), th_ref, th0, 1, TOL_F32, cfg.steps)
        assert ok, (loss, opt, worst)


def test_write_streamed_empty_scene_zero_losses():
    cfg = _cfg(views=1, heads=16)
    theta = torch.randn((16, 3 * 64 * 128), device=DEV)
    before = theta.clone()
    losses = torch.full((2, 16), 7.0, device=DEV)
    empty = torch.empty((0, 1024), dtype=torch.bfloat16, pin_memory=True)
    tla.ttt_write_streamed(empty, empty, theta, 0.1, 2, 16, 512, loss_out=losses)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(theta), bits(before))
    assert torch.all(losses == 0)


@pytest.mark.parametrize("chunk", [1000, 4122, 7, 100_000])
@pytest.mark.parametrize("streams", ["side", "one_copy_stream", "compute_only"])
def test_read_streamed_equals_read_bitwise(chunk, streams):
    cfg = _cfg(views=3, heads=16)
    print(f"[stream] read chunk {chunk} {streams}", flush=True)
    inp = make_inputs(cfg, DEV, with_q=True)
    theta = inp.theta0 * 5.0  # larger weights so outputs are not tiny
    ref = tla.ttt_read(inp.Q, theta, cfg.n_heads)
    Qh = _pinned(inp.Q)
    cur = torch.cuda.current_stream()
    if streams == "side":
        kw = {}
    elif streams == "one_copy_stream":
        s = torch.cuda.Stream()
        kw = dict(h2d_stream=s, d2h_stream=s)
    else:
        kw = dict(h2d_stream=cur, d2h_stream=cur)
    out = tla.ttt_read_streamed(Qh, theta, cfg.n_heads, chunk, **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), bits(ref))


def test_read_streamed_f32_and_empty():
    cfg = CONFIGS["tiny_f32"]
    inp = make_inputs(cfg, DEV, with_q=True)
    ref = tla.ttt_read(inp.Q, inp.theta0, 1)
    out = tla.ttt_read_streamed(_pinned(inp.Q), inp.theta0, 1, 40)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), bits(ref))
    O_ref = oracle.ttt_read(to64(inp.Q), inp.theta0.cpu().numpy(), 1, 16, 32)
    assert rel_err_per_head(to64(out), O_ref, 1).max() <= TOL_F32
    empty = torch.empty((0, 16), dtype=torch.float32, pin_memory=True)
    out = tla.ttt_read_streamed(empty, inp.theta0, 1, 40)
    torch.cuda.synchronize()
    assert out.shape == (0, 16)


def test_views1000_streamed_write_and_read_bitwise():
    """The 1000-view scene (1,374,000 tokens) streamed in 131,072-token chunks
    (10 full chunks and a ragged one) through the staging slots."""
    cfg = CONFIGS["views1000"]
    chunk = 131_072
    print("[stream] views1000 streamed write + read", flush=True)
    inp, Vp = _scene(cfg)
    ref_theta, ref_losses = _chunked_reference(inp.K, Vp, inp.theta0, cfg, chunk, "mse", "gd")
    Kh, Vh = _pinned(inp.K), _pinned(Vp)
    del inp.V
    theta = inp.theta0.clone()
    losses = torch.empty((cfg.steps, cfg.n_heads), device=DEV)
    tla.ttt_write_streamed(Kh, Vh, theta, cfg.lr, cfg.steps, cfg.n_heads, chunk, loss_out=losses)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(theta), bits(ref_theta))
    np.testing.assert_array_equal(bits(losses), bits(ref_losses))
    del Kh, Vh, Vp
    O_ref = tla.ttt_read(inp.Q, theta, cfg.n_heads)
    O = tla.ttt_read_streamed(_pinned(inp.Q), theta, cfg.n_heads, chunk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(O), bits(O_ref))


# ---------------------------------------------------------------------------
# the full-width 1024 -> 4096 -> 1024 MLP streamed from host memory
# ---------------------------------------------------------------------------


def _wide_cfg(views=2, steps=2):
    return replace(CONFIGS["views24"], n_views=views, n_heads=1, d_head=1024, d_hidden=4096, steps=steps,
                   name=f"wide_stream{views}v")


@pytest.mark.parametrize("recipe", [("mse", "gd"), ("dot", "muon")], ids=["mse_gd", "dot_muon"])
def test_wide_write_streamed_equals_chunked_grad_bitwise(recipe):
    """2 views (2,748 tokens) in chunks of 1,000: three chunks through the two
    slots, the last ragged; each chunk's gradient is the full-width GEMM pass."""
    loss, opt = recipe
    cfg = _wide_cfg()
    print(f"[stream] wide write {loss}/{opt}", flush=True)
    inp, Vp = _scene(cfg)
    ref_theta, ref_losses = _chunked_reference(inp.K, Vp, inp.theta0, cfg, 1000, loss, opt)
    theta = inp.theta0.clone()
    losses = torch.empty((cfg.steps, 1), device=DEV)
    tla.ttt_write_streamed(_pinned(inp.K), _pinned(Vp), theta, cfg.lr, cfg.steps, 1, 1000, loss_out=losses,
                           loss=loss, optimizer=opt)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(theta), bits(ref_theta))
    np.testing.assert_array_equal(bits(losses), bits(ref_losses))


def test_wide_read_streamed_equals_read_bitwise():
    cfg = _wide_cfg()
    inp = make_inputs(cfg, DEV, with_q=True)
    theta = inp.theta0 * 10.0
    ref = tla.ttt_read(inp.Q, theta, 1)
    out = tla.ttt_read_streamed(_pinned(inp.Q), theta, 1, 1000)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), bits(ref))
