"""vggt3_ttt_write_noalloc: the write without a caller workspace (the library's
fixed per-GPU scratch array instead), for callers that cannot allocate.

GPU: two calls in a row, the second with a smaller input (fewer tokens and
heads, another recipe), each compared with vggt3_ttt_write_ex on its own
workspace: same bits, and within the 2e-2 bar of the bf16 path.
CPU: the size limit and the unsupported shape are rejected before any HIP call.
"""
from __future__ import annotations

import ctypes
from dataclasses import replace

import numpy as np
import pytest
import torch

import test_layer_amd as tla
from synth import CONFIGS, make_inputs
from tests.gpu_util import bits, rel_err_per_head

TOL_BF16 = 2e-2
DEV = "cuda"


def _err(lib):
    return lib.vggt3_last_error().decode()


def test_noalloc_rejects_sizes_beyond_its_scratch():
    lib = tla.lib()
    dummy = ctypes.c_void_p(0x7000000000)
    # 1024 heads of the (64, 128) MLP need ~100 MB of chunk partials
    need = lib.vggt3_ttt_workspace_bytes(4096, 1024, 64, 128, tla.BF16)
    assert need > tla.NOALLOC_SCRATCH_BYTES
    rc = lib.vggt3_ttt_write_noalloc(dummy, dummy, dummy, 4096, 1024, 64, 128, 0.1, 1, 0, 0, 0, tla.BF16, None,
                                     None)
    assert rc == tla.EWORKSPACE and "scratch" in _err(lib)
    # the full-width MLP needs a workspace of gigabytes
    rc = lib.vggt3_ttt_write_noalloc(dummy, dummy, dummy, 4096, 1, 1024, 4096, 0.1, 1, 0, 0, 0, tla.BF16, None, None)
    assert rc == tla.EUNSUPPORTED
    # ordinary argument checks still apply
    rc = lib.vggt3_ttt_write_noalloc(dummy, dummy, dummy, 4096, 16, 64, 128, 0.1, 0, 0, 0, 0, tla.BF16, None, None)
    assert rc == tla.EINVAL and "steps" in _err(lib)
    # the 1000-view layer (16 heads) fits
    assert lib.vggt3_ttt_workspace_bytes(1_374_000, 16, 64, 128, tla.BF16) <= tla.NOALLOC_SCRATCH_BYTES


def _case(views, heads, steps):
    return replace(CONFIGS["views24"], n_views=views, n_heads=heads, steps=steps, name=f"noalloc{views}v{heads}h")


@pytest.mark.gpu
def test_noalloc_write_matches_the_workspace_write_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tla.lib()
    for cfg, loss, opt in ((_case(3, 16, 2), "mse", "gd"), (_case(1, 4, 2), "dot", "muon")):
        print(f"[noalloc] n={cfg.n_tokens} heads={cfg.n_heads} {loss}+{opt}", flush=True)
        inp = make_inputs(cfg, DEV, with_q=False)
        Vp = tla.shortconv(inp.V, inp.conv_w, cfg.n_views, cfg.grid_h, cfg.grid_w, cfg.n_special)
        ref = inp.theta0.clone()
        ref_loss = torch.empty((cfg.steps, cfg.n_heads), device=DEV)
        tla.ttt_write(inp.K, Vp, ref, cfg.lr, cfg.steps, cfg.n_heads, loss_out=ref_loss, loss=loss, optimizer=opt)
        got = inp.theta0.clone()
        got_loss = torch.empty((cfg.steps, cfg.n_heads), device=DEV)
        tla.ttt_write_noalloc(inp.K, Vp, got, cfg.lr, cfg.steps, cfg.n_heads, loss_out=got_loss, loss=loss,
                              optimizer=opt)
        torch.cuda.synchronize()
        th0 = inp.theta0.cpu().numpy().astype(np.float64)
        d = rel_err_per_head(got.cpu().numpy() - th0, ref.cpu().numpy() - th0, cfg.n_heads, axis_cols=False)
        print(f"  delta-theta rel diff {d.max():.3e}", flush=True)
        assert d.max() <= TOL_BF16
        np.testing.assert_array_equal(bits(got), bits(ref))
        np.testing.assert_array_equal(bits(got_loss), bits(ref_loss))
