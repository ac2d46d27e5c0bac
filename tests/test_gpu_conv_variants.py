"""The pages' ShortConv2D variants of Table 9 (Appendix C) on the GPU.

"V-5": a 5x5 depthwise filter on the values, checked bit for bit against the
oracle's conv contract (row offset outer, column offset inner, separately
rounded fp32 product and sum, bf16 round to nearest even). "KV-3": the 3x3
conv applied to the keys as well (own filters), checked through a whole layer
against the oracle doing the same.
"""
from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import test_layer_amd as tla
from synth import CONFIGS, make_inputs
from tests.gpu_util import bits, f32_to_bits, rel_err_per_head, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tla.lib()


def _filters(C, k, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn((C, k, k), generator=g) / k).to(DEV)


V5_CASES = [
    # (views, grid_h, grid_w, n_special, heads, d_head, dtype)
    (3, 37, 37, 5, 16, 64, "bf16"),
    (2, 5, 7, 2, 1, 64, "bf16"),
    (2, 1, 3, 1, 1, 8, "bf16"),
    (2, 8, 8, 0, 1, 16, "f32"),
    (1, 14, 27, 0, 2, 32, "bf16"),
]


@pytest.mark.parametrize("case", V5_CASES, ids=lambda c: "x".join(map(str, c)))
def test_shortconv_5x5_bitexact(case):
    views, gh, gw, ns, H, d, dt = case
    print(f"[conv5] {case}", flush=True)
    cfg = replace(CONFIGS["tiny_f32"], n_views=views, grid_h=gh, grid_w=gw, n_special=ns, n_heads=H, d_head=d,
                  d_hidden=2 * d, dtype=dt, normalize=(dt == "bf16"), name="conv5")
    inp = make_inputs(cfg, DEV, with_q=False)
    w5 = _filters(cfg.channels, 5, 31)
    Vp = tla.shortconv(inp.V, w5, views, gh, gw, ns)
    torch.cuda.synchronize()
    ref = oracle.shortconv(to64(inp.V).astype(np.float32), w5.cpu().numpy(), views, gh, gw, ns,
                           out="bf16" if dt == "bf16" else "f32")
    np.testing.assert_array_equal(bits(Vp), f32_to_bits(ref, dt == "bf16"))


def test_shortconv_5x5_delta_is_identity():
    cfg = replace(CONFIGS["views24"], n_views=2, name="conv5id")
    inp = make_inputs(cfg, DEV, with_q=False)
    w = torch.zeros((cfg.channels, 5, 5), device=DEV)
    w[:, 2, 2] = 1.0
    Vp = tla.shortconv(inp.V, w, cfg.n_views, cfg.grid_h, cfg.grid_w, cfg.n_special)
    np.testing.assert_array_equal(bits(Vp), bits(inp.V))


def test_kv3_layer_parity():
    cfg = replace(CONFIGS["views24"], n_views=3, steps=2, name="kv3")
    print("[kv3] layer", flush=True)
    inp = make_inputs(cfg, DEV)
    wk = _filters(cfg.channels, 3, 41)
    theta = inp.theta0.clone()
    O, Vp = tla.ttt_layer(inp.K, inp.V, inp.Q, theta, inp.conv_w, cfg.n_views, cfg.grid_h, cfg.grid_w,
                          cfg.n_special, cfg.n_heads, cfg.lr, cfg.steps, conv_k=wk)
    Kp = tla.shortconv(inp.K, wk, cfg.n_views, cfg.grid_h, cfg.grid_w, cfg.n_special)
    torch.cuda.synchronize()
    args = (cfg.n_views, cfg.grid_h, cfg.grid_w, cfg.n_special)
    Kp_ref = oracle.shortconv(to64(inp.K).astype(np.float32), wk.cpu().numpy(), *args, out="bf16")
    Vp_ref = oracle.shortconv(to64(inp.V).astype(np.float32), inp.conv_w.cpu().numpy(), *args, out="bf16")
    np.testing.assert_array_equal(bits(Kp), f32_to_bits(Kp_ref, True))
    np.testing.assert_array_equal(bits(Vp), f32_to_bits(Vp_ref, True))
    th0 = inp.theta0.cpu().numpy()
    th_ref, _, _ = oracle.ttt_write(Kp_ref.astype(np.float64), Vp_ref.astype(np.float64), th0, cfg.n_heads,
                                    cfg.d_head, cfg.d_hidden, cfg.lr, cfg.steps)
    th = theta.cpu().numpy().astype(np.float64)
    dth = rel_err_per_head(th - th0, th_ref - th0, cfg.n_heads, axis_cols=False)
    O_ref = oracle.ttt_read(to64(inp.Q), th_ref, cfg.n_heads, cfg.d_head, cfg.d_hidden)
    oerr = rel_err_per_head(to64(O), O_ref, cfg.n_heads)
    print(f"  delta-theta {dth.max():.3e}, read {oerr.max():.3e}", flush=True)
    assert dth.max() <= 2e-2, dth
    assert oerr.max() <= 2e-2, oerr
