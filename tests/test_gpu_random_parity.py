"""Randomized parity sweep (fixed seed): the write and the read against the
oracle on drawn shapes, across dtypes (bf16, fp32), head shapes (64, 128) and
(16, 32), both inner losses, both updates, 1 to 3 steps, token counts around
the kernels' tile and chunk edges, and small or large fast weights ([GRAPH]
"VGG-T3: Offline Feed-Forward 3D Reconstruction at Scale", section 3.4,
Eq. 3 (write) and Eq. 4 (read), "TTT MLP Architecture and Inner
Optimization", "Muon optimizer for inner loop").

Bars are the contract's: 2e-2 for bf16 compute, 1e-4 for fp32 arithmetic (the
fp32 mode, and bf16 tokens at (16, 32), which the fp32 kernels serve), with the
fp32-storage floor on Delta-theta that `dtheta_ok` states. One exception: with
fewer tokens than hidden units the gradient is rank-deficient, and the
Newton-Schulz map amplifies rounding in its null space (a one-token gradient
is exactly rank 1, and the oracle's own Muon update then moves by about 1e-4
when its gradient is perturbed at fp32 rounding level). So for an fp32 Muon
write the bar is the larger of 1e-4 and twice that measured sensitivity of the
oracle; bf16 keeps the plain 2e-2. The read is checked on the GPU's own theta*,
so that its error is the read's alone.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import test_layer_amd as tla
from tests.gpu_util import dtheta_ok, rel_err_per_head

pytestmark = pytest.mark.gpu

DEV = "cuda"
SPECIAL_N = [1, 15, 16, 17, 31, 32, 33, 47, 48, 63, 64, 65, 1023, 1024, 1025, 4096, 4097]
N_CASES = 24


def _case(i: int):
    rng = np.random.default_rng(1000 + i)
    dt = ["bf16", "f32"][i % 2]
    d, m = [(64, 128), (16, 32)][(i // 2) % 2]
    loss = ["mse", "dot"][(i // 4) % 2]
    opt = ["gd", "muon"][(i // 8) % 2]
    H = int(rng.choice([1, 2, 3, 5, 8, 16]))
    n = int(rng.choice(SPECIAL_N)) if rng.random() < 0.5 else int(rng.integers(1, 6000))
    steps = int(rng.integers(1, 4))
    scale = float(rng.choice([0.02, 0.3]))
    return dict(dt=dt, d=d, m=m, loss=loss, opt=opt, H=H, n=n, steps=steps, scale=scale, seed=2000 + i)


def _muon_sensitivity(K64, V64, t0, H, d, m, c):
    """Largest per-head relative change of the oracle's first Muon update when
    its gradient is perturbed by relative noise at fp32 rounding level (2^-24)."""
    grad, _ = oracle.ttt_grad(K64, V64, t0, H, d, m, loss=c["loss"])
    upd = oracle.muon_apply(t0, grad, 0.1, H, d, m, 5) - t0
    rng = np.random.default_rng(c["seed"])
    worst = 0.0
    for _ in range(3):
        gp = grad * (1.0 + 2.0 ** -24 * rng.standard_normal(grad.shape))
        up = oracle.muon_apply(t0, gp, 0.1, H, d, m, 5) - t0
        worst = max(worst, max(float(np.abs(up[h] - upd[h]).max() / np.abs(upd[h]).max()) for h in range(H)))
    return worst


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tla.lib()


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_write_and_read_match_the_oracle(i):
    c = _case(i)
    print(f"[random parity {i}] {c}", flush=True)
    d, m, H, n = c["d"], c["m"], c["H"], c["n"]
    g = torch.Generator(device="cpu").manual_seed(c["seed"])
    tdt = torch.bfloat16 if c["dt"] == "bf16" else torch.float32
    K, V, Q = ((torch.randn((n, H * d), generator=g) / np.sqrt(d)).to(tdt) for _ in range(3))
    th0 = torch.randn((H, 3 * d * m), generator=g) * c["scale"]
    th = th0.to(DEV)
    tla.ttt_write(K.to(DEV), V.to(DEV), th, 0.1, c["steps"], H, d_hidden=m, loss=c["loss"], optimizer=c["opt"])
    O = tla.ttt_read(Q.to(DEV), th, H, d_hidden=m)
    torch.cuda.synchronize()
    th_gpu = th.cpu().numpy().astype(np.float64)
    t0 = th0.numpy().astype(np.float64)
    K64, V64, Q64 = (x.to(torch.float64).numpy() for x in (K, V, Q))
    th_ref, _, _ = oracle.ttt_write(K64, V64, t0, H, d, m, 0.1, c["steps"], loss=c["loss"], opt=c["opt"])
    exact32 = c["dt"] == "f32" or (d, m) == (16, 32)
    bar_w = 1e-4 if exact32 else 2e-2
    if exact32 and c["opt"] == "muon":
        bar_w = max(bar_w, 2.0 * _muon_sensitivity(K64, V64, t0, H, d, m, c))
    dth = rel_err_per_head(th_gpu - t0, th_ref - t0, H, axis_cols=False).max()
    ok_w = dth <= bar_w or (exact32 and dtheta_ok(th_gpu, th_ref, t0, H, bar_w, c["steps"])[0])
    O_ref = oracle.ttt_read(Q64, th_gpu, H, d, m)
    oerr = rel_err_per_head(O.cpu().to(torch.float64).numpy(), O_ref, H).max()
    bar_o = 1e-4 if c["dt"] == "f32" else 2e-2
    print(f"  delta-theta {dth:.2e} (bar {bar_w:g}), read {oerr:.2e} (bar {bar_o:g})", flush=True)
    assert ok_w, dth
    assert oerr <= bar_o, oerr
