"""Pins of the oracle's ShortConv2D and bf16 rounding (CPU only).

ShortConv2D: paper-graph summary "VGG-T3: Offline Feed-Forward 3D
Reconstruction at Scale", section 3.4 "Non-Linear Spatial Mixing via
ShortConv2D" and its Appendix A note on special tokens.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import bf16_round, shortconv, shortconv_direct

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def test_handworked_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "shortconv_handworked.json")))
    V = np.array(g["V"], dtype=np.float32)
    w = np.array(g["w"], dtype=np.float32)
    out = shortconv(V, w, g["n_views"], g["grid_h"], g["grid_w"], g["n_special"], out="f32")
    np.testing.assert_array_equal(out, np.array(g["expected"], dtype=np.float32))
    c = g["positive_zero_channel"]
    for r in g["positive_zero_rows"]:
        assert out[r, c] == 0.0 and not np.signbit(out[r, c])
    # bf16 output of small integers is exact as well
    out16 = shortconv(V, w, g["n_views"], g["grid_h"], g["grid_w"], g["n_special"], out="bf16")
    np.testing.assert_array_equal(out16, out)


@pytest.mark.parametrize("layout", [(2, 5, 7, 0), (3, 4, 4, 2), (1, 1, 1, 1), (2, 1, 6, 3)])
def test_contract_matches_bruteforce(layout):
    n_views, gh, gw, ns = layout
    C = 6
    n = n_views * (ns + gh * gw)
    V = _rand((n, C), 1)
    w = _rand((C, 3, 3), 2, 1 / 3)
    ref = shortconv_direct(V, w, n_views, gh, gw, ns)
    out = shortconv(V, w, n_views, gh, gw, ns, out="f32")
    scale = np.abs(ref).max()
    assert np.abs(out - ref).max() <= 1e-6 * scale
    # special tokens bit-identical
    tpv = ns + gh * gw
    for v in range(n_views):
        np.testing.assert_array_equal(out[v * tpv:v * tpv + ns], V[v * tpv:v * tpv + ns])


def test_contract_matches_torch_conv2d():
    n_views, gh, gw, ns, C = 3, 9, 11, 2, 8
    tpv = ns + gh * gw
    V = _rand((n_views * tpv, C), 3)
    w = _rand((C, 3, 3), 4, 1 / 3)
    grid = torch.from_numpy(V.astype(np.float64)).view(n_views, tpv, C)[:, ns:, :]
    x = grid.reshape(n_views, gh, gw, C).permute(0, 3, 1, 2)
    y = torch.nn.functional.conv2d(x, torch.from_numpy(w.astype(np.float64)).unsqueeze(1),
                                   padding=1, groups=C)
    ref = y.permute(0, 2, 3, 1).reshape(n_views, gh * gw, C).numpy()
    out = shortconv(V, w, n_views, gh, gw, ns, out="f32").reshape(n_views, tpv, C)[:, ns:, :]
    assert np.abs(out - ref).max() <= 1e-6 * np.abs(ref).max()


def test_delta_kernel_is_identity_bitexact():
    n_views, gh, gw, ns, C = 2, 6, 5, 3, 4
    V = bf16_round(_rand((n_views * (ns + gh * gw), C), 5))
    w = np.zeros((C, 3, 3), np.float32)
    w[:, 1, 1] = 1.0
    np.testing.assert_array_equal(shortconv(V, w, n_views, gh, gw, ns, out="bf16"), V)


@pytest.mark.parametrize("dy,dx", [(-1, 0), (1, 0), (0, -1), (0, 1), (1, 1), (-1, 1)])
def test_shift_kernels(dy, dx):
    n_views, gh, gw, ns, C = 2, 5, 6, 1, 3
    tpv = ns + gh * gw
    V = _rand((n_views * tpv, C), 6)
    w = np.zeros((C, 3, 3), np.float32)
    w[:, dy + 1, dx + 1] = 1.0
    out = shortconv(V, w, n_views, gh, gw, ns, out="f32").reshape(n_views, tpv, C)[:, ns:, :]
    grid = V.reshape(n_views, tpv, C)[:, ns:, :].reshape(n_views, gh, gw, C)
    exp = np.zeros_like(grid)
    for y in range(gh):
        for x in range(gw):
            if 0 <= y + dy < gh and 0 <= x + dx < gw:
                exp[:, y, x] = grid[:, y + dy, x + dx]
    np.testing.assert_array_equal(out.reshape(n_views, gh, gw, C), exp)


def test_views_do_not_mix():
    # changing view 1 must leave view 0's output untouched (conv stays within one view)
    n_views, gh, gw, ns, C = 2, 4, 4, 2, 3
    tpv = ns + gh * gw
    V = _rand((n_views * tpv, C), 7)
    w = _rand((C, 3, 3), 8)
    a = shortconv(V, w, n_views, gh, gw, ns)
    V2 = V.copy()
    V2[tpv:] += 1.0
    b = shortconv(V2, w, n_views, gh, gw, ns)
    np.testing.assert_array_equal(a[:tpv], b[:tpv])
    assert not np.array_equal(a[tpv:], b[tpv:])


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(9)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),  # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                  -(1.0 + 2 ** -8), 1.0 + 2 ** -8 + 2 ** -20], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    out = bf16_round(x)
    np.testing.assert_array_equal(out.view(np.uint32), ref.view(np.uint32))
    # ties to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> 1
    assert bf16_round(np.float32(1.0 + 2 ** -8)) == 1.0
    assert bf16_round(np.float32(1.0 + 3 * 2 ** -8)) == np.float32(1.0 + 2 ** -6)
    assert np.isnan(bf16_round(np.float32(np.nan)))


def test_contract_rounding_order_matters():
    """The contract is a specific float32 evaluation order; a fused or fp64
    evaluation differs in the last bit on some inputs. This guards against the
    oracle silently computing in higher precision."""
    n_views, gh, gw, ns, C = 4, 8, 8, 0, 16
    V = _rand((n_views * gh * gw, C), 10)
    w = _rand((C, 3, 3), 11, 1 / 3)
    out = shortconv(V, w, n_views, gh, gw, ns, out="f32")
    ref64 = shortconv_direct(V[:gh * gw * 1], w, 1, gh, gw, ns).astype(np.float32)
    assert not np.array_equal(out[:gh * gw], ref64)


# ---- k x k filters: the pages' V-5 variant of ShortConv2D (Table 9) --------


@pytest.mark.parametrize("layout", [(2, 6, 7, 1), (1, 2, 3, 0), (2, 1, 1, 2)])
def test_5x5_contract_matches_bruteforce(layout):
    n_views, gh, gw, ns = layout
    C = 4
    V = _rand((n_views * (ns + gh * gw), C), 21)
    w = _rand((C, 5, 5), 22, 1 / 5)
    ref = shortconv_direct(V, w, n_views, gh, gw, ns)
    out = shortconv(V, w, n_views, gh, gw, ns, out="f32")
    assert np.abs(out - ref).max() <= 1e-6 * max(np.abs(ref).max(), 1e-30)


def test_5x5_contract_matches_torch_conv2d():
    n_views, gh, gw, ns, C = 2, 9, 8, 3, 6
    tpv = ns + gh * gw
    V = _rand((n_views * tpv, C), 23)
    w = _rand((C, 5, 5), 24, 1 / 5)
    grid = torch.from_numpy(V.astype(np.float64)).view(n_views, tpv, C)[:, ns:, :]
    x = grid.reshape(n_views, gh, gw, C).permute(0, 3, 1, 2)
    y = torch.nn.functional.conv2d(x, torch.from_numpy(w.astype(np.float64)).unsqueeze(1), padding=2, groups=C)
    ref = y.permute(0, 2, 3, 1).reshape(n_views, gh * gw, C).numpy()
    out = shortconv(V, w, n_views, gh, gw, ns, out="f32").reshape(n_views, tpv, C)[:, ns:, :]
    assert np.abs(out - ref).max() <= 1e-6 * np.abs(ref).max()
    np.testing.assert_array_equal(shortconv(V, w, n_views, gh, gw, ns, out="f32").reshape(n_views, tpv, C)[:, :ns],
                                  V.reshape(n_views, tpv, C)[:, :ns])


@pytest.mark.parametrize("dy,dx", [(0, 0), (-2, 0), (2, 1), (-1, -2), (2, 2)])
def test_5x5_delta_and_shift_kernels(dy, dx):
    n_views, gh, gw, ns, C = 2, 6, 5, 1, 3
    tpv = ns + gh * gw
    V = bf16_round(_rand((n_views * tpv, C), 25))
    w = np.zeros((C, 5, 5), np.float32)
    w[:, dy + 2, dx + 2] = 1.0
    out = shortconv(V, w, n_views, gh, gw, ns, out="bf16").reshape(n_views, tpv, C)[:, ns:, :]
    grid = V.reshape(n_views, tpv, C)[:, ns:, :].reshape(n_views, gh, gw, C)
    exp = np.zeros_like(grid)
    for y in range(gh):
        for x in range(gw):
            if 0 <= y + dy < gh and 0 <= x + dx < gw:
                exp[:, y, x] = grid[:, y + dy, x + dx]
    np.testing.assert_array_equal(out.reshape(n_views, gh, gw, C), exp)


def test_filter_shape_is_checked():
    V = _rand((4, 2), 26)
    with pytest.raises(ValueError):
        shortconv(V, _rand((2, 4, 4), 27), 1, 2, 2, 0)
