"""Bounds guards of the kernels' ragged tails.

The kernels address token rows through buffer descriptors whose range ends at
the caller's last row: loads past it read zeros and stores past it are dropped.
These tests hand the library views of the first n rows of larger buffers whose
remaining rows (and the bytes after each workspace, staging buffer and loss
output) hold a sentinel, then check that
  * no output byte past the caller's extent changed, and
  * no input byte past it was read (results are bit-identical to a call on
    exact-size copies, although the rows after the view hold NaNs).
Token counts are ragged (not multiples of any tile) and every head is present,
so the last head's columns, which end each row, are covered.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import test_layer_amd as tla

pytestmark = pytest.mark.gpu

DEV = "cuda"
PAD = 64  # sentinel rows after each token view
TAIL = 4096  # sentinel bytes after each workspace / staging buffer
SENT16 = 0x7FA5  # a bf16 NaN
SENT32 = 0x7FC0DEAD  # an fp32 NaN
SENT8 = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tla.lib()


def _ibits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _sent(dtype):
    return SENT16 if dtype == torch.bfloat16 else SENT32


def _padded_tokens(n, C, dtype, src=None, device=DEV, pin=False):
    """[n + PAD, C] buffer: rows < n from src (or sentinel), rows >= n sentinel; returns (buffer, view)."""
    if device == "cpu":
        big = torch.empty((n + PAD, C), dtype=dtype, pin_memory=pin)
    else:
        big = torch.empty((n + PAD, C), dtype=dtype, device=device)
    _ibits(big).fill_(_sent(dtype))
    if src is not None:
        big[:n].copy_(src)
    return big, big[:n]


def _assert_tail_intact(big, n, what):
    tail = _ibits(big[n:]).cpu()
    assert bool((tail == _sent(big.dtype)).all()), f"{what}: rows past the caller's {n} rows were written"


def _padded_bytes(nbytes, device=DEV):
    buf = torch.full((nbytes + TAIL,), SENT8, dtype=torch.uint8, device=device)
    return buf, buf[:nbytes]


def _assert_bytes_intact(buf, nbytes, what):
    assert bool((buf[nbytes:].cpu() == SENT8).all()), f"{what}: bytes past its {nbytes}-byte extent were written"


def _rand_tokens(n, C, dtype, seed, scale=1.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn((n, C), generator=g, device=DEV) * scale).to(dtype)


def _rand_theta(H, d, m, seed, scale=0.02):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randn((H, 3 * d * m), generator=g, device=DEV) * scale


def _bits_equal(a, b):
    return torch.equal(_ibits(a.contiguous()), _ibits(b.contiguous()))


READ_CASES = [
    # (n, heads, d, m, dtype)
    (1, 16, 64, 128, torch.bfloat16),
    (16, 16, 64, 128, torch.bfloat16),
    (17, 5, 64, 128, torch.bfloat16),
    (31, 16, 64, 128, torch.bfloat16),
    (48, 16, 64, 128, torch.bfloat16),
    (997, 16, 64, 128, torch.bfloat16),
    (4122, 3, 64, 128, torch.bfloat16),
    (37, 2, 16, 32, torch.float32),
    (37, 2, 16, 32, torch.bfloat16),  # the fp32 kernels with bf16 tokens
    (300, 4, 64, 128, torch.float32),
    (257, 1, 1024, 4096, torch.bfloat16),  # the full-width MLP
]


@pytest.mark.parametrize("case", READ_CASES, ids=lambda c: f"n{c[0]}h{c[1]}d{c[2]}m{c[3]}{str(c[4])[6:]}")
def test_read_stays_within_its_rows(case):
    n, H, d, m, dt = case
    print(f"[guard read] n={n} H={H} d={d} m={m} {dt}", flush=True)
    C = H * d
    Q = _rand_tokens(n, C, dt, 11, 1.0 / np.sqrt(d))
    theta = _rand_theta(H, d, m, 12)
    ref = tla.ttt_read(Q.clone(), theta, H, d_hidden=m)
    qbig, qv = _padded_tokens(n, C, dt, Q)
    obig, ov = _padded_tokens(n, C, dt)
    need = tla.read_workspace_bytes(n, H, d, m, tla.BF16 if dt == torch.bfloat16 else tla.F32)
    wbuf, wv = _padded_bytes(need) if need > 0 else (None, None)
    tla.ttt_read(qv, theta, H, d_hidden=m, out=ov, workspace=wv)
    torch.cuda.synchronize()
    _assert_tail_intact(obig, n, "read output")
    assert _bits_equal(ov, ref), "read output differs when the rows after Q hold NaNs"
    if wbuf is not None:
        _assert_bytes_intact(wbuf, need, "read workspace")


GRAD_CASES = [
    (1, 16, 64, 128, torch.bfloat16),
    (33, 16, 64, 128, torch.bfloat16),
    (997, 16, 64, 128, torch.bfloat16),
    (37, 1, 16, 32, torch.float32),
    (45, 2, 16, 32, torch.bfloat16),
    (301, 2, 64, 128, torch.float32),
    (257, 1, 1024, 4096, torch.bfloat16),
]


@pytest.mark.parametrize("loss", ["mse", "dot"])
@pytest.mark.parametrize("case", GRAD_CASES, ids=lambda c: f"n{c[0]}h{c[1]}d{c[2]}m{c[3]}{str(c[4])[6:]}")
def test_gradient_reads_only_its_rows(case, loss):
    """The gradient kernels load K/V' tiles ahead of use; past the last token
    those loads must read zeros, not the NaN rows after the view."""
    n, H, d, m, dt = case
    print(f"[guard grad] n={n} H={H} d={d} m={m} {dt} {loss}", flush=True)
    C = H * d
    K = _rand_tokens(n, C, dt, 21, 1.0 / np.sqrt(d))
    Vp = _rand_tokens(n, C, dt, 22, 1.0 / np.sqrt(d))
    theta = _rand_theta(H, d, m, 23)
    code = tla.BF16 if dt == torch.bfloat16 else tla.F32
    need = tla.workspace_bytes(n, H, d, m, code)
    ref = tla.ttt_grad(K.clone(), Vp.clone(), theta, H, d_hidden=m, loss=loss)
    kbig, kv = _padded_tokens(n, C, dt, K)
    vbig, vv = _padded_tokens(n, C, dt, Vp)
    wbuf, wv = _padded_bytes(need)
    lbuf = torch.full((H + 8,), float("nan"), device=DEV)
    lbuf[H:].view(torch.int32).fill_(SENT32)
    g = tla.ttt_grad(kv, vv, theta, H, d_hidden=m, workspace=wv, loss_out=lbuf[:H], loss=loss)
    torch.cuda.synchronize()
    assert _bits_equal(g, ref), "gradient differs when the rows after K/V' hold NaNs"
    _assert_bytes_intact(wbuf, need, "gradient workspace")
    assert bool((lbuf[H:].view(torch.int32).cpu() == SENT32).all()), "loss output overrun"
    assert bool(torch.isfinite(lbuf[:H]).all())


CONV_CASES = [
    # (views, grid_h, grid_w, n_special, C, ksize, dtype)
    (2, 37, 37, 5, 1024, 3, torch.bfloat16),  # LDS ring kernel, 128-channel strips
    (3, 5, 7, 2, 128, 3, torch.bfloat16),
    (2, 7, 40, 3, 192, 3, torch.bfloat16),    # LDS ring kernel, 64-channel strips
    (1, 4, 127, 1, 64, 3, torch.bfloat16),    # register-window kernel
    (2, 8, 8, 0, 16, 3, torch.float32),
    (2, 9, 11, 3, 64, 5, torch.bfloat16),     # V-5
]


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: "x".join(str(v) for v in c[:6]) + str(c[6])[6:])
def test_shortconv_stays_within_its_views(case):
    views, gh, gw, ns, C, k, dt = case
    print(f"[guard conv] {case}", flush=True)
    n = views * (ns + gh * gw)
    V = _rand_tokens(n, C, dt, 31)
    g = torch.Generator(device=DEV).manual_seed(32)
    w = torch.randn((C, k, k), generator=g, device=DEV) / k
    ref = tla.shortconv(V.clone(), w, views, gh, gw, ns)
    vbig, vv = _padded_tokens(n, C, dt, V)
    obig, ov = _padded_tokens(n, C, dt)
    tla.shortconv(vv, w, views, gh, gw, ns, out=ov)
    torch.cuda.synchronize()
    _assert_tail_intact(obig, n, "conv output")
    assert _bits_equal(ov, ref), "conv output differs when the rows after V hold NaNs"


@pytest.mark.parametrize("chunk", [100, 997, 4096])
def test_streamed_read_stays_within_its_rows_and_stage(chunk):
    n, H, d, m = 997, 16, 64, 128
    print(f"[guard streamed read] n={n} chunk={chunk}", flush=True)
    C = H * d
    Q = _rand_tokens(n, C, torch.bfloat16, 41, 0.125)
    theta = _rand_theta(H, d, m, 42)
    ref = tla.ttt_read(Q, theta, H).cpu()
    qbig, qv = _padded_tokens(n, C, torch.bfloat16, Q.cpu(), device="cpu", pin=True)
    obig, ov = _padded_tokens(n, C, torch.bfloat16, device="cpu", pin=True)
    ct = min(chunk, n)
    sneed = tla.stage_bytes(ct, H, d, tla.BF16)
    sbuf, sv = _padded_bytes(sneed)
    tla.ttt_read_streamed(qv, theta, H, chunk, out=ov, stage=sv)
    torch.cuda.synchronize()
    _assert_tail_intact(obig, n, "streamed read output")
    _assert_bytes_intact(sbuf, sneed, "streamed read stage")
    assert _bits_equal(ov, ref)


@pytest.mark.parametrize("chunk", [100, 997])
def test_streamed_write_stays_within_its_stage_and_workspace(chunk):
    n, H, d, m = 997, 16, 64, 128
    print(f"[guard streamed write] n={n} chunk={chunk}", flush=True)
    C = H * d
    K = _rand_tokens(n, C, torch.bfloat16, 51, 0.125)
    Vp = _rand_tokens(n, C, torch.bfloat16, 52, 0.125)
    theta0 = _rand_theta(H, d, m, 53)
    ref = theta0.clone()
    tla.ttt_write_streamed(K.cpu().pin_memory(), Vp.cpu().pin_memory(), ref, 0.1, 2, H, chunk)
    kbig, kv = _padded_tokens(n, C, torch.bfloat16, K.cpu(), device="cpu", pin=True)
    vbig, vv = _padded_tokens(n, C, torch.bfloat16, Vp.cpu(), device="cpu", pin=True)
    ct = min(chunk, n)
    sneed = tla.stage_bytes(ct, H, d, tla.BF16)
    wneed = tla.workspace_bytes(ct, H, d, m, tla.BF16)
    sbuf, sv = _padded_bytes(sneed)
    wbuf, wv = _padded_bytes(wneed)
    theta = theta0.clone()
    tla.ttt_write_streamed(kv, vv, theta, 0.1, 2, H, chunk, stage=sv, workspace=wv)
    torch.cuda.synchronize()
    _assert_bytes_intact(sbuf, sneed, "streamed write stage")
    _assert_bytes_intact(wbuf, wneed, "streamed write workspace")
    assert _bits_equal(theta, ref)
