"""The C ABI loads, exports every declared symbol, and validates arguments on
the host before touching the GPU (CPU only: no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import test_layer_amd as tla
from test_layer_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vggt3.h")

# a fake, 16-byte aligned "device" address: validation must reject before use
FAKE = ctypes.c_void_p(0x10000)
FAKE2 = ctypes.c_void_p(0x20000000)
FAKE3 = ctypes.c_void_p(0x40000000)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vggt3_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"{n} has no ctypes signature"
    assert set(_lib.SIGNATURES) == set(names)


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, 7):
        assert lib.vggt3_status_str(code)
    assert lib.vggt3_version() >= 10000


def test_workspace_bytes(lib):
    nb = lib.vggt3_ttt_workspace_bytes(1_374_000, 16, 64, 128, tla.BF16)
    assert nb >= 16 * 3 * 64 * 128 * 4  # at least one fp32 partial per head
    assert nb < 256 << 20
    assert lib.vggt3_ttt_workspace_bytes(0, 16, 64, 128, tla.BF16) == 0
    assert lib.vggt3_ttt_workspace_bytes(100, 16, 32, 128, tla.BF16) == 0  # unsupported
    assert lib.vggt3_ttt_workspace_bytes(128, 1, 16, 32, tla.F32) > 0
    assert lib.vggt3_ttt_workspace_bytes(100, 1, 16, 32, 9) == 0
    # chunking depends only on (n, heads, dtype): monotone, bounded
    a = lib.vggt3_ttt_workspace_bytes(1000, 16, 64, 128, tla.BF16)
    b = lib.vggt3_ttt_workspace_bytes(10_000_000, 16, 64, 128, tla.BF16)
    assert 0 < a <= b


def _err(lib):
    return lib.vggt3_last_error().decode()


def test_shortconv_validation(lib):
    ok_args = dict(V=FAKE, Vp=FAKE2, w=FAKE3, n=2, gh=37, gw=37, ns=5, C=1024, dt=tla.BF16)

    def call(**kw):
        a = dict(ok_args, **kw)
        return lib.vggt3_shortconv(a["V"], a["Vp"], a["w"], a["n"], a["gh"], a["gw"], a["ns"], a["C"], a["dt"], None)

    assert call(dt=5) == tla.EINVAL
    assert call(n=-1) == tla.EINVAL
    assert call(gh=0) == tla.EINVAL
    assert call(ns=-1) == tla.EINVAL
    assert call(C=12) == tla.EUNSUPPORTED  # not a multiple of 8 in bf16
    assert call(gw=5000) == tla.EUNSUPPORTED  # wider than the kernel accepts
    assert call(V=None) == tla.EINVAL
    assert call(V=ctypes.c_void_p(0x10008)) == tla.EINVAL  # misaligned
    assert call(Vp=FAKE) == tla.EINVAL and "overlap" in _err(lib)  # in place
    assert call(n=0) == tla.OK  # empty scene: no-op, nothing enqueued


def test_write_validation(lib):
    n, H, d, m = 4096, 16, 64, 128
    ws_need = lib.vggt3_ttt_workspace_bytes(n, H, d, m, tla.BF16)

    def call(K=FAKE, Vp=FAKE2, theta=FAKE3, n=n, H=H, d=d, m=m, lr=0.1, steps=1, dt=tla.BF16,
             ws=ctypes.c_void_p(0x60000000), wsb=ws_need, loss=None):
        return lib.vggt3_ttt_write(K, Vp, theta, n, H, d, m, lr, steps, dt, ws, wsb, loss, None)

    assert call(steps=0) == tla.EINVAL
    assert call(lr=float("nan")) == tla.EINVAL
    assert call(lr=float("inf")) == tla.EINVAL
    assert call(n=-5) == tla.EINVAL
    assert call(d=32) == tla.EUNSUPPORTED
    assert call(m=64) == tla.EUNSUPPORTED
    assert call(dt=tla.F32, d=16, m=64) == tla.EUNSUPPORTED
    assert call(theta=None) == tla.EINVAL
    assert call(K=None) == tla.EINVAL
    assert call(ws=None) == tla.EWORKSPACE
    assert call(wsb=ws_need - 1) == tla.EWORKSPACE
    assert call(theta=FAKE) == tla.EINVAL and "overlap" in _err(lib)
    assert call(theta=ctypes.c_void_p(0x40000004)) == tla.EINVAL  # misaligned
    assert call(H=0) == tla.EINVAL
    # empty scene with no loss output: nothing to do, nothing enqueued
    assert call(n=0, K=None, Vp=None, ws=None, wsb=0) == tla.OK


def test_grad_reduce_apply_read_validation(lib):
    n, H, d, m = 4096, 16, 64, 128
    wsb = lib.vggt3_ttt_workspace_bytes(n, H, d, m, tla.BF16)
    ws = ctypes.c_void_p(0x60000000)
    assert lib.vggt3_ttt_grad(FAKE, FAKE2, FAKE3, FAKE3, 0, n, H, d, m, tla.BF16, ws, wsb, None, None) == tla.EINVAL
    assert lib.vggt3_ttt_grad(FAKE, FAKE2, FAKE3, None, 0, n, H, d, m, tla.BF16, ws, wsb, None, None) == tla.EINVAL
    assert lib.vggt3_ttt_grad(FAKE, FAKE2, FAKE3, ctypes.c_void_p(0x70000000), 0, n, H, d, m, tla.BF16, ws, 16,
                              None, None) == tla.EWORKSPACE
    assert lib.vggt3_ttt_grad_partials(FAKE, FAKE2, FAKE3, n, H, d, m, tla.BF16, None, 0, None) == tla.EWORKSPACE
    assert lib.vggt3_ttt_grad_partials(FAKE, FAKE2, FAKE3, n, H, 48, m, tla.BF16, ws, wsb, None) == tla.EUNSUPPORTED
    assert lib.vggt3_ttt_reduce(ws, wsb, n, H, d, m, tla.BF16, 3, FAKE3, 0.1, None, None) == tla.EINVAL
    assert lib.vggt3_ttt_reduce(ws, wsb, n, H, d, m, tla.BF16, 0, None, 0.1, None, None) == tla.EINVAL
    assert lib.vggt3_ttt_reduce(ws, wsb, n, H, d, m, tla.BF16, 0, ws, 0.1, None, None) == tla.EINVAL
    assert lib.vggt3_ttt_apply(FAKE, FAKE, 0.1, H, d, m, None) == tla.EINVAL
    assert lib.vggt3_ttt_apply(FAKE, FAKE2, float("nan"), H, d, m, None) == tla.EINVAL
    assert lib.vggt3_ttt_apply(FAKE, FAKE2, 0.1, 0, d, m, None) == tla.OK  # nothing to update
    assert lib.vggt3_ttt_read(FAKE, FAKE3, FAKE, n, H, d, m, tla.BF16, None) == tla.EINVAL
    assert lib.vggt3_ttt_read(FAKE, FAKE3, FAKE2, n, H, d, 96, tla.BF16, None) == tla.EUNSUPPORTED
    assert lib.vggt3_ttt_read(None, FAKE3, FAKE2, n, H, d, m, tla.BF16, None) == tla.EINVAL
    assert lib.vggt3_ttt_read(None, None, None, 0, H, d, m, tla.BF16, None) == tla.OK


def test_binding_refuses_cpu_tensors():
    import torch
    V = torch.zeros(10, 16)
    w = torch.zeros(16, 3, 3)
    with pytest.raises(ValueError):
        tla.shortconv(V, w, 1, 3, 3, 1)


def test_product_path_does_not_import_oracle():
    """The package never reaches for the CPU oracle (no fallback)."""
    pkg = os.path.join(ROOT, "test_layer_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, flags=re.M), f


def test_recipe_entry_points_validate(lib):
    n, H, d, m = 4096, 16, 64, 128
    ws_need = lib.vggt3_ttt_workspace_bytes(n, H, d, m, tla.BF16)
    big = ctypes.c_void_p(0x7000000000)

    def write_ex(loss=0, opt=1, ns=5, dt=tla.BF16, lr=0.1):
        return lib.vggt3_ttt_write_ex(FAKE, FAKE2, FAKE3, n, H, d, m, lr, 2, loss, opt, ns, dt, big, ws_need,
                                      None, None)

    assert write_ex(loss=2) == tla.EINVAL and "loss" in _err(lib)
    assert write_ex(opt=7) == tla.EINVAL and "optimizer" in _err(lib)
    assert write_ex(ns=-1) == tla.EINVAL and "ns_steps" in _err(lib)
    assert write_ex(ns=65) == tla.EINVAL
    assert write_ex(lr=float("nan")) == tla.EINVAL
    assert lib.vggt3_ttt_grad_ex(FAKE, FAKE2, FAKE3, big, 0, n, H, d, m, 3, tla.BF16, big, ws_need, None,
                                 None) == tla.EINVAL
    assert lib.vggt3_ttt_grad_partials_ex(FAKE, FAKE2, FAKE3, n, H, d, m, -1, 1, tla.BF16, big, ws_need,
                                          None) == tla.EINVAL
    # Muon apply: unsupported shape, bad step count, aliasing, empty
    assert lib.vggt3_ttt_muon_apply(FAKE, FAKE2, 0.1, H, 32, 64, 5, None) == tla.EUNSUPPORTED
    assert lib.vggt3_ttt_muon_apply(FAKE, FAKE2, 0.1, H, d, m, 99, None) == tla.EINVAL
    assert lib.vggt3_ttt_muon_apply(FAKE, FAKE, 0.1, H, d, m, 5, None) == tla.EINVAL and "overlap" in _err(lib)
    assert lib.vggt3_ttt_muon_apply(FAKE, None, 0.1, H, d, m, 5, None) == tla.EINVAL
    assert lib.vggt3_ttt_muon_apply(FAKE, FAKE2, 0.1, 0, d, m, 5, None) == tla.OK


def test_shortconv_ex_validation(lib):
    def call(k, dt=tla.BF16, C=1024):
        return lib.vggt3_shortconv_ex(FAKE, FAKE2, FAKE3, 2, 37, 37, 5, C, k, dt, None)

    assert call(4) == tla.EUNSUPPORTED and "filter size" in _err(lib)
    assert call(7) == tla.EUNSUPPORTED
    assert call(5, dt=9) == tla.EINVAL
    assert call(5, C=12) == tla.EUNSUPPORTED
    assert lib.vggt3_shortconv_ex(FAKE, FAKE, FAKE3, 2, 37, 37, 5, 1024, 5, tla.BF16, None) == tla.EINVAL
    assert lib.vggt3_shortconv_ex(FAKE, FAKE2, FAKE3, 0, 37, 37, 5, 1024, 5, tla.BF16, None) == tla.OK


def test_streamed_entry_points_validate(lib):
    n, H, d, m = 100_000, 16, 64, 128
    ct = 8192
    stage_need = lib.vggt3_ttt_stream_stage_bytes(ct, H, d, tla.BF16)
    assert stage_need == 4 * ((ct * H * d * 2 + 255) // 256 * 256)
    assert lib.vggt3_ttt_stream_stage_bytes(0, H, d, tla.BF16) == 0
    assert lib.vggt3_ttt_stream_stage_bytes(ct, H, d, 9) == 0
    assert lib.vggt3_ttt_stream_stage_bytes(1, 1, 16, tla.F32) == 4 * 256
    ws_need = lib.vggt3_ttt_workspace_bytes(ct, H, d, m, tla.BF16)
    stage = ctypes.c_void_p(0x7000000000)
    ws = ctypes.c_void_p(0x7800000000)

    def write(K=FAKE, Vp=FAKE2, theta=FAKE3, n=n, ct=ct, stage=stage, sb=stage_need, ws=ws, wsb=ws_need, steps=2,
              loss=0, opt=0, ns=5, lr=0.1, loss_out=None, d=d, m=m):
        return lib.vggt3_ttt_write_streamed(K, Vp, theta, n, H, d, m, lr, steps, loss, opt, ns, tla.BF16, ct, stage,
                                            sb, ws, wsb, loss_out, None, None)

    assert write(ct=0) == tla.EINVAL and "chunk_tokens" in _err(lib)
    assert write(steps=0) == tla.EINVAL
    assert write(lr=float("nan")) == tla.EINVAL
    assert write(loss=5) == tla.EINVAL
    assert write(opt=3) == tla.EINVAL
    assert write(opt=1, ns=65) == tla.EINVAL
    assert write(d=32) == tla.EUNSUPPORTED
    assert write(K=None) == tla.EINVAL
    assert write(theta=None) == tla.EINVAL
    assert write(stage=None) == tla.EINVAL
    assert write(sb=stage_need - 1) == tla.EWORKSPACE and "stage" in _err(lib)
    assert write(ws=None) == tla.EWORKSPACE
    assert write(wsb=ws_need - 1) == tla.EWORKSPACE
    # the workspace is sized for one chunk, not for the scene
    assert ws_need <= lib.vggt3_ttt_workspace_bytes(n, H, d, m, tla.BF16)
    assert lib.vggt3_ttt_workspace_bytes(256, H, d, m, tla.BF16) < lib.vggt3_ttt_workspace_bytes(n, H, d, m, tla.BF16)
    assert write(stage=ws) == tla.EINVAL and "overlap" in _err(lib)
    assert write(theta=stage) == tla.EINVAL and "overlap" in _err(lib)
    assert write(loss_out=stage) == tla.EINVAL and "overlap" in _err(lib)
    # a chunk larger than the scene needs only the scene's staging
    small = lib.vggt3_ttt_stream_stage_bytes(1000, H, d, tla.BF16)
    assert write(n=1000, ct=10**9, sb=small - 1, wsb=10**9) == tla.EWORKSPACE
    # empty scene without loss output: nothing enqueued
    assert write(n=0, K=None, Vp=None, stage=None, ws=None) == tla.OK

    def read(Q=FAKE, theta=FAKE3, O=FAKE2, n=n, ct=ct, stage=stage, sb=stage_need):
        return lib.vggt3_ttt_read_streamed(Q, theta, O, n, H, d, m, tla.BF16, ct, stage, sb, None, None, None)

    assert read(ct=-1) == tla.EINVAL
    assert read(Q=None) == tla.EINVAL
    assert read(O=FAKE) == tla.EINVAL and "overlap" in _err(lib)
    assert read(stage=None) == tla.EINVAL
    assert read(sb=stage_need - 16) == tla.EWORKSPACE
    assert read(stage=FAKE3) == tla.EINVAL and "overlap" in _err(lib)
    assert read(n=0, Q=None, O=None, stage=None) == tla.OK


def test_streamed_binding_refuses_device_layout_mixups():
    import torch
    theta = torch.zeros(16, 3 * 64 * 128)
    K = torch.zeros(64, 1024, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tla.ttt_write_streamed(K, K, theta, 0.1, 1, 16, 32)  # theta must be a device tensor
    with pytest.raises(ValueError):
        tla.ttt_read_streamed(K[:, ::2], theta, 16, 32, out=K[:, ::2])  # non-contiguous host tensor


def test_wide_mlp_shape_rules(lib):
    # the full-width 1024 -> 4096 -> 1024 MLP: one head, bf16, gradient descent
    n, d, m = 5000, 1024, 4096
    ws = lib.vggt3_ttt_workspace_bytes(n, 1, d, m, tla.BF16)
    assert ws > 3 * d * m * 4  # holds at least the reduced gradient
    assert lib.vggt3_ttt_workspace_bytes(n, 2, d, m, tla.BF16) == 0  # two heads: unsupported
    assert lib.vggt3_ttt_workspace_bytes(n, 1, d, m, tla.F32) == 0  # no fp32 kernel
    # the workspace stops growing once the scene exceeds one token chunk
    big = lib.vggt3_ttt_workspace_bytes(10_000_000, 1, d, m, tla.BF16)
    assert big == lib.vggt3_ttt_workspace_bytes(1_000_000, 1, d, m, tla.BF16)
    assert big < 8 << 30
    rws = lib.vggt3_ttt_read_workspace_bytes(n, 1, d, m, tla.BF16)
    assert 0 < rws < ws
    assert lib.vggt3_ttt_read_workspace_bytes(n, 16, 64, 128, tla.BF16) == 0  # per-head: none needed
    big_ptr = ctypes.c_void_p(0x7000000000)
    assert lib.vggt3_ttt_write(FAKE, FAKE2, FAKE3, n, 2, d, m, 0.1, 1, tla.BF16, big_ptr, ws, None,
                               None) == tla.EUNSUPPORTED and "n_heads = 1" in _err(lib)
    assert lib.vggt3_ttt_write_ex(FAKE, FAKE2, FAKE3, n, 1, d, m, 0.1, 1, tla.LOSS_DOT, tla.OPT_MUON, 99, tla.BF16,
                                  big_ptr, ws, None, None) == tla.EINVAL and "ns_steps" in _err(lib)
    assert lib.vggt3_ttt_read(FAKE, FAKE3, FAKE2, n, 1, d, m, tla.BF16, None) == tla.EUNSUPPORTED
    assert "vggt3_ttt_read_ex" in _err(lib)
    assert lib.vggt3_ttt_read_ex(FAKE, FAKE3, FAKE2, n, 1, d, m, tla.BF16, None, 0, None) == tla.EWORKSPACE
    assert lib.vggt3_ttt_read_ex(FAKE, FAKE3, FAKE2, n, 1, d, m, tla.BF16, big_ptr, rws - 1, None) == tla.EWORKSPACE
    assert lib.vggt3_ttt_read_ex(FAKE, FAKE3, FAKE, n, 1, d, m, tla.BF16, big_ptr, rws, None) == tla.EINVAL
    assert lib.vggt3_ttt_grad_partials(FAKE, FAKE2, FAKE3, n, 1, d, m, tla.BF16, big_ptr, ws,
                                       None) == tla.EUNSUPPORTED
    assert lib.vggt3_ttt_reduce(big_ptr, ws, n, 1, d, m, tla.BF16, 0, FAKE3, 0.1, None, None) == tla.EUNSUPPORTED
    stage = lib.vggt3_ttt_stream_stage_bytes(4096, 1, d, tla.BF16)
    ws_chunk = lib.vggt3_ttt_workspace_bytes(4096, 1, d, m, tla.BF16)
    assert lib.vggt3_ttt_write_streamed(FAKE, FAKE2, FAKE3, n, 1, d, m, 0.1, 1, 0, 0, 5, tla.BF16, 4096, big_ptr,
                                        stage, ctypes.c_void_p(0x7800000000), ws_chunk - 1, None, None,
                                        None) == tla.EWORKSPACE
    rws_chunk = lib.vggt3_ttt_read_workspace_bytes(4096, 1, d, m, tla.BF16)
    assert lib.vggt3_ttt_read_streamed_ex(FAKE, FAKE3, FAKE2, n, 1, d, m, tla.BF16, 4096, big_ptr, stage, None, 0,
                                          None, None, None) == tla.EWORKSPACE
    assert lib.vggt3_ttt_read_streamed_ex(FAKE, FAKE3, FAKE2, n, 1, d, m, tla.BF16, 4096, big_ptr, stage,
                                          ctypes.c_void_p(0x7800000000), rws_chunk - 2, None, None,
                                          None) == tla.EWORKSPACE
    assert lib.vggt3_ttt_read_streamed(FAKE, FAKE3, FAKE2, n, 1, d, m, tla.BF16, 4096, big_ptr, stage, None, None,
                                       None) == tla.EWORKSPACE
    mws = lib.vggt3_ttt_muon_workspace_bytes(1, d, m)
    assert mws > 2 * d * m * 4 and lib.vggt3_ttt_muon_workspace_bytes(16, 64, 128) == 0
    assert lib.vggt3_ttt_muon_apply(FAKE, FAKE2, 0.1, 1, d, m, 5, None) == tla.EUNSUPPORTED
    assert lib.vggt3_ttt_muon_apply_ex(FAKE, FAKE2, 0.1, 1, d, m, 5, None, 0, None) == tla.EWORKSPACE
    assert lib.vggt3_ttt_muon_apply_ex(FAKE, FAKE2, 0.1, 1, d, m, 5, big_ptr, mws - 4, None) == tla.EWORKSPACE
    assert lib.vggt3_ttt_muon_apply_ex(FAKE, FAKE2, 0.1, 1, d, m, 70, big_ptr, mws, None) == tla.EINVAL
    assert lib.vggt3_ttt_muon_apply_ex(FAKE, FAKE, 0.1, 1, d, m, 5, big_ptr, mws, None) == tla.EINVAL
    assert lib.vggt3_ttt_muon_apply_ex(FAKE, FAKE2, 0.1, 2, d, m, 5, big_ptr, mws, None) == tla.EUNSUPPORTED
    # the workspace must not overlap the token inputs
    assert lib.vggt3_ttt_grad(FAKE, FAKE2, FAKE3, big_ptr, 0, n, 1, d, m, tla.BF16, FAKE, ws, None,
                              None) == tla.EINVAL


def test_write_conv_validation(lib):
    nv, gh, gw, ns, H = 2, 37, 37, 5, 16
    n = nv * (ns + gh * gw)
    ws_need = lib.vggt3_ttt_workspace_bytes(n, H, 64, 128, tla.BF16)
    CW = ctypes.c_void_p(0x50000000)
    WS = ctypes.c_void_p(0x60000000)

    def call(K=FAKE, V=FAKE2, w=CW, nv=nv, gh=gh, gw=gw, ns=ns, theta=FAKE3, H=H, d=64, m=128, lr=0.1, steps=2,
             loss=0, opt=0, nsteps=5, vp=None, ws=WS, wsb=ws_need, lo=None):
        return lib.vggt3_ttt_write_conv(K, V, w, nv, gh, gw, ns, theta, H, d, m, lr, steps, loss, opt, nsteps, vp, ws,
                                        wsb, lo, None)

    assert call(gw=48) == tla.EUNSUPPORTED and "47" in _err(lib)  # the ring holds a 47-wide window
    assert call(ns=70000) == tla.EUNSUPPORTED
    assert call(d=16, m=32) == tla.EUNSUPPORTED
    assert call(d=1024, m=4096, H=1) == tla.EUNSUPPORTED
    assert call(nv=-1) == tla.EINVAL
    assert call(gh=0) == tla.EINVAL
    assert call(ns=-1) == tla.EINVAL
    assert call(steps=0) == tla.EINVAL
    assert call(loss=7) == tla.EINVAL
    assert call(w=None) == tla.EINVAL
    assert call(w=ctypes.c_void_p(0x50000004)) == tla.EINVAL  # misaligned filters
    assert call(vp=ctypes.c_void_p(0x20000000)) == tla.EINVAL and "overlap" in _err(lib)  # V' over V
    assert call(vp=ctypes.c_void_p(0x70000008)) == tla.EINVAL  # misaligned V'
    assert call(ws=None) == tla.EWORKSPACE
    assert call(wsb=ws_need - 1) == tla.EWORKSPACE
    assert call(theta=CW) == tla.EINVAL and "overlap" in _err(lib)
    assert call(nv=0, K=None, V=None, w=None, ws=None, wsb=0) == tla.OK  # empty scene, nothing enqueued
