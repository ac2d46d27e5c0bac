"""The C ABI used from plain C (tests/c_caller.c, built with gcc against
include/vggt3.h, libvggt3.so and the HIP runtime; no Python in the caller).

CPU: the program's argument-validation calls return the documented statuses.
GPU: the program runs ShortConv2D, a 2-step write and the read on a small
scene and writes its inputs and outputs to a file; the oracle recomputes the
layer from those inputs (conv bit-exact; write and read at the bf16 bar 2e-2).
"""
from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from tests.gpu_util import dtheta_ok, rel_err_per_head

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_caller.c")
LIBDIR = os.path.join(ROOT, "test_layer_amd")
ROCM = "/opt/rocm"


def _build(out_dir) -> str:
    if shutil.which("gcc") is None or not os.path.exists(os.path.join(LIBDIR, "libvggt3.so")):
        pytest.skip("gcc or the built library is missing")
    exe = os.path.join(str(out_dir), "c_caller")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{ROCM}/include", SRC, "-o", exe, f"-L{LIBDIR}", "-lvggt3",
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{ROCM}/lib", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_caller_validation(tmp_path):
    exe = _build(tmp_path)
    r = subprocess.run([exe, "validate"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "validate: ok" in r.stdout


def _bf16(u16):
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@pytest.mark.gpu
def test_c_caller_layer_parity(tmp_path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = _build(tmp_path)
    out = os.path.join(str(tmp_path), "layer.bin")
    print("[c_caller] run", flush=True)
    r = subprocess.run([exe, "run", out], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    raw = open(out, "rb").read()
    hdr = np.frombuffer(raw, dtype=np.int32, count=8)
    n_views, gh, gw, ns, H, d, m, steps = (int(x) for x in hdr)
    lr = float(np.frombuffer(raw, dtype=np.float32, count=1, offset=32)[0])
    n, C = n_views * (ns + gh * gw), H * d
    off = 36

    def take(dtype, count):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=count, offset=off)
        off += a.nbytes
        return a

    K = _bf16(take(np.uint16, n * C)).reshape(n, C)
    V = _bf16(take(np.uint16, n * C)).reshape(n, C)
    Q = _bf16(take(np.uint16, n * C)).reshape(n, C)
    w = take(np.float32, C * 9).reshape(C, 3, 3)
    th0 = take(np.float32, H * 3 * d * m).reshape(H, -1)
    Vp_gpu = take(np.uint16, n * C).reshape(n, C)
    th1 = take(np.float32, H * 3 * d * m).reshape(H, -1)
    O_gpu = _bf16(take(np.uint16, n * C)).reshape(n, C)
    loss = take(np.float32, steps * H).reshape(steps, H)
    assert off == len(raw)

    Vp_ref = oracle.shortconv(V, w, n_views, gh, gw, ns, out="bf16")
    np.testing.assert_array_equal(Vp_gpu, (Vp_ref.view(np.uint32) >> 16).astype(np.uint16))
    th_ref, L_ref, _ = oracle.ttt_write(K.astype(np.float64), Vp_ref.astype(np.float64), th0, H, d, m, lr, steps)
    ok, worst = dtheta_ok(th1.astype(np.float64), th_ref, th0.astype(np.float64), H, 2e-2, steps)
    print(f"  dtheta worst/allowance {worst:.3f}", flush=True)
    assert ok, worst
    np.testing.assert_allclose(loss, L_ref, rtol=2e-2)
    O_ref = oracle.ttt_read(Q.astype(np.float64), th_ref, H, d, m)
    e = rel_err_per_head(O_gpu.astype(np.float64), O_ref, H)
    assert e.max() <= 2e-2, e
