"""Build libvggt3.so (the gfx950 HIP kernels and their C ABI) in-tree.

    python -m test_layer_amd.build [--asm DIR]

Compiles every source under csrc/ with hipcc for gfx950 and links the shared
library next to this file. Always recompiles (the caller asked for a build).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libvggt3.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "shortconv.hip", "ttt_write_bf16.hip", "ttt_read_bf16.hip", "ttt_f32.hip", "reduce.hip",
           "muon.hip", "wide_mlp.hip", "wide_muon.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay disabled on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
]
# The conv's result is fixed bit for bit by a separately-rounded fp32 order.
EXTRA_FLAGS = {"shortconv.hip": ["-ffp-contract=off"]}


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str, asm_dir: str | None) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        out = os.path.join(asm_dir, os.path.splitext(src)[0] + ".s")
        cmd = [_hipcc(), *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-S", "--cuda-device-only",
               os.path.join(CSRC, src), "-o", out]
        subprocess.run(cmd, check=True, capture_output=True)
    return obj


def build(verbose: bool = False, asm_dir: str | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm_dir), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="also write device assembly to this directory")
    args = ap.parse_args()
    build(verbose=True, asm_dir=args.asm)
    sys.exit(0)
