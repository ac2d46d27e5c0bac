"""ctypes loader for libvggt3.so: declares the C ABI of include/vggt3.h.

Loading never touches the GPU. If the library has not been built, loading
raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvggt3.so")

c_void_p = ctypes.c_void_p
c_int = ctypes.c_int32
c_i64 = ctypes.c_int64
c_size = ctypes.c_size_t
c_float = ctypes.c_float

# name -> (restype, argtypes), mirroring include/vggt3.h
SIGNATURES = {
    "vggt3_version": (c_int, []),
    "vggt3_status_str": (ctypes.c_char_p, [c_int]),
    "vggt3_last_error": (ctypes.c_char_p, []),
    "vggt3_shortconv": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_int, c_int, c_int, c_int, c_int,
                                c_void_p]),
    "vggt3_shortconv_ex": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_int, c_int, c_int, c_int, c_int, c_int,
                                   c_void_p]),
    "vggt3_ttt_workspace_bytes": (c_size, [c_i64, c_int, c_int, c_int, c_int]),
    "vggt3_ttt_write": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_int, c_int, c_int, c_float, c_int,
                                c_int, c_void_p, c_size, c_void_p, c_void_p]),
    "vggt3_ttt_write_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_int, c_int, c_int, c_float, c_int,
                                        c_int, c_int, c_int, c_int, c_void_p, c_void_p]),
    "vggt3_ttt_write_conv": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_int, c_int, c_int, c_void_p, c_int,
                                     c_int, c_int, c_float, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_size,
                                     c_void_p, c_void_p]),
    "vggt3_ttt_grad": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_i64, c_int, c_int, c_int,
                               c_int, c_void_p, c_size, c_void_p, c_void_p]),
    "vggt3_ttt_grad_partials": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_int, c_int, c_int, c_int,
                                        c_void_p, c_size, c_void_p]),
    "vggt3_ttt_reduce": (c_int, [c_void_p, c_size, c_i64, c_int, c_int, c_int, c_int, c_int, c_void_p, c_float,
                                 c_void_p, c_void_p]),
    "vggt3_ttt_apply": (c_int, [c_void_p, c_void_p, c_float, c_int, c_int, c_int, c_void_p]),
    "vggt3_ttt_read": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_int, c_int, c_int, c_int, c_void_p]),
    "vggt3_ttt_write_ex": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_int, c_int, c_int, c_float, c_int,
                                   c_int, c_int, c_int, c_int, c_void_p, c_size, c_void_p, c_void_p]),
    "vggt3_ttt_grad_ex": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_i64, c_int, c_int, c_int,
                                  c_int, c_int, c_void_p, c_size, c_void_p, c_void_p]),
    "vggt3_ttt_grad_partials_ex": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_int, c_int, c_int, c_int, c_int,
                                           c_int, c_void_p, c_size, c_void_p]),
    "vggt3_ttt_muon_apply": (c_int, [c_void_p, c_void_p, c_float, c_int, c_int, c_int, c_int, c_void_p]),
    "vggt3_ttt_stream_stage_bytes": (c_size, [c_i64, c_int, c_int, c_int]),
    "vggt3_ttt_read_workspace_bytes": (c_size, [c_i64, c_int, c_int, c_int, c_int]),
    "vggt3_ttt_muon_workspace_bytes": (c_size, [c_int, c_int, c_int]),
    "vggt3_ttt_muon_apply_ex": (c_int, [c_void_p, c_void_p, c_float, c_int, c_int, c_int, c_int, c_void_p, c_size,
                                        c_void_p]),
    "vggt3_ttt_read_ex": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_int, c_int, c_int, c_int, c_void_p, c_size,
                                  c_void_p]),
    "vggt3_ttt_write_streamed": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_int, c_int, c_int, c_float, c_int,
                                         c_int, c_int, c_int, c_int, c_i64, c_void_p, c_size, c_void_p, c_size,
                                         c_void_p, c_void_p, c_void_p]),
    "vggt3_ttt_read_streamed": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_int, c_int, c_int, c_int, c_i64,
                                        c_void_p, c_size, c_void_p, c_void_p, c_void_p]),
    "vggt3_ttt_read_streamed_ex": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_int, c_int, c_int, c_int, c_i64,
                                           c_void_p, c_size, c_void_p, c_size, c_void_p, c_void_p, c_void_p]),
}

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m test_layer_amd.build, or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
