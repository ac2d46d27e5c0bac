"""Helpers shared by the GPU parity tests (comparison metrics, tensor transfer)."""
from __future__ import annotations

import numpy as np
import torch


def to64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a (bf16 / fp32) tensor to a float64 numpy array."""
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def to32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float32).cpu().numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns (int16 for bf16, int32 for fp32)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    return t.view(torch.int32).numpy()


def f32_to_bits(x: np.ndarray, bf16: bool) -> np.ndarray:
    """Bit patterns of float32 values (which, in bf16 mode, are bf16-representable)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if bf16:
        return (x.view(np.uint32) >> 16).astype(np.uint16).view(np.int16)
    return x.view(np.int32)


def rel_err(x: np.ndarray, ref: np.ndarray) -> float:
    """Normwise max error max|x - ref| / max|ref| (0 if both are 0)."""
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den


def rel_err_per_head(x: np.ndarray, ref: np.ndarray, n_heads: int, axis_cols: bool = True) -> np.ndarray:
    """rel_err per head: theta-like [H, P] arrays by row, token arrays [n, H*d] by column block."""
    if not axis_cols:
        return np.array([rel_err(x[h], ref[h]) for h in range(n_heads)])
    d = x.shape[1] // n_heads
    return np.array([rel_err(x[:, h * d:(h + 1) * d], ref[:, h * d:(h + 1) * d]) for h in range(n_heads)])


def dtheta_ok(th: np.ndarray, th_ref: np.ndarray, th0: np.ndarray, n_heads: int, tol: float, steps: int):
    """Per head: |(th - th0) - (th_ref - th0)| <= tol * max|th_ref - th0| + floor.

    theta is stored in fp32 between steps, so each update theta - lr*g is
    rounded to fp32: an absolute error of up to one fp32 ulp of |theta| per
    step that no compute precision removes. floor = steps * 2^-23 * max|theta|.
    Returns (ok, worst ratio of error to allowance).
    """
    th = th.reshape(n_heads, -1)
    th_ref = th_ref.reshape(n_heads, -1)
    th0 = th0.reshape(n_heads, -1)
    worst = 0.0
    for h in range(n_heads):
        d, dr = th[h] - th0[h], th_ref[h] - th0[h]
        floor = steps * 2.0 ** -23 * float(np.max(np.abs(th_ref[h])))
        allow = tol * float(np.max(np.abs(dr))) + floor
        worst = max(worst, float(np.max(np.abs(d - dr))) / allow)
    return worst <= 1.0, worst
