"""VGG-T^3 test-time-training layer on MI355X (gfx950).

Thin binding over the C ABI in include/vggt3.h (libvggt3.so, built from
test_layer_amd/csrc). Every function marshals torch tensors (device memory and
the current stream) into the C calls; all layer arithmetic runs in the HIP
kernels. There is no CPU or PyTorch fallback: without the built library, or
without a GPU, calls raise.

    Vp    = shortconv(V, w, n_views, grid_h, grid_w, n_special)
    theta = ttt_write(K, Vp, theta, lr, steps, n_heads)        # in place
    O     = ttt_read(Q, theta, n_heads)
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

BF16 = 0
F32 = 1

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4


class Vggt3Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = _lib.load()
        detail = lib.vggt3_last_error().decode()
        super().__init__(f"{fn}: {lib.vggt3_status_str(status).decode()} ({status}): {detail}")
        self.status = status


def lib():
    return _lib.load()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}; token tensors are bfloat16 or float32")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU (HIP device memory)")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _check_tokens(name: str, t: torch.Tensor) -> None:
    if t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D [tokens, channels] tensor, got shape {tuple(t.shape)}")
    _dtype_code(t)


def _check_same(name: str, t: Optional[torch.Tensor], ref: torch.Tensor, ref_name: str) -> None:
    if t is None:
        return
    if t.shape != ref.shape or t.dtype != ref.dtype:
        raise ValueError(f"{name} {tuple(t.shape)} {t.dtype} does not match {ref_name} {tuple(ref.shape)} {ref.dtype}")


def _check_f32(name: str, t: Optional[torch.Tensor], numel: int, at_least: bool = False) -> None:
    if t is None:
        return
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32, got {t.dtype}")
    if (t.numel() < numel) if at_least else (t.numel() != numel):
        raise ValueError(f"{name} has {t.numel()} elements, {'at least ' if at_least else ''}{numel} expected")


def _check_theta(theta: torch.Tensor, n_heads: int, d: int, m: int) -> None:
    _check_f32("theta", theta, n_heads * 3 * d * m)


def _call(name: str, *args) -> int:
    rc = getattr(lib(), name)(*args)
    if rc != OK:
        raise Vggt3Error(name, rc)
    return rc


def shortconv(V: torch.Tensor, w: torch.Tensor, n_views: int, grid_h: int, grid_w: int, n_special: int,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """V' = depthwise k x k ShortConv2D of each view's patch grid (k = w.shape[-1],
    3 or 5); special tokens copied."""
    _check_tokens("V", V)
    if w.dtype != torch.float32 or w.dim() != 3 or w.shape[1] != w.shape[2]:
        raise TypeError("conv weights are float32 [C, k, k]")
    if w.shape[0] != V.shape[1]:
        raise ValueError(f"conv weights have {w.shape[0]} channels, V has {V.shape[1]}")
    if V.shape[0] != n_views * (n_special + grid_h * grid_w):
        raise ValueError(f"V has {V.shape[0]} tokens, {n_views} views x ({n_special} + {grid_h}x{grid_w}) expected")
    _check_same("out", out, V, "V")
    if out is None:
        out = torch.empty_like(V)
    _check_dev(V, w, out)
    k = int(w.shape[-1])
    if k == 3:
        _call("vggt3_shortconv", _ptr(V), _ptr(out), _ptr(w), n_views, grid_h, grid_w, n_special, V.shape[1],
              _dtype_code(V), _stream())
    else:
        _call("vggt3_shortconv_ex", _ptr(V), _ptr(out), _ptr(w), n_views, grid_h, grid_w, n_special, V.shape[1], k,
              _dtype_code(V), _stream())
    return out


def workspace_bytes(n_tokens: int, n_heads: int, d_head: int, d_hidden: int, dtype_code: int) -> int:
    return int(lib().vggt3_ttt_workspace_bytes(n_tokens, n_heads, d_head, d_hidden, dtype_code))


def make_workspace(n_tokens: int, n_heads: int, d_head: int, d_hidden: int, dtype_code: int,
                   device="cuda") -> Optional[torch.Tensor]:
    nb = workspace_bytes(n_tokens, n_heads, d_head, d_hidden, dtype_code)
    if nb == 0:
        return None
    return torch.empty(nb, dtype=torch.uint8, device=device)


def _mlp_dims(theta: torch.Tensor, X: torch.Tensor, n_heads: int, d_hidden: Optional[int]):
    C = X.shape[1]
    if C % n_heads:
        raise ValueError("channels not divisible by n_heads")
    d = C // n_heads
    per = theta.shape[-1] if theta.dim() == 2 else theta.numel() // n_heads
    m = d_hidden if d_hidden is not None else per // (3 * d)
    return d, m


LOSS_MSE, LOSS_DOT = 0, 1
OPT_GD, OPT_MUON = 0, 1
_LOSSES = {"mse": LOSS_MSE, "dot": LOSS_DOT}
_OPTS = {"gd": OPT_GD, "muon": OPT_MUON}


def _loss_code(loss) -> int:
    return _LOSSES[loss] if isinstance(loss, str) else int(loss)


def _opt_code(opt) -> int:
    return _OPTS[opt] if isinstance(opt, str) else int(opt)


def ttt_write(K: torch.Tensor, Vp: torch.Tensor, theta: torch.Tensor, lr: float, steps: int, n_heads: int,
              d_hidden: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
              loss_out: Optional[torch.Tensor] = None, loss="mse", optimizer="gd", ns_steps: int = 5) -> torch.Tensor:
    """`steps` write steps of the inner loss; theta (fp32) is updated in place.

    loss: "mse" (default) or "dot"; optimizer: "gd" (default) or "muon" with
    `ns_steps` Newton-Schulz iterations.
    """
    _check_tokens("K", K)
    _check_same("Vp", Vp, K, "K")
    d, m = _mlp_dims(theta, K, n_heads, d_hidden)
    _check_theta(theta, n_heads, d, m)
    _check_f32("loss_out", loss_out, max(int(steps), 0) * n_heads, at_least=True)
    _check_dev(K, Vp, theta, workspace, loss_out)
    dt = _dtype_code(K)
    if workspace is None:
        workspace = make_workspace(K.shape[0], n_heads, d, m, dt, K.device)
    nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lc, oc = _loss_code(loss), _opt_code(optimizer)
    if lc == LOSS_MSE and oc == OPT_GD:
        _call("vggt3_ttt_write", _ptr(K), _ptr(Vp), _ptr(theta), K.shape[0], n_heads, d, m, float(lr), int(steps),
              dt, _ptr(workspace), nb, _ptr(loss_out), _stream())
    else:
        _call("vggt3_ttt_write_ex", _ptr(K), _ptr(Vp), _ptr(theta), K.shape[0], n_heads, d, m, float(lr),
              int(steps), lc, oc, int(ns_steps), dt, _ptr(workspace), nb, _ptr(loss_out), _stream())
    return theta


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


def ttt_write_noalloc(K: torch.Tensor, Vp: torch.Tensor, theta: torch.Tensor, lr: float, steps: int, n_heads: int,
                      d_hidden: Optional[int] = None, loss_out: Optional[torch.Tensor] = None, loss="mse",
                      optimizer="gd", ns_steps: int = 5) -> torch.Tensor:
    """ttt_write through vggt3_ttt_write_noalloc: no workspace, nothing allocated
    (the library's fixed per-GPU scratch array serves as the workspace)."""
    _check_tokens("K", K)
    _check_same("Vp", Vp, K, "K")
    d, m = _mlp_dims(theta, K, n_heads, d_hidden)
    _check_theta(theta, n_heads, d, m)
    _check_f32("loss_out", loss_out, max(int(steps), 0) * n_heads, at_least=True)
    _check_dev(K, Vp, theta, loss_out)
    _call("vggt3_ttt_write_noalloc", _ptr(K), _ptr(Vp), _ptr(theta), K.shape[0], n_heads, d, m, float(lr),
          int(steps), _loss_code(loss), _opt_code(optimizer), int(ns_steps), _dtype_code(K), _ptr(loss_out),
          _stream())
    return theta


def ttt_write_conv(K: torch.Tensor, V: torch.Tensor, conv_w: torch.Tensor, n_views: int, grid_h: int, grid_w: int,
                   n_special: int, theta: torch.Tensor, lr: float, steps: int, n_heads: int,
                   Vp_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   loss_out: Optional[torch.Tensor] = None, loss="mse", optimizer="gd",
                   ns_steps: int = 5) -> torch.Tensor:
    """ShortConv2D + write with the 3x3 conv formed inside each gradient pass
    (vggt3_ttt_write_conv): V' never has to exist in device memory. With
    Vp_out, the first step also writes V' there and later steps read it.
    bf16, (d_head, d_hidden) = (64, 128); theta is updated in place."""
    _check_tokens("K", K)
    _check_same("V", V, K, "K")
    if conv_w.dtype != torch.float32 or tuple(conv_w.shape) != (K.shape[1], 3, 3):
        raise ValueError(f"conv_w must be float32 [{K.shape[1]}, 3, 3]")
    if K.shape[0] != n_views * (n_special + grid_h * grid_w):
        raise ValueError(f"K has {K.shape[0]} tokens, {n_views} views x ({n_special} + {grid_h}x{grid_w}) expected")
    _check_same("Vp_out", Vp_out, K, "K")
    d, m = _mlp_dims(theta, K, n_heads, None)
    _check_theta(theta, n_heads, d, m)
    _check_f32("loss_out", loss_out, max(int(steps), 0) * n_heads, at_least=True)
    _check_dev(K, V, conv_w, theta, Vp_out, workspace, loss_out)
    dt = _dtype_code(K)
    if workspace is None:
        workspace = make_workspace(K.shape[0], n_heads, d, m, dt, K.device)
    nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("vggt3_ttt_write_conv", _ptr(K), _ptr(V), _ptr(conv_w), n_views, grid_h, grid_w, n_special, _ptr(theta),
          n_heads, d, m, float(lr), int(steps), _loss_code(loss), _opt_code(optimizer), int(ns_steps),
          _ptr(Vp_out), _ptr(workspace), nb, _ptr(loss_out), _stream())
    return theta


def ttt_grad(K: torch.Tensor, Vp: torch.Tensor, theta: torch.Tensor, n_heads: int,
             grad: Optional[torch.Tensor] = None, accumulate: bool = False, d_hidden: Optional[int] = None,
             workspace: Optional[torch.Tensor] = None, loss_out: Optional[torch.Tensor] = None,
             loss="mse") -> torch.Tensor:
    """Gradient of the inner loss at theta (Eq. 5 split: accumulate=True adds to grad)."""
    _check_tokens("K", K)
    _check_same("Vp", Vp, K, "K")
    d, m = _mlp_dims(theta, K, n_heads, d_hidden)
    _check_theta(theta, n_heads, d, m)
    _check_f32("grad", grad, n_heads * 3 * d * m)
    _check_f32("loss_out", loss_out, n_heads, at_least=True)
    if grad is None:
        grad = torch.empty_like(theta)
    _check_dev(K, Vp, theta, grad, workspace, loss_out)
    dt = _dtype_code(K)
    if workspace is None:
        workspace = make_workspace(K.shape[0], n_heads, d, m, dt, K.device)
    nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lc = _loss_code(loss)
    if lc == LOSS_MSE:
        _call("vggt3_ttt_grad", _ptr(K), _ptr(Vp), _ptr(theta), _ptr(grad), int(bool(accumulate)), K.shape[0],
              n_heads, d, m, dt, _ptr(workspace), nb, _ptr(loss_out), _stream())
    else:
        _call("vggt3_ttt_grad_ex", _ptr(K), _ptr(Vp), _ptr(theta), _ptr(grad), int(bool(accumulate)), K.shape[0],
              n_heads, d, m, lc, dt, _ptr(workspace), nb, _ptr(loss_out), _stream())
    return grad


REDUCE_APPLY, REDUCE_STORE, REDUCE_ACCUMULATE = 0, 1, 2


def ttt_grad_partials(K: torch.Tensor, Vp: torch.Tensor, theta: torch.Tensor, n_heads: int,
                      workspace: torch.Tensor, d_hidden: Optional[int] = None, loss="mse",
                      want_loss: bool = True) -> None:
    """Per-(head, chunk) gradient and loss partials into `workspace` (Eq. 5 inner sums).
    With want_loss=False the loss partials are not computed (a later reduce's loss is NaN)."""
    _check_tokens("K", K)
    _check_same("Vp", Vp, K, "K")
    d, m = _mlp_dims(theta, K, n_heads, d_hidden)
    _check_theta(theta, n_heads, d, m)
    _check_dev(K, Vp, theta, workspace)
    lc = _loss_code(loss)
    if lc == LOSS_MSE and want_loss:
        _call("vggt3_ttt_grad_partials", _ptr(K), _ptr(Vp), _ptr(theta), K.shape[0], n_heads, d, m,
              _dtype_code(K), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream())
    else:
        _call("vggt3_ttt_grad_partials_ex", _ptr(K), _ptr(Vp), _ptr(theta), K.shape[0], n_heads, d, m, lc,
              int(bool(want_loss)), _dtype_code(K), _ptr(workspace), workspace.numel() * workspace.element_size(),
              _stream())


def muon_workspace_bytes(n_heads: int, d_head: int, d_hidden: int) -> int:
    return int(lib().vggt3_ttt_muon_workspace_bytes(n_heads, d_head, d_hidden))


def ttt_muon_apply(theta: torch.Tensor, grad: torch.Tensor, lr: float, n_heads: int, d_head: int,
                   d_hidden: int, ns_steps: int = 5, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """theta -= lr * NS(grad) per head and weight matrix (Muon update), in place
    (the full-width 1024 -> 4096 MLP takes a workspace)."""
    _check_theta(theta, n_heads, d_head, d_hidden)
    _check_f32("grad", grad, n_heads * 3 * d_head * d_hidden)
    _check_dev(theta, grad, workspace)
    need = muon_workspace_bytes(n_heads, d_head, d_hidden)
    if need == 0 and workspace is None:
        _call("vggt3_ttt_muon_apply", _ptr(theta), _ptr(grad), float(lr), n_heads, d_head, d_hidden, int(ns_steps),
              _stream())
        return theta
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=theta.device)
    _call("vggt3_ttt_muon_apply_ex", _ptr(theta), _ptr(grad), float(lr), n_heads, d_head, d_hidden, int(ns_steps),
          _ptr(workspace), workspace.numel() * workspace.element_size(), _stream())
    return theta


def ttt_reduce(workspace: torch.Tensor, n_tokens: int, n_heads: int, d_head: int, d_hidden: int, dtype_code: int,
               mode: int, dst: torch.Tensor, lr: float = 0.0, loss_out: Optional[torch.Tensor] = None) -> None:
    """Fixed-tree sum of the partials, then apply to theta / store / accumulate into dst."""
    _check_f32("dst", dst, n_heads * 3 * d_head * d_hidden)
    _check_f32("loss_out", loss_out, n_heads, at_least=True)
    _check_dev(workspace, dst, loss_out)
    _call("vggt3_ttt_reduce", _ptr(workspace), workspace.numel() * workspace.element_size(), n_tokens, n_heads,
          d_head, d_hidden, dtype_code, mode, _ptr(dst), float(lr), _ptr(loss_out), _stream())


def ttt_apply(theta: torch.Tensor, grad: torch.Tensor, lr: float, n_heads: int, d_head: int,
              d_hidden: int) -> torch.Tensor:
    _check_theta(theta, n_heads, d_head, d_hidden)
    _check_f32("grad", grad, n_heads * 3 * d_head * d_hidden)
    _check_dev(theta, grad)
    _call("vggt3_ttt_apply", _ptr(theta), _ptr(grad), float(lr), n_heads, d_head, d_hidden, _stream())
    return theta


def read_workspace_bytes(n_tokens: int, n_heads: int, d_head: int, d_hidden: int, dtype_code: int) -> int:
    return int(lib().vggt3_ttt_read_workspace_bytes(n_tokens, n_heads, d_head, d_hidden, dtype_code))


def ttt_read(Q: torch.Tensor, theta: torch.Tensor, n_heads: int, d_hidden: Optional[int] = None,
             out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """O = T_theta(Q) per head (the full-width 1024 -> 4096 MLP reads through a workspace)."""
    _check_tokens("Q", Q)
    _check_same("out", out, Q, "Q")
    d, m = _mlp_dims(theta, Q, n_heads, d_hidden)
    _check_theta(theta, n_heads, d, m)
    if out is None:
        out = torch.empty_like(Q)
    _check_dev(Q, theta, out, workspace)
    dt = _dtype_code(Q)
    need = read_workspace_bytes(Q.shape[0], n_heads, d, m, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    # vggt3_ttt_read_ex serves every shape (the per-head ones ignore the workspace)
    _call("vggt3_ttt_read_ex", _ptr(Q), _ptr(theta), _ptr(out), Q.shape[0], n_heads, d, m, dt, _ptr(workspace), nb,
          _stream())
    return out


def ttt_layer(K, V, Q, theta, conv_w, n_views, grid_h, grid_w, n_special, n_heads, lr, steps,
              workspace=None, loss_out=None, Vp=None, O=None, loss="mse", optimizer="gd", ns_steps=5,
              conv_k=None):
    """The whole layer: V' = ShortConv2D(V); write theta (in place); O = read(Q).

    conv_w may be [C, 3, 3] (the pages' ShortConv2D) or [C, 5, 5] (their "V-5"
    variant); conv_k, if given, convolves the keys as well before the write
    (their "KV-3" variant, with its own filters)."""
    Vp = shortconv(V, conv_w, n_views, grid_h, grid_w, n_special, out=Vp)
    if conv_k is not None:
        K = shortconv(K, conv_k, n_views, grid_h, grid_w, n_special)
    ttt_write(K, Vp, theta, lr, steps, n_heads, workspace=workspace, loss_out=loss_out, loss=loss,
              optimizer=optimizer, ns_steps=ns_steps)
    return ttt_read(Q, theta, n_heads, out=O), Vp


# ---------------------------------------------------------------------------
# Streamed (offloaded) write and read over host-resident token tensors
# ---------------------------------------------------------------------------

_side_streams = {}


def _side_stream(device: torch.device, key: str) -> torch.cuda.Stream:
    """A per-device copy stream of default priority, created once."""
    idx = device.index if device.index is not None else torch.cuda.current_device()
    s = _side_streams.get((idx, key))
    if s is None:
        s = torch.cuda.Stream(device=idx)
        _side_streams[(idx, key)] = s
    return s


def _check_host(*ts):
    for t in ts:
        if t.is_cuda:
            raise ValueError("streamed token tensors live in host memory (pinned for overlap)")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def stage_bytes(chunk_tokens: int, n_heads: int, d_head: int, dtype_code: int) -> int:
    """Device staging a streamed call needs: two slots of two token chunks."""
    return int(lib().vggt3_ttt_stream_stage_bytes(chunk_tokens, n_heads, d_head, dtype_code))


def ttt_write_streamed(K_host: torch.Tensor, Vp_host: torch.Tensor, theta: torch.Tensor, lr: float, steps: int,
                       n_heads: int, chunk_tokens: int, d_hidden: Optional[int] = None,
                       stage: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       loss_out: Optional[torch.Tensor] = None, loss="mse", optimizer="gd", ns_steps: int = 5,
                       copy_stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """ttt_write over host-resident K and V' streamed in chunks of `chunk_tokens`
    (Eq. 5 offload schedule); theta is a device tensor updated in place.

    The copies run on `copy_stream` (default: a side stream of this device)
    while the kernels run on the current stream; the host tensors must stay
    untouched until the current stream has been synchronised."""
    _check_tokens("K_host", K_host)
    _check_same("Vp_host", Vp_host, K_host, "K_host")
    d, m = _mlp_dims(theta, K_host, n_heads, d_hidden)
    _check_theta(theta, n_heads, d, m)
    _check_f32("loss_out", loss_out, max(int(steps), 0) * n_heads, at_least=True)
    _check_host(K_host, Vp_host)
    _check_dev(theta, stage, workspace, loss_out)
    dt = _dtype_code(K_host)
    n = K_host.shape[0]
    ct = max(1, min(int(chunk_tokens), n))
    if stage is None:
        stage = torch.empty(stage_bytes(ct, n_heads, d, dt), dtype=torch.uint8, device=theta.device)
    if workspace is None:
        workspace = make_workspace(ct, n_heads, d, m, dt, theta.device)
    if copy_stream is None:
        copy_stream = _side_stream(theta.device, "h2d")
    ws_nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("vggt3_ttt_write_streamed", _ptr(K_host), _ptr(Vp_host), _ptr(theta), n, n_heads, d, m, float(lr),
          int(steps), _loss_code(loss), _opt_code(optimizer), int(ns_steps), dt, int(chunk_tokens), _ptr(stage),
          stage.numel() * stage.element_size(), _ptr(workspace), ws_nb, _ptr(loss_out), _stream(),
          ctypes.c_void_p(copy_stream.cuda_stream))
    return theta


def ttt_read_streamed(Q_host: torch.Tensor, theta: torch.Tensor, n_heads: int, chunk_tokens: int,
                      d_hidden: Optional[int] = None, out: Optional[torch.Tensor] = None,
                      stage: Optional[torch.Tensor] = None, h2d_stream: Optional[torch.cuda.Stream] = None,
                      d2h_stream: Optional[torch.cuda.Stream] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """O = T_theta(Q) for host-resident Q, written to a host tensor (query mode
    over a frozen theta), streamed in chunks of `chunk_tokens`. `out` defaults
    to a new pinned tensor; read it after synchronising the current stream."""
    _check_tokens("Q_host", Q_host)
    _check_same("out", out, Q_host, "Q_host")
    d, m = _mlp_dims(theta, Q_host, n_heads, d_hidden)
    _check_theta(theta, n_heads, d, m)
    if out is None:
        out = torch.empty(Q_host.shape, dtype=Q_host.dtype, pin_memory=True)
    _check_host(Q_host, out)
    _check_dev(theta, stage)
    dt = _dtype_code(Q_host)
    n = Q_host.shape[0]
    ct = max(1, min(int(chunk_tokens), n))
    if stage is None:
        stage = torch.empty(stage_bytes(ct, n_heads, d, dt), dtype=torch.uint8, device=theta.device)
    if h2d_stream is None:
        h2d_stream = _side_stream(theta.device, "h2d")
    if d2h_stream is None:
        d2h_stream = _side_stream(theta.device, "d2h")
    if workspace is None:
        need = read_workspace_bytes(ct, n_heads, d, m, dt)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=theta.device)
    _check_dev(workspace)
    nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("vggt3_ttt_read_streamed_ex", _ptr(Q_host), _ptr(theta), _ptr(out), n, n_heads, d, m, dt,
          int(chunk_tokens), _ptr(stage), stage.numel() * stage.element_size(), _ptr(workspace), nb, _stream(),
          ctypes.c_void_p(h2d_stream.cuda_stream), ctypes.c_void_p(d2h_stream.cuda_stream))
    return out
