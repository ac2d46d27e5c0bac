"""Seeded synthetic inputs with the shapes of the VGG-T^3 workloads.

Token geometry (paper-graph summary of VGG-T^3, section 3.4 "Tokenization"):
a 518x518 view cut into 14x14 patches gives a 37x37 patch grid; camera and
register tokens ride along with each view. Per view the tokens are laid out as
``[n_special special tokens][grid_h*grid_w patch tokens, row-major]`` and views
follow one another, so a token tensor is ``[n_views * tokens_per_view, C]`` with
``C = n_heads * d_head`` channels and head ``h`` owning channels
``h*d_head .. h*d_head + d_head - 1``.

Value distributions follow the layer's synthetic workload recipe:
K, V, Q ~ N(0, 1) in fp32; in the VGGT-shaped workloads each head's slice is
then scaled to unit L2 norm (the pages replace LayerNorm on Q and K by a plain
L2 normalisation; the synthetic recipe applies it to V as well) and rounded to
bf16 (round to nearest even, done by torch's dtype cast). Fast weights theta_0
are N(0, 0.02^2) in fp32 (std 0.02); depthwise 3x3 conv weights are N(0, 1/9)
in fp32 (std 1/3).

Generation uses torch generators on the device the tensors are wanted on, so a
1000-view scene is drawn in HBM in milliseconds. Values drawn on the CPU and on
a GPU differ; every consumer that needs the same bytes (the oracle in a GPU
test) copies them from the tensors made here.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import torch

# Random streams: each tensor kind has its own generator so that the presence
# or size of one input never shifts the values of another.
_STREAM = {"K": 1, "V": 2, "Q": 3, "theta": 4, "conv_w": 5}

# Views drawn per randn call (bounds the fp32 temporaries at large scene sizes).
_VIEW_CHUNK = 64


@dataclass(frozen=True)
class LayerConfig:
    name: str
    n_views: int
    grid_h: int
    grid_w: int
    n_special: int
    n_heads: int
    d_head: int
    d_hidden: int
    steps: int
    lr: float
    dtype: str  # "bf16" or "f32": storage/compute type of K, V, V', Q, O
    normalize: bool  # per-head L2 normalisation of K, V, Q
    seed: int = 0
    # Query-mode read (frozen theta applied to unseen views, drawn from query_seed).
    query_views: int = 0
    query_seed: int = 1
    description: str = field(default="", compare=False)

    @property
    def tokens_per_view(self) -> int:
        return self.n_special + self.grid_h * self.grid_w

    @property
    def n_tokens(self) -> int:
        return self.n_views * self.tokens_per_view

    @property
    def channels(self) -> int:
        return self.n_heads * self.d_head

    @property
    def theta_per_head(self) -> int:
        return 3 * self.d_head * self.d_hidden

    @property
    def n_query_tokens(self) -> int:
        return self.query_views * self.tokens_per_view

    def with_views(self, n_views: int, **kw) -> "LayerConfig":
        return replace(self, n_views=n_views, name=f"{self.name}@{n_views}v", **kw)


def view_token_count(grid_h: int, grid_w: int, n_special: int) -> int:
    return n_special + grid_h * grid_w


_VGGT = dict(grid_h=37, grid_w=37, n_special=5, n_heads=16, d_head=64, d_hidden=128,
             lr=0.1, dtype="bf16", normalize=True)

CONFIGS = {
    "tiny_f32": LayerConfig(
        name="tiny_f32", n_views=2, grid_h=8, grid_w=8, n_special=0, n_heads=1,
        d_head=16, d_hidden=32, steps=1, lr=0.1, dtype="f32", normalize=False,
        description="2 views of 8x8 patches (128 tokens), 1 head, d 16, hidden 32, fp32, 1 step"),
    "views24": LayerConfig(
        name="views24", n_views=24, steps=1, **_VGGT,
        description="24 views x (37x37 + 5) = 32,976 tokens, 16 heads x 64, hidden 128, 1 step"),
    "views100": LayerConfig(
        name="views100", n_views=100, steps=2, **_VGGT,
        description="100 views = 137,400 tokens, 2 steps"),
    "views1000": LayerConfig(
        name="views1000", n_views=1000, steps=2, **_VGGT,
        description="1000 views = 1,374,000 tokens, 2 steps + full read"),
    "views2000": LayerConfig(
        name="views2000", n_views=2000, steps=2, query_views=50, **_VGGT,
        description="2000 views = 2,748,000 tokens, 2 steps; read of 50 unseen views (68,700 queries)"),
}


@dataclass
class LayerInputs:
    cfg: LayerConfig
    K: torch.Tensor  # [n, C] bf16 or fp32
    V: torch.Tensor  # [n, C]
    Q: Optional[torch.Tensor]  # [n, C] (or [n_query, C] in query mode)
    theta0: torch.Tensor  # [n_heads, 3*d*m] fp32: per head [W_g (d x m) | W_u (d x m) | W_d (m x d)]
    conv_w: torch.Tensor  # [C, 3, 3] fp32


def _generator(device: torch.device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + stream)
    return g


def _token_tensor(cfg: LayerConfig, n_views: int, seed: int, stream: int,
                  device: torch.device) -> torch.Tensor:
    """N(0,1) draws, optionally per-head unit-L2-normalised, stored in cfg.dtype."""
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    tpv = cfg.tokens_per_view
    C = cfg.channels
    out = torch.empty((n_views * tpv, C), dtype=dt, device=device)
    g = _generator(device, seed, stream)
    for v0 in range(0, n_views, _VIEW_CHUNK):
        v1 = min(n_views, v0 + _VIEW_CHUNK)
        x = torch.randn(((v1 - v0) * tpv, C), generator=g, device=device, dtype=torch.float32)
        if cfg.normalize:
            xh = x.view(-1, cfg.n_heads, cfg.d_head)
            nrm = torch.linalg.vector_norm(xh, dim=-1, keepdim=True).clamp_min(1e-12)
            x = (xh / nrm).view(-1, C)
        out[v0 * tpv:v1 * tpv] = x.to(dt)
        del x
    return out


def make_inputs(cfg: LayerConfig, device="cpu", with_q: bool = True) -> LayerInputs:
    """Draw the layer's inputs for `cfg` on `device`.

    With ``cfg.query_views > 0`` the returned Q holds the unseen query views
    (drawn from ``cfg.query_seed``) instead of the scene's own queries.
    """
    device = torch.device(device)
    K = _token_tensor(cfg, cfg.n_views, cfg.seed, _STREAM["K"], device)
    V = _token_tensor(cfg, cfg.n_views, cfg.seed, _STREAM["V"], device)
    Q = None
    if with_q:
        if cfg.query_views > 0:
            Q = _token_tensor(cfg, cfg.query_views, cfg.query_seed, _STREAM["Q"], device)
        else:
            Q = _token_tensor(cfg, cfg.n_views, cfg.seed, _STREAM["Q"], device)
    g = _generator(device, cfg.seed, _STREAM["theta"])
    theta0 = torch.randn((cfg.n_heads, cfg.theta_per_head), generator=g, device=device,
                         dtype=torch.float32) * 0.02
    g = _generator(device, cfg.seed, _STREAM["conv_w"])
    conv_w = torch.randn((cfg.channels, 3, 3), generator=g, device=device,
                         dtype=torch.float32) * (1.0 / 3.0)
    return LayerInputs(cfg=cfg, K=K, V=V, Q=Q, theta0=theta0, conv_w=conv_w)
