"""Seeded synthetic inputs for the VSA-H3 attention forward.

This module is shared by the HIP path's tests and bench and by the oracle's
tests.  It holds no arithmetic of the method itself: it only lays out the
packed token stream (segment tags and video grid positions) and draws the
q / k / v / gate tensors.

Shapes follow the FastH3 pages: a 1344x768, 243-frame clip packs 73.6k tokens
(FastH3 NVFP4 on RTX PRO 6000, "Results"); a 480p, 124-frame clip packs 15.1k
tokens (same section); the transformer has 56 heads (same page, "Per-block
measurements"); the tokens are packed as [text | cond | audio | video]
(FastH3 4-step Preview, "Video Sparse Attention is not optional here").

No trained activations or gates exist here, so every tensor is synthetic:
q, k, v ~ N(0, 1) and gate ~ N(0, 0.1) (0.1 is the standard deviation).  The
"smooth" workloads give q and k a low-frequency spatiotemporal component
(a sum of four random sinusoids over t, y, x) plus N(0, 0.5) noise on video
tokens, so pooled tile scores carry structure instead of being uniform.

All draws use torch's CPU generator seeded with ``seed`` and happen in a fixed
order (sinusoid parameters first, then q, k, v, gate), in float32; bf16
workloads round with round-to-nearest-even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

# Segment tags of the packed stream.  Text tags travel as int64 on the pages'
# wire format (FastH3 4-step Preview, "Split across two Spaces").
TEXT, COND, AUDIO, VIDEO = 0, 1, 2, 3
TAG_NAMES = {TEXT: "text", COND: "cond", AUDIO: "audio", VIDEO: "video"}


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    head_dim: int
    io_dtype: str                  # "f32" or "bf16"
    prefix: tuple                  # ((tag, n_tokens), ...) in packed order
    grid: tuple                    # post-patchify video grid (T, H, W)
    sparsity: float
    smooth: bool = False
    description: str = ""
    tile: tuple = (4, 4, 4)        # video tile box (64 or 128 grid cells)
    ref_keep: float = 1.0          # reference keep ratio (1: every cond tile visited)

    @property
    def n_prefix_tokens(self) -> int:
        return sum(n for _, n in self.prefix)

    @property
    def n_video_tokens(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def L(self) -> int:
        return self.n_prefix_tokens + self.n_video_tokens

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload(
        "tiny", 2, 64, "f32", ((TEXT, 64),), (8, 8, 8), 0.5,
        description="2 heads, head_dim 64, fp32 I/O; 64 text tokens + 8x8x8 video grid "
                    "(576 tokens, 8 video tiles); sparsity 0.5"),
    "480p5s": Workload(
        "480p5s", 56, 128, "bf16", ((TEXT, 512), (COND, 256), (AUDIO, 512)), (16, 24, 36), 0.9,
        description="480p 5-s shape: 15,104 tokens (1,280 prefix + 16x24x36 video), "
                    "56 heads, head_dim 128, bf16, sparsity 0.9"),
    "768p10s": Workload(
        "768p10s", 56, 128, "bf16", ((TEXT, 512), (AUDIO, 512)), (18, 48, 84), 0.8,
        description="768p 10-s shape: 73,600 tokens (1,024 prefix + 18x48x84 video; the last "
                    "temporal tile row holds 2 frames), 56 heads, head_dim 128, bf16, sparsity 0.8"),
    "768p10s_smooth": Workload(
        "768p10s_smooth", 56, 128, "bf16", ((TEXT, 512), (AUDIO, 512)), (18, 48, 84), 0.9,
        smooth=True,
        description="768p 10-s shape at sparsity 0.9 with smooth+noise q/k"),
    "768p15s_smooth": Workload(
        "768p15s_smooth", 56, 128, "bf16", ((TEXT, 512), (COND, 1536), (AUDIO, 1024)),
        (27, 48, 84), 0.9, smooth=True,
        description="768p 15-s shape: 111,936 tokens (3,072 prefix + 27x48x84 video; last "
                    "temporal tile row 3 frames), smooth+noise q/k, sparsity 0.9"),
    # The OmniRef profile: VSA at sparsity 0.9 with 128-token tiles and
    # reference keep 0.1 (the OmniRef page, "Device profiles").  Its reference
    # prefix here is 4 images of 896x896 at one vision token per 28x28 pixels
    # (4 x 1,024 cond tokens); the pages give no token counts for it.
    "omniref768p10s": Workload(
        "omniref768p10s", 56, 128, "bf16", ((TEXT, 512), (COND, 4096), (AUDIO, 512)),
        (18, 48, 84), 0.9, tile=(4, 8, 4), ref_keep=0.1,
        description="OmniRef 768p 10-s shape: 77,696 tokens (512 text + 4,096 reference + "
                    "512 audio + 18x48x84 video), 56 heads, head_dim 128, bf16, sparsity 0.9, "
                    "(4,8,4) 128-token tiles (the last temporal tile row holds 2 frames: "
                    "64 tokens), reference keep 0.1"),
    "omniref_small": Workload(
        "omniref_small", 2, 128, "bf16", ((TEXT, 100), (COND, 700), (AUDIO, 60), (COND, 200)),
        (10, 16, 12), 0.7, tile=(4, 8, 4), ref_keep=0.3,
        description="small OmniRef layout: 2,980 tokens (1,060 prefix tokens in 10 tiles, 8 "
                    "of them reference tiles, + 10x16x12 video in 18 tiles, those of the last "
                    "temporal row 64 tokens each), 2 heads, head_dim 128, bf16, sparsity 0.7, "
                    "reference keep 0.3"),
}


def make_layout(w: Workload, video_order: str = "raster", seed: int = 0):
    """Packed token tags [L] int64 and position ids [L, 3] int64 (t, y, x).

    Prefix tokens come first, one run per segment, and carry position 0.
    Video tokens follow; ``video_order="raster"`` lists them in (t, y, x)
    raster order, as a patchify emits them, ``"shuffled"`` in a seeded random
    order (the packing carries its positions, so any order is legal).
    """
    tags = []
    for tag, n in w.prefix:
        tags.append(torch.full((n,), tag, dtype=torch.int64))
    T, H, W = w.grid
    nv = T * H * W
    tags.append(torch.full((nv,), VIDEO, dtype=torch.int64))
    tags = torch.cat(tags) if tags else torch.zeros(0, dtype=torch.int64)
    pos = torch.zeros((w.L, 3), dtype=torch.int64)
    if nv:
        tt, yy, xx = torch.meshgrid(torch.arange(T), torch.arange(H), torch.arange(W),
                                    indexing="ij")
        vpos = torch.stack([tt.reshape(-1), yy.reshape(-1), xx.reshape(-1)], dim=1)
        if video_order == "shuffled":
            g = torch.Generator().manual_seed(seed + 7919)
            vpos = vpos[torch.randperm(nv, generator=g)]
        elif video_order != "raster":
            raise ValueError(video_order)
        pos[w.n_prefix_tokens:] = vpos
    return tags, pos


def _round_bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def _smooth_component(g: torch.Generator, heads: int, head_dim: int, pos_video: torch.Tensor,
                      grid, n_terms: int = 4) -> torch.Tensor:
    """sqrt(2/n) * sum_m sin(2*pi*(a_m t/T + b_m y/H + c_m x/W) + phi_m) per (head, channel).

    a_m in {0,1,2}, b_m, c_m in {0..3} (not all zero), phi_m ~ U[0, 2*pi).
    Unit variance per channel.  Returns [n_video, heads, head_dim] float32.
    """
    T, H, W = grid
    C = heads * head_dim
    a = torch.randint(0, 3, (n_terms, C), generator=g)
    b = torch.randint(0, 4, (n_terms, C), generator=g)
    c = torch.randint(0, 4, (n_terms, C), generator=g)
    phi = torch.rand((n_terms, C), generator=g, dtype=torch.float32) * (2 * math.pi)
    zero = (a == 0) & (b == 0) & (c == 0)
    c = torch.where(zero, torch.ones_like(c), c)          # no constant term
    t = pos_video[:, 0:1].to(torch.float32) / T
    y = pos_video[:, 1:2].to(torch.float32) / H
    x = pos_video[:, 2:3].to(torch.float32) / W
    out = torch.zeros((pos_video.shape[0], C), dtype=torch.float32)
    for m in range(n_terms):
        arg = (t * a[m].to(torch.float32) + y * b[m].to(torch.float32)
               + x * c[m].to(torch.float32)) * (2 * math.pi) + phi[m]
        out += torch.sin(arg)
        del arg
    out *= math.sqrt(2.0 / n_terms)
    return out.view(-1, heads, head_dim)


def make_inputs(w: Workload, seed: int = 0, video_order: str = "raster"):
    """Returns dict(q, k, v, gate, token_tags, position_ids) as CPU tensors.

    q, k, v, gate: [L, heads, head_dim] in the workload's I/O dtype
    (torch.float32 or torch.bfloat16), sequence-major and contiguous.
    """
    tags, pos = make_layout(w, video_order, seed)
    L, Hh, D = w.L, w.heads, w.head_dim
    g = torch.Generator().manual_seed(seed)
    smooth_q = smooth_k = None
    pv = pos[w.n_prefix_tokens:]
    if w.smooth and w.n_video_tokens:
        smooth_q = _smooth_component(g, Hh, D, pv, w.grid)
        smooth_k = _smooth_component(g, Hh, D, pv, w.grid)
    out = {}
    for name, sm in (("q", smooth_q), ("k", smooth_k), ("v", None)):
        x = torch.randn((L, Hh, D), generator=g, dtype=torch.float32)
        if sm is not None:
            # video tokens: smooth part + N(0, 0.5) noise; prefix tokens stay N(0, 1)
            xv = x[w.n_prefix_tokens:]
            xv.mul_(0.5).add_(sm)
        out[name] = x
    out["gate"] = torch.randn((L, Hh, D), generator=g, dtype=torch.float32).mul_(0.1)
    if w.io_dtype == "bf16":
        for name in ("q", "k", "v", "gate"):
            out[name] = _round_bf16(out[name])
    elif w.io_dtype != "f32":
        raise ValueError(w.io_dtype)
    out["token_tags"] = tags
    out["position_ids"] = pos
    return out


def make_qk_prep_inputs(w: Workload, position_ids, seed: int = 0, theta: float = 10000.0):
    """Synthetic inputs of the optional QK-norm + RoPE step (the H3 weights and
    frequencies are not published): norm weights for q and k drawn from
    U(0.5, 1.5), eps 1e-6, and per-token cos/sin tables [L, D/2] of a 3D RoPE
    whose pairs are split over (t, y, x) as (D/2 - 2*(D/6), D/6, D/6) with
    frequencies theta^(-j/n) inside each axis; prefix tokens get angle 0.
    Returns dict(q_weight, k_weight, eps, cos, sin) of CPU float32 tensors."""
    D = w.head_dim
    g = torch.Generator().manual_seed(seed + 7919)
    qw = torch.rand(D, generator=g, dtype=torch.float32) + 0.5
    kw = torch.rand(D, generator=g, dtype=torch.float32) + 0.5
    pairs = D // 2
    ny = nx = D // 6
    nt = pairs - ny - nx
    pos = torch.as_tensor(position_ids, dtype=torch.float64).reshape(-1, 3)
    L = pos.shape[0]
    ang = torch.zeros((L, pairs), dtype=torch.float64)
    start = 0
    n_pre = w.n_prefix_tokens
    for axis, n in enumerate((nt, ny, nx)):
        freqs = theta ** (-torch.arange(n, dtype=torch.float64) / max(n, 1))
        ang[n_pre:, start:start + n] = pos[n_pre:, axis:axis + 1] * freqs[None, :]
        start += n
    return {"q_weight": qw, "k_weight": kw, "eps": 1e-6,
            "cos": torch.cos(ang).to(torch.float32), "sin": torch.sin(ang).to(torch.float32)}
