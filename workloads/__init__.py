"""Seeded synthetic inputs for gated, tile-sparse video attention.

This module only *draws* inputs: it holds no step of the attention method
(no tiling, pooling, scoring, selection, softmax or gate projection). Both the
CPU oracle and the HIP path consume what it produces; neither imports the
other.

Every tensor is drawn on the host with torch's CPU generator from a seed that
is a pure function of (workload seed, stream id), sampled in fp32 and rounded
once to bf16 (round-to-nearest-even, torch's own conversion). Stream ids:
0 = Q, 1 = K, 2 = V, 3 = x, 4 = W_gate, 5 = per-head scales, 6 = low-rank
fields, 7 = low-rank per-head bases, 8-10 = W_q, W_k, W_v (for the layer run
from its input x).

The shapes follow the workloads these pages measure: MiniMax-H3-like layers
(42 heads x 128, hidden 5376) with a segment-pure prefix of text, reference
image and reference audio tokens ahead of a t-major video latent grid
(Ref2VA VSA news item, "The two-tier attention patch"; SnackOnAI analysis,
"It In Action", step two). Real H3 activations are neither public nor
available; these synthetic tensors stand in for them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

import torch

STREAM_Q, STREAM_K, STREAM_V, STREAM_X, STREAM_W = 0, 1, 2, 3, 4
STREAM_HEAD_SCALE, STREAM_FIELDS, STREAM_LOWRANK_U = 5, 6, 7
STREAM_WQ, STREAM_WK, STREAM_WV = 8, 9, 10


@dataclass(frozen=True)
class Workload:
    """One attention-layer shape plus the recipe for its values."""

    name: str
    seed: int
    heads: int
    head_dim: int
    hidden: int
    prefix_segments: Tuple[int, ...]
    grid: Tuple[int, int, int]          # latent (T, H, W) of the generated video
    tile: Tuple[int, int, int]          # tile shape (t, h, w)
    sparsity: Optional[float] = None    # fraction of video key tiles dropped
    keep_k: Optional[int] = None        # integer keep-count (overrides sparsity)
    values: str = "normal"              # "normal" | "normal_head_scaled" | "lowrank_smooth"
    w_gate_std: float = 0.02
    note: str = field(default="", compare=False)

    @property
    def prefix_tokens(self) -> int:
        return int(sum(self.prefix_segments))

    @property
    def video_tokens(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def tokens(self) -> int:
        return self.prefix_tokens + self.video_tokens

    @property
    def tile_rows(self) -> int:
        a, b, c = self.tile
        return a * b * c


# The five layer shapes, plus the worked geometry of the SnackOnAI analysis
# ("It In Action", step two: 150 text + 1,008 reference + 414 audio tokens and a
# 37 x 24 x 42 latent grid) as an extra, untimed parity case.
WORKLOADS = {
    "tiny": Workload("tiny", 1001, 2, 64, 128, (20, 40), (4, 8, 8), (4, 4, 4),
                     keep_k=2, note="2 sink tiles + 4 video tiles"),
    "mid": Workload("mid", 1002, 8, 128, 1024, (77, 1024, 200), (8, 16, 32), (4, 4, 4),
                    sparsity=0.75, note="22 prefix + 64 video tiles, k=16"),
    "h3": Workload("h3", 1003, 42, 128, 5376, (512, 512, 512, 128), (24, 48, 84), (4, 4, 4),
                   sparsity=0.75, values="normal_head_scaled",
                   note="H3-shaped layer, 98,432 tokens, 26 + 1512 tiles, k=378"),
    "veda": Workload("veda", 1004, 42, 128, 5376, (512, 512, 512, 128), (32, 48, 84), (4, 8, 4),
                     keep_k=101, values="lowrank_smooth",
                     note="128-row tiles, 13 + 1008 tiles, 90% sparsity as integer k=101"),
    "long": Workload("long", 1005, 42, 128, 5376, (512, 512, 512, 128), (88, 48, 84), (4, 4, 4),
                     sparsity=0.95, note="356,480 tokens, 26 + 5544 tiles, k=277"),
    "page5": Workload("page5", 1006, 2, 128, 256, (150, 1008, 414), (37, 24, 42), (4, 4, 4),
                      sparsity=0.75, note="worked geometry with partial edge tiles"),
}


def _gen(seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) * 1_000_003 + int(stream) * 7_919 + 17)
    return g


def _normal(shape, seed: int, stream: int) -> torch.Tensor:
    return torch.randn(*shape, generator=_gen(seed, stream), dtype=torch.float32)


def _uniform(shape, seed: int, stream: int) -> torch.Tensor:
    return torch.rand(*shape, generator=_gen(seed, stream), dtype=torch.float32)


def _video_positions(wl: Workload) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(t, y, x) of each video token; the video is flattened t-major, then h, then w."""
    T, Hg, Wg = wl.grid
    t = torch.arange(T, dtype=torch.float32).view(T, 1, 1).expand(T, Hg, Wg).reshape(-1)
    y = torch.arange(Hg, dtype=torch.float32).view(1, Hg, 1).expand(T, Hg, Wg).reshape(-1)
    x = torch.arange(Wg, dtype=torch.float32).view(1, 1, Wg).expand(T, Hg, Wg).reshape(-1)
    return t, y, x


def _lowrank_video(wl: Workload, rank: int = 8) -> torch.Tensor:
    """Spatially smooth low-rank component shared by Q and K: [S_video][H][D] fp32.

    Eight fields f_m(t,y,x) = sqrt(2) cos(2 pi (a t/T + b y/Hg + c x/Wg) + phi),
    a in {0,1,2}, b,c in {0..3}, phi ~ U[0, 2 pi); per head U_h ~ N(0,1)^{8 x D}/sqrt(8).
    """
    T, Hg, Wg = wl.grid
    u = _uniform((rank, 4), wl.seed, STREAM_FIELDS)
    a = torch.floor(u[:, 0] * 3.0)
    b = torch.floor(u[:, 1] * 4.0)
    c = torch.floor(u[:, 2] * 4.0)
    phi = u[:, 3] * (2.0 * math.pi)
    t, y, x = _video_positions(wl)
    arg = (2.0 * math.pi) * (a[None, :] * t[:, None] / T + b[None, :] * y[:, None] / Hg
                             + c[None, :] * x[:, None] / Wg) + phi[None, :]
    f = math.sqrt(2.0) * torch.cos(arg)                                    # [S_v][rank]
    U = _normal((wl.heads, rank, wl.head_dim), wl.seed, STREAM_LOWRANK_U) / math.sqrt(rank)
    return torch.einsum("sr,hrd->shd", f, U)                               # [S_v][H][D]


def head_scales(wl: Workload) -> torch.Tensor:
    """Per-head scale s_h ~ U(0.5, 2) applied to Q, K and V of the H3-shaped layer."""
    return 0.5 + 1.5 * _uniform((wl.heads,), wl.seed, STREAM_HEAD_SCALE)


def make_qkv(wl: Workload) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Q, K, V as bf16 CPU tensors [S][H][D] in natural (prefix-then-video) token order."""
    shape = (wl.tokens, wl.heads, wl.head_dim)
    out = []
    for stream in (STREAM_Q, STREAM_K, STREAM_V):
        x = _normal(shape, wl.seed, stream)
        if wl.values == "normal_head_scaled":
            x.mul_(head_scales(wl).view(1, -1, 1))
        elif wl.values == "lowrank_smooth" and stream in (STREAM_Q, STREAM_K):
            # Video rows: smooth low-rank signal + 0.5 * noise; prefix rows stay N(0,1).
            p = wl.prefix_tokens
            x[p:].mul_(0.5).add_(_lowrank_video(wl))
        out.append(x.to(torch.bfloat16))
        del x
    return out[0], out[1], out[2]


def make_x(wl: Workload) -> torch.Tensor:
    """Layer input x ~ N(0,1), bf16 [S][hidden]."""
    return _normal((wl.tokens, wl.hidden), wl.seed, STREAM_X).to(torch.bfloat16)


def make_w_gate(wl: Workload) -> torch.Tensor:
    """Bias-free gate weight W_gate ~ N(0, std^2), bf16 [H*D][hidden] (nn.Linear out x in)."""
    w = _normal((wl.heads * wl.head_dim, wl.hidden), wl.seed, STREAM_W)
    return (w * wl.w_gate_std).to(torch.bfloat16)


def make_w_qkvg(wl: Workload) -> torch.Tensor:
    """Stacked bias-free projection weights [W_q; W_k; W_v; W_gate], bf16
    [4][H*D][hidden]: W_q, W_k, W_v ~ N(0, 1/hidden) (unit-variance projections of
    a unit-variance x), W_gate as make_w_gate."""
    HD = wl.heads * wl.head_dim
    ws = [(_normal((HD, wl.hidden), wl.seed, st) * wl.hidden ** -0.5).to(torch.bfloat16)
          for st in (STREAM_WQ, STREAM_WK, STREAM_WV)]
    return torch.stack(ws + [make_w_gate(wl)])


def bf16_bits(t: torch.Tensor):
    """uint16 numpy view of a bf16 CPU tensor (the raw bit patterns)."""
    assert t.dtype == torch.bfloat16 and t.device.type == "cpu"
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def custom(name: str = "custom", **kw) -> Workload:
    """A workload with explicit fields (tests use this for small random geometries)."""
    base = dict(seed=7, heads=1, head_dim=64, hidden=64, prefix_segments=(), grid=(4, 4, 4),
                tile=(4, 4, 4))
    base.update(kw)
    return Workload(name=name, **base)
