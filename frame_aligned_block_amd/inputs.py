"""Seeded synthetic inputs for frame-aligned windowed attention.

This module draws random tensors and nothing else: it holds none of the
attention arithmetic, so both the HIP path and the fp64 oracle can take their
inputs from it without sharing any of the method's code.

The workloads stand in for the unpublished production data of the source page
("HeyGen 与 Google Cloud：将 Avatar IV 部署到 TPU", news.xcc.im/article/5328,
sections "Deleting the Mask" and "Unchaining the Softmax"): a chunk of F video
frames of T tokens each, tokens frame-major, H heads of width d.

Recipe (one independent stream per (batch, head), so any single head can be
regenerated without drawing the others):
  * generator: ``torch.Generator(device)`` seeded with ``head_seed(seed, b, h)``;
  * draws, in this order, all float32:
      q = N(0,1) [N, d];  e = N(0,1) [N, d];
      c = 4 * N(0,1) [1, d]        (only when keys carry a shared mean);
      v = N(0,1) [N, d];
      p = randint(0, T) [F]        (only for a loose head);
      u = randint(0, T - R + 1) [F] (only for configs with R = hot_rows > 0);
  * k = sigma * e + c  (or k = sigma * e), sigma = key_sigma (1 by default);
  * a loose head multiplies, in every frame g (or only in the frames a config
    lists), the raw key at token g*T + p[g] (shared mean included) by 20;
  * with hot rows, the queries at tokens g*T + u[g] + [0, R) of every frame g
    are multiplied by hot_scale;
  * finally q, k, v are cast to the config dtype (bf16 rounds to nearest even).
The cast tensors are the inputs; the oracle upcasts exactly these values.

The stream differs between a CPU and a GPU generator; a comparison always
feeds one set of drawn values to both sides.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import torch


@dataclass(frozen=True)
class Config:
    name: str
    F: int            # frames in the chunk
    T: int            # tokens per frame
    H: int            # heads
    d: int            # head width
    dtype: str        # "bf16" or "f32"
    window: int       # frames on each side of the query frame
    ref_frame: int    # the global reference frame
    shared_mean: bool  # keys = c + N(0,1) with one c ~ N(0, 4^2) per head
    loose_period: int = 0   # head h is loose iff loose_period and h % loose_period == loose_phase
    loose_phase: int = 0
    loose_frames: tuple = ()  # frames holding a loose head's outlier key; () = every frame
    B: int = 1
    M: int = 0        # cross-attention: reference tokens every query attends to (0 = self)
    grid: tuple = ()  # (Hg, Wg) latent patch grid of a frame (T = Hg*Wg); producer workloads
    key_sigma: float = 1.0  # spread of the keys around their shared mean
    hot_rows: int = 0       # a band of this many query rows per frame is scaled ...
    hot_scale: float = 1.0  # ... by this factor

    @property
    def N(self) -> int:
        return self.F * self.T

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def is_loose(self, h: int) -> bool:
        return self.loose_period > 0 and h % self.loose_period == self.loose_phase

    def with_(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


# The five workloads: a tiny fp32 plumbing case, a small bf16 case whose frame
# span (22x40 patches = 880 tokens) is not a multiple of 128, the 720p- and
# 1080p-shaped super-resolution chunks (45x80 and 68x120 latent patch grids),
# and the 720p shape with 40 heads of which one in fifty has a loose bound.
# A sixth runs the 720p shape with a window that covers every frame: dense
# self-attention over the chunk through the same kernel. A seventh has loose
# heads whose outlier key sits in one frame only (frame 6), so only the frames
# whose slice holds frame 6 have a loose bound: the case for eligibility per
# (head, frame). The last two are cross-attention: every token of the chunk
# attends to the M tokens of a separate reference set (one 3600-token
# reference image at 720p; 720 tokens in the small case, whose head 3 has a
# loose reference key), through the same kernel.
CONFIGS = {
    "tiny": Config("tiny", F=5, T=48, H=2, d=64, dtype="f32", window=1,
                   ref_frame=0, shared_mean=False),
    "small": Config("small", F=9, T=880, H=16, d=128, dtype="bf16", window=2,
                    ref_frame=0, shared_mean=True),
    "720p": Config("720p", F=13, T=3600, H=24, d=128, dtype="bf16", window=2,
                   ref_frame=0, shared_mean=True),
    "1080p": Config("1080p", F=9, T=8160, H=24, d=128, dtype="bf16", window=1,
                    ref_frame=0, shared_mean=True),
    "stress": Config("stress", F=13, T=3600, H=40, d=128, dtype="bf16",
                     window=2, ref_frame=0, shared_mean=True, loose_period=50,
                     loose_phase=7),
    "720p-dense": Config("720p-dense", F=13, T=3600, H=24, d=128, dtype="bf16",
                         window=12, ref_frame=0, shared_mean=True),
    "outlier-frame": Config("outlier-frame", F=13, T=3600, H=8, d=128, dtype="bf16",
                            window=2, ref_frame=0, shared_mean=True, loose_period=4,
                            loose_phase=1, loose_frames=(6,)),
    "720p-xref": Config("720p-xref", F=13, T=3600, H=24, d=128, dtype="bf16", window=0,
                        ref_frame=0, shared_mean=True, M=3600),
    "xref-small": Config("xref-small", F=4, T=880, H=4, d=128, dtype="bf16", window=0,
                         ref_frame=0, shared_mean=True, M=720, loose_period=4,
                         loose_phase=3),
    # Looser heads: keys spread twice as wide (every head's largest row bound
    # is above the per-head threshold, so the per-head and per-frame checks
    # send everything online) and, in every frame, a band of 256 query rows
    # with 2.5x the norm. Only the rows of that band have a gap bound too
    # loose for the fixed max: the case for the per-row-block check.
    "loose-rows": Config("loose-rows", F=13, T=3600, H=24, d=128, dtype="bf16", window=2,
                         ref_frame=0, shared_mean=True, key_sigma=2.0, hot_rows=256,
                         hot_scale=2.5),
    "loose-rows-small": Config("loose-rows-small", F=5, T=880, H=4, d=128, dtype="bf16",
                               window=2, ref_frame=0, shared_mean=True, key_sigma=2.0,
                               hot_rows=160, hot_scale=2.5),
    # Producer workloads: the tokens of a chunk (C = H*d channels) go through
    # RMSNorm, the Q/K/V projection, 3-D rotary embedding and head packing
    # into the attention's layout. The 720p one is the SR transformer layer
    # that feeds the 720p attention (45x80 patches per frame, 24 heads of 128).
    "prep-small": Config("prep-small", F=4, T=880, H=4, d=128, dtype="bf16", window=2,
                         ref_frame=0, shared_mean=True, grid=(22, 40)),
    "720p-prep": Config("720p-prep", F=13, T=3600, H=24, d=128, dtype="bf16", window=2,
                        ref_frame=0, shared_mean=True, grid=(45, 80)),
}


def head_seed(seed: int, b: int, h: int) -> int:
    """Seed of the (b, h) stream: distinct for every seed < 2^20, b, h < 4096."""
    return (seed << 24) + (b << 12) + h


def make_head(cfg: Config, seed: int, b: int, h: int, device="cpu"):
    """Draw one head's (q, k, v), each [N, d] in the config dtype."""
    g = torch.Generator(device=device)
    g.manual_seed(head_seed(seed, b, h))
    N, d = cfg.N, cfg.d
    kw = dict(generator=g, device=device, dtype=torch.float32)
    q = torch.randn((N, d), **kw)
    k = torch.randn((N, d), **kw)
    if cfg.key_sigma != 1.0:
        k *= cfg.key_sigma
    if cfg.shared_mean:
        k += 4.0 * torch.randn((1, d), **kw)
    v = torch.randn((N, d), **kw)
    if cfg.is_loose(h):
        p = torch.randint(0, cfg.T, (cfg.F,), generator=g, device=device)
        rows = torch.arange(cfg.F, device=device) * cfg.T + p
        if cfg.loose_frames:
            rows = rows[list(cfg.loose_frames)]
        k[rows] *= 20.0
    if cfg.hot_rows:
        u = torch.randint(0, cfg.T - cfg.hot_rows + 1, (cfg.F,), generator=g, device=device)
        rows = (torch.arange(cfg.F, device=device) * cfg.T + u)[:, None] \
            + torch.arange(cfg.hot_rows, device=device)[None, :]
        q[rows.reshape(-1)] *= cfg.hot_scale
    dt = cfg.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt)


def make_cross_head(cfg: Config, seed: int, b: int, h: int, device="cpu"):
    """Draw one head's (q, kr, vr) of a cross-attention workload: q [N, d] for
    the chunk's tokens, kr and vr [M, d] for the reference tokens. Draw order:
    q = N(0,1); e = N(0,1) [M, d]; c = 4 N(0,1) [1, d] (shared-mean configs);
    vr = N(0,1) [M, d]; a loose head then multiplies the reference key at a
    seeded position p = randint(0, M) by 20. kr = e + c."""
    g = torch.Generator(device=device)
    g.manual_seed(head_seed(seed, b, h))
    N, M, d = cfg.N, cfg.M, cfg.d
    kw = dict(generator=g, device=device, dtype=torch.float32)
    q = torch.randn((N, d), **kw)
    k = torch.randn((M, d), **kw)
    if cfg.shared_mean:
        k += 4.0 * torch.randn((1, d), **kw)
    v = torch.randn((M, d), **kw)
    if cfg.is_loose(h):
        p = int(torch.randint(0, M, (1,), generator=g, device=device))
        k[p] *= 20.0
    dt = cfg.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt)


def make_inputs(cfg: Config, seed: int = 0, device="cpu"):
    """Draw Q, K, V (contiguous, the config dtype): Q [B, H, N, d]; K and V
    [B, H, N, d], or [B, H, M, d] for a cross-attention workload (M > 0)."""
    shape = (cfg.B, cfg.H, cfg.N, cfg.d)
    Q = torch.empty(shape, dtype=cfg.torch_dtype, device=device)
    kshape = (cfg.B, cfg.H, cfg.M, cfg.d) if cfg.M else shape
    K = torch.empty(kshape, dtype=cfg.torch_dtype, device=device)
    V = torch.empty_like(K)
    draw = make_cross_head if cfg.M else make_head
    for b in range(cfg.B):
        for h in range(cfg.H):
            q, k, v = draw(cfg, seed, b, h, device)
            Q[b, h], K[b, h], V[b, h] = q, k, v
    return Q, K, V


def make_prep_inputs(cfg: Config, seed: int = 0, device="cpu"):
    """Draw the producer's inputs for a workload with a grid: tokens X
    [B, N, C] (bf16), the joint projection W [3C, C] (bf16, (out, in)
    convention) and the RMSNorm weight gamma [C] (float32), C = H*d.

    Draw order from one generator seeded with head_seed(seed, 4095, 4095):
    gamma = 1 + 0.1 N(0,1); W = N(0,1) / sqrt(C); then per batch b:
    z = N(0,1) [N, C] and a shared offset c = N(0,1) [1, C] (shared-mean
    workloads), x = z + c. The shared offset gives the keys the common
    component that centring removes."""
    C = cfg.H * cfg.d
    g = torch.Generator(device=device)
    g.manual_seed(head_seed(seed, 4095, 4095))
    kw = dict(generator=g, device=device, dtype=torch.float32)
    gamma = 1.0 + 0.1 * torch.randn((C,), **kw)
    W = (torch.randn((3 * C, C), **kw) / math.sqrt(C)).to(torch.bfloat16)
    X = torch.empty((cfg.B, cfg.N, C), dtype=torch.bfloat16, device=device)
    for b in range(cfg.B):
        x = torch.randn((cfg.N, C), **kw)
        if cfg.shared_mean:
            x += torch.randn((1, C), **kw)
        X[b] = x.to(torch.bfloat16)
    return X, W, gamma


def to_f64(t: torch.Tensor):
    """Exact upcast of drawn values to a float64 numpy array on the host."""
    return t.detach().to("cpu", torch.float64).numpy()
