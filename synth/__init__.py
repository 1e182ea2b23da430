"""Seeded synthetic inputs for the CSA / HCA forward (shared by tests and bench).

This module holds only shapes, seeds and value distributions -- none of the
method's arithmetic.  Distributions follow the workload descriptions: KV streams
C^a, C^b, C, raw window KV and the indexer-key streams ~ N(0, 1); compression
logits Z ~ N(0, 1) per channel; queries ~ N(0, sigma = 1/sqrt(d)) with d the
per-head dim of that query; indexer head weights ~ U(0, 1); sink logits ~ N(0, 1).
Values are drawn in fp32 and then stored in the workload's dtype (bf16 rounding by
torch's cast).  No public dataset is used; these stand in for the pages' 1M-token
workloads.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


class Gen:
    """A torch generator on `device`, seeded once; draws happen in call order."""

    def __init__(self, seed: int, device="cuda"):
        self.device = torch.device(device)
        self.g = torch.Generator(device=self.device)
        self.g.manual_seed(seed)

    def normal(self, shape, std: float = 1.0, dtype=torch.float32):
        x = torch.randn(tuple(shape), generator=self.g, device=self.device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        return x.to(dtype)

    def uniform(self, shape, lo: float = 0.0, hi: float = 1.0, dtype=torch.float32):
        x = torch.rand(tuple(shape), generator=self.g, device=self.device, dtype=torch.float32)
        if (lo, hi) != (0.0, 1.0):
            x.mul_(hi - lo).add_(lo)
        return x.to(dtype)

    def integers(self, lo: int, hi: int, shape):
        return torch.randint(lo, hi, tuple(shape), generator=self.g, device=self.device, dtype=torch.int64)


def qstd(d: int) -> float:
    return 1.0 / math.sqrt(d)


@dataclass
class Config:
    """One workload: shapes, dtypes and the seed of its inputs."""
    idx: int
    name: str
    mode: str                 # "csa" or "hca"
    dtype: str                # "f32" or "bf16" (streams, queries, caches)
    B: int
    ctx: int                  # tokens of context per sequence
    Tq: int                   # query tokens per sequence (the last Tq positions, or ctx for decode)
    decode: bool              # queries at t = ctx (after the context) rather than inside it
    m: int
    D: int = 512
    R: int = 64
    rope_base: float = 10000.0
    HI: int = 64
    DI: int = 128
    k: int = 1024
    H: int = 128
    n_win: int = 128
    softmax_scale: float = 1.0
    kv_format: str = "same"   # "same" (dtype) or "fp8mix"
    ik_format: str = "same"   # "same" or "mxfp4"
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return 7000 + self.idx

    @property
    def N(self) -> int:
        return self.ctx // self.m


CONFIGS = {
    0: Config(0, "tiny CSA prefill fp32, T=1024, m=4, D=128, HI=4x32, k=64, H=8", "csa", "f32",
              B=1, ctx=1024, Tq=1024, decode=False, m=4, D=128, HI=4, DI=32, k=64, H=8),
    1: Config(1, "CSA decode bf16, B=16, 128K context, m=4, D=512, HI=64x128, k=1024, H=128", "csa", "bf16",
              B=16, ctx=131072, Tq=1, decode=True, m=4),
    2: Config(2, "CSA chunked prefill bf16, 1M context, last 2048 queries", "csa", "bf16",
              B=1, ctx=1 << 20, Tq=2048, decode=False, m=4),
    3: Config(3, "HCA bf16, m'=128, 1M context (decode B=32 / 2048-query prefill)", "hca", "bf16",
              B=32, ctx=1 << 20, Tq=1, decode=True, m=128),
    4: Config(4, "mixed-precision CSA decode, B=8, 1M context, FP8-mixed KV, MXFP4 indexer", "csa", "bf16",
              B=8, ctx=1 << 20, Tq=1, decode=True, m=4, kv_format="fp8mix", ik_format="mxfp4"),
}


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def query_positions(cfg: Config, B: int | None = None, device="cuda"):
    """Absolute positions of the query tokens, [B, Tq] int64."""
    B = cfg.B if B is None else B
    if cfg.decode:
        pos = torch.full((B, cfg.Tq), cfg.ctx, dtype=torch.int64)
    else:
        pos = torch.arange(cfg.ctx - cfg.Tq, cfg.ctx, dtype=torch.int64).expand(B, cfg.Tq).contiguous()
    return pos.to(device)


def window_span(cfg: Config):
    """(first position, rows) of the raw window buffer covering every query's window."""
    last = cfg.ctx if cfg.decode else cfg.ctx - 1
    first_q = cfg.ctx if cfg.decode else cfg.ctx - cfg.Tq
    first = max(0, first_q - cfg.n_win + 1)
    return first, last - first + 1
