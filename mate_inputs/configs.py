"""Workload shapes for the MATE token mixer.

Five shapes are used throughout (tests, benchmark, smoke check):

  0  tiny fp32      4x8x8 grid (256 tokens), SSD 2 heads x P=32, N=16, chunk 16,
                    TESA 2 heads x 32, window 2x4x4
  1  bf16           16x32x32 (16,384 tokens), SSD 16x64, N=64, chunk 64,
                    TESA 16x64, window 4x8x8
  2  bf16 512p-like 32x64x64 (131,072 tokens), SSD 32x64, N=128, chunk 128,
                    TESA 32x64, window 4x8x8
  3  bf16 minute    128x64x64 (524,288 tokens), dims as 2 (4x the tokens of 2)
  4  bf16 768p-like 32x96x96 (294,912 tokens), dims as 2, plus 64 review tokens
                    (mean-pooled 2x12x12 blocks -> 16x8x8 grid -> 4x4x4 sample)

The pages give no latent shapes for their 512p / 768p, 17-68 s workloads
(QbitAI article, 评估 section; LinGen abstract).  Shapes 2, 3 and 4 stand in for
them: 2 for 512p at 17 s, 3 for four times the length, 4 for 768p (1.5x the
height and width of 2).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class MateShape:
    """Mirror of the C struct ``lingen_mate_shape`` (include/lingen_mate.h)."""

    batch: int
    T: int
    H: int
    W: int
    ssd_heads: int          # Hs
    headdim: int            # P
    d_state: int            # N
    ngroups: int            # G (1: B and C shared by all heads)
    chunk: int              # Q
    attn_heads: int         # Ha
    attn_headdim: int       # d
    win: Tuple[int, int, int]          # (wt, wh, ww)
    dtype: str                          # "f32" or "bf16": x, B, C, q, k, v, y
    n_review: int = 0                   # R = prod(rgrid) or 0
    rpool: Tuple[int, int, int] = (1, 1, 1)
    rgrid: Tuple[int, int, int] = (1, 1, 1)

    @property
    def L(self) -> int:
        return self.T * self.H * self.W

    @property
    def d_inner(self) -> int:
        return self.ssd_heads * self.headdim

    @property
    def n_w(self) -> int:
        return self.win[0] * self.win[1] * self.win[2]

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "MateShape":
        return replace(self, **kw)


_C2 = dict(ssd_heads=32, headdim=64, d_state=128, ngroups=1, chunk=128,
           attn_heads=32, attn_headdim=64, win=(4, 8, 8), dtype="bf16")

CONFIGS = (
    MateShape(batch=1, T=4, H=8, W=8, ssd_heads=2, headdim=32, d_state=16,
              ngroups=1, chunk=16, attn_heads=2, attn_headdim=32,
              win=(2, 4, 4), dtype="f32"),
    MateShape(batch=1, T=16, H=32, W=32, ssd_heads=16, headdim=64, d_state=64,
              ngroups=1, chunk=64, attn_heads=16, attn_headdim=64,
              win=(4, 8, 8), dtype="bf16"),
    MateShape(batch=1, T=32, H=64, W=64, **_C2),
    MateShape(batch=1, T=128, H=64, W=64, **_C2),
    MateShape(batch=1, T=32, H=96, W=96, n_review=64, rpool=(2, 12, 12),
              rgrid=(4, 4, 4), **_C2),
)

CONFIG_NOTES = (
    "tiny fp32 4x8x8",
    "bf16 16x32x32",
    "bf16 512p-like 32x64x64",
    "bf16 minute-length 128x64x64",
    "bf16 768p-like 32x96x96 + 64 review tokens",
)


def config_shape(i: int) -> MateShape:
    return CONFIGS[i]
