"""Scan distance of grid neighbours under the Rotary Major Scan (host only).

The pages credit the four alternating scan orders with bringing the average
distance, after the scan, of tokens that were adjacent in the video grid down
to the level of special scan patterns (page "视频生成模子太贵太慢如何办？",
section 要领; page "LinGen：基于Mamba机制的线性复杂度高清长视频生成框架", section
关键算法创新 > Rotary Major Scan).  They give neither the definition nor the
numbers.  Reading taken here: two tokens are adjacent when their (t, h, w)
differ by one along exactly one axis; their scan distance under an order is
|inv[a] - inv[b]|, inv being the scan position of each canonical token (the
library's lingen_rms_index).  Reported per order, per axis and over all
adjacent pairs, and for the four orders used in turn: the mean over orders,
and the mean over pairs of the smallest distance a pair gets in any of the
four consecutive layers.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .binding import lingen_rms_index

AXES = ("t", "h", "w")


def _pair_distances(inv: np.ndarray, T: int, H: int, W: int) -> Dict[str, np.ndarray]:
    g = inv.reshape(T, H, W).astype(np.int64)
    return {
        "t": np.abs(g[1:] - g[:-1]).ravel(),
        "h": np.abs(g[:, 1:] - g[:, :-1]).ravel(),
        "w": np.abs(g[:, :, 1:] - g[:, :, :-1]).ravel(),
    }


def adjacent_scan_distance(mode: int, T: int, H: int, W: int) -> Dict[str, float]:
    """Mean scan distance of adjacent tokens along each axis and over all
    adjacent pairs, for scan order ``mode``."""
    _, inv = lingen_rms_index(mode, T, H, W)
    d = _pair_distances(inv, T, H, W)
    out = {a: float(d[a].mean()) if d[a].size else float("nan") for a in AXES}
    allp = np.concatenate([d[a] for a in AXES])
    out["all"] = float(allp.mean()) if allp.size else float("nan")
    return out


def rms_adjacent_distance(T: int, H: int, W: int) -> Dict[str, object]:
    """The four orders one by one, their mean (the distance averaged over four
    consecutive layers), and the mean over adjacent pairs of the smallest
    distance any of the four layers gives the pair."""
    per_mode = {m: adjacent_scan_distance(m, T, H, W) for m in range(4)}
    best = None
    for m in range(4):
        _, inv = lingen_rms_index(m, T, H, W)
        d = _pair_distances(inv, T, H, W)
        allp = np.concatenate([d[a] for a in AXES])
        best = allp if best is None else np.minimum(best, allp)
    return {
        "per_mode": per_mode,
        "mean_over_modes": float(np.mean([per_mode[m]["all"] for m in range(4)])),
        "min_over_modes": float(best.mean()) if best is not None and best.size else float("nan"),
    }
