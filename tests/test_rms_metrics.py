"""The scan distance of grid neighbours under the four Rotary Major Scan
orders (host metric over the library's index maps): closed forms and brute
force over the oracle's scan orders."""
import itertools

import numpy as np
import pytest

import oracle
from linear_complexity_video_mate_amd.rms_metrics import adjacent_scan_distance, rms_adjacent_distance

GRIDS = [(2, 3, 4), (4, 8, 8), (32, 64, 64)]


def _strides(mode, T, H, W):
    # step in scan position when one coordinate grows by one: the fastest
    # axis of the order moves by 1, the next by its length, the last by both
    return {
        0: {"w": 1, "h": W, "t": H * W},
        1: {"h": 1, "w": H, "t": H * W},
        2: {"t": 1, "w": T, "h": T * W},
        3: {"t": 1, "h": T, "w": T * H},
    }[mode]


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("mode", range(4))
def test_axis_distance_is_the_axis_stride(mode, grid):
    T, H, W = grid
    got = adjacent_scan_distance(mode, T, H, W)
    st = _strides(mode, T, H, W)
    n = {"t": (T - 1) * H * W, "h": T * (H - 1) * W, "w": T * H * (W - 1)}
    for a in "thw":
        assert got[a] == st[a]
    assert got["all"] == pytest.approx(sum(n[a] * st[a] for a in "thw") / sum(n.values()), rel=1e-12)


@pytest.mark.parametrize("grid", GRIDS)
def test_four_orders_make_every_neighbour_adjacent_once(grid):
    r = rms_adjacent_distance(*grid)
    assert r["min_over_modes"] == 1.0
    assert r["mean_over_modes"] == pytest.approx(np.mean([r["per_mode"][m]["all"] for m in range(4)]))


def test_brute_force_over_oracle_orders():
    T, H, W = 2, 3, 4
    for mode in range(4):
        perm = oracle.rms_scan_order(mode, T, H, W)
        pos = {int(c): s for s, c in enumerate(perm)}
        dist = {"t": [], "h": [], "w": []}
        for t, h, w in itertools.product(range(T), range(H), range(W)):
            c = (t * H + h) * W + w
            if t + 1 < T:
                dist["t"].append(abs(pos[c + H * W] - pos[c]))
            if h + 1 < H:
                dist["h"].append(abs(pos[c + W] - pos[c]))
            if w + 1 < W:
                dist["w"].append(abs(pos[c + 1] - pos[c]))
        got = adjacent_scan_distance(mode, T, H, W)
        for a in "thw":
            assert got[a] == pytest.approx(np.mean(dist[a]), rel=0, abs=0)
        assert got["all"] == pytest.approx(np.mean(dist["t"] + dist["h"] + dist["w"]), rel=1e-15)
