"""Pins for the oracle's Rotary Major Scan orders and layer schedule."""
import os

import numpy as np
import pytest

import oracle
from mate_inputs import CONFIGS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_rms_fixture():
    out = {}
    with open(os.path.join(GOLDEN, "rms_scan_orders_T2H2W3.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, vals = line.split(":")
            out[int(name.replace("mode", ""))] = np.array([int(v) for v in vals.split()])
    return out


def test_rms_hand_enumerated_fixture():
    fix = _load_rms_fixture()
    assert sorted(fix) == [0, 1, 2, 3]
    for mode, want in fix.items():
        got = oracle.rms_scan_order(mode, 2, 2, 3)
        np.testing.assert_array_equal(got, want, err_msg=f"mode {mode}")


def _closed_form(mode, T, H, W):
    """Mixed-radix position formulas, written independently of the oracle's
    reshape/transpose: scan position of token (t, h, w)."""
    pos = np.empty(T * H * W, dtype=np.int64)
    for t in range(T):
        for h in range(H):
            for w in range(W):
                c = (t * H + h) * W + w
                if mode == 0:
                    s = (t * H + h) * W + w
                elif mode == 1:
                    s = (t * W + w) * H + h
                elif mode == 2:
                    s = (h * W + w) * T + t
                else:
                    s = (w * H + h) * T + t
                pos[s] = c
    return pos


@pytest.mark.parametrize("dims", [(2, 3, 5), (4, 8, 8), (3, 1, 7), (1, 4, 1)])
@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_rms_closed_form(mode, dims):
    T, H, W = dims
    np.testing.assert_array_equal(oracle.rms_scan_order(mode, T, H, W), _closed_form(mode, T, H, W))


@pytest.mark.parametrize("cfg", range(len(CONFIGS)))
@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_rms_bijection_on_configs(mode, cfg):
    s = CONFIGS[cfg]
    perm = oracle.rms_scan_order(mode, s.T, s.H, s.W)
    inv = oracle.rms_inverse(perm)
    L = s.L
    ar = np.arange(L)
    np.testing.assert_array_equal(perm[inv], ar)
    np.testing.assert_array_equal(inv[perm], ar)
    np.testing.assert_array_equal(np.sort(perm), ar)


def test_rms_mode0_is_identity():
    np.testing.assert_array_equal(oracle.rms_scan_order(0, 5, 6, 7), np.arange(210))


def test_rms_neighbours_along_fastest_axis():
    # In each mode, consecutive scan positions inside a run differ by exactly
    # one step of the fastest axis (stride 1 for W, W for H, H*W for T).
    T, H, W = 3, 4, 5
    strides = {0: 1, 1: W, 2: H * W, 3: H * W}
    runs = {0: W, 1: H, 2: T, 3: T}
    for mode in range(4):
        p = oracle.rms_scan_order(mode, T, H, W)
        r = runs[mode]
        for s in range(T * H * W - 1):
            if (s + 1) % r:
                assert p[s + 1] - p[s] == strides[mode]


def test_layer_schedule():
    assert [oracle.rms_mode(i) for i in range(9)] == [0, 1, 2, 3, 0, 1, 2, 3, 0]
    assert oracle.tesa_shift(0, (4, 8, 8)) == (0, 0, 0)
    assert oracle.tesa_shift(1, (4, 8, 8)) == (2, 4, 4)
    assert oracle.tesa_shift(3, (2, 4, 4)) == (1, 2, 2)
    assert oracle.tesa_shift(2, (2, 4, 4)) == (0, 0, 0)
    with pytest.raises(ValueError):
        oracle.rms_mode(-1)
