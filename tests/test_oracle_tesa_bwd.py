"""Pins for the oracle's TESA gradients: central finite differences of the
(separately pinned) forward, closed forms at zero queries, and the softmax
invariant that a window's key gradients sum to zero."""
import numpy as np
import pytest

import oracle


def _qkv(rng, L, Ha, d, scale=1.0):
    return (rng.standard_normal((L, Ha, d)) * scale, rng.standard_normal((L, Ha, d)) * scale,
            rng.standard_normal((L, Ha, d)))


CASES = [((2, 4, 4), (2, 4, 4), (0, 0, 0), False),     # one window
         ((4, 4, 4), (2, 2, 2), (1, 1, 1), False),     # cut border windows
         ((4, 4, 4), (2, 2, 2), (1, 1, 1), True),      # cyclic windows
         ((3, 3, 6), (3, 3, 3), (1, 1, 1), False)]     # odd window


@pytest.mark.parametrize("grid,win,shift,cyclic", CASES)
def test_gradients_match_finite_differences(grid, win, shift, cyclic):
    T, H, W = grid
    L, Ha, d = T * H * W, 2, 3
    rng = np.random.default_rng(sum(grid) + sum(shift) + 7 * cyclic)
    q, k, v = _qkv(rng, L, Ha, d)
    dO = rng.standard_normal((L, Ha, d))
    grads = oracle.tesa_backward(q, k, v, dO, T, H, W, win, shift, cyclic)
    loss = lambda a, b, c: float((oracle.tesa(a, b, c, T, H, W, win, shift, cyclic=cyclic) * dO).sum())
    eps = 1e-6
    for which in range(3):
        for _ in range(6):
            i, h, e = int(rng.integers(L)), int(rng.integers(Ha)), int(rng.integers(d))
            args_p = [x.copy() for x in (q, k, v)]
            args_m = [x.copy() for x in (q, k, v)]
            args_p[which][i, h, e] += eps
            args_m[which][i, h, e] -= eps
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(grads[which][i, h, e] - fd) <= 1e-7 * max(1.0, abs(fd)), (which, i, h, e)


def test_zero_queries_closed_form():
    # q = 0: uniform weights inside each window, so dv is the window mean of
    # dO, dk vanishes, and dq = s * (mean_j (dO.v_j) k_j - mean(dO.v) mean(k)).
    rng = np.random.default_rng(21)
    T, H, W, win = 2, 4, 4, (2, 4, 4)
    L, Ha, d = T * H * W, 2, 4
    _, k, v = _qkv(rng, L, Ha, d)
    q = np.zeros_like(k)
    dO = rng.standard_normal((L, Ha, d))
    dq, dk, dv = oracle.tesa_backward(q, k, v, dO, T, H, W, win, (0, 0, 0))
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv, np.broadcast_to(dO.mean(axis=0), dv.shape), rtol=1e-13, atol=1e-14)
    s = 1 / np.sqrt(d)
    for h in range(Ha):
        g = dO[:, h] @ v[:, h].T                              # dP[i, j]
        want = s * (g @ k[:, h] / L - g.mean(axis=1, keepdims=True) * k[:, h].mean(axis=0))
        np.testing.assert_allclose(dq[:, h], want, rtol=1e-12, atol=1e-13)


def test_key_gradients_sum_to_zero_per_window():
    rng = np.random.default_rng(22)
    T, H, W, win, shift = 4, 8, 8, (2, 4, 4), (1, 2, 2)
    L, Ha, d = T * H * W, 2, 4
    q, k, v = _qkv(rng, L, Ha, d)
    dO = rng.standard_normal((L, Ha, d))
    _, dk, _ = oracle.tesa_backward(q, k, v, dO, T, H, W, win, shift)
    keys = oracle.tesa_window_keys(T, H, W, win, shift)
    for key in np.unique(keys, axis=0):
        members = np.all(keys == key, axis=1)
        np.testing.assert_allclose(dk[members].sum(axis=0), 0.0, atol=1e-12)
