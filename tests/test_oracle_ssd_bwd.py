"""Pins for the oracle's backward of the MA branch (ssd_scan_backward,
ssd_bidir_backward): every gradient against central finite differences of
the pinned forward scan, per input tensor, with one and two B/C groups and
every scan order; independence from the checkpoint spacing; the closed-form
skip gradient."""
import numpy as np
import pytest

import oracle


def _inputs(rng, L, Hs, P, N, G):
    x = rng.standard_normal((L, Hs, P))
    dt = rng.uniform(0.05, 0.6, (L, Hs))
    A = -rng.uniform(0.3, 2.0, Hs)
    shape_bc = (L, N) if G == 1 else (L, G, N)
    B = rng.standard_normal(shape_bc)
    C = rng.standard_normal(shape_bc)
    D = rng.standard_normal(Hs)
    dy = rng.standard_normal((L, Hs, P))
    return [x, dt, A, B, C, D], dy


def _loss(params, dy, perm):
    return float(np.sum(dy * oracle.ssd_bidir(*params, perm)))


@pytest.mark.parametrize("G,mode", [(1, 0), (2, 3), (1, 2)])
def test_bidir_backward_matches_finite_differences(G, mode):
    rng = np.random.default_rng(50 + G + mode)
    T, H, W, Hs, P, N = 2, 2, 3, 2, 3, 2
    params, dy = _inputs(rng, T * H * W, Hs, P, N, G)
    perm = oracle.rms_scan_order(mode, T, H, W)
    grads = oracle.ssd_bidir_backward(*params, dy, perm)
    names = ("x", "dt", "A", "B", "C", "D")
    eps = 1e-6
    for i, name in enumerate(names):
        assert grads[i].shape == np.shape(params[i]), name
        v = rng.standard_normal(np.shape(params[i]))
        plus = [p.copy() for p in params]
        minus = [p.copy() for p in params]
        plus[i] = plus[i] + eps * v
        minus[i] = minus[i] - eps * v
        fd = (_loss(plus, dy, perm) - _loss(minus, dy, perm)) / (2 * eps)
        an = float(np.sum(grads[i] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)


def test_single_direction_backward_matches_finite_differences():
    rng = np.random.default_rng(57)
    L, Hs, P, N = 9, 3, 2, 4
    params, dy = _inputs(rng, L, Hs, P, N, 3)
    order = rng.permutation(L)
    grads = oracle.ssd_scan_backward(*params, dy, order, segment=4)
    eps = 1e-6
    for i in range(6):
        v = rng.standard_normal(np.shape(params[i]))
        plus = [p.copy() for p in params]
        minus = [p.copy() for p in params]
        plus[i] = plus[i] + eps * v
        minus[i] = minus[i] - eps * v
        lp = np.sum(dy * oracle.ssd_scan(*plus, order)[0])
        lm = np.sum(dy * oracle.ssd_scan(*minus, order)[0])
        fd = (lp - lm) / (2 * eps)
        assert abs(fd - float(np.sum(grads[i] * v))) <= 1e-6 * max(1.0, abs(fd)), i


def test_checkpoint_spacing_does_not_matter_and_skip_gradient():
    rng = np.random.default_rng(58)
    L, Hs, P, N = 13, 2, 3, 2
    params, dy = _inputs(rng, L, Hs, P, N, 1)
    order = rng.permutation(L)
    a = oracle.ssd_scan_backward(*params, dy, order, segment=64)
    b = oracle.ssd_scan_backward(*params, dy, order, segment=3)
    for u, v in zip(a, b):
        np.testing.assert_allclose(u, v, rtol=1e-12, atol=1e-12)
    # y carries D x once per direction: dD = 2 sum dy . x for the bidirectional scan
    full = oracle.ssd_bidir_backward(*params, dy, order)
    np.testing.assert_allclose(full[5], 2 * np.sum(dy * params[0], axis=(0, 2)), rtol=1e-12)
