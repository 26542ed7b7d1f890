"""Pins for the oracle's steps either side of the scan: the scan-order causal
convolution with SiLU, softplus, and the gated RMS norm (brute-force loops,
closed forms and special cases)."""
import math

import numpy as np
import pytest

import oracle


def _silu(v):
    return v / (1.0 + math.exp(-v))


def test_conv_brute_force_loops():
    rng = np.random.default_rng(31)
    L, Ch, K = 7, 3, 4
    u = rng.standard_normal((L, Ch))
    w = rng.standard_normal((Ch, K))
    b = rng.standard_normal(Ch)
    order = rng.permutation(L)
    got = oracle.scan_conv_silu(u, w, b, order)
    for s in range(L):
        for c in range(Ch):
            acc = b[c]
            for k in range(K):
                p = s - (K - 1) + k
                if p >= 0:
                    acc += w[c, k] * u[order[p], c]
            assert abs(got[order[s], c] - _silu(acc)) < 1e-13


def test_conv_special_kernels():
    rng = np.random.default_rng(32)
    L, Ch = 9, 2
    u = rng.standard_normal((L, Ch))
    ident = np.arange(L)
    w_now = np.zeros((Ch, 4))
    w_now[:, 3] = 1.0              # the current token only
    np.testing.assert_allclose(oracle.scan_conv_silu(u, w_now, np.zeros(Ch), ident), u / (1 + np.exp(-u)), rtol=1e-14)
    w_old = np.zeros((Ch, 4))
    w_old[:, 0] = 1.0              # the token three positions back
    got = oracle.scan_conv_silu(u, w_old, np.zeros(Ch), ident)
    np.testing.assert_allclose(got[3:], u[:-3] / (1 + np.exp(-u[:-3])), rtol=1e-14)
    np.testing.assert_array_equal(got[:3], 0.0)


def test_prep_splits_and_reverses():
    rng = np.random.default_rng(33)
    L, Hs, P, G, N = 10, 2, 3, 2, 2
    Ch = Hs * P + 2 * G * N
    xbc = rng.standard_normal((L, Ch))
    wf, wb = rng.standard_normal((Ch, 4)), rng.standard_normal((Ch, 4))
    bf, bb = rng.standard_normal(Ch), rng.standard_normal(Ch)
    dt_raw, dt_bias = rng.standard_normal((L, Hs)), rng.standard_normal(Hs)
    order = rng.permutation(L)
    xf, Bf, Cf, xb, Bb, Cb, dt = oracle.ma_prep(xbc, dt_raw, wf, bf, wb, bb, dt_bias, order, Hs, P, G, N)
    # backward direction: the taps are the tokens at scan positions s .. s+3
    for s in range(L):
        for c in range(Ch):
            acc = bb[c]
            for k in range(4):
                p = s + 3 - k
                if p < L:
                    acc += wb[c, k] * xbc[order[p], c]
            full = np.concatenate([xb[order[s]].ravel(), Bb[order[s]].ravel(), Cb[order[s]].ravel()])
            assert abs(full[c] - _silu(acc)) < 1e-13
    f = oracle.scan_conv_silu(xbc, wf, bf, order)
    np.testing.assert_array_equal(np.concatenate([xf.reshape(L, -1), Bf.reshape(L, -1), Cf.reshape(L, -1)], 1), f)
    np.testing.assert_allclose(dt, np.log1p(np.exp(dt_raw + dt_bias)), rtol=1e-14)


def test_softplus_values():
    np.testing.assert_allclose(oracle.softplus([0.0, 50.0, -50.0]), [math.log(2.0), 50.0, math.exp(-50.0)], rtol=1e-14)


def test_gated_rmsnorm_loops_and_invariants():
    rng = np.random.default_rng(34)
    rows, dim, group = 3, 8, 4
    y, z = rng.standard_normal((rows, dim)), rng.standard_normal((rows, dim))
    w = rng.standard_normal(dim)
    got = oracle.gated_rmsnorm(y, z, w, 1e-5, group)
    for r in range(rows):
        for g0 in range(0, dim, group):
            gv = [y[r, c] * _silu(z[r, c]) for c in range(g0, g0 + group)]
            rms = math.sqrt(sum(v * v for v in gv) / group + 1e-5)
            for i, c in enumerate(range(g0, g0 + group)):
                assert abs(got[r, c] - gv[i] / rms * w[c]) < 1e-13
    # without eps: scale invariance in y and unit RMS of out / w per group
    a = oracle.gated_rmsnorm(y, z, np.ones(dim), 0.0, group)
    np.testing.assert_allclose(oracle.gated_rmsnorm(3.5 * y, z, np.ones(dim), 0.0, group), a, rtol=1e-13)
    np.testing.assert_allclose(np.sqrt((a.reshape(rows, -1, group) ** 2).mean(-1)), 1.0, rtol=1e-13)
