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


# ---------------------------------------------------------------------------
# The whole block (projections around the mixer): wiring pins.
# ---------------------------------------------------------------------------

def _block_weights(rng, Dm, Hs, P, G, N, K):
    d = Hs * P
    ch = d + 2 * G * N
    w = {
        "w_z": rng.standard_normal((d, Dm)) / np.sqrt(Dm),
        "w_xbc": rng.standard_normal((ch, Dm)) / np.sqrt(Dm),
        "w_dt": rng.standard_normal((Hs, Dm)) / np.sqrt(Dm),
        "conv_w_f": rng.standard_normal((ch, K)), "conv_b_f": rng.standard_normal(ch),
        "conv_w_b": rng.standard_normal((ch, K)), "conv_b_b": rng.standard_normal(ch),
        "dt_bias": rng.standard_normal(Hs), "A_f": -rng.uniform(1, 4, Hs), "A_b": -rng.uniform(1, 4, Hs),
        "D_f": rng.standard_normal(Hs), "D_b": rng.standard_normal(Hs), "norm_w": 1 + 0.1 * rng.standard_normal(d),
        "w_out_ma": rng.standard_normal((Dm, d)) / np.sqrt(d),
        "w_q": rng.standard_normal((d, Dm)), "w_k": rng.standard_normal((d, Dm)),
        "w_v": rng.standard_normal((d, Dm)), "w_o": rng.standard_normal((Dm, d)) / np.sqrt(d),
    }
    return w


def test_block_te_branch_one_window_is_dense_attention():
    """With the MA output projection zeroed and one window over the whole
    grid, the block is textbook softmax attention of the projected q, k, v,
    projected by w_o (scipy's softmax, no oracle helper)."""
    from scipy.special import softmax

    rng = np.random.default_rng(41)
    T, H, W, Hs, P, G, N, Dm = 2, 2, 3, 2, 3, 1, 2, 5
    w = _block_weights(rng, Dm, Hs, P, G, N, 4)
    w["w_out_ma"] = np.zeros_like(w["w_out_ma"])
    u = rng.standard_normal((T * H * W, Dm))
    got = oracle.mate_block(u, w, 0, T, H, W, Hs, P, G, N, Hs, (T, H, W))
    q, k, v = ((u @ w[n].T).reshape(-1, Hs, P) for n in ("w_q", "w_k", "w_v"))
    o = np.empty_like(q)
    for h in range(Hs):
        a = softmax(q[:, h] @ k[:, h].T / np.sqrt(P), axis=1)
        o[:, h] = a @ v[:, h]
    np.testing.assert_allclose(got, o.reshape(len(u), -1) @ w["w_o"].T, rtol=1e-12, atol=1e-12)


def test_block_ma_branch_infinite_decay_closed_form():
    """With w_o zeroed, one-tap convolutions and a decay that empties the
    state at every token, each direction's scan output is (dt B.C + D) x at
    the token itself, so the MA branch has a closed form: written out here
    with numpy alone (logaddexp for softplus, x * sigmoid for SiLU), with
    different weights per direction, two B/C groups and two norm groups."""
    rng = np.random.default_rng(42)
    T, H, W, Hs, P, G, N, Dm = 2, 2, 2, 4, 2, 2, 3, 6
    d, L = Hs * P, T * H * W
    w = _block_weights(rng, Dm, Hs, P, G, N, 1)
    w["w_o"] = np.zeros_like(w["w_o"])
    w["A_f"] = np.full(Hs, -1e6)
    w["A_b"] = np.full(Hs, -1e6)
    w["dt_bias"] = np.full(Hs, 2.0)          # dt >= softplus(2 - |raw|), far above 1e6^-1
    u = rng.standard_normal((L, Dm)) * 0.5
    sig = lambda a: 1 / (1 + np.exp(-a))
    xbc = u @ w["w_xbc"].T
    z = u @ w["w_z"].T
    dt = np.logaddexp(0.0, u @ w["w_dt"].T + w["dt_bias"])
    y = np.zeros((L, Hs, P))
    for tag in ("f", "b"):
        c = xbc * w["conv_w_" + tag][:, 0] + w["conv_b_" + tag]
        c = c * sig(c)
        x = c[:, :d].reshape(L, Hs, P)
        Bm = c[:, d:d + G * N].reshape(L, G, N)
        Cm = c[:, d + G * N:].reshape(L, G, N)
        for h in range(Hs):
            g = h // (Hs // G)
            bc = np.sum(Bm[:, g] * Cm[:, g], axis=1)
            y[:, h] += (dt[:, h] * bc + w["D_" + tag][h])[:, None] * x[:, h]
    gte = y.reshape(L, d) * z * sig(z)
    grp = gte.reshape(L, G, d // G)
    yn = (grp / np.sqrt((grp ** 2).mean(axis=2, keepdims=True) + 1e-5)).reshape(L, d) * w["norm_w"]
    want = yn @ w["w_out_ma"].T
    for layer in (0, 1, 2, 3):       # every scan order: the decay leaves no neighbour term
        got = oracle.mate_block(u, w, layer, T, H, W, Hs, P, G, N, Hs, (2, 2, 2))
        np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-12)


def test_block_branches_add_and_layers_repeat():
    rng = np.random.default_rng(43)
    T, H, W, Hs, P, G, N, Dm = 2, 4, 4, 2, 4, 1, 4, 7
    w = _block_weights(rng, Dm, Hs, P, G, N, 4)
    u = rng.standard_normal((T * H * W, Dm))
    args = (T, H, W, Hs, P, G, N, Hs, (2, 2, 2))
    full = oracle.mate_block(u, w, 1, *args)
    ma = oracle.mate_block(u, dict(w, w_o=np.zeros_like(w["w_o"])), 1, *args)
    te = oracle.mate_block(u, dict(w, w_out_ma=np.zeros_like(w["w_out_ma"])), 1, *args)
    np.testing.assert_allclose(full, ma + te, rtol=1e-12, atol=1e-12)
    # scan orders repeat every 4 layers, window phases every 2
    np.testing.assert_allclose(oracle.mate_block(u, w, 5, *args), full, rtol=1e-12, atol=1e-12)
    assert np.abs(oracle.mate_block(u, w, 3, *args) - full).max() > 1e-3
