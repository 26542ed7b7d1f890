"""Pins for the oracle's review tokens and the whole-mixer composition."""
import math

import numpy as np
import pytest

import oracle


def _case(rng, T, H, W, Hs, P, N):
    L = T * H * W
    x = rng.standard_normal((L, Hs, P))
    dt = np.log1p(np.exp(rng.standard_normal((L, Hs)) - 1.0))
    A = -np.exp(rng.uniform(0.0, math.log(4.0), Hs))
    B = rng.standard_normal((L, N)) / math.sqrt(N)
    C = rng.standard_normal((L, N)) / math.sqrt(N)
    D = rng.standard_normal(Hs)
    return x, dt, A, B, C, D


T, H, W = 8, 6, 6
RPOOL, RGRID = (2, 3, 3), (2, 2, 2)     # pooled grid 4x2x2, sampled at stride (2,1,1)


def _review_by_loops(a):
    """Block means at the sampled block positions, by explicit loops."""
    pt, ph, pw = RPOOL
    a = np.asarray(a).reshape((T, H, W) + a.shape[1:])
    out = []
    for i in range(RGRID[0]):
        for j in range(RGRID[1]):
            for k in range(RGRID[2]):
                bt, bh, bw = 2 * i, 1 * j, 1 * k            # sampled block (stride 2,1,1)
                blk = a[bt * pt:(bt + 1) * pt, bh * ph:(bh + 1) * ph, bw * pw:(bw + 1) * pw]
                out.append(blk.reshape((-1,) + a.shape[3:]).sum(axis=0) / (pt * ph * pw))
    return np.stack(out)


def test_review_tokens_are_sampled_block_means():
    rng = np.random.default_rng(1)
    x, dt, A, B, C, D = _case(rng, T, H, W, 2, 3, 4)
    xr, dtr, Br, Cr = oracle.review_tokens(x, dt, B, C, T, H, W, RPOOL, RGRID)
    for got, src in ((xr, x), (dtr, dt), (Br, B), (Cr, C)):
        np.testing.assert_allclose(got, _review_by_loops(src), rtol=1e-13, atol=1e-14)


def test_review_state_closed_form():
    # h_R = sum_r exp(sum_{tau=r+1..R-1} a_tau) dt_r x_r B_r^T over the review tokens.
    rng = np.random.default_rng(2)
    x, dt, A, B, C, D = _case(rng, T, H, W, 2, 3, 4)
    hR = oracle.review_state(x, dt, A, B, C, T, H, W, RPOOL, RGRID)
    xr, dtr, Br = _review_by_loops(x), _review_by_loops(dt), _review_by_loops(B)
    R = xr.shape[0]
    for hd in range(2):
        a = dtr[:, hd] * A[hd]
        want = sum(math.exp(a[r + 1:].sum()) * dtr[r, hd] * np.outer(xr[r, hd], Br[r]) for r in range(R))
        np.testing.assert_allclose(hR[hd], want, rtol=1e-12, atol=1e-14)


def test_review_equals_prepending_tokens():
    # Using h_R as the initial state equals scanning [review tokens, main
    # tokens] as one sequence, in each direction.
    rng = np.random.default_rng(3)
    x, dt, A, B, C, D = _case(rng, T, H, W, 2, 3, 4)
    mode = 3
    perm = oracle.rms_scan_order(mode, T, H, W)
    y = oracle.ma_fwd(x, dt, A, B, C, D, mode, T, H, W, review=(RPOOL, RGRID))
    xr, dtr, Br, Cr = oracle.review_tokens(x, dt, B, C, T, H, W, RPOOL, RGRID)
    R, L = xr.shape[0], T * H * W
    cat = lambda a, b: np.concatenate([a, b], axis=0)
    X, DT, BB, CC = cat(xr, x), cat(dtr, dt), cat(Br, B), cat(Cr, C)
    yf, _, _ = oracle.ssd_scan(X, DT, A, BB, CC, D, np.concatenate([np.arange(R), R + perm]))
    yb, _, _ = oracle.ssd_scan(X, DT, A, BB, CC, D, np.concatenate([np.arange(R), R + perm[::-1]]))
    np.testing.assert_allclose(y, (yf + yb)[R:], rtol=1e-12, atol=1e-13)


def test_zero_review_input_changes_nothing():
    rng = np.random.default_rng(4)
    x, dt, A, B, C, D = _case(rng, T, H, W, 2, 3, 4)
    # zero x inside the sampled blocks: the review state is then exactly zero
    xx = x.reshape(T, H, W, 2, 3).copy()
    for i in range(2):
        for j in range(2):
            for k in range(2):
                xx[2 * i * 2:(2 * i + 1) * 2, j * 3:(j + 1) * 3, k * 3:(k + 1) * 3] = 0.0
    xx = xx.reshape(-1, 2, 3)
    a = oracle.ma_fwd(xx, dt, A, B, C, D, 1, T, H, W, review=(RPOOL, RGRID))
    b = oracle.ma_fwd(xx, dt, A, B, C, D, 1, T, H, W, review=None)
    np.testing.assert_array_equal(a, b)


def test_mate_is_sum_of_branches():
    rng = np.random.default_rng(5)
    Tt, Hh, Ww, Hs, P, N = 4, 8, 8, 2, 4, 3
    x, dt, A, B, C, D = _case(rng, Tt, Hh, Ww, Hs, P, N)
    q, k, v = (rng.standard_normal((Tt * Hh * Ww, Hs, P)) for _ in range(3))
    for layer in range(4):
        y = oracle.mate_fwd(x, dt, A, B, C, D, q, k, v, layer, Tt, Hh, Ww, (2, 4, 4))
        ym = oracle.ma_fwd(x, dt, A, B, C, D, layer % 4, Tt, Hh, Ww)
        o = oracle.tesa(q, k, v, Tt, Hh, Ww, (2, 4, 4), (1, 2, 2) if layer % 2 else (0, 0, 0))
        np.testing.assert_allclose(y, ym.reshape(-1, Hs * P) + o.reshape(-1, Hs * P), rtol=0, atol=0)


def _prepend_scan(x, dt, A, B, C, D, order, R):
    """Scan [review tokens, main tokens] as one sequence (review tokens first,
    in canonical order, then the main tokens along ``order``) and return the
    main tokens' outputs: the review tokens written out as a prefix, with no
    initial state."""
    xr, dtr, Br, Cr = oracle.review_tokens(x, dt, B, C, T, H, W, RPOOL, RGRID)
    cat = lambda a, b: np.concatenate([a, b], axis=0)
    X, DT, BB, CC = cat(xr, x), cat(dtr, dt), cat(Br, B), cat(Cr, C)
    y, _, _ = oracle.ssd_scan(X, DT, A, BB, CC, D, np.concatenate([np.arange(R), R + np.asarray(order)]))
    return y[R:]


@pytest.mark.parametrize("mode", [0, 2])
def test_dirs_review_equals_prepending_own_tokens(mode):
    # Per-direction parameters: each direction prepends review tokens pooled
    # from its own inputs and scans them with its own A; two B/C groups.
    rng = np.random.default_rng(6 + mode)
    G = 2
    f = _case(rng, T, H, W, 4, 3, 5)
    b = _case(rng, T, H, W, 4, 3, 5)
    L = T * H * W
    fwd = (f[0], f[1], f[2], rng.standard_normal((L, G, 5)) / 2, rng.standard_normal((L, G, 5)) / 2, f[5])
    bwd = (b[0], b[1], b[2], rng.standard_normal((L, G, 5)) / 2, rng.standard_normal((L, G, 5)) / 2, b[5])
    perm = oracle.rms_scan_order(mode, T, H, W)
    R = int(np.prod(RGRID))
    y = oracle.ssd_dirs(fwd, bwd, perm, review=(RPOOL, RGRID), grid=(T, H, W))
    want = _prepend_scan(*fwd, perm, R) + _prepend_scan(*bwd, perm[::-1], R)
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-13)
    # and the review state does change the result
    assert np.abs(y - oracle.ssd_dirs(fwd, bwd, perm)).max() > 1e-3


def test_dirs_review_with_shared_sets_is_the_mixer_branch():
    # the same set in both directions reduces to the shared-parameter branch
    rng = np.random.default_rng(9)
    s = _case(rng, T, H, W, 2, 3, 4)
    perm = oracle.rms_scan_order(1, T, H, W)
    y = oracle.ssd_dirs(s, s, perm, review=(RPOOL, RGRID), grid=(T, H, W))
    np.testing.assert_allclose(y, oracle.ma_fwd(*s, 1, T, H, W, review=(RPOOL, RGRID)), rtol=1e-13, atol=1e-14)
