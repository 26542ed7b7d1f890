"""Pins for the oracle's TEmporal Swin Attention and the linear-cost claim."""
import math
import os
import time

import numpy as np
import pytest
from scipy.special import softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _qkv(rng, L, Ha, d, scale=1.0):
    return (rng.standard_normal((L, Ha, d)) * scale,
            rng.standard_normal((L, Ha, d)) * scale,
            rng.standard_normal((L, Ha, d)))


def test_one_window_covering_everything_is_full_attention():
    rng = np.random.default_rng(1)
    T, H, W, Ha, d = 2, 3, 4, 2, 5
    L = T * H * W
    q, k, v = _qkv(rng, L, Ha, d)
    got = oracle.tesa(q, k, v, T, H, W, (T, H, W), (0, 0, 0))
    for h in range(Ha):
        p = softmax(q[:, h] @ k[:, h].T / math.sqrt(d), axis=1)
        np.testing.assert_allclose(got[:, h], p @ v[:, h], rtol=1e-12, atol=1e-13)


def test_unit_window_returns_v():
    rng = np.random.default_rng(2)
    q, k, v = _qkv(rng, 2 * 2 * 3, 3, 4)
    np.testing.assert_allclose(oracle.tesa(q, k, v, 2, 2, 3, (1, 1, 1), (0, 0, 0)), v, rtol=0, atol=1e-15)


def _load_segments():
    rows = []
    with open(os.path.join(GOLDEN, "tesa_partition_segments.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split(":")
            n, w, s = (int(t) for t in lhs.split())
            rows.append((n, w, s, [int(t) for t in rhs.split()]))
    return rows


@pytest.mark.parametrize("row", _load_segments())
def test_partition_segments_fixture(row):
    n, w, s, want = row
    # along the T axis (H = W = 1): keys of consecutive tokens
    keys = oracle.tesa_window_keys(n, 1, 1, (w, 1, 1), (s, 0, 0))[:, 0]
    lengths = [int(c) for c in np.unique(keys, return_counts=True)[1]]
    assert lengths == want
    # every key value must form one contiguous run
    assert np.all(np.diff(keys) >= 0)


def _segments(n, w, s):
    cuts = sorted(set([0, n] + [c for c in range(s, n, w)]))
    return [(cuts[i], cuts[i + 1]) for i in range(len(cuts) - 1)]


def test_zero_query_gives_window_mean():
    rng = np.random.default_rng(3)
    T, H, W, Ha, d = 4, 8, 8, 2, 3
    win, shift = (2, 4, 4), (1, 2, 2)
    q = np.zeros((T * H * W, Ha, d))
    k = rng.standard_normal(q.shape)
    v = rng.standard_normal(q.shape)
    got = oracle.tesa(q, k, v, T, H, W, win, shift)
    vv = v.reshape(T, H, W, Ha, d)
    for (t0, t1) in _segments(T, win[0], shift[0]):
        for (h0, h1) in _segments(H, win[1], shift[1]):
            for (w0, w1) in _segments(W, win[2], shift[2]):
                mean = vv[t0:t1, h0:h1, w0:w1].reshape(-1, Ha, d).mean(axis=0)
                g = got.reshape(T, H, W, Ha, d)[t0:t1, h0:h1, w0:w1].reshape(-1, Ha, d)
                np.testing.assert_allclose(g, np.broadcast_to(mean, g.shape), rtol=1e-12, atol=1e-13)


def _swin_roll_mask(q, k, v, T, H, W, win, shift):
    """Second, independent construction of shifted-window attention: roll the
    grid by -shift, cut it into whole windows, give every rolled position a
    region label per axis (0 for the part that was never wrapped, 1 and 2 for
    the two pieces at the end), attend only between equal labels, roll back."""
    L, Ha, d = q.shape
    st, sh, sw = shift
    wt, wh, ww = win
    g = lambda a: np.roll(a.reshape(T, H, W, Ha, d), (-st, -sh, -sw), axis=(0, 1, 2))
    qr, kr, vr = g(q), g(k), g(v)

    def labels(n, w, s):
        lab = np.zeros(n, dtype=int)
        if s:
            lab[n - w:n - s] = 1
            lab[n - s:] = 2
        return lab

    lt, lh, lw = labels(T, wt, st), labels(H, wh, sh), labels(W, ww, sw)
    out = np.zeros_like(qr)
    for a in range(0, T, wt):
        for b in range(0, H, wh):
            for c in range(0, W, ww):
                sl = (slice(a, a + wt), slice(b, b + wh), slice(c, c + ww))
                lab = (lt[sl[0]][:, None, None] * 9 + lh[sl[1]][None, :, None] * 3 + lw[sl[2]][None, None, :]).ravel()
                mask = lab[:, None] == lab[None, :]
                qq = qr[sl].reshape(-1, Ha, d)
                kk = kr[sl].reshape(-1, Ha, d)
                vv = vr[sl].reshape(-1, Ha, d)
                for h in range(Ha):
                    s_ = qq[:, h] @ kk[:, h].T / math.sqrt(d)
                    s_ = np.where(mask, s_, -np.inf)
                    p = softmax(s_, axis=1)
                    blk = (p @ vv[:, h]).reshape(wt, wh, ww, d)
                    out[sl + (h,)] = blk
    return np.roll(out, (st, sh, sw), axis=(0, 1, 2)).reshape(L, Ha, d)


@pytest.mark.parametrize("shifted", [False, True])
def test_swin_roll_and_mask_agrees(shifted):
    rng = np.random.default_rng(4)
    T, H, W, Ha, d = 4, 8, 8, 2, 4
    win = (2, 4, 4)
    shift = (1, 2, 2) if shifted else (0, 0, 0)
    q, k, v = _qkv(rng, T * H * W, Ha, d)
    got = oracle.tesa(q, k, v, T, H, W, win, shift)
    want = _swin_roll_mask(q, k, v, T, H, W, win, shift)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_tesa_for_queries_matches_full():
    rng = np.random.default_rng(5)
    T, H, W, Ha, d = 4, 8, 8, 2, 4
    q, k, v = _qkv(rng, T * H * W, Ha, d)
    full = oracle.tesa(q, k, v, T, H, W, (2, 4, 4), (1, 2, 2))
    idx = rng.choice(T * H * W, 40, replace=False)
    part = oracle.tesa_for_queries(q, k, v, T, H, W, (2, 4, 4), (1, 2, 2), idx)
    np.testing.assert_allclose(part, full[idx], rtol=1e-13, atol=1e-14)


def test_work_is_linear_in_T():
    # Attention pairs: fixed windows give L * n_w pairs per head when unshifted
    # and an affine function of T when shifted; the scan takes 2 L steps.
    Ha, d, H, W = 1, 2, 8, 8
    win = (2, 4, 4)
    res = {}
    for T in (4, 8, 16):
        L = T * H * W
        rng = np.random.default_rng(T)
        q, k, v = _qkv(rng, L, Ha, d)
        for shift in ((0, 0, 0), (1, 2, 2)):
            st = {}
            oracle.tesa(q, k, v, T, H, W, win, shift, stats=st)
            res[(T, shift)] = st["tesa_pairs"]
        st = {}
        x = rng.standard_normal((L, 1, 2))
        oracle.ssd_bidir(x, np.ones((L, 1)), -np.ones(1), np.ones((L, 1)), np.ones((L, 1)), np.zeros(1),
                         np.arange(L), stats=st)
        assert st["ssd_steps"] == 2 * L
    for T in (4, 8, 16):
        assert res[(T, (0, 0, 0))] == T * H * W * 32
    s = (1, 2, 2)
    assert res[(16, s)] - res[(8, s)] == 2 * (res[(8, s)] - res[(4, s)])


@pytest.mark.slow
def test_oracle_time_grows_linearly_in_T():
    # The oracle's own cost at T, 2T, 4T (tiny dims): about 2x per doubling.
    def run(T):
        H = W = 4
        L = T * H * W
        rng = np.random.default_rng(0)
        x = rng.standard_normal((L, 1, 4))
        q = rng.standard_normal((L, 1, 4))
        best = float("inf")
        for _ in range(7):   # best of several: a timing under a loaded host
            t0 = time.perf_counter()
            oracle.mate_fwd(x, np.full((L, 1), 0.1), -np.ones(1), rng.standard_normal((L, 4)),
                            rng.standard_normal((L, 4)), np.ones(1), q, q, q, 1, T, H, W, (2, 2, 2))
            best = min(best, time.perf_counter() - t0)
        return best

    run(16)   # warm the code paths before either measurement
    t1, t4 = run(16), run(64)
    assert 2.0 < t4 / t1 < 8.0, (t1, t4)


def _load_cyclic():
    rows = []
    with open(os.path.join(GOLDEN, "tesa_cyclic_windows.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split(":")
            n, w, s = (int(t) for t in lhs.split())
            rows.append((n, w, s, [int(t) for t in rhs.split()]))
    return rows


@pytest.mark.parametrize("row", _load_cyclic())
def test_cyclic_windows_fixture(row):
    n, w, s, want = row
    keys = oracle.tesa_window_keys(n, 1, 1, (w, 1, 1), (s, 0, 0), cyclic=True)[:, 0]
    assert keys.tolist() == want
    assert np.all(np.bincount(keys) == w)      # every cyclic window is whole


@pytest.mark.parametrize("win,shift", [((2, 4, 4), (1, 2, 2)), ((3, 3, 3), (1, 1, 1)), ((2, 4, 4), (1, 3, 1))])
def test_cyclic_equals_roll_then_plain_windows(win, shift):
    # Cyclic shifted windows = roll the grid back by the offset, attend in the
    # plain (unshifted) windows, roll the result forward again.
    rng = np.random.default_rng(6)
    T, H, W, Ha, d = 6 if win[0] == 3 else 4, 6 if win[1] == 3 else 8, 6 if win[2] == 3 else 8, 2, 4
    L = T * H * W
    q, k, v = _qkv(rng, L, Ha, d)
    roll = lambda a, sgn: np.roll(a.reshape(T, H, W, Ha, d), tuple(sgn * s for s in shift), axis=(0, 1, 2))
    plain = oracle.tesa(roll(q, -1).reshape(L, Ha, d), roll(k, -1).reshape(L, Ha, d), roll(v, -1).reshape(L, Ha, d),
                        T, H, W, win, (0, 0, 0))
    want = roll(plain, 1).reshape(L, Ha, d)
    got = oracle.tesa(q, k, v, T, H, W, win, shift, cyclic=True)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    assert np.allclose(oracle.tesa(q, k, v, T, H, W, win, (0, 0, 0), cyclic=True),
                       oracle.tesa(q, k, v, T, H, W, win, (0, 0, 0)), rtol=0, atol=0)


@pytest.mark.parametrize("win,shift", [((3, 3, 3), (1, 1, 1)), ((2, 4, 4), (1, 3, 1))])
def test_swin_roll_and_mask_agrees_odd_and_uneven(win, shift):
    rng = np.random.default_rng(7)
    T, H, W, Ha, d = (6, 6, 6, 2, 4) if win[0] == 3 else (4, 8, 8, 2, 4)
    q, k, v = _qkv(rng, T * H * W, Ha, d)
    got = oracle.tesa(q, k, v, T, H, W, win, shift)
    want = _swin_roll_mask(q, k, v, T, H, W, win, shift)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


# Pins of the softmax denominator the backward pass reuses (oracle.tesa_lse).
def test_lse_two_keys_closed_form():
    # d = 1, two tokens in one window, keys 0 and ln 3: sum exp = 1 + 3
    q = np.ones((2, 1, 1))
    k = np.array([0.0, math.log(3.0)]).reshape(2, 1, 1)
    got = oracle.tesa_lse(q, k, 1, 1, 2, (1, 1, 2), (0, 0, 0))
    np.testing.assert_allclose(got, np.full((2, 1), 2.0), rtol=0, atol=1e-15)


@pytest.mark.parametrize("shift", [(0, 0, 0), (1, 2, 1)])
def test_lse_zero_keys_counts_the_window(shift):
    # every score 0: lse = log2 of the size of the query's window, with the
    # window sizes counted by brute force over the grid (cut border windows)
    T, H, W, win = 3, 5, 4, (2, 4, 2)
    L, Ha = T * H * W, 2
    rng = np.random.default_rng(7)
    q = rng.standard_normal((L, Ha, 3))
    k = np.zeros((L, Ha, 3))
    got = oracle.tesa_lse(q, k, T, H, W, win, shift)
    coords = [(t, h, w) for t in range(T) for h in range(H) for w in range(W)]
    def cell(c):
        return tuple((c[a] - shift[a]) // win[a] for a in range(3))
    for i, c in enumerate(coords):
        n = sum(1 for c2 in coords if cell(c2) == cell(c))
        np.testing.assert_allclose(got[i], math.log2(n), rtol=0, atol=1e-12)


def test_lse_one_window_is_logsumexp():
    from scipy.special import logsumexp
    rng = np.random.default_rng(8)
    T, H, W, Ha, d = 2, 3, 4, 2, 5
    L = T * H * W
    q, k, _ = _qkv(rng, L, Ha, d, scale=2.0)
    got = oracle.tesa_lse(q, k, T, H, W, (T, H, W), (0, 0, 0))
    for h in range(Ha):
        ref = logsumexp(q[:, h] @ k[:, h].T / math.sqrt(d), axis=1) / math.log(2.0)
        np.testing.assert_allclose(got[:, h], ref, rtol=1e-13, atol=1e-13)


def test_lse_gives_the_tesa_weights():
    # 2^(s log2(e) - lse) are the softmax weights: with them, sum_j w_ij v_j
    # is the pinned tesa output, on a shifted (cut) partition
    rng = np.random.default_rng(9)
    T, H, W, Ha, d, win, shift = 4, 4, 4, 2, 8, (2, 2, 4), (1, 1, 2)
    L = T * H * W
    q, k, v = _qkv(rng, L, Ha, d)
    lse = oracle.tesa_lse(q, k, T, H, W, win, shift)
    ref = oracle.tesa(q, k, v, T, H, W, win, shift)
    keys = oracle.tesa_window_keys(T, H, W, win, shift)
    for i in range(0, L, 5):
        same = np.all(keys == keys[i], axis=1)
        for h in range(Ha):
            s = k[same, h] @ q[i, h] / math.sqrt(d)
            w = np.exp2(s * math.log2(math.e) - lse[i, h])
            assert abs(w.sum() - 1.0) < 1e-12
            np.testing.assert_allclose(w @ v[same, h], ref[i, h], rtol=1e-11, atol=1e-12)
