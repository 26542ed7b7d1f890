"""Pins for the oracle's bidirectional selective-SSM scan (MA branch).

Each check uses a computation that is independent of the oracle's sequential
recurrence: explicit full matrices built from the closed-form solution of the
recurrence, cumulative sums, or exact special cases.
"""
import math

import numpy as np
import pytest

import oracle


def _rand_case(rng, T, H, W, Hs, P, N, dt_scale=1.0):
    L = T * H * W
    x = rng.standard_normal((L, Hs, P))
    dt = np.log1p(np.exp(rng.standard_normal((L, Hs)) - 1.0)) * dt_scale
    A = -np.exp(rng.uniform(0.0, math.log(4.0), Hs))
    B = rng.standard_normal((L, N)) / math.sqrt(N)
    C = rng.standard_normal((L, N)) / math.sqrt(N)
    D = rng.standard_normal(Hs)
    return x, dt, A, B, C, D


def _brute_bidir(x, dt, A, B, C, D, perm, h0=None):
    """y[c] from explicit sums over all (t, s) pairs of scan positions.

    Forward:  y_f(t) = sum_{s<=t} exp(sum_{tau=s+1..t} a_tau) dt_s (C_t.B_s) x_s
    Backward: y_b(t) = sum_{s>=t} exp(sum_{tau=t..s-1} a_tau) dt_s (C_t.B_s) x_s
    with a_tau = dt_tau * A; plus D x_t per direction, plus the initial state
    decayed by every a up to and including t (forward) or from t (backward).
    """
    L, Hs, P = x.shape
    y = np.zeros_like(x)
    for hd in range(Hs):
        a = np.array([dt[perm[s], hd] * A[hd] for s in range(L)])
        for t in range(L):
            ct = perm[t]
            acc = np.zeros(P)
            for s in range(L):
                cs = perm[s]
                cb = float(C[ct] @ B[cs])
                if s <= t:
                    acc += math.exp(a[s + 1:t + 1].sum()) * dt[cs, hd] * cb * x[cs, hd]
                if s >= t:
                    acc += math.exp(a[t:s].sum()) * dt[cs, hd] * cb * x[cs, hd]
            acc += 2.0 * D[hd] * x[ct, hd]
            if h0 is not None:
                acc += math.exp(a[0:t + 1].sum()) * (h0[hd] @ C[ct])
                acc += math.exp(a[t:L].sum()) * (h0[hd] @ C[ct])
            y[ct, hd] = acc
    return y


def _rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("with_h0", [False, True])
def test_bidir_matches_bruteforce_matrix(mode, with_h0):
    rng = np.random.default_rng(100 + mode)
    T, H, W, Hs, P, N = 2, 3, 4, 2, 3, 5
    x, dt, A, B, C, D = _rand_case(rng, T, H, W, Hs, P, N)
    perm = oracle.rms_scan_order(mode, T, H, W)
    h0 = rng.standard_normal((Hs, P, N)) if with_h0 else None
    got = oracle.ssd_bidir(x, dt, A, B, C, D, perm, h0=h0)
    want = _brute_bidir(x, dt, A, B, C, D, perm, h0=h0)
    assert _rel(got, want) < 1e-12


def test_single_direction_and_recorded_states():
    # Forward direction alone and its states at chunk boundaries, against the
    # explicit sums h(k) = sum_{s<k} exp(sum_{tau=s+1..k-1} a_tau) dt_s x_s B_s^T.
    rng = np.random.default_rng(7)
    T, H, W, Hs, P, N = 2, 2, 4, 2, 3, 4
    x, dt, A, B, C, D = _rand_case(rng, T, H, W, Hs, P, N)
    perm = oracle.rms_scan_order(2, T, H, W)
    L = T * H * W
    h0 = rng.standard_normal((Hs, P, N))
    ks = [0, 4, 8, 12, 16]
    y, hL, rec = oracle.ssd_scan(x, dt, A, B, C, D, perm, h0=h0, record_after=ks)
    for hd in range(Hs):
        a = np.array([dt[perm[s], hd] * A[hd] for s in range(L)])
        for k in ks:
            want = math.exp(a[:k].sum()) * h0[hd]
            for s in range(k):
                cs = perm[s]
                want = want + math.exp(a[s + 1:k].sum()) * dt[cs, hd] * np.outer(x[cs, hd], B[cs])
            np.testing.assert_allclose(rec[k][hd], want, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(hL[hd], rec[16][hd], rtol=0, atol=0)
        # outputs: y_t = h(t+1) C_t + D x_t
        for t in range(L):
            ct = perm[t]
            want = math.exp(a[:t + 1].sum()) * (h0[hd] @ C[ct]) + D[hd] * x[ct, hd]
            for s in range(t + 1):
                cs = perm[s]
                want = want + math.exp(a[s + 1:t + 1].sum()) * dt[cs, hd] * float(C[ct] @ B[cs]) * x[cs, hd]
            np.testing.assert_allclose(y[ct, hd], want, rtol=1e-12, atol=1e-13)


def test_cumulative_sum_case_scalar():
    # A = 0, dt = 1, N = 1, B = C = 1, D = 0: the forward scan is a running
    # sum and the bidirectional result is (sum of all x) + x_t.
    rng = np.random.default_rng(3)
    L, Hs, P = 24, 3, 2
    x = rng.standard_normal((L, Hs, P))
    dt = np.ones((L, Hs))
    A = np.zeros(Hs)
    B = np.ones((L, 1))
    C = np.ones((L, 1))
    D = np.zeros(Hs)
    perm = np.arange(L)
    y_f, _, _ = oracle.ssd_scan(x, dt, A, B, C, D, perm)
    np.testing.assert_allclose(y_f, np.cumsum(x, axis=0), rtol=1e-13, atol=1e-13)
    y = oracle.ssd_bidir(x, dt, A, B, C, D, perm)
    np.testing.assert_allclose(y, x.sum(axis=0, keepdims=True) + x, rtol=1e-13, atol=1e-13)


def test_cumulative_sum_case_general_N():
    # A = 0, dt = 1: y_f(t) = C_t . (cumulative sum over s <= t of x_s B_s^T) + D x_t
    rng = np.random.default_rng(4)
    L, Hs, P, N = 20, 2, 3, 4
    x = rng.standard_normal((L, Hs, P))
    B = rng.standard_normal((L, N))
    C = rng.standard_normal((L, N))
    D = rng.standard_normal(Hs)
    perm = oracle.rms_scan_order(1, 2, 2, 5)
    outer = x[perm][:, :, :, None] * B[perm][:, None, None, :]        # [L,Hs,P,N] in scan order
    cs = np.cumsum(outer, axis=0)
    want_scan = np.einsum("shpn,sn->shp", cs, C[perm]) + D[None, :, None] * x[perm]
    y_f, _, _ = oracle.ssd_scan(x, np.ones((L, Hs)), np.zeros(Hs), B, C, D, perm)
    np.testing.assert_allclose(y_f[perm], want_scan, rtol=1e-12, atol=1e-12)


def test_reversal_symmetry():
    # Scanning the reversed order swaps the two directions, so the
    # bidirectional result is unchanged.
    rng = np.random.default_rng(5)
    x, dt, A, B, C, D = _rand_case(rng, 3, 3, 3, 2, 4, 3)
    perm = oracle.rms_scan_order(3, 3, 3, 3)
    y1 = oracle.ssd_bidir(x, dt, A, B, C, D, perm)
    y2 = oracle.ssd_bidir(x, dt, A, B, C, D, perm[::-1])
    np.testing.assert_allclose(y1, y2, rtol=1e-12, atol=1e-13)


def test_zero_B_leaves_only_skip():
    rng = np.random.default_rng(6)
    x, dt, A, B, C, D = _rand_case(rng, 2, 2, 2, 3, 4, 3)
    y = oracle.ssd_bidir(x, dt, A, np.zeros_like(B), C, D, np.arange(8))
    np.testing.assert_allclose(y, 2.0 * D[None, :, None] * x, rtol=1e-15, atol=0)


def test_infinite_decay_keeps_only_self_term():
    # exp(dt*A) = 0 for every token: each direction sees only its own token,
    # y_t = 2 (dt_t C_t.B_t + D) x_t.
    rng = np.random.default_rng(8)
    x, dt, A, B, C, D = _rand_case(rng, 2, 2, 3, 2, 3, 4)
    A = np.full_like(A, -1e30)
    y = oracle.ssd_bidir(x, dt, A, B, C, D, oracle.rms_scan_order(1, 2, 2, 3))
    cb = np.einsum("ln,ln->l", C, B)
    want = 2.0 * (dt * cb[:, None] + D[None, :])[:, :, None] * x
    np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-14)


def test_linear_in_x():
    rng = np.random.default_rng(9)
    x1, dt, A, B, C, D = _rand_case(rng, 2, 2, 4, 2, 3, 3)
    x2 = rng.standard_normal(x1.shape)
    perm = oracle.rms_scan_order(2, 2, 2, 4)
    f = lambda xx: oracle.ssd_bidir(xx, dt, A, B, C, D, perm)
    np.testing.assert_allclose(f(1.5 * x1 - 0.25 * x2), 1.5 * f(x1) - 0.25 * f(x2), rtol=1e-11, atol=1e-12)


def test_heads_are_independent():
    # A head subset gives the same values as the full run (used by the
    # full-size parity checks, which run the oracle head by head).
    rng = np.random.default_rng(10)
    x, dt, A, B, C, D = _rand_case(rng, 2, 2, 2, 4, 3, 3)
    perm = np.arange(8)
    full = oracle.ssd_bidir(x, dt, A, B, C, D, perm)
    sub = oracle.ssd_bidir(x[:, [1, 3]], dt[:, [1, 3]], A[[1, 3]], B, C, D[[1, 3]], perm)
    np.testing.assert_allclose(sub, full[:, [1, 3]], rtol=0, atol=0)


def test_grouped_bc_reduce_to_shared_and_split_by_group():
    # G groups of B and C: head h reads group h // (Hs // G).  Identical groups
    # give the shared (one-group) scan; and each group's heads alone, scanned
    # with that group's B and C shared, give the same outputs.
    rng = np.random.default_rng(40)
    L, Hs, P, N, G = 24, 4, 3, 5, 2
    x = rng.standard_normal((L, Hs, P))
    dt = rng.uniform(0.05, 0.5, (L, Hs))
    A = -rng.uniform(0.5, 2.0, Hs)
    D = rng.standard_normal(Hs)
    B1, C1 = rng.standard_normal((L, N)), rng.standard_normal((L, N))
    perm = rng.permutation(L)
    same = oracle.ssd_bidir(x, dt, A, np.stack([B1] * G, 1), np.stack([C1] * G, 1), D, perm)
    np.testing.assert_allclose(same, oracle.ssd_bidir(x, dt, A, B1, C1, D, perm), rtol=1e-13, atol=1e-13)
    Bg, Cg = rng.standard_normal((L, G, N)), rng.standard_normal((L, G, N))
    got = oracle.ssd_bidir(x, dt, A, Bg, Cg, D, perm)
    hpg = Hs // G
    for g in range(G):
        hs = slice(g * hpg, (g + 1) * hpg)
        want = oracle.ssd_bidir(x[:, hs], dt[:, hs], A[hs], Bg[:, g], Cg[:, g], D[hs], perm)
        np.testing.assert_allclose(got[:, hs], want, rtol=1e-13, atol=1e-13)
    with pytest.raises(ValueError):
        oracle.ssd_bidir(x, dt, A, rng.standard_normal((L, 3, N)), rng.standard_normal((L, 3, N)), D, perm)


def test_grouped_review_state_splits_by_group():
    rng = np.random.default_rng(41)
    T, H, W, Hs, P, N, G = 4, 4, 4, 4, 2, 3, 2
    L = T * H * W
    x = rng.standard_normal((L, Hs, P))
    dt = rng.uniform(0.05, 0.5, (L, Hs))
    A = -rng.uniform(0.5, 2.0, Hs)
    Bg, Cg = rng.standard_normal((L, G, N)), rng.standard_normal((L, G, N))
    got = oracle.review_state(x, dt, A, Bg, Cg, T, H, W, (2, 2, 2), (2, 2, 2))
    for g in range(G):
        hs = slice(g * 2, g * 2 + 2)
        want = oracle.review_state(x[:, hs], dt[:, hs], A[hs], Bg[:, g], Cg[:, g], T, H, W, (2, 2, 2), (2, 2, 2))
        np.testing.assert_allclose(got[hs], want, rtol=1e-13, atol=1e-13)


def _brute_dirs(fwd, bwd, perm):
    """Explicit sums with a parameter set per direction: the lower triangle
    (s <= t) from the forward set, the upper (s >= t) from the backward set,
    and D x per direction."""
    xf, dtf, Af, Bf, Cf, Df = fwd
    xb, dtb, Ab, Bb, Cb, Db = bwd
    L, Hs, P = xf.shape
    y = np.zeros_like(xf)
    for hd in range(Hs):
        af = np.array([dtf[perm[s], hd] * Af[hd] for s in range(L)])
        ab = np.array([dtb[perm[s], hd] * Ab[hd] for s in range(L)])
        for t in range(L):
            ct = perm[t]
            acc = Df[hd] * xf[ct, hd] + Db[hd] * xb[ct, hd]
            for s in range(L):
                cs = perm[s]
                if s <= t:
                    acc = acc + math.exp(af[s + 1:t + 1].sum()) * dtf[cs, hd] * float(Cf[ct] @ Bf[cs]) * xf[cs, hd]
                if s >= t:
                    acc = acc + math.exp(ab[t:s].sum()) * dtb[cs, hd] * float(Cb[ct] @ Bb[cs]) * xb[cs, hd]
            y[ct, hd] = acc
    return y


@pytest.mark.parametrize("mode", [0, 3])
def test_direction_specific_parameters_match_bruteforce(mode):
    rng = np.random.default_rng(60 + mode)
    T, H, W = 2, 2, 3
    fwd = _rand_case(rng, T, H, W, 2, 3, 4)
    bwd = _rand_case(rng, T, H, W, 2, 3, 4)
    perm = oracle.rms_scan_order(mode, T, H, W)
    got = oracle.ssd_dirs(fwd, bwd, perm)
    assert _rel(got, _brute_dirs(fwd, bwd, perm)) < 1e-12
    # one set for both directions is the shared-weight scan
    assert _rel(oracle.ssd_dirs(fwd, fwd, perm), oracle.ssd_bidir(*fwd, perm)) < 1e-13
