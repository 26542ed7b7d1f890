"""Pins for the oracle's backward of the MA branch (ssd_scan_backward,
ssd_bidir_backward, ma_bwd): every gradient against central finite
differences of the pinned forward scan, per input tensor, with one and two
B/C groups and every scan order, with and without review tokens;
independence from the checkpoint spacing; the closed-form skip gradient."""
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


def test_transposed_scan_identity_in_chunks():
    """The identity behind the GPU backward's dx: yhat = (dx - 2 D dy) / dt of
    the oracle equals the bidirectional scan with B and C exchanged, unit
    token weights and the prefix sums trading places (pairs i < o decay by
    e^{exc_o - exc_i}, pairs i > o by e^{cum_i - cum_o}, weight 2 on the
    diagonal), evaluated chunk by chunk: within a chunk densely, across
    chunks through states that carry the chunk-local weights e^{cum_end -
    exc_i} (forward) and e^{cum_i} (reverse), i.e. the states of dy e^{dt A}
    / dt against C, with the factors e^{exc_o} and e^{cum_end - cum_o} on the
    output side."""
    rng = np.random.default_rng(71)
    T, H, W, Hs, P, N, Q = 2, 2, 4, 2, 3, 2, 4
    L = T * H * W
    params, dy = _inputs(rng, L, Hs, P, N, 1)
    x, dt, A, B, C, D = params
    perm = oracle.rms_scan_order(1, T, H, W)
    dx = oracle.ssd_bidir_backward(*params, dy, perm)[0]
    yhat_oracle = (dx - 2.0 * D[None, :, None] * dy) / dt[:, :, None]
    nc = L // Q
    yhat = np.zeros_like(dy)
    for h in range(Hs):
        a = dt[perm, h] * A[h]                      # scan order
        Bs, Cs, us = B[perm], C[perm], dy[perm, h]  # [L, N], [L, N], [L, P]
        cum = np.zeros(L)
        exc = np.zeros(L)
        for c in range(nc):                         # chunk-local prefix sums
            blk = slice(c * Q, (c + 1) * Q)
            cum[blk] = np.cumsum(a[blk])
            exc[blk] = cum[blk] - a[blk]
        g = np.array([np.exp(cum[(c + 1) * Q - 1]) for c in range(nc)])
        # chunk states of u against C with the adjoint weights
        sf = np.zeros((nc, N, P))
        sb = np.zeros((nc, N, P))
        for c in range(nc):
            end = (c + 1) * Q - 1
            for i in range(c * Q, (c + 1) * Q):
                sf[c] += np.exp(cum[end] - exc[i]) * np.outer(Cs[i], us[i])
                sb[c] += np.exp(cum[i]) * np.outer(Cs[i], us[i])
        hf = np.zeros((nc, N, P))
        hb = np.zeros((nc, N, P))
        for c in range(1, nc):
            hf[c] = g[c - 1] * hf[c - 1] + sf[c - 1]
        for c in range(nc - 2, -1, -1):
            hb[c] = g[c + 1] * hb[c + 1] + sb[c + 1]
        out = np.zeros((L, P))
        for c in range(nc):
            end = (c + 1) * Q - 1
            for o in range(c * Q, (c + 1) * Q):
                acc = np.zeros(P)
                for i in range(c * Q, (c + 1) * Q):
                    lam = 2.0 if i == o else (np.exp(exc[o] - exc[i]) if i < o else np.exp(cum[i] - cum[o]))
                    acc += (Bs[o] @ Cs[i]) * lam * us[i]
                acc += np.exp(exc[o]) * (Bs[o] @ hf[c]) + np.exp(cum[end] - cum[o]) * (Bs[o] @ hb[c])
                out[o] = acc
        yhat[perm, h] = out
    np.testing.assert_allclose(yhat, yhat_oracle, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("G,mode", [(1, 0), (2, 3)])
def test_review_backward_matches_finite_differences(G, mode):
    """ma_bwd with review tokens: the review state starts both directions and
    depends on pooled x, dt, B and on A, so every input but C gets a share
    through it; central finite differences of the pinned forward
    (oracle.ma_fwd with review) check every gradient."""
    rng = np.random.default_rng(90 + G + mode)
    T, H, W, Hs, P, N = 4, 6, 6, 2, 3, 4
    review = ((2, 3, 3), (2, 2, 2))          # pooled grid 2x2x2, every block sampled
    params, dy = _inputs(rng, T * H * W, Hs, P, N, G)
    grads = oracle.ma_bwd(*params, dy, mode, T, H, W, review=review)

    def loss(ps):
        return float(np.sum(dy * oracle.ma_fwd(*ps, mode, T, H, W, review=review)))

    eps = 1e-6
    for i, name in enumerate(("x", "dt", "A", "B", "C", "D")):
        assert grads[i].shape == np.shape(params[i]), name
        v = rng.standard_normal(np.shape(params[i]))
        plus = [p.copy() for p in params]
        minus = [p.copy() for p in params]
        plus[i] = plus[i] + eps * v
        minus[i] = minus[i] - eps * v
        fd = (loss(plus) - loss(minus)) / (2 * eps)
        an = float(np.sum(grads[i] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)
    # the review path changes the gradients (it is not a no-op)
    plain = oracle.ma_bwd(*params, dy, mode, T, H, W)
    assert np.abs(plain[0] - grads[0]).max() > 1e-3


def test_review_backward_without_review_is_bidir_backward():
    rng = np.random.default_rng(95)
    T, H, W = 2, 2, 3
    params, dy = _inputs(rng, T * H * W, 2, 3, 2, 1)
    a = oracle.ma_bwd(*params, dy, 1, T, H, W)
    b = oracle.ssd_bidir_backward(*params, dy, oracle.rms_scan_order(1, T, H, W))
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_initial_state_adjoint_matches_finite_differences():
    """return_dh0: the adjoint of the initial state, and g_final: an adjoint
    on the final state, against finite differences of sum(dy * y) +
    <gf, h_final> in h0."""
    rng = np.random.default_rng(96)
    L, Hs, P, N = 7, 2, 3, 2
    params, dy = _inputs(rng, L, Hs, P, N, 1)
    order = rng.permutation(L)
    h0 = rng.standard_normal((Hs, P, N))
    gf = rng.standard_normal((Hs, P, N))
    out = oracle.ssd_scan_backward(*params, dy, order, h0=h0, g_final=gf, return_dh0=True, segment=3)

    def loss(h, ps=params):
        y, hf, _ = oracle.ssd_scan(*ps, order, h0=h)
        return float(np.sum(dy * y) + np.sum(gf * hf))

    eps = 1e-6
    v = rng.standard_normal(h0.shape)
    fd = (loss(h0 + eps * v) - loss(h0 - eps * v)) / (2 * eps)
    assert abs(fd - float(np.sum(out[6] * v))) <= 1e-6 * max(1.0, abs(fd))
    for i in range(6):
        w = rng.standard_normal(np.shape(params[i]))
        plus = [p.copy() for p in params]
        minus = [p.copy() for p in params]
        plus[i] = plus[i] + eps * w
        minus[i] = minus[i] - eps * w
        fd = (loss(h0, plus) - loss(h0, minus)) / (2 * eps)
        assert abs(fd - float(np.sum(out[i] * w))) <= 1e-6 * max(1.0, abs(fd)), i
