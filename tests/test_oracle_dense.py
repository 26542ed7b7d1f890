"""Pins for the oracle's dense (full) softmax attention, the quadratic mixer
that MATE replaces: brute force on tiny inputs, closed forms and invariances
of softmax attention."""
import math

import numpy as np

import oracle


def _qkv(rng, L, Ha, d, scale=1.0):
    return (rng.standard_normal((L, Ha, d)) * scale,
            rng.standard_normal((L, Ha, d)) * scale,
            rng.standard_normal((L, Ha, d)))


def test_brute_force_loops():
    # Scalar loops straight from o_i = sum_j e^{s_ij} v_j / sum_j e^{s_ij},
    # s_ij = q_i . k_j / sqrt(d): no max subtraction, no library softmax.
    rng = np.random.default_rng(11)
    L, Ha, d = 6, 2, 3
    q, k, v = _qkv(rng, L, Ha, d)
    got = oracle.dense_attention(q, k, v)
    for h in range(Ha):
        for i in range(L):
            w = [math.exp(sum(q[i, h, c] * k[j, h, c] for c in range(d)) / math.sqrt(d)) for j in range(L)]
            z = sum(w)
            for c in range(d):
                ref = sum(w[j] * v[j, h, c] for j in range(L)) / z
                assert abs(got[i, h, c] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_zero_query_gives_mean_of_all_values():
    rng = np.random.default_rng(12)
    q, k, v = _qkv(rng, 37, 3, 4)
    q[:] = 0.0
    got = oracle.dense_attention(q, k, v)
    np.testing.assert_allclose(got, np.broadcast_to(v.mean(axis=0), got.shape), rtol=1e-13, atol=1e-14)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(13)
    q, k, v = _qkv(rng, 1, 2, 5)
    np.testing.assert_array_equal(oracle.dense_attention(q, k, v), v)


def test_key_permutation_invariance_and_query_equivariance():
    rng = np.random.default_rng(14)
    q, k, v = _qkv(rng, 29, 2, 4)
    base = oracle.dense_attention(q, k, v)
    pk = rng.permutation(29)
    np.testing.assert_allclose(oracle.dense_attention(q, k[pk], v[pk]), base, rtol=1e-12, atol=1e-13)
    pq = rng.permutation(29)
    np.testing.assert_allclose(oracle.dense_attention(q[pq], k, v), base[pq], rtol=1e-12, atol=1e-13)


def test_common_key_offset_cancels():
    # q_i . (k_j + u) = q_i . k_j + q_i . u: the same shift for every key j.
    rng = np.random.default_rng(15)
    q, k, v = _qkv(rng, 23, 2, 6)
    u = rng.standard_normal((1, 2, 6))
    np.testing.assert_allclose(oracle.dense_attention(q, k + u, v), oracle.dense_attention(q, k, v),
                               rtol=1e-10, atol=1e-12)


def test_sharp_scores_select_the_best_key():
    rng = np.random.default_rng(16)
    L, Ha, d = 17, 2, 8
    q, k, v = _qkv(rng, L, Ha, d)
    q *= 1e3
    got = oracle.dense_attention(q, k, v)
    for h in range(Ha):
        best = np.argmax(q[:, h] @ k[:, h].T, axis=1)
        np.testing.assert_allclose(got[:, h], v[best, h], rtol=0, atol=1e-6)


def test_outputs_are_convex_combinations():
    rng = np.random.default_rng(17)
    q, k, v = _qkv(rng, 50, 3, 4, scale=2.0)
    got = oracle.dense_attention(q, k, v)
    assert np.all(got <= v.max(axis=0) + 1e-12) and np.all(got >= v.min(axis=0) - 1e-12)


def test_equals_one_window_tesa_and_query_subset():
    rng = np.random.default_rng(18)
    T, H, W = 2, 3, 5
    q, k, v = _qkv(rng, T * H * W, 2, 4)
    full = oracle.dense_attention(q, k, v)
    np.testing.assert_allclose(full, oracle.tesa(q, k, v, T, H, W, (T, H, W), (0, 0, 0)), rtol=1e-12, atol=1e-13)
    idx = [29, 0, 7, 7]
    np.testing.assert_allclose(oracle.dense_attention_for_queries(q, k, v, idx, head_block=1), full[idx],
                               rtol=1e-12, atol=1e-13)
