"""The seeded input generator: determinism, head independence, bf16 rounding."""
import math

import numpy as np
import pytest

from mate_inputs import CONFIGS, make_inputs, bf16_bits_from_f32, f32_from_bf16_bits


def test_deterministic_and_head_independent():
    s = CONFIGS[1].with_(T=2, H=8, W=8)
    a = make_inputs(s, 1)
    b = make_inputs(s, 1)
    for name in a.store:
        np.testing.assert_array_equal(a.store[name], b.store[name])
    sub = make_inputs(s, 1, heads=[3, 11])
    np.testing.assert_array_equal(sub.store["x"], a.store["x"][:, [3, 11]])
    np.testing.assert_array_equal(sub.store["q"], a.store["q"][:, [3, 11]])
    np.testing.assert_array_equal(sub.store["dt"], a.store["dt"][:, [3, 11]])
    np.testing.assert_array_equal(sub.store["A"], a.store["A"][[3, 11]])
    np.testing.assert_array_equal(sub.store["B"], a.store["B"])
    c = make_inputs(s, 2)
    assert not np.array_equal(c.store["x"], a.store["x"])


def test_bf16_round_to_nearest_even_cases():
    one = np.float32(1.0)
    vals = np.array([
        1.0,
        1.0 + 2.0 ** -8,          # halfway between 1 and 1+2^-7: ties to even -> 1
        1.0 + 3 * 2.0 ** -8,      # halfway between 1+2^-7 and 1+2^-6: -> 1+2^-6
        1.0 + 2.0 ** -8 + 2.0 ** -20,  # just above halfway -> 1+2^-7
        -2.5, 0.0, -0.0, 3.0e38, 1e-40,
    ], dtype=np.float32)
    want = np.array([1.0, 1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -2.5, 0.0, -0.0, 2.9941e38, 1e-40])
    got = f32_from_bf16_bits(bf16_bits_from_f32(vals))
    np.testing.assert_array_equal(got[:7], want[:7].astype(np.float32))
    assert abs(got[7] / 3.0e38 - 1) < 2 ** -8
    assert got[8] > 0


def test_bf16_matches_torch_conversion():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ours = bf16_bits_from_f32(a).view(np.int16)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_distributions():
    s = CONFIGS[1].with_(T=4, H=32, W=32)
    inp = make_inputs(s, 1)
    dt = inp.f64("dt")
    A = inp.f64("A")
    assert np.all(dt > 0)
    assert np.all((A <= -1.0) & (A >= -16.0))
    assert abs(np.median(dt) - math.log1p(math.exp(-3.0))) < 0.01
    B = inp.f64("B")
    assert abs(B.std() - 1 / math.sqrt(s.d_state)) < 0.01
    x = inp.f64("x")
    assert abs(x.std() - 1.0) < 0.01
    # bf16 storage: every value is exactly representable in bf16
    np.testing.assert_array_equal(bf16_bits_from_f32(inp.f32("q")), inp.store["q"])


def test_fp32_config_is_not_rounded():
    inp = make_inputs(CONFIGS[0], 0)
    assert inp.store["x"].dtype == np.float32
    assert inp.store["x"].shape == (256, 2, 32)
    assert inp.store["q"].shape == (256, 2, 32)
