"""Full-size parity in the benchmark's launch configuration: one
lingen_mate_fwd call over the whole tensor (131k, 524k and 295k+64 review
tokens), checked against the fp64 oracle on sampled heads.

Heads are independent in both branches (an SSD head reads only its own x,
dt, A, D plus the shared B, C; an attention head only its own q, k, v), so
the oracle runs the full sequence for the sampled head and the whole column
block of that head in y is compared, over every token."""
import numpy as np
import pytest

import oracle
from mate_inputs import CONFIGS, make_inputs
from gpu_util import need_gpu, say, upload, head_f64, review_of, check_rows

pytestmark = pytest.mark.gpu

_cache = {}


def _inputs(cfg):
    if cfg not in _cache:
        _cache.clear()
        _cache[cfg] = make_inputs(CONFIGS[cfg], cfg, threads=16)
    return _cache[cfg]


def _run(cfg, layer, head):
    torch, mate = need_gpu()
    s = CONFIGS[cfg]
    inp = _inputs(cfg)
    d = upload(inp)
    say(f"full-size mate_fwd cfg{cfg} ({s.L} tokens) layer{layer} sampled head {head}")
    y = mate.lingen_mate_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["q"], d["k"], d["v"], layer, s)
    torch.cuda.synchronize()
    got = y[0, :, head * s.headdim:(head + 1) * s.headdim].double().cpu().numpy()
    assert not np.isnan(got).any()
    del y, d
    torch.cuda.empty_cache()
    B = inp.f64("B")
    C = inp.f64("C")
    hx = {n: head_f64(inp, n, head) for n in ("x", "dt", "A", "D", "q", "k", "v")}
    shift = tuple(w // 2 for w in s.win) if layer % 2 else (0, 0, 0)
    y_ma = oracle.ma_fwd(hx["x"], hx["dt"], hx["A"], B, C, hx["D"], layer % 4, s.T, s.H, s.W, review=review_of(s))
    o = oracle.tesa(hx["q"], hx["k"], hx["v"], s.T, s.H, s.W, s.win, shift)
    ref = y_ma[:, 0, :] + o[:, 0, :]
    check_rows(got, ref, s.headdim, s, what=f"head {head}, all tokens")


@pytest.mark.parametrize("layer,head", [(0, 0), (1, 13), (2, 22), (3, 31)])
def test_cfg2_512p_like(layer, head):
    _run(2, layer, head)


@pytest.mark.parametrize("layer,head", [(0, 7), (1, 18), (2, 3), (3, 30)])
def test_cfg3_minute_length(layer, head):
    _run(3, layer, head)


@pytest.mark.parametrize("layer,head", [(0, 11), (1, 5), (2, 26), (3, 20)])
def test_cfg4_768p_review(layer, head):
    _run(4, layer, head)
