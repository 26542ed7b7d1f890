"""GPU parity of the MA branch's backward (lingen_ma_bwd) against the fp64
oracle's ssd_bidir_backward: the 16k-token bf16 workload in several scan
orders with one and two B/C groups, a batch of two, and the 512p-like
workload in its launch configuration and the minute-length workload
(524,288 tokens) with dy nonzero on one head only (the gradients are linear
in dy, so every gradient -- dB and dC included -- is that head's, which the
oracle computes over all tokens; the other heads' dx, ddt, dA, dD must be
zero).  Bar: relative L2 error at most 2e-2
per gradient (bf16 storage)."""
import numpy as np
import pytest

import oracle
from mate_inputs import CONFIGS, make_inputs, make_block_inputs
from gpu_util import need_gpu, say, rel_l2, to_np, head_f64

pytestmark = pytest.mark.gpu

SCAN = ("x", "dt", "A", "B", "C", "D")
NAMES = ("dx", "ddt", "dA", "dB", "dC", "dD")
TOL = 2e-2


def _dy(s, cfg_id, seed):
    return make_block_inputs(s, cfg_id, seed=seed, tensors=("y",)).store["y"].reshape(s.L, s.ssd_heads, s.headdim)


def _check(got, ref, what):
    for name, g, r in zip(NAMES, got, ref):
        g = to_np(g).reshape(np.shape(r))
        e = rel_l2(g, r)
        say(f"  {what} {name}: rel L2 {e:.3e}")
        assert e <= TOL, (what, name)


@pytest.mark.parametrize("mode,G", [(0, 1), (1, 2), (3, 1)])
def test_ma_bwd_parity(mode, G):
    torch, mate = need_gpu()
    s = CONFIGS[1].with_(ngroups=G)
    inp = make_inputs(s, 1, seed=111, tensors=list(SCAN))
    dy_bits = _dy(s, 1, 112)
    say(f"ma_bwd {s.T}x{s.H}x{s.W} bf16 groups={G} mode{mode}")
    d = {n: inp.torch(n, "cuda") for n in SCAN}
    dy = torch.from_numpy(dy_bits.view(np.int16)).view(torch.bfloat16).cuda()
    got = mate.lingen_ma_bwd(*(d[n] for n in SCAN), dy, mode, s)
    torch.cuda.synchronize()
    f = {n: inp.f64(n) for n in SCAN}
    from mate_inputs import f32_from_bf16_bits
    dy64 = f32_from_bf16_bits(dy_bits).astype(np.float64)
    ref = oracle.ssd_bidir_backward(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], dy64,
                                    oracle.rms_scan_order(mode, s.T, s.H, s.W))
    _check(got, ref, "")


def test_ma_bwd_batch_of_two():
    torch, mate = need_gpu()
    from mate_inputs import f32_from_bf16_bits
    base = CONFIGS[1].with_(T=4)
    s = base.with_(batch=2)
    mode = 2
    parts = [make_inputs(base, 1, seed=121 + b, tensors=list(SCAN)) for b in range(2)]
    dys = [_dy(base, 1, 131 + b) for b in range(2)]
    say(f"ma_bwd batch 2, {base.T}x{base.H}x{base.W} mode{mode}")
    cat = lambda n: torch.stack([p.torch(n, "cuda") for p in parts])
    x, dt, B, C = cat("x"), cat("dt"), cat("B"), cat("C")
    # A and D are per head, shared by the batch: take the first element's
    A, D = parts[0].torch("A", "cuda"), parts[0].torch("D", "cuda")
    dy = torch.stack([torch.from_numpy(v.view(np.int16)).view(torch.bfloat16) for v in dys]).cuda()
    got = mate.lingen_ma_bwd(x, dt, A, B, C, D, dy, mode, s)
    torch.cuda.synchronize()
    perm = oracle.rms_scan_order(mode, base.T, base.H, base.W)
    refs = []
    for b in range(2):
        f = {n: parts[b].f64(n) for n in SCAN}
        refs.append(oracle.ssd_bidir_backward(f["x"], f["dt"], parts[0].f64("A"), f["B"], f["C"],
                                              parts[0].f64("D"), f32_from_bf16_bits(dys[b]).astype(np.float64),
                                              perm))
    for i, name in enumerate(NAMES):
        g = to_np(got[i])
        if name in ("dA", "dD"):
            r = refs[0][i] + refs[1][i]
        else:
            r = np.stack([refs[0][i], refs[1][i]]).reshape(g.shape)
        e = rel_l2(g, r)
        say(f"  {name}: rel L2 {e:.3e}")
        assert e <= TOL, name


def test_ma_bwd_512p_one_head():
    torch, mate = need_gpu()
    from mate_inputs import f32_from_bf16_bits
    s, cfg_id, head, mode = CONFIGS[2], 2, 13, 3
    inp = make_inputs(s, cfg_id, seed=141, tensors=list(SCAN), threads=16)
    dy_bits = _dy(s, cfg_id, 142)
    dy_bits[:, :head] = 0
    dy_bits[:, head + 1:] = 0
    say(f"ma_bwd 512p-like mode{mode}, dy on head {head} only")
    d = {n: inp.torch(n, "cuda") for n in SCAN}
    dy = torch.from_numpy(dy_bits.view(np.int16)).view(torch.bfloat16).cuda()
    got = mate.lingen_ma_bwd(*(d[n] for n in SCAN), dy, mode, s)
    torch.cuda.synchronize()
    dx, ddt, dA, dB, dC, dD = got
    others = [h for h in range(s.ssd_heads) if h != head]
    assert float(dx[0][:, others].abs().max()) == 0.0
    assert float(ddt[0][:, others].abs().max()) == 0.0
    assert float(dA[others].abs().max()) == 0.0 and float(dD[others].abs().max()) == 0.0
    hx = {n: head_f64(inp, n, head) for n in ("x", "dt", "A", "D")}
    dy64 = f32_from_bf16_bits(dy_bits[:, [head]]).astype(np.float64)
    ref = oracle.ssd_bidir_backward(hx["x"], hx["dt"], hx["A"], inp.f64("B"), inp.f64("C"), hx["D"], dy64,
                                    oracle.rms_scan_order(mode, s.T, s.H, s.W))
    got_head = (dx[0][:, [head]], ddt[0][:, [head]], dA[[head]], dB[0], dC[0], dD[[head]])
    _check(got_head, ref, f"head {head}")


def test_ma_bwd_minute_length_one_head():
    """The largest workload (128x64x64 = 524,288 tokens; 4096 chunks, about
    10^9 state elements per direction), dy on one head, scan order 1."""
    torch, mate = need_gpu()
    from mate_inputs import f32_from_bf16_bits
    s, cfg_id, head, mode = CONFIGS[3], 3, 5, 1
    inp = make_inputs(s, cfg_id, seed=151, tensors=list(SCAN), threads=16)
    dy_bits = _dy(s, cfg_id, 152)
    dy_bits[:, :head] = 0
    dy_bits[:, head + 1:] = 0
    say(f"ma_bwd minute-length mode{mode}, dy on head {head} only")
    d = {n: inp.torch(n, "cuda") for n in SCAN}
    dy = torch.from_numpy(dy_bits.view(np.int16)).view(torch.bfloat16).cuda()
    got = mate.lingen_ma_bwd(*(d[n] for n in SCAN), dy, mode, s)
    torch.cuda.synchronize()
    dx, ddt, dA, dB, dC, dD = got
    got_head = (dx[0][:, [head]].clone(), ddt[0][:, [head]].clone(), dA[[head]].clone(), dB[0].clone(), dC[0].clone(),
                dD[[head]].clone())
    del got, dx, ddt, d, dy
    say("  oracle over all tokens (one head)")
    hx = {n: head_f64(inp, n, head) for n in ("x", "dt", "A", "D")}
    dy64 = f32_from_bf16_bits(dy_bits[:, [head]]).astype(np.float64)
    ref = oracle.ssd_bidir_backward(hx["x"], hx["dt"], hx["A"], inp.f64("B"), inp.f64("C"), hx["D"], dy64,
                                    oracle.rms_scan_order(mode, s.T, s.H, s.W))
    _check(got_head, ref, f"head {head}")
