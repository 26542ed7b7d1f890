"""GPU parity of the MA branch's backward (lingen_ma_bwd) against the fp64
oracle's ssd_bidir_backward: the 16k-token bf16 workload in several scan
orders with one and two B/C groups, a batch of two, and the 512p-like
workload in its launch configuration and the minute-length workload
(524,288 tokens) with dy nonzero on one head only (the gradients are linear
in dy, so every gradient -- dB and dC included -- is that head's, which the
oracle computes over all tokens; the other heads' dx, ddt, dA, dD must be
zero); and review tokens (the 16k-token workload with 64 review tokens,
and the 768p-like workload with its 64 review tokens, dy on one head),
against the oracle's ma_bwd, whose review path is pinned by finite
differences.  Bar: relative L2 error at most 2e-2 per gradient (bf16
storage).  The fp32 family (the 4x8x8 grid: every scan order, one and two
groups, review tokens, a batch of two) at 1e-4.  The saved-state pair
(lingen_ma_fwd_saved, lingen_ma_bwd_saved) against lingen_ma_fwd and
lingen_ma_bwd on the same inputs: y_ma and dx bit for bit, the other
gradients to 1e-6 (the order of float atomic sums)."""
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


@pytest.mark.parametrize("mode,G", [(0, 1), (2, 2)])
def test_ma_bwd_review_parity(mode, G):
    torch, mate = need_gpu()
    from mate_inputs import f32_from_bf16_bits
    rv = ((2, 4, 4), (4, 4, 4))
    s = CONFIGS[1].with_(ngroups=G, n_review=64, rpool=rv[0], rgrid=rv[1])
    inp = make_inputs(s, 1, seed=161, tensors=list(SCAN))
    dy_bits = _dy(s, 1, 162)
    say(f"ma_bwd {s.T}x{s.H}x{s.W} bf16 groups={G} mode{mode} review={s.n_review}")
    d = {n: inp.torch(n, "cuda") for n in SCAN}
    dy = torch.from_numpy(dy_bits.view(np.int16)).view(torch.bfloat16).cuda()
    got = mate.lingen_ma_bwd(*(d[n] for n in SCAN), dy, mode, s)
    torch.cuda.synchronize()
    f = {n: inp.f64(n) for n in SCAN}
    dy64 = f32_from_bf16_bits(dy_bits).astype(np.float64)
    ref = oracle.ma_bwd(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], dy64, mode, s.T, s.H, s.W, review=rv)
    _check(got, ref, "")


def test_ma_bwd_768p_review_one_head():
    """The 768p-like workload (32x96x96 = 294,912 tokens) with its 64 review
    tokens, dy on one head, scan order 2: the review state's adjoint
    reaches the pooled x, dt and B of that head (and B of all)."""
    torch, mate = need_gpu()
    from mate_inputs import f32_from_bf16_bits
    s, cfg_id, head, mode = CONFIGS[4], 4, 21, 2
    inp = make_inputs(s, cfg_id, seed=171, tensors=list(SCAN), threads=16)
    dy_bits = _dy(s, cfg_id, 172)
    dy_bits[:, :head] = 0
    dy_bits[:, head + 1:] = 0
    say(f"ma_bwd 768p-like + review mode{mode}, dy on head {head} only")
    d = {n: inp.torch(n, "cuda") for n in SCAN}
    dy = torch.from_numpy(dy_bits.view(np.int16)).view(torch.bfloat16).cuda()
    got = mate.lingen_ma_bwd(*(d[n] for n in SCAN), dy, mode, s)
    torch.cuda.synchronize()
    dx, ddt, dA, dB, dC, dD = got
    others = [h for h in range(s.ssd_heads) if h != head]
    assert float(dx[0][:, others].abs().max()) == 0.0
    assert float(ddt[0][:, others].abs().max()) == 0.0
    assert float(dA[others].abs().max()) == 0.0 and float(dD[others].abs().max()) == 0.0
    got_head = (dx[0][:, [head]].clone(), ddt[0][:, [head]].clone(), dA[[head]].clone(), dB[0].clone(), dC[0].clone(),
                dD[[head]].clone())
    del got, dx, ddt, d, dy
    say("  oracle over all tokens (one head)")
    hx = {n: head_f64(inp, n, head) for n in ("x", "dt", "A", "D")}
    dy64 = f32_from_bf16_bits(dy_bits[:, [head]]).astype(np.float64)
    ref = oracle.ma_bwd(hx["x"], hx["dt"], hx["A"], inp.f64("B"), inp.f64("C"), hx["D"], dy64, mode, s.T, s.H, s.W,
                        review=(s.rpool, s.rgrid))
    _check(got_head, ref, f"head {head}")


def test_ma_bwd_review_path_isolated():
    """The review tokens' share of the gradients is small at these decays
    (1e-5 of dx, 3e-4 of dB), below what a bf16 bar sees in the whole
    gradient, so it is checked on its own: dx and dB take nothing from the
    review state on the main path (dx from the adjoint alone, dB from the
    adjoint and x), so the difference between the gradients with and
    without review tokens is exactly the review tokens' share, in fp32 on
    both sides; it must match the oracle's difference."""
    torch, mate = need_gpu()
    from mate_inputs import f32_from_bf16_bits
    rv = ((2, 4, 4), (4, 4, 4))
    plain = CONFIGS[1].with_(T=8)
    s = plain.with_(n_review=64, rpool=rv[0], rgrid=rv[1])
    mode = 3
    inp = make_inputs(s, 1, seed=181, tensors=list(SCAN))
    dy_bits = _dy(s, 1, 182)
    say(f"ma_bwd review share {s.T}x{s.H}x{s.W} mode{mode}: with minus without review tokens")
    d = {n: inp.torch(n, "cuda") for n in SCAN}
    dy = torch.from_numpy(dy_bits.view(np.int16)).view(torch.bfloat16).cuda()
    got_r = [g.clone() for g in mate.lingen_ma_bwd(*(d[n] for n in SCAN), dy, mode, s)]
    got_p = mate.lingen_ma_bwd(*(d[n] for n in SCAN), dy, mode, plain)
    torch.cuda.synchronize()
    f = [inp.f64(n) for n in SCAN]
    dy64 = f32_from_bf16_bits(dy_bits).astype(np.float64)
    ref_r = oracle.ma_bwd(*f, dy64, mode, s.T, s.H, s.W, review=rv)
    ref_p = oracle.ma_bwd(*f, dy64, mode, s.T, s.H, s.W)
    for i, name in ((0, "dx"), (3, "dB")):
        dg = to_np(got_r[i]).reshape(np.shape(ref_r[i])) - to_np(got_p[i]).reshape(np.shape(ref_p[i]))
        dr = ref_r[i] - ref_p[i]
        e = rel_l2(dg, dr)
        say(f"  review share of {name}: rel L2 {e:.3e} (share {rel_l2(ref_r[i], ref_p[i]):.2e} of the gradient)")
        assert e <= TOL, name


# The fp32 family (4x8x8 grid, 2 heads of 32, N = Q = 16): fp32 storage and
# fp32 arithmetic throughout (fp32 loops for the crossing sums), so the bar
# is 1e-4 relative L2 per gradient.
TOL_F32 = 1e-4


def _check_f32(got, ref, what):
    for name, g, r in zip(NAMES, got, ref):
        g = to_np(g).reshape(np.shape(r))
        e = rel_l2(g, r)
        say(f"  {what} {name}: rel L2 {e:.3e}")
        assert e <= TOL_F32, (what, name, e)


@pytest.mark.parametrize("mode,G,review", [(0, 1, False), (1, 2, False), (2, 1, False), (3, 2, False),
                                           (1, 1, True), (2, 2, True)])
def test_ma_bwd_fp32(mode, G, review):
    torch, mate = need_gpu()
    rv = ((2, 2, 2), (1, 2, 2))
    s = CONFIGS[0].with_(ngroups=G)
    if review:
        s = s.with_(n_review=4, rpool=rv[0], rgrid=rv[1])
    inp = make_inputs(s, 0, seed=181, tensors=list(SCAN))
    dy = _dy(s, 0, 182)
    say(f"ma_bwd {s.T}x{s.H}x{s.W} fp32 groups={G} mode{mode} review={s.n_review}")
    d = {n: inp.torch(n, "cuda") for n in SCAN}
    got = mate.lingen_ma_bwd(*(d[n] for n in SCAN), torch.from_numpy(dy).cuda(), mode, s)
    torch.cuda.synchronize()
    f = {n: inp.f64(n) for n in SCAN}
    ref = oracle.ma_bwd(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], dy.astype(np.float64), mode, s.T, s.H, s.W,
                        review=rv if review else None)
    _check_f32(got, ref, "")


def test_ma_bwd_fp32_batch_of_two():
    torch, mate = need_gpu()
    base = CONFIGS[0]
    s = base.with_(batch=2)
    mode = 3
    parts = [make_inputs(base, 0, seed=191 + b, tensors=list(SCAN)) for b in range(2)]
    dys = [_dy(base, 0, 193 + b) for b in range(2)]
    say(f"ma_bwd fp32 batch 2, {base.T}x{base.H}x{base.W} mode{mode}")
    cat = lambda n: torch.stack([p.torch(n, "cuda") for p in parts])
    x, dt, B, C = cat("x"), cat("dt"), cat("B"), cat("C")
    A, D = parts[0].torch("A", "cuda"), parts[0].torch("D", "cuda")
    dy = torch.stack([torch.from_numpy(v) for v in dys]).cuda()
    got = mate.lingen_ma_bwd(x, dt, A, B, C, D, dy, mode, s)
    torch.cuda.synchronize()
    perm = oracle.rms_scan_order(mode, base.T, base.H, base.W)
    refs = []
    for b in range(2):
        f = {n: parts[b].f64(n) for n in SCAN}
        refs.append(oracle.ssd_bidir_backward(f["x"], f["dt"], parts[0].f64("A"), f["B"], f["C"],
                                              parts[0].f64("D"), dys[b].astype(np.float64), perm))
    for i, name in enumerate(NAMES):
        g = to_np(got[i])
        if name in ("dA", "dD"):   # summed over the batch
            r = refs[0][i] + refs[1][i]
            e = rel_l2(g.reshape(np.shape(r)), r)
        else:
            e = max(rel_l2(g[b].reshape(np.shape(refs[b][i])), refs[b][i]) for b in range(2))
        say(f"  {name}: rel L2 {e:.3e}")
        assert e <= TOL_F32, (name, e)


# The saved-state pair: same kernels as lingen_ma_fwd + lingen_ma_bwd, with
# the forward's scan states kept instead of computed again.
SAVED_CASES = {
    "bf16-16k-g2-mode1": dict(cfg=1, kw=dict(ngroups=2), mode=1, batch=1),
    "bf16-16k-batch2-mode2": dict(cfg=1, kw=dict(T=4), mode=2, batch=2),
    "bf16-16k-review-mode3": dict(cfg=1, kw=dict(n_review=64, rpool=(2, 4, 4), rgrid=(4, 4, 4)), mode=3, batch=1),
    "bf16-512p-like-mode3": dict(cfg=2, kw={}, mode=3, batch=1),
    "fp32-review-g2-mode2": dict(cfg=0, kw=dict(ngroups=2, n_review=4, rpool=(2, 2, 2), rgrid=(1, 2, 2)), mode=2,
                                 batch=1),
    "fp32-batch2-mode0": dict(cfg=0, kw={}, mode=0, batch=2),
}


@pytest.mark.parametrize("case", list(SAVED_CASES))
def test_ma_saved_matches_recompute(case):
    torch, mate = need_gpu()
    c = SAVED_CASES[case]
    base = CONFIGS[c["cfg"]].with_(**c["kw"])
    s = base.with_(batch=c["batch"])
    mode = c["mode"]
    parts = [make_inputs(base, c["cfg"], seed=201 + b, tensors=list(SCAN), threads=16) for b in range(c["batch"])]
    dys = [_dy(base, c["cfg"], 211 + b) for b in range(c["batch"])]
    say(f"ma saved vs recompute: {case} ({s.T}x{s.H}x{s.W} batch {s.batch} {s.dtype} mode{mode})")
    cat = lambda n: torch.stack([p.torch(n, "cuda") for p in parts])
    x, dt, B, C = cat("x"), cat("dt"), cat("B"), cat("C")
    A, D = parts[0].torch("A", "cuda"), parts[0].torch("D", "cuda")
    if s.dtype == "bf16":
        dy = torch.stack([torch.from_numpy(v.view(np.int16)).view(torch.bfloat16) for v in dys]).cuda()
    else:
        dy = torch.stack([torch.from_numpy(v) for v in dys]).cuda()
    y_ref = mate.lingen_ma_fwd(x, dt, A, B, C, D, mode, s)
    ref = [g.clone() for g in mate.lingen_ma_bwd(x, dt, A, B, C, D, dy, mode, s)]
    y, saved = mate.lingen_ma_fwd_saved(x, dt, A, B, C, D, mode, s)
    got = mate.lingen_ma_bwd_saved(x, dt, A, B, C, D, dy, saved, mode, s)
    torch.cuda.synchronize()
    assert saved.numel() == mate.lingen_ma_saved_bytes(s)
    assert torch.equal(y.view(torch.int16 if s.dtype == "bf16" else torch.int32),
                       y_ref.view(torch.int16 if s.dtype == "bf16" else torch.int32)), "y_ma"
    assert torch.equal(got[0], ref[0]), "dx"
    for name, g, r in zip(NAMES, got, ref):
        e = rel_l2(to_np(g), to_np(r))
        say(f"  {name}: rel L2 to the recomputing backward {e:.2e}")
        assert e <= 1e-6, name
