"""GPU parity of the TE-branch backward pass (lingen_te_bwd) through the C
ABI against the fp64 oracle's tesa_backward on the same inputs: plain,
shifted (cut border windows), cyclic and uneven offsets, batch 2, and sampled
heads at the 512p-like workload in the benchmark's launch configuration;
the odd 3x3x3 window (bf16) and the fp32 family of the smallest grid.
The saved-statistics pair (lingen_te_fwd_saved, lingen_te_bwd_saved): its
output equals lingen_te_fwd_shift's bit for bit, its log2 softmax
denominators match oracle.tesa_lse within 4e-3 (the bound from summing
bf16-rounded weights: log2(1 + 2^-9)), and its gradients meet the bars
below against the oracle.

Bar (bf16 storage, fp32 accumulation, bf16 rounding of P and dS as MFMA
operands): relative L2 error at most 2e-2 for each of dq, dk and dv, and
every (token, head) row within 5e-2 of the largest row norm."""
import numpy as np
import pytest

import oracle
from mate_inputs import CONFIGS, make_inputs
from gpu_util import need_gpu, say, head_f64, rel_l2

pytestmark = pytest.mark.gpu

TOL, ROW_TOL = 2e-2, 5e-2


def _check(got, ref, what):
    e = rel_l2(got, ref)
    rows = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1).max()
    say(f"  {what}: rel L2 {e:.3e}, worst row {rows.max():.3e}")
    assert e <= TOL and rows.max() <= ROW_TOL


def _grad_out(torch, shape, seed):
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("shift,masked", [((0, 0, 0), 1), ((2, 4, 4), 1), ((2, 4, 4), 0), ((1, 5, 3), 1)])
def test_te_bwd_cfg1(shift, masked):
    torch, mate = need_gpu()
    s = CONFIGS[1]
    inp = make_inputs(s, 1, tensors=["q", "k", "v"])
    shape = (s.L, s.attn_heads, s.attn_headdim)
    d = {n: inp.torch(n, "cuda") for n in ("q", "k", "v")}
    g = _grad_out(torch, shape, 50)
    say(f"te_bwd cfg1 shift{shift} masked{masked}")
    dq, dk, dv = mate.lingen_te_bwd(d["q"], d["k"], d["v"], g.cuda(), shift, masked, s)
    torch.cuda.synchronize()
    f = {n: inp.f64(n) for n in ("q", "k", "v")}
    ref = oracle.tesa_backward(f["q"], f["k"], f["v"], g.double().numpy(), s.T, s.H, s.W, s.win, shift,
                               cyclic=not masked)
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        _check(got.double().cpu().numpy().reshape(want.shape), want, name)


def test_te_bwd_batch2():
    torch, mate = need_gpu()
    s = CONFIGS[1].with_(batch=2, T=8, H=16, W=16)
    shape = (2, s.L, s.attn_heads, s.attn_headdim)
    rng = np.random.default_rng(51)
    q, k, v, g = (torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16) for _ in range(4))
    say("te_bwd batch 2, 8x16x16, shifted")
    dq, dk, dv = mate.lingen_te_bwd(q.cuda(), k.cuda(), v.cuda(), g.cuda(), (2, 4, 4), 1, s)
    torch.cuda.synchronize()
    for b in range(2):
        ref = oracle.tesa_backward(q[b].double().numpy(), k[b].double().numpy(), v[b].double().numpy(),
                                   g[b].double().numpy(), s.T, s.H, s.W, s.win, (2, 4, 4))
        for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            _check(got[b].double().cpu().numpy(), want, f"batch {b} {name}")


@pytest.mark.parametrize("shift", [(0, 0, 0), (2, 4, 4)])
def test_te_bwd_512p_sampled_heads(shift):
    torch, mate = need_gpu()
    s = CONFIGS[2]
    inp = make_inputs(s, 2, tensors=["q", "k", "v"], threads=16)
    shape = (s.L, s.attn_heads, s.attn_headdim)
    d = {n: inp.torch(n, "cuda") for n in ("q", "k", "v")}
    g = _grad_out(torch, shape, 52)
    say(f"te_bwd 512p-like shift{shift}")
    grads = mate.lingen_te_bwd(d["q"], d["k"], d["v"], g.cuda(), shift, 1, s)
    torch.cuda.synchronize()
    grads = [t.view(shape) for t in grads]
    for h in (0, 17, 31):
        f = {n: head_f64(inp, n, h) for n in ("q", "k", "v")}
        ref = oracle.tesa_backward(f["q"], f["k"], f["v"], g[:, [h]].double().numpy(), s.T, s.H, s.W, s.win, shift)
        for name, got, want in zip(("dq", "dk", "dv"), grads, ref):
            _check(got[:, [h]].double().cpu().numpy(), want, f"head {h} {name}")


# The small-window families (fp32 loops, one workgroup per window and head):
# the odd 3x3x3 window with bf16 storage (the bars above), and the fp32
# family of the 4x8x8 grid (2x4x4 windows, d = 32), where fp32 arithmetic
# from fp32 inputs leaves relative errors of order 1e-6: bar 1e-5.
ODD = CONFIGS[1].with_(T=12, H=12, W=12, win=(3, 3, 3))


@pytest.mark.parametrize("shift,masked", [((0, 0, 0), 1), ((1, 1, 1), 1), ((1, 2, 1), 0), ((2, 1, 0), 1)])
def test_te_bwd_odd_window(shift, masked):
    torch, mate = need_gpu()
    s = ODD
    inp = make_inputs(s, 1, tensors=["q", "k", "v"])
    shape = (s.L, s.attn_heads, s.attn_headdim)
    d = {n: inp.torch(n, "cuda") for n in ("q", "k", "v")}
    g = _grad_out(torch, shape, 53)
    say(f"te_bwd 3x3x3 windows {s.T}x{s.H}x{s.W} shift{shift} masked{masked}")
    dq, dk, dv = mate.lingen_te_bwd(d["q"], d["k"], d["v"], g.cuda(), shift, masked, s)
    torch.cuda.synchronize()
    f = {n: inp.f64(n) for n in ("q", "k", "v")}
    ref = oracle.tesa_backward(f["q"], f["k"], f["v"], g.double().numpy(), s.T, s.H, s.W, s.win, shift,
                               cyclic=not masked)
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        _check(got.double().cpu().numpy().reshape(want.shape), want, name)


@pytest.mark.parametrize("shift,masked", [((0, 0, 0), 1), ((1, 2, 2), 1), ((1, 2, 2), 0), ((1, 1, 3), 1)])
def test_te_bwd_fp32(shift, masked):
    torch, mate = need_gpu()
    s = CONFIGS[0].with_(batch=2)
    rng = np.random.default_rng(54)
    shape = (2, s.L, s.attn_heads, s.attn_headdim)
    q, k, v, g = (torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)) for _ in range(4))
    say(f"te_bwd fp32 {s.T}x{s.H}x{s.W} windows {s.win} shift{shift} masked{masked}, batch 2")
    dq, dk, dv = mate.lingen_te_bwd(q.cuda(), k.cuda(), v.cuda(), g.cuda(), shift, masked, s)
    torch.cuda.synchronize()
    for b in range(2):
        ref = oracle.tesa_backward(q[b].double().numpy(), k[b].double().numpy(), v[b].double().numpy(),
                                   g[b].double().numpy(), s.T, s.H, s.W, s.win, shift, cyclic=not masked)
        for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            got = got[b].double().cpu().numpy()
            e = rel_l2(got, want)
            say(f"  batch {b} {name}: rel L2 {e:.3e}")
            assert e <= 1e-5, (name, e)


# The saved-statistics pair.  LSE_TOL: the forward sums the weights as bf16
# MFMA operands, each within a relative 2^-9 of its value, so the sum and
# its log2 are off by at most log2(1 + 2^-9) = 2.8e-3.
LSE_TOL = 4e-3


@pytest.mark.parametrize("cfg,shift,masked,heads", [(1, (0, 0, 0), 1, None), (1, (2, 4, 4), 1, None),
                                                     (1, (2, 4, 4), 0, None), (1, (1, 5, 3), 1, None),
                                                     (2, (2, 4, 4), 1, (0, 17, 31))])
def test_te_saved_pair(cfg, shift, masked, heads):
    torch, mate = need_gpu()
    s = CONFIGS[cfg]
    inp = make_inputs(s, cfg, tensors=["q", "k", "v"], threads=16)
    shape = (s.L, s.attn_heads, s.attn_headdim)
    d = {n: inp.torch(n, "cuda") for n in ("q", "k", "v")}
    g = _grad_out(torch, shape, 54)
    say(f"te saved pair cfg{cfg} shift{shift} masked{masked}")
    y_ref = mate.lingen_te_fwd_shift(d["q"], d["k"], d["v"], shift, masked, s)
    y, lse = mate.lingen_te_fwd_saved(d["q"], d["k"], d["v"], shift, masked, s)
    grads = mate.lingen_te_bwd_saved(d["q"], d["k"], d["v"], y, g.cuda(), lse, shift, masked, s)
    torch.cuda.synchronize()
    assert torch.equal(y.reshape(-1).view(torch.int16), y_ref.reshape(-1).view(torch.int16)), "y_te"
    grads = [t.view(shape) for t in grads]
    lse = lse.view(s.L, s.attn_heads)
    for h in (heads if heads is not None else range(s.attn_heads)):
        f = {n: head_f64(inp, n, h) for n in ("q", "k", "v")}
        want = oracle.tesa_lse(f["q"], f["k"], s.T, s.H, s.W, s.win, shift, cyclic=not masked)
        err = float(np.abs(lse[:, [h]].double().cpu().numpy() - want).max())
        if heads is not None or h == 0:
            say(f"  head {h} lse: max abs error {err:.2e}")
        assert err <= LSE_TOL, (h, err)
        if heads is None and h > 1:
            continue
        ref = oracle.tesa_backward(f["q"], f["k"], f["v"], g[:, [h]].double().numpy(), s.T, s.H, s.W, s.win,
                                   shift, cyclic=not masked)
        for name, got, want in zip(("dq", "dk", "dv"), grads, ref):
            _check(got[:, [h]].double().cpu().numpy(), want, f"head {h} {name}")


def test_te_saved_pair_batch2():
    torch, mate = need_gpu()
    s = CONFIGS[1].with_(batch=2, T=8, H=16, W=16)
    shape = (2, s.L, s.attn_heads, s.attn_headdim)
    rng = np.random.default_rng(55)
    q, k, v, g = (torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16) for _ in range(4))
    say("te saved pair batch 2, 8x16x16, shifted")
    y, lse = mate.lingen_te_fwd_saved(q.cuda(), k.cuda(), v.cuda(), (2, 4, 4), 1, s)
    dq, dk, dv = mate.lingen_te_bwd_saved(q.cuda(), k.cuda(), v.cuda(), y, g.cuda(), lse, (2, 4, 4), 1, s)
    torch.cuda.synchronize()
    for b in range(2):
        want = oracle.tesa_lse(q[b].double().numpy(), k[b].double().numpy(), s.T, s.H, s.W, s.win, (2, 4, 4))
        err = float(np.abs(lse[b].double().cpu().numpy() - want).max())
        say(f"  batch {b} lse: max abs error {err:.2e}")
        assert err <= LSE_TOL
        ref = oracle.tesa_backward(q[b].double().numpy(), k[b].double().numpy(), v[b].double().numpy(),
                                   g[b].double().numpy(), s.T, s.H, s.W, s.win, (2, 4, 4))
        for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            _check(got[b].double().cpu().numpy(), want, f"batch {b} {name}")
