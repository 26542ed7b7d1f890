"""GPU parity of the TE-branch backward pass (lingen_te_bwd) through the C
ABI against the fp64 oracle's tesa_backward on the same inputs: plain,
shifted (cut border windows), cyclic and uneven offsets, batch 2, and sampled
heads at the 512p-like workload in the benchmark's launch configuration.

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
