"""GPU parity of the dense softmax attention (the quadratic mixer that MATE
replaces) through the C ABI against the fp64 oracle on the same inputs.

Small cases cover one and several key blocks, ragged tails of the 64-key
blocks and of the 512-query workgroup tiles, batch > 1, sharper softmax
(scaled queries) and the empty problem.  The full-size cases run the launch
configuration the benchmark times (131,072 and 524,288 tokens, 32 heads of 64)
and check sampled queries, each against all keys.

Bar (bf16 storage, fp32 accumulation): relative L2 error at most 2e-2 over
the whole output, and at most 5e-2 for every single (token, head) row, so
that one wrong row cannot hide in a large tensor."""
import numpy as np
import pytest

import oracle
from mate_inputs import CONFIGS, make_inputs
from gpu_util import need_gpu, say, head_f64, rel_l2

pytestmark = pytest.mark.gpu

TOL, ROW_TOL = 2e-2, 5e-2


def _row_errors(got, ref):
    """Relative L2 error of every (token, head) row of [n, heads, d] arrays."""
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return num / np.maximum(den, 1e-30)


def _check(got, ref, what):
    err = rel_l2(got, ref)
    rows = _row_errors(got, ref)
    say(f"  {what}: rel L2 {err:.3e}, worst row {rows.max():.3e}")
    assert err <= TOL
    assert rows.max() <= ROW_TOL


@pytest.mark.parametrize("batch,L,heads,scale", [
    (1, 1, 1, 1.0),
    (1, 17, 2, 1.0),
    (1, 64, 1, 1.0),
    (1, 65, 3, 1.0),
    (2, 1000, 2, 1.0),
    (1, 4099, 2, 1.0),
    (1, 1536, 1, 3.0),
])
def test_dense_small(batch, L, heads, scale):
    torch, mate = need_gpu()
    rng = np.random.default_rng(7000 + L)
    shape = (batch, L, heads, 64)
    q, k, v = (torch.from_numpy(rng.standard_normal(shape, dtype=np.float32) * s).to(torch.bfloat16)
               for s in (scale, scale, 1.0))
    say(f"dense_attn batch={batch} L={L} heads={heads} scale={scale}")
    o = mate.lingen_dense_attn_fwd(q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    got = o.double().cpu().numpy()
    for b in range(batch):
        ref = oracle.dense_attention(q[b].double().numpy(), k[b].double().numpy(), v[b].double().numpy())
        _check(got[b], ref, f"batch {b}")
    if L == 1:
        assert torch.equal(o.cpu(), v)       # one key: the weight is exactly 1


def test_dense_empty_and_unsupported():
    torch, mate = need_gpu()
    say("dense_attn empty inputs and unsupported head size")
    for shape in ((1, 0, 2, 64), (0, 5, 2, 64), (1, 5, 0, 64)):
        t = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        assert mate.lingen_dense_attn_fwd(t, t, t).shape == shape
    t = torch.zeros((1, 8, 2, 32), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mate.LingenError):
        mate.lingen_dense_attn_fwd(t, t, t)
    t = torch.zeros((1, 8, 2, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(mate.LingenError):
        mate.lingen_dense_attn_fwd(t, t, t)


@pytest.mark.parametrize("cfg,heads_checked,n_queries", [(2, None, 24), (3, (0, 9, 22, 31), 12)])
def test_dense_fullsize_sampled(cfg, heads_checked, n_queries):
    torch, mate = need_gpu()
    s = CONFIGS[cfg]
    inp = make_inputs(s, cfg, tensors=["q", "k", "v"], threads=16)
    shape = (1, s.L, s.attn_heads, s.attn_headdim)
    d = {n: inp.torch(n, "cuda").view(shape) for n in ("q", "k", "v")}
    say(f"dense_attn full size cfg{cfg}: L={s.L} heads={s.attn_heads}")
    o = mate.lingen_dense_attn_fwd(d["q"], d["k"], d["v"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(cfg)
    edge = [0, 1, 511, 512, s.L - 513, s.L - 1]
    idx = np.array(sorted(set(edge) | set(rng.integers(0, s.L, n_queries - len(edge)).tolist())))
    got = o[0, torch.from_numpy(idx).cuda()].double().cpu().numpy()        # [nq, heads, d]
    del d, o
    for h in (heads_checked or range(s.attn_heads)):
        q, k, v = (head_f64(inp, n, h) for n in ("q", "k", "v"))
        ref = oracle.dense_attention_for_queries(q, k, v, idx)
        _check(got[:, [h]], ref, f"head {h}, {idx.size} queries")
