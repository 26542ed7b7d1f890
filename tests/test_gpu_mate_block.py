"""GPU parity of the whole MATE block (lingen_mate_block_fwd: rocBLAS
projections around the library's kernels) against the oracle's mate_block:
the fp32 workload at every layer phase with a model width different from
the mixer width, the 16k-token bf16 workload with one and two B/C groups,
and the 512p-like workload at model width 2048 in the launch configuration
of the full-size run, where the attention half is checked on sampled tokens
(each computed by the oracle from its window alone) and the whole output by
the additivity of the two branches; and review tokens in the MA branch at
the small workloads.  Bars: relative L2 error at most 1e-5 with fp32
storage and 2e-2 with bf16 storage."""
import numpy as np
import pytest

import oracle
from mate_inputs import CONFIGS, make_block_weights
from gpu_util import need_gpu, say, rel_l2, to_np, tol

pytestmark = pytest.mark.gpu


def _upload(inp, mate):
    return {n: inp.torch(n, "cuda") for n in mate.BLOCK_WEIGHTS}


def _oracle_block(inp, s, layer):
    w = {n: inp.f64(n) for n in inp.store if n != "u"}
    return oracle.mate_block(inp.f64("u"), w, layer, s.T, s.H, s.W, s.ssd_heads, s.headdim, s.ngroups, s.d_state,
                             s.attn_heads, s.win)


@pytest.mark.parametrize("cfg_id,G,d_model,layer", [(0, 1, 96, 0), (0, 1, 96, 1), (0, 1, 96, 2), (0, 1, 96, 3),
                                                    (1, 1, 1024, 1), (1, 1, 1024, 2), (1, 2, 768, 3)])
def test_block_parity(cfg_id, G, d_model, layer):
    torch, mate = need_gpu()
    s = CONFIGS[cfg_id].with_(ngroups=G)
    inp = make_block_weights(s, cfg_id, d_model, seed=808)
    say(f"mate_block {s.T}x{s.H}x{s.W} {s.dtype} groups={G} d_model={d_model} layer={layer}")
    u = inp.torch("u", "cuda").reshape(1, s.L, d_model)
    out = mate.lingen_mate_block_fwd(u, _upload(inp, mate), layer, s)
    torch.cuda.synchronize()
    ref = _oracle_block(inp, s, layer)
    e = rel_l2(to_np(out)[0], ref)
    say(f"  rel L2 {e:.3e}")
    assert e <= tol(s)


@pytest.mark.parametrize("cfg_id,G,d_model,layer,rv", [
    (0, 1, 96, 1, ((2, 2, 2), (1, 2, 2))),
    (1, 1, 1024, 2, ((2, 4, 4), (4, 4, 4))),
    (1, 2, 768, 3, ((2, 4, 4), (4, 4, 4))),
])
def test_block_review_parity(cfg_id, G, d_model, layer, rv):
    # review tokens in the MA branch, pooled from each direction's scan
    # inputs (after the convolution)
    torch, mate = need_gpu()
    rpool, rgrid = rv
    s = CONFIGS[cfg_id].with_(ngroups=G, n_review=int(np.prod(rgrid)), rpool=rpool, rgrid=rgrid)
    inp = make_block_weights(s, cfg_id, d_model, seed=818)
    say(f"mate_block {s.T}x{s.H}x{s.W} {s.dtype} groups={G} d_model={d_model} layer={layer} review={s.n_review}")
    u = inp.torch("u", "cuda").reshape(1, s.L, d_model)
    out = mate.lingen_mate_block_fwd(u, _upload(inp, mate), layer, s)
    torch.cuda.synchronize()
    w = {n: inp.f64(n) for n in inp.store if n != "u"}
    ref = oracle.mate_block(inp.f64("u"), w, layer, s.T, s.H, s.W, s.ssd_heads, s.headdim, s.ngroups, s.d_state,
                            s.attn_heads, s.win, review=(rpool, rgrid))
    e = rel_l2(to_np(out)[0], ref)
    say(f"  rel L2 {e:.3e}")
    assert e <= tol(s)
    if s.dtype == "f32":
        # the review state reaches the output far above the fp32 error (in
        # bf16 its share, 1e-3 of the output at these decays, is below the
        # storage's rounding)
        plain = oracle.mate_block(inp.f64("u"), w, layer, s.T, s.H, s.W, s.ssd_heads, s.headdim, s.ngroups,
                                  s.d_state, s.attn_heads, s.win)
        assert rel_l2(plain, ref) > 100 * e


def test_block_512p():
    """512p-like workload (131,072 tokens), model width 2048."""
    torch, mate = need_gpu()
    s, cfg_id, Dm, layer = CONFIGS[2], 2, 2048, 1
    inp = make_block_weights(s, cfg_id, Dm, seed=909)
    w = _upload(inp, mate)
    u = inp.torch("u", "cuda").reshape(1, s.L, Dm)
    say("mate_block 512p-like, d_model 2048, layer 1: full, MA only, TE only")
    full = mate.lingen_mate_block_fwd(u, w, layer, s)
    ma = mate.lingen_mate_block_fwd(u, dict(w, w_o=torch.zeros_like(w["w_o"])), layer, s)
    te = mate.lingen_mate_block_fwd(u, dict(w, w_out_ma=torch.zeros_like(w["w_out_ma"])), layer, s)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(full.float()).all())
    e_add = float(torch.linalg.vector_norm((ma.float() + te.float() - full.float())) /
                  torch.linalg.vector_norm(full.float()))
    say(f"  additivity: rel L2 {e_add:.3e}")
    assert e_add <= 1e-2

    # attention half on sampled tokens: each from the projections of its own window
    rng = np.random.default_rng(7)
    sample = sorted(set([0, s.L - 1]) | set(rng.choice(s.L, 30, replace=False).tolist()))
    keys = oracle.tesa_window_keys(s.T, s.H, s.W, s.win, oracle.tesa_shift(layer, s.win))
    u64 = inp.f32("u")
    wq, wk, wv, wo = (inp.f64(n) for n in ("w_q", "w_k", "w_v", "w_o"))
    got = to_np(te[0, sample])
    ref = np.empty_like(got)
    dh = s.attn_headdim
    for i, t in enumerate(sample):
        members = np.flatnonzero((keys == keys[t]).all(axis=1))
        uu = u64[members].astype(np.float64)
        q, k, v = ((uu @ m.T).reshape(len(members), s.attn_heads, dh) for m in (wq, wk, wv))
        o = oracle.dense_attention_for_queries(q, k, v, [int(np.flatnonzero(members == t)[0])])
        ref[i] = o.reshape(-1) @ wo.T
    e = rel_l2(got, ref)
    say(f"  attention half, {len(sample)} sampled tokens: rel L2 {e:.3e}")
    assert e <= tol(s)
