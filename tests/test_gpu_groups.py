"""GPU parity with several B, C groups (Mamba2's head grouping: head h reads
group h // (Hs / G)) against the fp64 oracle: the chunk-boundary states,
the whole mixer, with and without review tokens.  Bars: relative L2 error of
the output at most 1e-5 with fp32 storage and 2e-2 with bf16 storage."""
import numpy as np
import pytest

import oracle
from mate_inputs import CONFIGS, make_inputs
from gpu_util import need_gpu, say, upload, f64_all, rel_l2, to_np, tol, review_of

pytestmark = pytest.mark.gpu


def _mate(s, cfg_id, layer):
    torch, mate = need_gpu()
    inp = make_inputs(s, cfg_id)
    d = upload(inp)
    say(f"mate_fwd {s.T}x{s.H}x{s.W} {s.dtype} heads={s.ssd_heads} groups={s.ngroups} review={s.n_review} "
        f"layer{layer}")
    y = mate.lingen_mate_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["q"], d["k"], d["v"], layer, s)
    torch.cuda.synchronize()
    f = f64_all(inp)
    ref = oracle.mate_fwd(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["q"], f["k"], f["v"], layer,
                          s.T, s.H, s.W, s.win, review=review_of(s))
    e = rel_l2(to_np(y).reshape(ref.shape), ref)
    say(f"  rel L2 {e:.3e}")
    assert e <= tol(s)


@pytest.mark.parametrize("layer", range(4))
def test_mate_two_groups_fp32(layer):
    _mate(CONFIGS[0].with_(ngroups=2), 40, layer)           # one head per group


@pytest.mark.parametrize("layer", range(4))
def test_mate_four_groups_bf16(layer):
    _mate(CONFIGS[1].with_(ngroups=4), 41, layer)           # four heads per group


@pytest.mark.parametrize("G", [2, 16])
def test_mate_groups_review_bf16(G):
    _mate(CONFIGS[1].with_(ngroups=G, n_review=64, rpool=(2, 4, 4), rgrid=(4, 4, 4)), 42, 1)


def test_mate_groups_512p_heads():
    # workload-2 head and state sizes (N = 128, chunk 128) with 8 groups on a
    # smaller grid that the oracle scans in seconds
    _mate(CONFIGS[2].with_(T=8, H=16, W=16, ssd_heads=8, attn_heads=8, ngroups=4), 43, 2)


def test_chunk_states_groups():
    torch, mate = need_gpu()
    s = CONFIGS[1].with_(ngroups=8)
    inp = make_inputs(s, 44)
    d = upload(inp)
    mode = 3
    say(f"ssd_chunk_states groups={s.ngroups} mode{mode}")
    hf, hb = mate.lingen_ssd_chunk_states(d["x"], d["dt"], d["A"], d["B"], mode, s)
    torch.cuda.synchronize()
    f = f64_all(inp)
    L, Q = s.L, s.chunk
    nc = L // Q
    perm = oracle.rms_scan_order(mode, s.T, s.H, s.W)
    _, _, recf = oracle.ssd_scan(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], perm,
                                 record_after=[c * Q for c in range(nc)])
    _, _, recb = oracle.ssd_scan(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], perm[::-1],
                                 record_after=[L - (c + 1) * Q for c in range(nc)])
    ef = rel_l2(to_np(hf)[0], np.stack([recf[c * Q] for c in range(nc)]))
    eb = rel_l2(to_np(hb)[0], np.stack([recb[L - (c + 1) * Q] for c in range(nc)]))
    say(f"  rel L2 fwd {ef:.3e} bwd {eb:.3e}")
    assert ef <= tol(s) and eb <= tol(s)
