"""GPU parity of the MA branch with a parameter set per scan direction
(lingen_ma_fwd_dirs) against the fp64 oracle's ssd_dirs: every scan order at
the fp32 workload, bf16 orders with one and two B, C groups, one set for both
directions (which is the shared-weight scan), review tokens (each direction
starting from the state its own review tokens leave), and one head of the
512p-like and of the 768p-like workload (with its 64 review tokens) over all
their tokens in the benchmark's launch configuration.  Bars: relative L2
error at most 1e-5 with fp32 storage and 2e-2 with bf16 storage, and every
(token, head) row within 1e-4 / 5e-2 of its norm."""
import numpy as np
import pytest

import oracle
from mate_inputs import CONFIGS, make_inputs
from gpu_util import need_gpu, say, upload, f64_all, head_f64, rel_l2, to_np, tol, check_rows, review_of

pytestmark = pytest.mark.gpu

SCAN = ("x", "dt", "A", "B", "C", "D")


def _sets(s, cfg_id, same=False):
    fi = make_inputs(s, cfg_id, seed=101, tensors=list(SCAN))
    bi = fi if same else make_inputs(s, cfg_id, seed=202, tensors=list(SCAN))
    return fi, bi


def _case(s, cfg_id, mode, same=False):
    torch, mate = need_gpu()
    fi, bi = _sets(s, cfg_id, same)
    df, db = upload(fi, SCAN), upload(bi, SCAN)
    say(f"ma_fwd_dirs {s.T}x{s.H}x{s.W} {s.dtype} groups={s.ngroups} review={s.n_review} mode{mode} same={same}")
    y = mate.lingen_ma_fwd_dirs(tuple(df[n] for n in SCAN), tuple(db[n] for n in SCAN), mode, s)
    torch.cuda.synchronize()
    ff, fb = f64_all(fi, SCAN), f64_all(bi, SCAN)
    perm = oracle.rms_scan_order(mode, s.T, s.H, s.W)
    ref = oracle.ssd_dirs(tuple(ff[n] for n in SCAN), tuple(fb[n] for n in SCAN), perm, review=review_of(s),
                          grid=(s.T, s.H, s.W))
    check_rows(to_np(y).reshape(ref.shape), ref, s.headdim, s)
    if s.n_review and s.dtype == "f32":
        # the review states reach the output far above the fp32 error
        plain = oracle.ssd_dirs(tuple(ff[n] for n in SCAN), tuple(fb[n] for n in SCAN), perm)
        assert rel_l2(plain, ref) > 100 * rel_l2(to_np(y).reshape(ref.shape), ref)
    return y


@pytest.mark.parametrize("mode", range(4))
def test_dirs_fp32(mode):
    _case(CONFIGS[0], 0, mode)


@pytest.mark.parametrize("mode,G", [(0, 1), (2, 1), (3, 2)])
def test_dirs_bf16(mode, G):
    _case(CONFIGS[1].with_(ngroups=G), 1, mode)


def test_dirs_same_set_is_shared_scan():
    torch, mate = need_gpu()
    s = CONFIGS[1]
    y = _case(s, 1, 1, same=True)
    fi, _ = _sets(s, 1, same=True)
    d = upload(fi, SCAN)
    y2 = mate.lingen_ma_fwd(*(d[n] for n in SCAN), 1, s)
    torch.cuda.synchronize()
    e = rel_l2(to_np(y), to_np(y2))
    say(f"  against lingen_ma_fwd: rel L2 {e:.3e}")
    assert e <= tol(s)


@pytest.mark.parametrize("mode", [1, 3])
def test_dirs_review_fp32(mode):
    _case(CONFIGS[0].with_(n_review=4, rpool=(2, 2, 2), rgrid=(1, 2, 2)), 0, mode)


@pytest.mark.parametrize("mode,G", [(0, 1), (2, 2)])
def test_dirs_review_bf16(mode, G):
    _case(CONFIGS[1].with_(ngroups=G, n_review=64, rpool=(2, 4, 4), rgrid=(4, 4, 4)), 1, mode)


def _one_head(cfg, head, mode):
    torch, mate = need_gpu()
    s = CONFIGS[cfg]
    fi = make_inputs(s, cfg, seed=101, tensors=list(SCAN), threads=16)
    bi = make_inputs(s, cfg, seed=202, tensors=list(SCAN), threads=16)
    df, db = upload(fi, SCAN), upload(bi, SCAN)
    say(f"ma_fwd_dirs cfg{cfg} ({s.L} tokens, review={s.n_review}) mode{mode}, head {head} over all tokens")
    y = mate.lingen_ma_fwd_dirs(tuple(df[n] for n in SCAN), tuple(db[n] for n in SCAN), mode, s)
    torch.cuda.synchronize()
    got = y[0, :, head * s.headdim:(head + 1) * s.headdim].double().cpu().numpy()
    del y, df, db
    torch.cuda.empty_cache()
    perm = oracle.rms_scan_order(mode, s.T, s.H, s.W)
    sets = []
    for inp in (fi, bi):
        hx = {n: head_f64(inp, n, head) for n in ("x", "dt", "A", "D")}
        sets.append((hx["x"], hx["dt"], hx["A"], inp.f64("B"), inp.f64("C"), hx["D"]))
    ref = oracle.ssd_dirs(sets[0], sets[1], perm, review=review_of(s), grid=(s.T, s.H, s.W))[:, 0, :]
    check_rows(got, ref, s.headdim, s, what=f"head {head}, all tokens")


def test_dirs_768p_review_one_head():
    _one_head(4, 17, 2)


def test_dirs_512p_one_head():
    _one_head(2, 9, 3)
