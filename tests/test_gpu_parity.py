"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs, at sizes the oracle finishes in seconds (configurations
0 and 1 and variants of them), plus robustness checks.

Bars: Rotary Major Scan index maps bit-exact; relative L2 error of y at most
1e-5 with fp32 storage and 2e-2 with bf16 storage (fp32 accumulation); for
the whole mixer also every (token, head) row of y within 1e-4 (fp32) or
5e-2 (bf16) of the oracle's row, relative to the row's norm."""
import numpy as np
import pytest

import oracle
from mate_inputs import CONFIGS, make_inputs
from gpu_util import need_gpu, say, upload, f64_all, rel_l2, to_np, tol, review_of, check_rows

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------------------
# Rotary Major Scan maps and gather
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", range(len(CONFIGS)))
def test_rms_index_device_bitexact(cfg):
    torch, mate = need_gpu()
    s = CONFIGS[cfg]
    for mode in range(4):
        say(f"rms_index_device cfg{cfg} mode{mode}")
        got = mate.lingen_rms_index_device(mode, s.T, s.H, s.W).cpu().numpy()
        np.testing.assert_array_equal(got, oracle.rms_scan_order(mode, s.T, s.H, s.W).astype(np.int32))


@pytest.mark.parametrize("mode", range(4))
def test_rms_gather_bitexact(mode):
    torch, mate = need_gpu()
    s = CONFIGS[1]
    inp = make_inputs(s, 1, tensors=["x"])
    x = inp.torch("x")
    say(f"rms_gather cfg1 mode{mode}")
    got = mate.lingen_rms_gather(x, mode, s.T, s.H, s.W)
    perm = torch.from_numpy(oracle.rms_scan_order(mode, s.T, s.H, s.W)).cuda()
    assert torch.equal(got.view(torch.int16), x[perm].view(torch.int16))


# --------------------------------------------------------------------------
# Chunk-boundary states (phase A + state pass)
# --------------------------------------------------------------------------

def _state_case(cfg_shape, cfg_id, mode):
    torch, mate = need_gpu()
    s = cfg_shape
    inp = make_inputs(s, cfg_id)
    d = upload(inp)
    say(f"ssd_chunk_states {s.T}x{s.H}x{s.W} {s.dtype} review={s.n_review} mode{mode}")
    hf, hb = mate.lingen_ssd_chunk_states(d["x"], d["dt"], d["A"], d["B"], mode, s)
    torch.cuda.synchronize()
    f = f64_all(inp)
    L, Q = s.L, s.chunk
    nc = L // Q
    perm = oracle.rms_scan_order(mode, s.T, s.H, s.W)
    h0 = None
    if s.n_review:
        h0 = oracle.review_state(f["x"], f["dt"], f["A"], f["B"], f["C"], s.T, s.H, s.W, s.rpool, s.rgrid)
    _, _, recf = oracle.ssd_scan(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], perm, h0=h0,
                                 record_after=[c * Q for c in range(nc)])
    _, _, recb = oracle.ssd_scan(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], perm[::-1], h0=h0,
                                 record_after=[L - (c + 1) * Q for c in range(nc)])
    ref_f = np.stack([recf[c * Q] for c in range(nc)])
    ref_b = np.stack([recb[L - (c + 1) * Q] for c in range(nc)])
    ef = rel_l2(to_np(hf)[0], ref_f)
    eb = rel_l2(to_np(hb)[0], ref_b)
    say(f"  rel L2 fwd {ef:.3e} bwd {eb:.3e}")
    bound = tol(s)
    assert ef <= bound and eb <= bound


@pytest.mark.parametrize("mode", range(4))
def test_chunk_states_cfg0(mode):
    _state_case(CONFIGS[0], 0, mode)


@pytest.mark.parametrize("mode", [0, 3])
def test_chunk_states_cfg1(mode):
    _state_case(CONFIGS[1], 1, mode)


def test_chunk_states_review_small():
    _state_case(CONFIGS[1].with_(n_review=64, rpool=(2, 4, 4), rgrid=(4, 4, 4)), 11, 2)


# --------------------------------------------------------------------------
# Branches separately, every (mode, shift) combination
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [0, 1])
@pytest.mark.parametrize("mode", range(4))
def test_ma_branch(cfg, mode):
    torch, mate = need_gpu()
    s = CONFIGS[cfg]
    inp = make_inputs(s, cfg)
    d = upload(inp)
    say(f"ma_fwd cfg{cfg} mode{mode}")
    y = mate.lingen_ma_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], mode, s)
    torch.cuda.synchronize()
    f = f64_all(inp)
    ref = oracle.ma_fwd(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], mode, s.T, s.H, s.W)
    e = rel_l2(to_np(y).reshape(ref.shape), ref)
    say(f"  rel L2 {e:.3e}")
    assert e <= tol(s)


@pytest.mark.parametrize("cfg", [0, 1])
@pytest.mark.parametrize("shifted", [0, 1])
def test_te_branch(cfg, shifted):
    torch, mate = need_gpu()
    s = CONFIGS[cfg]
    inp = make_inputs(s, cfg, tensors=["q", "k", "v"])
    d = upload(inp, ("q", "k", "v"))
    say(f"te_fwd cfg{cfg} shifted{shifted}")
    y = mate.lingen_te_fwd(d["q"], d["k"], d["v"], shifted, s)
    torch.cuda.synchronize()
    f = f64_all(inp, ("q", "k", "v"))
    shift = tuple(w // 2 for w in s.win) if shifted else (0, 0, 0)
    ref = oracle.tesa(f["q"], f["k"], f["v"], s.T, s.H, s.W, s.win, shift)
    e = rel_l2(to_np(y).reshape(ref.shape), ref)
    say(f"  rel L2 {e:.3e}")
    assert e <= tol(s)


# --------------------------------------------------------------------------
# The whole mixer
# --------------------------------------------------------------------------

def _mate_case(s, cfg_id, layer, inp=None):
    torch, mate = need_gpu()
    inp = inp or make_inputs(s, cfg_id)
    d = upload(inp)
    say(f"mate_fwd {s.T}x{s.H}x{s.W} {s.dtype} heads={s.ssd_heads} review={s.n_review} layer{layer}")
    y = mate.lingen_mate_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["q"], d["k"], d["v"], layer, s)
    torch.cuda.synchronize()
    f = f64_all(inp)
    ref = oracle.mate_fwd(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["q"], f["k"], f["v"], layer,
                          s.T, s.H, s.W, s.win, review=review_of(s))
    check_rows(to_np(y).reshape(ref.shape), ref, s.headdim, s)
    return y


@pytest.mark.parametrize("layer", range(4))
def test_mate_cfg0(layer):
    _mate_case(CONFIGS[0], 0, layer)


@pytest.mark.parametrize("layer", range(4))
def test_mate_cfg1(layer):
    _mate_case(CONFIGS[1], 1, layer)


@pytest.mark.parametrize("layer", [1, 2])
def test_mate_review_small(layer):
    _mate_case(CONFIGS[1].with_(n_review=64, rpool=(2, 4, 4), rgrid=(4, 4, 4)), 11, layer)


@pytest.mark.parametrize("layer", range(4))
def test_mate_ragged_grid_fp32(layer):
    # distinct T, H, W; 36 chunk workgroups (not a multiple of the XCD count);
    # shifted layers cut 3 border pieces per axis
    _mate_case(CONFIGS[0].with_(T=6, H=4, W=12), 20, layer)


@pytest.mark.parametrize("layer", [0, 1])
def test_mate_single_window_is_full_attention(layer):
    # one window covers the whole 2x4x4 grid on even layers
    _mate_case(CONFIGS[0].with_(T=2, H=4, W=4), 21, layer)


@pytest.mark.parametrize("layer", range(4))
def test_mate_single_frame(layer):
    # T = 1: the temporal scan orders degenerate to spatial ones
    _mate_case(CONFIGS[0].with_(T=1, H=8, W=8, win=(1, 4, 8)), 22, layer)


@pytest.mark.parametrize("heads,layer", [(3, 1), (5, 2)])
def test_mate_odd_head_groups_fp32(heads, layer):
    # 3 and 5 heads: chunk workgroups take all heads at once (an odd group)
    _mate_case(CONFIGS[0].with_(ssd_heads=heads, attn_heads=heads), 23, layer)


@pytest.mark.parametrize("heads,layer", [(10, 3), (12, 0)])
def test_mate_other_head_groups_bf16(heads, layer):
    # 10 heads: groups of 10 (output) and 5 (states); 12 heads: 12 and 6
    _mate_case(CONFIGS[1].with_(ssd_heads=heads, attn_heads=heads), 24, layer)


@pytest.mark.parametrize("A_value", [0.0, -1.0e4])
def test_mate_decay_extremes(A_value):
    # A = 0: no decay at all (plain cumulative sums); A = -1e4: every decay
    # underflows to zero inside one step
    s = CONFIGS[0]
    inp = make_inputs(s, 0)
    inp.store["A"][:] = np.float32(A_value)
    _mate_case(s, 0, 3, inp=inp)


# The kernel family of the large workloads (bf16, P 64, N 128, chunk 128,
# 4x8x8 windows) on a grid the oracle finishes in seconds: 8x16x16 tokens,
# 16 chunks per head, 8 windows, every layer phase.
_C2_SMALL = CONFIGS[2].with_(T=8, H=16, W=16)


@pytest.mark.parametrize("A_value", [0.0, -1.0e4])
@pytest.mark.parametrize("layer", [0, 3])
def test_mate_decay_extremes_bf16_large_family(A_value, layer):
    inp = make_inputs(_C2_SMALL, 25)
    inp.store["A"][:] = np.float32(A_value)
    _mate_case(_C2_SMALL, 25, layer, inp=inp)


@pytest.mark.parametrize("layer", range(4))
def test_mate_bf16_large_family_small_grid(layer):
    _mate_case(_C2_SMALL, 26, layer)


def test_batch_of_two_matches_single():
    torch, mate = need_gpu()
    for cfg in (0, 1):
        s1 = CONFIGS[cfg]
        s2 = s1.with_(batch=2)
        a = make_inputs(s1, cfg, seed=1)
        b = make_inputs(s1, cfg, seed=2)
        da, db = upload(a), upload(b)
        cat = {n: (torch.stack([da[n], db[n]]) if n not in ("A", "D") else da[n]) for n in da}
        say(f"batch=2 cfg{cfg}")
        y2 = mate.lingen_mate_fwd(*(cat[n] for n in ("x", "dt", "A", "B", "C", "D", "q", "k", "v")), 1, s2)
        # the per-head A and D of batch element b must equal those of a
        db["A"], db["D"] = da["A"], da["D"]
        ya = mate.lingen_mate_fwd(*(da[n] for n in ("x", "dt", "A", "B", "C", "D", "q", "k", "v")), 1, s1)
        yb = mate.lingen_mate_fwd(*(db[n] for n in ("x", "dt", "A", "B", "C", "D", "q", "k", "v")), 1, s1)
        torch.cuda.synchronize()
        assert torch.equal(y2[0], ya[0]) and torch.equal(y2[1], yb[0])


# --------------------------------------------------------------------------
# Robustness
# --------------------------------------------------------------------------

def test_repeatable_nan_workspace_and_canary():
    torch, mate = need_gpu()
    s = CONFIGS[1]
    inp = make_inputs(s, 1)
    d = upload(inp)
    args = [d[n] for n in ("x", "dt", "A", "B", "C", "D", "q", "k", "v")]
    say("robustness cfg1 layer3")
    y1 = mate.lingen_mate_fwd(*args, 3, s)
    ws = torch.full((mate.lingen_mate_workspace_bytes(s) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    n = s.L * s.d_inner
    big = torch.full((n + 4096,), 1.2345, dtype=torch.bfloat16, device="cuda")
    big[:n] = float("nan")
    out = big[:n].view(1, s.L, s.d_inner)
    y2 = mate.lingen_mate_fwd(*args, 3, s, out=out, workspace=ws.view(torch.uint8))
    y3 = mate.lingen_mate_fwd(*args, 3, s)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))
    assert bool(torch.all(big[n:] == torch.tensor(1.2345, dtype=torch.bfloat16, device="cuda")))
    assert not bool(torch.isnan(y1.float()).any())


def test_debug_sync_mode_same_results():
    # LINGEN_DEBUG=1 (sync and check after every launch), in a child process
    # since the variable is read once per process: the mixer's results are
    # unchanged and every launch reports success
    import os
    import subprocess
    import sys

    need_gpu()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import torch, numpy as np, oracle, linear_complexity_video_mate_amd as mate\n"
        "from mate_inputs import CONFIGS, make_inputs\n"
        "s = CONFIGS[0].with_(n_review=4, rpool=(2, 2, 2), rgrid=(1, 2, 2)); inp = make_inputs(s, 0)\n"
        "d = [inp.torch(n, 'cuda') for n in ('x', 'dt', 'A', 'B', 'C', 'D', 'q', 'k', 'v')]\n"
        "f = [inp.f64(n) for n in ('x', 'dt', 'A', 'B', 'C', 'D', 'q', 'k', 'v')]\n"
        "for layer in range(4):\n"
        "    y = mate.lingen_mate_fwd(*d, layer, s).double().cpu().numpy().reshape(s.L, -1)\n"
        "    ref = oracle.mate_fwd(*f, layer, s.T, s.H, s.W, s.win, review=(s.rpool, s.rgrid))\n"
        "    e = np.linalg.norm(y - ref) / np.linalg.norm(ref)\n"
        "    print(layer, e, flush=True)\n"
        "    assert e <= 1e-5\n"
    ) % root
    say("LINGEN_DEBUG=1 child process: tiny fp32 mixer with review tokens, layers 0-3")
    r = subprocess.run([sys.executable, "-c", code], env=dict(os.environ, LINGEN_DEBUG="1"), capture_output=True,
                       text=True, timeout=180)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stderr[-3000:]
    assert "lingen:" not in r.stderr


def test_rejects_bad_tensors():
    torch, mate = need_gpu()
    s = CONFIGS[0]
    inp = make_inputs(s, 0)
    d = upload(inp)
    args = [d[n] for n in ("x", "dt", "A", "B", "C", "D", "q", "k", "v")]
    bad = list(args)
    bad[0] = args[0].to(torch.bfloat16)
    with pytest.raises(TypeError):
        mate.lingen_mate_fwd(*bad, 0, s)
    with pytest.raises(mate.LingenError):
        mate.lingen_mate_fwd(*args, 0, s, workspace=torch.empty(64, dtype=torch.uint8, device="cuda"))
