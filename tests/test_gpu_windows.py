"""GPU parity of the TESA window variants through the C ABI against the fp64
oracle: explicit window-grid offsets (half windows and uneven ones), the
cyclic reading of a shifted partition (masked = 0), and the odd 3x3x3 window
of the TESA section (27 tokens, padded to 32 slots in the kernel), alone and
inside the whole mixer.  Bars as everywhere: relative L2 error of the output
at most 1e-5 with fp32 storage and 2e-2 with bf16 storage."""
import pytest

import oracle
from mate_inputs import CONFIGS, make_inputs
from gpu_util import need_gpu, say, upload, f64_all, rel_l2, to_np, tol

pytestmark = pytest.mark.gpu

ODD = CONFIGS[1].with_(T=12, H=12, W=12, win=(3, 3, 3))          # 64 windows, 27 chunks of 64
ODD_BIG = CONFIGS[1].with_(T=24, H=24, W=24, win=(3, 3, 3))      # 512 windows x 16 heads > one item per slot


def _te_case(s, cfg_id, shift, masked):
    torch, mate = need_gpu()
    inp = make_inputs(s, cfg_id, tensors=["q", "k", "v"])
    d = upload(inp, ("q", "k", "v"))
    say(f"te_fwd_shift {s.T}x{s.H}x{s.W} win{s.win} {s.dtype} shift{shift} masked{masked}")
    y = mate.lingen_te_fwd_shift(d["q"], d["k"], d["v"], shift, masked, s)
    torch.cuda.synchronize()
    f = f64_all(inp, ("q", "k", "v"))
    ref = oracle.tesa(f["q"], f["k"], f["v"], s.T, s.H, s.W, s.win, shift, cyclic=not masked)
    e = rel_l2(to_np(y).reshape(ref.shape), ref)
    say(f"  rel L2 {e:.3e}")
    assert e <= tol(s)


@pytest.mark.parametrize("shift,masked", [((1, 2, 2), 0), ((1, 3, 1), 1), ((1, 3, 1), 0), ((0, 0, 0), 0)])
def test_te_shift_fp32(shift, masked):
    _te_case(CONFIGS[0], 0, shift, masked)


@pytest.mark.parametrize("shift,masked", [((2, 4, 4), 0), ((1, 5, 3), 1), ((3, 1, 7), 0)])
def test_te_shift_bf16(shift, masked):
    _te_case(CONFIGS[1], 1, shift, masked)


@pytest.mark.parametrize("shift,masked", [((0, 0, 0), 1), ((1, 1, 1), 1), ((1, 1, 1), 0), ((2, 0, 1), 1)])
def test_te_odd_window(shift, masked):
    _te_case(ODD, 30, shift, masked)


@pytest.mark.parametrize("shift,masked", [((1, 1, 1), 1), ((1, 1, 1), 0)])
def test_te_odd_window_persistent(shift, masked):
    _te_case(ODD_BIG, 31, shift, masked)


@pytest.mark.parametrize("layer", range(4))
def test_mate_odd_window(layer):
    torch, mate = need_gpu()
    s = ODD
    inp = make_inputs(s, 32)
    d = upload(inp)
    say(f"mate_fwd {s.T}x{s.H}x{s.W} win{s.win} layer{layer}")
    y = mate.lingen_mate_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["q"], d["k"], d["v"], layer, s)
    torch.cuda.synchronize()
    f = f64_all(inp)
    ref = oracle.mate_fwd(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["q"], f["k"], f["v"], layer,
                          s.T, s.H, s.W, s.win)
    e = rel_l2(to_np(y).reshape(ref.shape), ref)
    say(f"  rel L2 {e:.3e}")
    assert e <= tol(s)


def test_te_shift_rejects_bad_offsets():
    torch, mate = need_gpu()
    s = CONFIGS[0]
    inp = make_inputs(s, 0, tensors=["q", "k", "v"])
    d = upload(inp, ("q", "k", "v"))
    say("te_fwd_shift argument checks")
    for shift, masked in (((2, 0, 0), 1), ((0, -1, 0), 1), ((0, 0, 4), 0), ((0, 0, 0), 2)):
        with pytest.raises(mate.LingenError):
            mate.lingen_te_fwd_shift(d["q"], d["k"], d["v"], shift, masked, s)
