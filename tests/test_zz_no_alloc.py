"""The no-allocation entry point (lingen_mate_fwd_noalloc) through the C ABI
against lingen_mate_fwd with a caller-provided workspace: the same kernels on
the same inputs, so the outputs must agree bit for bit.  Two calls in a row
share the device's scratch array, the second with a smaller input (and a
different layer phase), and a call with review tokens uses the array's
review buffers; each output is also within the parity bar of the fp64
oracle.  Shapes too large for the array are refused before any launch."""
import pytest

import oracle
from mate_inputs import CONFIGS, make_inputs
from gpu_util import need_gpu, say, upload, f64_all, to_np, review_of, check_rows


NAMES = ("x", "dt", "A", "B", "C", "D", "q", "k", "v")


def _pair(s, cfg_id, layer):
    torch, mate = need_gpu()
    inp = make_inputs(s, cfg_id)
    d = upload(inp)
    args = [d[n] for n in NAMES]
    say(f"noalloc mate_fwd {s.T}x{s.H}x{s.W} {s.dtype} review={s.n_review} layer{layer}")
    y_ref = mate.lingen_mate_fwd(*args, layer, s)
    y_na = torch.full_like(y_ref, float("nan"))
    mate.lingen_mate_fwd_noalloc(*args, layer, s, out=y_na)
    torch.cuda.synchronize()
    assert torch.equal(y_na.view(torch.int16 if y_na.dtype == torch.bfloat16 else torch.int32),
                       y_ref.view(torch.int16 if y_ref.dtype == torch.bfloat16 else torch.int32))
    f = f64_all(inp)
    ref = oracle.mate_fwd(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["q"], f["k"], f["v"], layer,
                          s.T, s.H, s.W, s.win, review=review_of(s))
    check_rows(to_np(y_na).reshape(ref.shape), ref, s.headdim, s)


@pytest.mark.gpu
def test_noalloc_two_calls_second_smaller():
    # 16,384 tokens (64 MiB of chunk states), then 4,096 tokens of the same
    # family: the second call reuses the array the first one filled
    _pair(CONFIGS[1], 1, 1)
    _pair(CONFIGS[1].with_(T=4), 31, 2)


@pytest.mark.gpu
def test_noalloc_review_then_fp32():
    _pair(CONFIGS[1].with_(n_review=64, rpool=(2, 4, 4), rgrid=(4, 4, 4)), 11, 3)
    _pair(CONFIGS[0], 0, 0)


def test_noalloc_rejects_too_large_before_launch():
    # host-side check only: no pointer is looked at and nothing is enqueued,
    # so this runs without a GPU
    import ctypes

    import linear_complexity_video_mate_amd as mate

    s = CONFIGS[2]            # 131,072 tokens: 1 GiB of chunk states
    assert mate.lingen_mate_workspace_bytes(s) > 256 << 20
    cs = mate.to_c_shape(s)
    rc = mate.lib().lingen_mate_fwd_noalloc(*([None] * 9), 0, ctypes.byref(cs), None, None)
    assert rc == -8 and mate.STATUS_NAMES[rc] == "LINGEN_ERR_SCRATCH"
    ok = CONFIGS[1]
    assert mate.lingen_mate_workspace_bytes(ok) <= 256 << 20
    bad = mate.to_c_shape(ok.with_(chunk=48))
    assert mate.lib().lingen_mate_fwd_noalloc(*([None] * 9), 0, ctypes.byref(bad), None, None) == -2
