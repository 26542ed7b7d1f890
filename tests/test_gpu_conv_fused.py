"""GPU parity of the fused per-direction scan, lingen_ma_fwd_dirs_conv: the
scan-order convolution, SiLU and dt softplus taken inside the scan kernels
instead of a pass of their own.

Two bars.  Against the two-call path on the same inputs (lingen_ma_prep,
then lingen_ma_fwd_dirs): bit-identical, since both form every value with
the same operations in the same order (taps padded with leading zero
weights add exact zeros).  Against the oracle's chain (oracle.ma_prep, then
oracle.ssd_dirs, in fp64): the whole-tensor and per-row bounds of the mixer
tests for bf16 storage.

Cases span both bf16 families (P64/N64/Q64 at the 16x32x32 grid, P64/N128/
Q128 at a 4x16x16 grid of the 512p-like dimensions and at the full 512p-like
and minute-length grids), every scan order, 1 to 4 taps, one and two B/C
groups and a batch of two (chunk halos must not cross batch elements or the
start of the sequence)."""
import numpy as np
import pytest

import oracle
from mate_inputs import CONFIGS, make_block_inputs, make_inputs
from gpu_util import need_gpu, say, to_np, check_rows

pytestmark = pytest.mark.gpu

PREP_IN = ("xbc", "dt_raw", "conv_w_f", "conv_b_f", "conv_w_b", "conv_b_b", "dt_bias")


def _inputs(torch, s, cfg_id, K, seed, batch):
    """Block inputs for `batch` elements (a seed each; the weights of the
    first), plus A and D per direction, on the GPU."""
    per = [make_block_inputs(s.with_(batch=1), cfg_id, seed=seed + b, conv_k=K, tensors=PREP_IN)
           for b in range(batch)]
    d = {n: per[0].torch(n, "cuda") for n in PREP_IN}
    d["xbc"] = torch.stack([p.torch("xbc", "cuda") for p in per])
    d["dt_raw"] = torch.stack([p.torch("dt_raw", "cuda") for p in per])
    ad_f = make_inputs(s.with_(batch=1), cfg_id, seed=101, tensors=["A", "D"])
    ad_b = make_inputs(s.with_(batch=1), cfg_id, seed=202, tensors=["A", "D"])
    for tag, ad in (("f", ad_f), ("b", ad_b)):
        d["A_" + tag], d["D_" + tag] = ad.torch("A", "cuda"), ad.torch("D", "cuda")
    return per, d, ad_f, ad_b


def _fused(mate, s, d, mode):
    return mate.lingen_ma_fwd_dirs_conv(d["xbc"], d["dt_raw"], (d["conv_w_f"], d["conv_b_f"]),
                                        (d["conv_w_b"], d["conv_b_b"]), d["dt_bias"], d["A_f"], d["D_f"],
                                        d["A_b"], d["D_b"], mode, s)


def _two_calls(mate, s, d, mode):
    xf, Bf, Cf, xb, Bb, Cb, dt = mate.lingen_ma_prep(d["xbc"], d["dt_raw"], (d["conv_w_f"], d["conv_b_f"]),
                                                     (d["conv_w_b"], d["conv_b_b"]), d["dt_bias"], mode, s)
    return mate.lingen_ma_fwd_dirs((xf, dt, d["A_f"], Bf, Cf, d["D_f"]), (xb, dt, d["A_b"], Bb, Cb, d["D_b"]),
                                   mode, s)


SMALL_C2 = dict(T=4, H=16, W=16)   # 1024 tokens: 8 chunks of the 512p-like family

BIT_CASES = [
    # cfg_id, grid override, mode, K, G, batch
    (1, None, 0, 4, 1, 1), (1, None, 1, 3, 1, 2), (1, None, 2, 2, 2, 1), (1, None, 3, 1, 1, 1),
    (2, SMALL_C2, 0, 4, 1, 2), (2, SMALL_C2, 1, 1, 2, 1), (2, SMALL_C2, 2, 4, 1, 1), (2, SMALL_C2, 3, 3, 2, 2),
]


@pytest.mark.parametrize("cfg_id,grid,mode,K,G,batch", BIT_CASES)
def test_fused_equals_two_calls(cfg_id, grid, mode, K, G, batch):
    torch, mate = need_gpu()
    s = CONFIGS[cfg_id].with_(ngroups=G, batch=batch, **(grid or {}))
    say(f"ma_fwd_dirs_conv {s.T}x{s.H}x{s.W} P{s.headdim} N{s.d_state} mode{mode} K={K} G={G} batch={batch}")
    _, d, _, _ = _inputs(torch, s, cfg_id, K, 808, batch)
    got = _fused(mate, s, d, mode)
    ref = _two_calls(mate, s, d, mode)
    torch.cuda.synchronize()
    diff = int((got.view(torch.int16) != ref.view(torch.int16)).sum())
    say(f"  elements differing from the two-call path: {diff} of {got.numel()}")
    assert diff == 0


ORACLE_CASES = [(1, None, 1, 4, 1), (1, None, 2, 2, 2), (2, SMALL_C2, 3, 4, 1), (2, SMALL_C2, 0, 3, 2)]


@pytest.mark.parametrize("cfg_id,grid,mode,K,G", ORACLE_CASES)
def test_fused_vs_oracle(cfg_id, grid, mode, K, G):
    torch, mate = need_gpu()
    s = CONFIGS[cfg_id].with_(ngroups=G, **(grid or {}))
    say(f"ma_fwd_dirs_conv vs oracle {s.T}x{s.H}x{s.W} P{s.headdim} N{s.d_state} mode{mode} K={K} G={G}")
    per, d, ad_f, ad_b = _inputs(torch, s, cfg_id, K, 909, 1)
    got = to_np(_fused(mate, s, d, mode)[0])
    torch.cuda.synchronize()
    f = {n: per[0].f64(n) for n in PREP_IN}
    order = oracle.rms_scan_order(mode, s.T, s.H, s.W)
    x_f, B_f, C_f, x_b, B_b, C_b, dt = oracle.ma_prep(f["xbc"], f["dt_raw"], f["conv_w_f"], f["conv_b_f"],
                                                      f["conv_w_b"], f["conv_b_b"], f["dt_bias"], order,
                                                      s.ssd_heads, s.headdim, s.ngroups, s.d_state)
    ref = oracle.ssd_dirs((x_f, dt, ad_f.f64("A"), B_f, C_f, ad_f.f64("D")),
                          (x_b, dt, ad_b.f64("A"), B_b, C_b, ad_b.f64("D")), order)
    check_rows(got.reshape(ref.shape), ref, s.headdim, s)


@pytest.mark.parametrize("cfg_id,modes", [(2, (0, 3)), (3, (1, 2))])
def test_fused_equals_two_calls_fullsize(cfg_id, modes):
    """The 512p-like and minute-length grids in the launch configuration of
    the block: bit-identical to the two-call path over every output."""
    torch, mate = need_gpu()
    s = CONFIGS[cfg_id]
    _, d, _, _ = _inputs(torch, s, cfg_id, 4, 1001, 1)
    for mode in modes:
        say(f"ma_fwd_dirs_conv {s.T}x{s.H}x{s.W} mode{mode}, all {s.L} tokens")
        got = _fused(mate, s, d, mode)
        ref = _two_calls(mate, s, d, mode)
        torch.cuda.synchronize()
        diff = int((got.view(torch.int16) != ref.view(torch.int16)).sum())
        say(f"  elements differing: {diff} of {got.numel()}")
        assert diff == 0
        del got, ref


def test_fused_unsupported_forms():
    """fp32 storage and review tokens are refused (they take the two calls)."""
    torch, mate = need_gpu()
    for cfg_id, s in ((0, CONFIGS[0]),
                      (1, CONFIGS[1].with_(n_review=64, rpool=(2, 4, 4), rgrid=(4, 4, 4)))):
        say(f"ma_fwd_dirs_conv refuses {s.dtype} storage, review={s.n_review}")
        _, d, _, _ = _inputs(torch, s, cfg_id, 4, 1111, 1)
        with pytest.raises(mate.LingenError) as e:
            _fused(mate, s, d, 0)
        assert "UNSUPPORTED" in str(e.value)
