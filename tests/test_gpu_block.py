"""GPU parity of the steps around the scan against the fp64 oracle:
lingen_ma_prep (scan-order causal convolution + SiLU in both directions,
softplus dt) against oracle.ma_prep, lingen_gated_rmsnorm against
oracle.gated_rmsnorm, and the chain prep -> lingen_ma_fwd_dirs -> gated norm
against the oracle's chain.

Bars.  fp32 storage: relative L2 error at most 1e-5, and for the elementwise
outputs every element within 1e-5 |ref| + 1e-6.  bf16 storage: every element
within 2^-8 |ref| + 1e-5 (the result rounded once to bf16 after fp32
arithmetic: half a bf16 ulp, 2^-9 |ref|, plus the fp32 arithmetic's error),
relative L2 at most 2e-2 for the chain through the scan.  dt (fp32 in both
storages) within 1e-6 relative."""
import numpy as np
import pytest

import oracle
from mate_inputs import CONFIGS, make_block_inputs
from gpu_util import need_gpu, say, rel_l2, to_np

pytestmark = pytest.mark.gpu

PREP_IN = ("xbc", "dt_raw", "conv_w_f", "conv_b_f", "conv_w_b", "conv_b_b", "dt_bias")


def _elementwise_ok(got, ref, bf16: bool, what: str):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bound = (2.0 ** -8 * np.abs(ref) + 1e-5) if bf16 else (1e-5 * np.abs(ref) + 1e-6)
    err = np.abs(got - ref)
    worst = float(np.max(err - bound)) if err.size else -1.0
    say(f"  {what}: max |err| {float(err.max()) if err.size else 0.0:.3e}, rel L2 {rel_l2(got, ref):.3e}")
    assert worst <= 0.0, what
    if not bf16:
        assert rel_l2(got, ref) <= 1e-5, what


def _upload(inp, names):
    return {n: inp.torch(n, "cuda") for n in names}


def _run_prep(mate, s, d, mode):
    return mate.lingen_ma_prep(d["xbc"], d["dt_raw"], (d["conv_w_f"], d["conv_b_f"]), (d["conv_w_b"], d["conv_b_b"]),
                               d["dt_bias"], mode, s)


def _prep_ref(inp, s, mode):
    f = {n: inp.f64(n) for n in PREP_IN}
    order = oracle.rms_scan_order(mode, s.T, s.H, s.W)
    return oracle.ma_prep(f["xbc"], f["dt_raw"], f["conv_w_f"], f["conv_b_f"], f["conv_w_b"], f["conv_b_b"],
                          f["dt_bias"], order, s.ssd_heads, s.headdim, s.ngroups, s.d_state)


PREP_CASES = [(0, 0, 4, 1), (0, 1, 4, 1), (0, 2, 3, 1), (0, 3, 1, 1),
              (1, 0, 4, 1), (1, 1, 2, 2), (1, 2, 4, 1), (1, 3, 4, 2)]


@pytest.mark.parametrize("cfg_id,mode,K,G", PREP_CASES)
def test_prep_parity(cfg_id, mode, K, G):
    torch, mate = need_gpu()
    s = CONFIGS[cfg_id].with_(ngroups=G)
    inp = make_block_inputs(s, cfg_id, seed=303, conv_k=K)
    say(f"ma_prep {s.T}x{s.H}x{s.W} {s.dtype} mode{mode} K={K} groups={G}")
    outs = _run_prep(mate, s, _upload(inp, PREP_IN), mode)
    torch.cuda.synchronize()
    ref = _prep_ref(inp, s, mode)
    bf16 = s.dtype == "bf16"
    for name, g, r in zip(("x_f", "B_f", "C_f", "x_b", "B_b", "C_b"), outs[:6], ref[:6]):
        _elementwise_ok(to_np(g)[0].reshape(r.shape), r, bf16, name)
    dt = to_np(outs[6])[0]
    np.testing.assert_allclose(dt, ref[6], rtol=1e-6, atol=0)


def _sampled_positions(L, n, rng):
    edge = [0, 1, 2, 3, 4, L // 2, L - 5, L - 4, L - 3, L - 2, L - 1]
    return sorted(set(edge) | set(rng.choice(L, n, replace=False).tolist()))


def test_prep_512p_sampled_positions():
    """The 512p-like workload (32x64x64 tokens, 2304 channels) in the
    launch configuration of the full-size run; the oracle computes sampled
    scan positions one by one from the K rows each output depends on."""
    torch, mate = need_gpu()
    s, cfg_id, K = CONFIGS[2], 2, 4
    inp = make_block_inputs(s, cfg_id, seed=404, conv_k=K, tensors=PREP_IN)
    rng = np.random.default_rng(5)
    xbc = inp.f32("xbc")
    wf, bf, wb, bb = (inp.f64(n) for n in ("conv_w_f", "conv_b_f", "conv_w_b", "conv_b_b"))
    L = s.L
    d = _upload(inp, PREP_IN)
    for mode in (1, 3):
        say(f"ma_prep 512p-like mode{mode}, sampled scan positions")
        outs = _run_prep(mate, s, d, mode)
        torch.cuda.synchronize()
        order = oracle.rms_scan_order(mode, s.T, s.H, s.W)
        pos = _sampled_positions(L, 48, rng)
        toks = torch.as_tensor(order[pos], dtype=torch.long, device="cuda")
        got_f = np.concatenate([to_np(t[0][toks].reshape(len(pos), -1)) for t in outs[0:3]], axis=1)
        got_b = np.concatenate([to_np(t[0][toks].reshape(len(pos), -1)) for t in outs[3:6]], axis=1)
        del outs
        for i, p in enumerate(pos):
            # forward: the rows at scan positions p-K+1 .. p, scanned in order
            taps = [q for q in range(p - K + 1, p + 1) if q >= 0]
            u = xbc[order[taps]].astype(np.float64)
            ref = oracle.scan_conv_silu(u, wf, bf, np.arange(len(taps)))[-1]
            _elementwise_ok(got_f[i], ref, True, f"forward p={p}")
            # backward: positions p+K-1 .. p visited in reversed order
            taps = [q for q in range(p + K - 1, p - 1, -1) if q < L]
            u = xbc[order[taps]].astype(np.float64)
            ref = oracle.scan_conv_silu(u, wb, bb, np.arange(len(taps)))[-1]
            _elementwise_ok(got_b[i], ref, True, f"backward p={p}")


NORM_CASES = [("f32", 64, 96, 32), ("f32", 33, 4096, 4096), ("f32", 7, 256, 4),
              ("bf16", 64, 2048, 2048), ("bf16", 64, 2048, 256), ("bf16", 5, 8192, 8192),
              ("bf16", 9, 1024, 8), ("bf16", 1, 72, 24)]


@pytest.mark.parametrize("dtype,rows,dim,group", NORM_CASES)
def test_gated_rmsnorm_parity(dtype, rows, dim, group):
    torch, mate = need_gpu()
    Hs = dim // 64 if dim % 64 == 0 else 1
    s = CONFIGS[0 if dtype == "f32" else 1].with_(ssd_heads=Hs, headdim=dim // Hs, T=1, H=1, W=max(rows, 1))
    inp = make_block_inputs(s, 7, seed=505, rows=rows, tensors=("y", "z", "norm_w"))
    say(f"gated_rmsnorm {dtype} rows={rows} dim={dim} group={group}")
    y, z, w = inp.torch("y", "cuda"), inp.torch("z", "cuda"), inp.torch("norm_w", "cuda")
    out = mate.lingen_gated_rmsnorm(y, z, w, 1e-5, group)
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(inp.f64("y"), inp.f64("z"), inp.f64("norm_w"), 1e-5, group)
    _elementwise_ok(to_np(out), ref, dtype == "bf16", "out")


def test_gated_rmsnorm_512p_rows():
    """All 131,072 rows of the 512p-like workload (2048 channels, one group),
    sampled rows checked against the oracle; every row's RMS of g / w equals
    one within rounding."""
    torch, mate = need_gpu()
    s = CONFIGS[2]
    inp = make_block_inputs(s, 2, seed=606, tensors=("y", "z", "norm_w"))
    say("gated_rmsnorm 512p-like, 131072 rows x 2048")
    out = mate.lingen_gated_rmsnorm(inp.torch("y", "cuda"), inp.torch("z", "cuda"), inp.torch("norm_w", "cuda"),
                                    1e-5, 2048)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    rows = sorted(set([0, s.L - 1]) | set(rng.choice(s.L, 254, replace=False).tolist()))
    got = to_np(out[rows])
    ref = oracle.gated_rmsnorm(inp.f32("y")[rows].astype(np.float64), inp.f32("z")[rows].astype(np.float64),
                               inp.f64("norm_w"), 1e-5, 2048)
    _elementwise_ok(got, ref, True, "sampled rows")
    w = torch.from_numpy(inp.f32("norm_w")).cuda()
    rms = (out.float() / w).pow(2).mean(dim=1).sqrt()
    assert float((rms - 1).abs().max()) < 1e-2


def test_gated_rmsnorm_zero_rows():
    torch, mate = need_gpu()
    say("gated_rmsnorm with zero rows")
    y = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    out = mate.lingen_gated_rmsnorm(y, y.clone(), torch.ones(64, device="cuda"), 1e-5, 64)
    assert out.shape == (0, 64)


@pytest.mark.parametrize("cfg_id,mode", [(0, 2), (1, 1)])
def test_block_chain(cfg_id, mode):
    """prep -> per-direction scan -> gated norm against the oracle's chain.
    A and D per direction come from the scan inputs' recipe; z and the norm
    weight from the block recipe; one norm group per B, C group."""
    torch, mate = need_gpu()
    from mate_inputs import make_inputs

    s = CONFIGS[cfg_id]
    inp = make_block_inputs(s, cfg_id, seed=707)
    ad_f = make_inputs(s, cfg_id, seed=101, tensors=["A", "D"])
    ad_b = make_inputs(s, cfg_id, seed=202, tensors=["A", "D"])
    say(f"prep -> ma_fwd_dirs -> gated_rmsnorm {s.T}x{s.H}x{s.W} {s.dtype} mode{mode}")
    d = _upload(inp, PREP_IN + ("z", "norm_w"))
    xf, Bf, Cf, xb, Bb, Cb, dt = _run_prep(mate, s, d, mode)
    A_f, D_f = ad_f.torch("A", "cuda"), ad_f.torch("D", "cuda")
    A_b, D_b = ad_b.torch("A", "cuda"), ad_b.torch("D", "cuda")
    y = mate.lingen_ma_fwd_dirs((xf, dt, A_f, Bf, Cf, D_f), (xb, dt, A_b, Bb, Cb, D_b), mode, s)
    dim = s.ssd_heads * s.headdim
    group = dim // s.ngroups
    out = mate.lingen_gated_rmsnorm(y[0], d["z"], d["norm_w"], 1e-5, group)
    torch.cuda.synchronize()

    rx_f, rB_f, rC_f, rx_b, rB_b, rC_b, rdt = _prep_ref(inp, s, mode)
    perm = oracle.rms_scan_order(mode, s.T, s.H, s.W)
    yr = oracle.ssd_dirs((rx_f, rdt, ad_f.f64("A"), rB_f, rC_f, ad_f.f64("D")),
                         (rx_b, rdt, ad_b.f64("A"), rB_b, rC_b, ad_b.f64("D")), perm)
    ref = oracle.gated_rmsnorm(yr.reshape(s.L, dim), inp.f64("z"), inp.f64("norm_w"), 1e-5, group)
    e = rel_l2(to_np(out), ref)
    say(f"  rel L2 {e:.3e}")
    assert e <= (1e-5 if s.dtype == "f32" else 2e-2)
