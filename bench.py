"""Benchmark of the MATE mixer forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3] [--no-cpu-baseline]

One step = one lingen_mate_fwd call over the whole token tensor: both MA
stages (chunk states, inter-chunk state pass, chunk outputs), windowed
attention and the branch sum.  Step k uses layer index k mod 4, so the four
scan orders and both window phases are timed in equal measure.  Inputs are
the seeded synthetic tensors of the workload, resident in GPU memory before
timing starts.  The default workload is the minute-length grid
(128x64x64 = 524,288 tokens), the largest that is run on one GPU.

Prints one JSON line: whole-job tokens/s, per-stage times from HIP events
recorded on the launch stream (lingen_mate_fwd_events), the roofline of the
dominant kernel (its bound taken from its arithmetic intensity against the
MFMA/HBM ridge), the linear-scaling check (the same forward on the first
quarter of the frames, i.e. the 512p-like 32x64x64 grid, timed in the same
run), and the fp64 oracle timed on host cores over a bounded sample of the
same workload (a process pool, run before the GPU is initialised).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MATE fwd tokens/s (bidir SSD + TESA) at 1 GPU; % MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
STAGES = ("review", "ssd_chunk_state", "ssd_state_pass", "ssd_chunk_out", "tesa_window")
# Sources that define the mixer's kernels (a traffic record is valid only for them as they stand).
KERNEL_SRCS = [os.path.join(ROOT, "linear_complexity_video_mate_amd", "csrc", n)
               for n in ("lingen_kernels.hip", "lingen_device.h", "lingen_window.h", "tesa_window.hip")]


def kernel_source_sha256() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# ---------------------------------------------------------------------------
# HIP events through the HIP runtime's C API
# ---------------------------------------------------------------------------

class HipEvents:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self) -> int:
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.made.append(e.value)
        return e.value

    def record(self, e: int, stream: int) -> None:
        if self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def sync(self, e: int) -> None:
        self.hip.hipEventSynchronize(ctypes.c_void_p(e))

    def ms(self, a: int, b: int) -> float:
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))
        self.made = []


# ---------------------------------------------------------------------------
# Algorithmic work per kernel launch (each input read once, each output
# written once, by that kernel), for one batch element.
# ---------------------------------------------------------------------------

def kernel_work(s):
    e = s.elem_bytes
    L, Hs, P, N, Q = s.L, s.ssd_heads, s.headdim, s.d_state, s.chunk
    Ha, d, nw = s.attn_heads, s.attn_headdim, s.n_w
    nc = L // Q
    states = 2 * nc * Hs * P * N * e          # chunk states are stored in the input dtype
    G = s.ngroups
    x, y, bc, dt = L * Hs * P * e, L * Hs * P * e, L * G * N * e, L * Hs * 4
    qkv = 3 * L * Ha * d * e
    work = {
        "ssd_chunk_state": dict(bytes=x + dt + bc + states + nc * Hs * 4,
                                flops=2 * 2 * nc * Hs * Q * N * P),
        "ssd_state_pass": dict(bytes=2 * states + nc * Hs * 4, flops=2 * states // 4),
        # C.B^T once per chunk and group (shared by the group's heads), then per
        # head the masked in-chunk product and the two inter-chunk read-outs
        "ssd_chunk_out": dict(bytes=x + dt + 2 * bc + states + y,
                              flops=nc * G * 2 * Q * Q * N + nc * Hs * (2 * Q * Q * P + 2 * 2 * Q * N * P)),
        "tesa_window": dict(bytes=qkv + 2 * y, flops=4 * L * nw * d * Ha),
    }
    if s.n_review:
        R = s.n_review
        blk = s.rpool[0] * s.rpool[1] * s.rpool[2]
        work["review"] = dict(bytes=R * blk * (Hs * P * e + Hs * 4 + G * N * e), flops=2 * R * Hs * P * N)
    return work


def compulsory_bytes(s):
    e = s.elem_bytes
    L = s.L
    return L * (2 * s.ssd_heads * s.headdim * e + s.ssd_heads * 4 + 2 * s.ngroups * s.d_state * e
                + 3 * s.attn_heads * s.attn_headdim * e)


TRAFFIC_PATH = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def _traffic_records():
    if not os.path.exists(TRAFFIC_PATH):
        return {}
    try:
        return json.load(open(TRAFFIC_PATH))
    except (OSError, ValueError):
        return {}


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` measured with rocprofv3
    counters, if a committed measurement exists for that workload and the
    current kernel source; else None."""
    rec = _traffic_records().get("workloads", {}).get(workload)
    if not rec or rec.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle, as it stands, on a bounded sample, in a
# process pool over heads (heads are independent in both branches).  It runs
# before anything initialises the GPU, so the forked workers hold no device
# state; they read the inputs copy-on-write from this process.
# ---------------------------------------------------------------------------

_CPU_SHARED = {}
MAX_CPU_WORKERS = 16     # the host share of one GPU


def _head_f64(inp, name, h):
    import numpy as np

    from mate_inputs import f32_from_bf16_bits

    a = inp.store[name]
    sl = a[[h]] if name in ("A", "D") else a[:, [h]]
    return (f32_from_bf16_bits(sl) if sl.dtype == np.uint16 else sl).astype(np.float64)


def _cpu_task(task):
    """One head of one branch through the oracle, single-threaded; returns its
    wall time (the extraction of the head's inputs is not timed)."""
    from threadpoolctl import threadpool_limits

    import oracle

    kind, h = task
    s, inp = _CPU_SHARED["shape"], _CPU_SHARED["inp"]
    with threadpool_limits(limits=1):
        if kind == "ssd":
            hx = {n: _head_f64(inp, n, h) for n in ("x", "dt", "A", "D")}
            review = (s.rpool, s.rgrid) if s.n_review else None
            t0 = time.perf_counter()
            oracle.ma_fwd(hx["x"], hx["dt"], hx["A"], _CPU_SHARED["B"], _CPU_SHARED["C"], hx["D"], 0,
                          s.T, s.H, s.W, review=review)
        else:
            hx = {n: _head_f64(inp, n, h) for n in ("q", "k", "v")}
            t0 = time.perf_counter()
            oracle.tesa(hx["q"], hx["k"], hx["v"], s.T, s.H, s.W, s.win, (0, 0, 0))
        return time.perf_counter() - t0


def cpu_workers(requested: int = 0) -> int:
    avail = len(os.sched_getaffinity(0))
    n = requested if requested > 0 else min(MAX_CPU_WORKERS, avail)
    return max(1, min(n, avail))


def cpu_baseline(s, inp, workers):
    """Layer 0 (scan order 0, plain windows) of the workload through the fp64
    oracle: `workers` SSD heads at once over every token (both directions),
    then `workers` attention heads at once, one head per process.  The whole
    job's time is each batch's wall time scaled by heads / workers."""
    import multiprocessing as mp

    _CPU_SHARED.update(shape=s, inp=inp, B=inp.f64("B"), C=inp.f64("C"))
    ns, na = min(workers, s.ssd_heads), min(workers, s.attn_heads)
    with mp.get_context("fork").Pool(workers) as pool:
        t0 = time.perf_counter()
        per_ssd = pool.map(_cpu_task, [("ssd", h) for h in range(ns)], chunksize=1)
        w_ssd = time.perf_counter() - t0
        t0 = time.perf_counter()
        per_att = pool.map(_cpu_task, [("tesa", h) for h in range(na)], chunksize=1)
        w_att = time.perf_counter() - t0
    _CPU_SHARED.clear()
    est = w_ssd * s.ssd_heads / ns + w_att * s.attn_heads / na
    return {
        "value": s.L / est,
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"fp64 NumPy oracle, {workers} processes of one thread each, layer 0, over all {s.L} tokens: "
                   f"SSD heads 0-{ns - 1} at once (both directions) {w_ssd:.2f} s wall "
                   f"(per head {min(per_ssd):.2f}-{max(per_ssd):.2f} s), then attention heads 0-{na - 1} at "
                   f"once {w_att:.2f} s wall; scaled by {s.ssd_heads}/{ns} SSD and {s.attn_heads}/{na} "
                   f"attention heads"),
    }


# Kernel (mangled-name fragment) -> the stage name bench.py reports it under.
KERNEL_STAGE = (("tesa_win256_pair_kernel", "tesa_window"), ("tesa_win256_kernel", "tesa_window"),
                ("tesa_window_kernel", "tesa_window"),
                ("ssd_chunk_state_kernel", "ssd_chunk_state"), ("ssd_state_pass_kernel", "ssd_state_pass"),
                ("ssd_chunk_out_kernel", "ssd_chunk_out"), ("review_pool_kernel", "review"),
                ("review_state_kernel", "review"), ("rms_gather_kernel", "rms_gather"))


def _pmc_means(path):
    """Mean counter value per launch of each stage from a rocprofv3 counter
    CSV (the review stage's two kernels summed per launch)."""
    import csv
    acc = {}
    for r in csv.DictReader(open(path)):
        for frag, stage in KERNEL_STAGE:
            if frag in r["Kernel_Name"]:
                acc.setdefault(stage, {}).setdefault(frag, []).append(float(r["Counter_Value"]))
                break
    return {stage: sum(sum(v) / len(v) for v in per.values()) for stage, per in acc.items()}


def record_traffic(mix_fetch, mix_write, copy_fetch, copy_write, config=2):
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for the plain copy kernel,
    whose true traffic is known (--copy-gib 1: 1 GiB read, 1 GiB written)."""
    from mate_inputs import CONFIG_NOTES

    true_kib = 2 ** 20
    fcal = true_kib / _pmc_means(copy_fetch)["rms_gather"]
    wcal = true_kib / _pmc_means(copy_write)["rms_gather"]
    fetch, write = _pmc_means(mix_fetch), _pmc_means(mix_write)
    kernels = {}
    for name in sorted(set(fetch) & set(write)):
        rd, wr = fetch[name] * fcal * 1024, write[name] * wcal * 1024
        kernels[name] = {"read_bytes": round(rd), "write_bytes": round(wr), "bytes_per_launch": round(rd + wr)}
    rec = {
        "kernel_source_sha256": kernel_source_sha256(),
        "calibration": {"FETCH_SIZE_scale": round(fcal, 4), "WRITE_SIZE_scale": round(wcal, 4),
                        "copy": "bench.py --copy-gib 1 (1 GiB read + 1 GiB written per launch)"},
        "counters": "rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE, each its own run",
        "kernels": kernels,
    }
    allrec = _traffic_records()
    allrec.setdefault("workloads", {})[CONFIG_NOTES[config]] = rec
    with open(TRAFFIC_PATH, "w") as f:
        json.dump({"workloads": allrec["workloads"]}, f, indent=1)
    print(json.dumps({CONFIG_NOTES[config]: rec}))
    return 0


def copy_calibration(args, mate, torch):
    """Plain copy of rows of 4 KiB through lingen_rms_gather (mode 0 is the
    identity order): reads and writes exactly copy_gib GiB each per launch."""
    rows = int(args.copy_gib * 2 ** 30) // 4096
    T, H, W = rows // 4096, 64, 64
    src = torch.empty((T * H * W, 2048), dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    nbytes = src.numel() * 2
    for _ in range(args.warmup):
        mate.lingen_rms_gather(src, 0, T, H, W, out=dst)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        mate.lingen_rms_gather(src, 0, T, H, W, out=dst)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    assert torch.equal(dst.view(torch.int16), src.view(torch.int16))
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "ms": round(ms, 4),
                      "GB/s_read+write": round(2 * nbytes / ms / 1e6, 1)}), flush=True)
    return 0


def gather_modes(args, mate, torch):
    """The scan-order gather (lingen_rms_gather) on the workload's grid with
    rows of one token's x (Hs*P elements): reads and writes L rows per launch,
    in each of the four scan orders."""
    from mate_inputs import CONFIGS, CONFIG_NOTES

    s = CONFIGS[args.config]
    src = torch.empty((s.L, s.d_inner), dtype=torch.bfloat16 if s.dtype == "bf16" else torch.float32,
                      device="cuda").normal_()
    dst = torch.empty_like(src)
    nbytes = src.numel() * src.element_size()
    out = {"workload": CONFIG_NOTES[args.config], "row_bytes": s.d_inner * src.element_size(), "modes": {}}
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for mode in range(4):
        for _ in range(args.warmup):
            mate.lingen_rms_gather(src, mode, s.T, s.H, s.W, out=dst)
        torch.cuda.synchronize()
        a.record()
        for _ in range(args.steps):
            mate.lingen_rms_gather(src, mode, s.T, s.H, s.W, out=dst)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / args.steps
        perm, _ = mate.lingen_rms_index(mode, s.T, s.H, s.W)
        assert torch.equal(dst.view(-1, s.d_inner).view(torch.int16),
                           src[torch.from_numpy(perm).long().cuda()].view(torch.int16)), f"gather mode {mode}"
        out["modes"][mode] = {"ms": round(ms, 4), "GB/s_read+write": round(2 * nbytes / ms / 1e6, 1),
                              "hbm_frac": round(2 * nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
    print(json.dumps(out), flush=True)
    return 0


def library_attention(torch, qkv, steps, flops, timed):
    """Context for the dense kernel: torch's fused scaled_dot_product_attention
    on the same tensors, restricted to its flash / memory-efficient backends
    (never the unfused math path).  Returns its latency, or why it could not
    run."""
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel

    q, k, v = (t.transpose(1, 2).contiguous() for t in qkv)      # [batch, heads, L, d]
    for backend in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
        try:
            with sdpa_kernel([backend]):
                ms = timed(lambda i: F.scaled_dot_product_attention(q, k, v), steps, 1)
        except RuntimeError as err:
            last = f"{backend.name}: {str(err).splitlines()[0][:200]}"
            continue
        tflops = flops / (ms / 1e3) / 1e12
        return {"op": "torch.nn.functional.scaled_dot_product_attention", "backend": backend.name,
                "ms": round(ms, 3), "TFLOP/s": round(tflops, 1), "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4)}
    return {"op": "torch.nn.functional.scaled_dot_product_attention", "unavailable": last}


def te_backward(args, mate, torch):
    """The TE branch's backward pass (lingen_te_bwd) on the workload against
    its forward (lingen_te_fwd), both timed with events on the launch stream,
    plain and shifted windows alternating by step as in the mixer; and the
    saved-statistics pair (lingen_te_fwd_saved, then lingen_te_bwd_saved
    reading that forward's output and log2 softmax denominators, one saved
    set per window offset)."""
    from mate_inputs import CONFIGS, CONFIG_NOTES, make_inputs

    s = CONFIGS[args.config]
    inp = make_inputs(s, args.config, tensors=["q", "k", "v"], threads=16)
    q, k, v = (inp.torch(n, "cuda") for n in ("q", "k", "v"))
    g = torch.empty_like(q).normal_()
    dq, dk, dv, y = (torch.empty_like(q) for _ in range(4))
    half = tuple(w // 2 for w in s.win)

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(args.steps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    bwd_ms = timed(lambda i: mate.lingen_te_bwd(q, k, v, g, half if i % 2 else (0, 0, 0), 1, s, dq=dq, dk=dk, dv=dv))
    fwd_ms = timed(lambda i: mate.lingen_te_fwd(q, k, v, i % 2, s, out=y))
    saved = [mate.lingen_te_fwd_saved(q, k, v, sh, 1, s) for sh in ((0, 0, 0), half)]
    fwd_saved_ms = timed(lambda i: mate.lingen_te_fwd_saved(q, k, v, half if i % 2 else (0, 0, 0), 1, s, out=y,
                                                            lse=saved[0][1]))
    bwd_saved_ms = timed(lambda i: mate.lingen_te_bwd_saved(q, k, v, saved[i % 2][0], g, saved[i % 2][1],
                                                            half if i % 2 else (0, 0, 0), 1, s, dq=dq, dk=dk, dv=dv))
    e = s.elem_bytes
    rows = s.L * s.attn_heads * s.attn_headdim
    nbytes = 7 * rows * e                                # q, k, v, dO read; dq, dk, dv written
    flops = 10 * s.n_w * rows                            # S, dP, dq, dk, dv: five products of 2 n_w d
    issued = 29 * s.n_w * rows // 2                      # S twice, o, dP, dq, dk, dv; row sums on a 16-wide ones operand
    out = {
        "kernel": "tesa_bwd", "workload": CONFIG_NOTES[args.config], "steps": args.steps,
        "bwd_ms": round(bwd_ms, 4), "fwd_ms": round(fwd_ms, 4), "bwd_over_fwd": round(bwd_ms / fwd_ms, 2),
        "algorithmic_bytes": nbytes, "GB/s": round(nbytes / bwd_ms / 1e6, 1),
        "hbm_frac": round(nbytes / bwd_ms / 1e6 / HBM_PEAK_GBS, 4),
        "algorithmic_flops": flops, "TFLOP/s": round(flops / bwd_ms / 1e9, 1),
        "mfma_frac": round(flops / bwd_ms / 1e9 / BF16_PEAK_TFLOPS, 4),
        "issued_mfma_TFLOP/s": round(issued / bwd_ms / 1e9, 1),
        "saved": {"fwd_ms": round(fwd_saved_ms, 4), "bwd_ms": round(bwd_saved_ms, 4),
                  "bwd_over_fwd": round(bwd_saved_ms / fwd_saved_ms, 2),
                  "lse_MiB": round(saved[0][1].numel() * 4 / 2 ** 20, 1)},
    }
    print(json.dumps(out), flush=True)
    return 0


def block_steps(args, mate, torch):
    """The steps either side of the scan on the workload (lingen_ma_prep:
    scan-order causal convolution + SiLU for both directions and softplus dt;
    lingen_gated_rmsnorm: SiLU(z) gate and RMS norm), each timed with events
    on the launch stream, scan order = step mod 4, against the algorithmic
    bytes each must move; and the per-direction scan they feed."""
    from mate_inputs import CONFIGS, CONFIG_NOTES, make_block_inputs, make_inputs

    s = CONFIGS[args.config]
    inp = make_block_inputs(s, args.config)
    names = ("xbc", "dt_raw", "conv_w_f", "conv_b_f", "conv_w_b", "conv_b_b", "dt_bias", "y", "z", "norm_w")
    d = {n: inp.torch(n, "cuda") for n in names}
    ad = make_inputs(s, args.config, tensors=["A", "D"])
    A, D = ad.torch("A", "cuda"), ad.torch("D", "cuda")
    outs = mate.lingen_ma_prep(d["xbc"], d["dt_raw"], (d["conv_w_f"], d["conv_b_f"]), (d["conv_w_b"], d["conv_b_b"]),
                               d["dt_bias"], 0, s)
    y_ma = torch.empty((s.batch, s.L, s.d_inner), dtype=outs[0].dtype, device="cuda")
    normed = torch.empty_like(d["y"])
    ws = torch.empty(max(mate.lingen_mate_workspace_bytes(s), 16), dtype=torch.uint8, device="cuda")

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(args.steps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    prep_ms = timed(lambda i: mate.lingen_ma_prep(
        d["xbc"], d["dt_raw"], (d["conv_w_f"], d["conv_b_f"]), (d["conv_w_b"], d["conv_b_b"]), d["dt_bias"], i % 4, s,
        outs=outs))
    norm_ms = timed(lambda i: mate.lingen_gated_rmsnorm(d["y"], d["z"], d["norm_w"], 1e-5, s.d_inner // s.ngroups,
                                                        out=normed))
    xf, Bf, Cf, xb, Bb, Cb, dt = outs
    dirs_ms = timed(lambda i: mate.lingen_ma_fwd_dirs((xf, dt, A, Bf, Cf, D), (xb, dt, A, Bb, Cb, D), i % 4, s,
                                                      out=y_ma, workspace=ws))
    fused_ms = None
    if s.dtype == "bf16" and not s.n_review:
        fused_ms = timed(lambda i: mate.lingen_ma_fwd_dirs_conv(
            d["xbc"], d["dt_raw"], (d["conv_w_f"], d["conv_b_f"]), (d["conv_w_b"], d["conv_b_b"]), d["dt_bias"],
            A, D, A, D, i % 4, s, out=y_ma, workspace=ws))
    e = s.elem_bytes
    ch = s.d_inner + 2 * s.ngroups * s.d_state
    prep_bytes = 3 * s.L * ch * e + 2 * s.L * s.ssd_heads * 4      # xbc in, both directions out; dt_raw in, dt out
    norm_bytes = 3 * s.L * s.d_inner * e                           # y, z in; out
    out = {"workload": CONFIG_NOTES[args.config], "steps": args.steps, "conv_k": 4, "channels": ch}
    for name, ms, nbytes in (("ma_prep", prep_ms, prep_bytes), ("gated_rmsnorm", norm_ms, norm_bytes)):
        out[name] = {"ms": round(ms, 4), "algorithmic_bytes": nbytes, "GB/s": round(nbytes / ms / 1e6, 1),
                     "hbm_frac": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
    out["ma_fwd_dirs_ms"] = round(dirs_ms, 4)
    out["block_ms"] = round(prep_ms + dirs_ms + norm_ms, 4)
    if fused_ms is not None:   # the convolution and softplus inside the scan kernels
        out["ma_fwd_dirs_conv_ms"] = round(fused_ms, 4)
        out["block_fused_ms"] = round(fused_ms + norm_ms, 4)
    print(json.dumps(out), flush=True)
    return 0


def mate_block(args, mate, torch):
    """The whole MATE block (lingen_mate_block_fwd) on the workload at model
    width d_model = Hs*P: rocBLAS projections around the library's kernels.
    Times the block (layer_idx = step mod 4) and, on the same intermediates,
    the library's own steps alone (convolution + softplus, per-direction
    scan, gated norm, window attention); the projections' share is the
    difference."""
    from mate_inputs import CONFIGS, CONFIG_NOTES, make_block_weights

    s = CONFIGS[args.config]
    dm = s.d_inner
    inp = make_block_weights(s, args.config, dm)
    w = {n: inp.torch(n, "cuda") for n in mate.BLOCK_WEIGHTS}
    u = inp.torch("u", "cuda").reshape(s.batch, s.L, dm)
    out = torch.empty_like(u)
    ws = torch.empty(mate.lingen_mate_block_workspace_bytes(s, dm), dtype=torch.uint8, device="cuda")

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(args.steps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    block_ms = timed(lambda i: mate.lingen_mate_block_fwd(u, w, i % 4, s, out=out, workspace=ws))
    # the library's steps alone, on tensors of the block's intermediate shapes
    td = u.dtype
    d, gn, ch = s.d_inner, s.ngroups * s.d_state, s.d_inner + 2 * s.ngroups * s.d_state
    xbc = torch.empty((s.batch, s.L, ch), dtype=td, device="cuda").normal_()
    dt_raw = torch.empty((s.batch, s.L, s.ssd_heads), dtype=torch.float32, device="cuda").normal_()
    outs = mate.lingen_ma_prep(xbc, dt_raw, (w["conv_w_f"], w["conv_b_f"]), (w["conv_w_b"], w["conv_b_b"]),
                               w["dt_bias"], 0, s)
    prep_ms = timed(lambda i: mate.lingen_ma_prep(xbc, dt_raw, (w["conv_w_f"], w["conv_b_f"]),
                                                  (w["conv_w_b"], w["conv_b_b"]), w["dt_bias"], i % 4, s, outs=outs))
    xf, Bf, Cf, xb, Bb, Cb, dt = outs
    y = torch.empty((s.batch, s.L, d), dtype=td, device="cuda")
    sws = torch.empty(max(mate.lingen_mate_workspace_bytes(s), 16), dtype=torch.uint8, device="cuda")
    dirs_ms = timed(lambda i: mate.lingen_ma_fwd_dirs((xf, dt, w["A_f"], Bf, Cf, w["D_f"]),
                                                      (xb, dt, w["A_b"], Bb, Cb, w["D_b"]), i % 4, s, out=y,
                                                      workspace=sws))
    # The fused form (convolution and softplus inside the scan kernels) is
    # timed beside the two-call form the block takes.
    fused = s.dtype == "bf16" and not s.n_review
    if fused:
        conv_ms = timed(lambda i: mate.lingen_ma_fwd_dirs_conv(
            xbc, dt_raw, (w["conv_w_f"], w["conv_b_f"]), (w["conv_w_b"], w["conv_b_b"]), w["dt_bias"], w["A_f"],
            w["D_f"], w["A_b"], w["D_b"], i % 4, s, out=y, workspace=sws))
    z = torch.empty_like(y).normal_()
    yn = torch.empty_like(y)
    norm_ms = timed(lambda i: mate.lingen_gated_rmsnorm(y, z, w["norm_w"], 1e-5, d // s.ngroups, out=yn))
    q, k, v = (torch.empty((s.batch, s.L, d), dtype=td, device="cuda").normal_() for _ in range(3))
    te_ms = timed(lambda i: mate.lingen_te_fwd(q, k, v, i % 2, s, out=yn))
    own = prep_ms + dirs_ms + norm_ms + te_ms
    rows = s.batch * s.L
    gemm_flops = 2 * rows * dm * (d + ch + s.ssd_heads + 3 * d) + 2 * rows * d * dm * 2
    gemm_ms = block_ms - own
    res = {"workload": CONFIG_NOTES[args.config], "d_model": dm, "steps": args.steps,
           "block_ms": round(block_ms, 4), "tokens_per_s": round(rows / (block_ms / 1e3), 1),
           "library_kernels_ms": {"ma_prep": round(prep_ms, 4), "ma_fwd_dirs": round(dirs_ms, 4),
                                  "ma_fwd_dirs_conv": round(conv_ms, 4) if fused else None,
                                  "gated_rmsnorm": round(norm_ms, 4), "te_fwd": round(te_ms, 4),
                                  "sum_of_the_blocks_own_steps": round(own, 4)},
           "projections": {"gemm_flops": gemm_flops, "ms_by_difference": round(gemm_ms, 4),
                           "TFLOP/s": round(gemm_flops / gemm_ms / 1e9, 1) if gemm_ms > 0 else None}}
    print(json.dumps(res), flush=True)
    return 0


def ma_backward(args, mate, torch):
    """The MA branch's backward pass (lingen_ma_bwd) on the workload against
    its forward (lingen_ma_fwd), both timed with events on the launch stream,
    scan order = step mod 4; and the saved-state pair (lingen_ma_fwd_saved,
    then lingen_ma_bwd_saved reading the scan states that forward kept, one
    saved buffer per scan order)."""
    from mate_inputs import CONFIGS, CONFIG_NOTES, make_inputs

    s = CONFIGS[args.config]
    inp = make_inputs(s, args.config, tensors=["x", "dt", "A", "B", "C", "D"], threads=16)
    d = {n: inp.torch(n, "cuda") for n in ("x", "dt", "A", "B", "C", "D")}
    dy = torch.empty((s.batch, s.L, s.d_inner), dtype=d["x"].dtype, device="cuda").normal_()
    grads = mate.lingen_ma_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], dy, 0, s)
    ws = torch.empty(mate.lingen_ma_bwd_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    y = torch.empty((s.batch, s.L, s.d_inner), dtype=d["x"].dtype, device="cuda")
    fws = torch.empty(max(mate.lingen_mate_workspace_bytes(s), 16), dtype=torch.uint8, device="cuda")
    args_f = [d[n] for n in ("x", "dt", "A", "B", "C", "D")]

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(args.steps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    bwd_ms = timed(lambda i: mate.lingen_ma_bwd(*args_f, dy, i % 4, s, grads=grads, workspace=ws))
    fwd_ms = timed(lambda i: mate.lingen_ma_fwd(*args_f, i % 4, s, out=y, workspace=fws))
    del ws
    saved = [mate.lingen_ma_fwd_saved(*args_f, m, s, out=y)[1] for m in range(4)]
    ws_s = torch.empty(mate.lingen_ma_bwd_saved_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    fwd_saved_ms = timed(lambda i: mate.lingen_ma_fwd_saved(*args_f, i % 4, s, out=y, saved=saved[i % 4]))
    bwd_saved_ms = timed(lambda i: mate.lingen_ma_bwd_saved(*args_f, dy, saved[i % 4], i % 4, s, grads=grads,
                                                             workspace=ws_s))
    e = s.elem_bytes
    rows = s.batch * s.L
    G, N, Hs, P = s.ngroups, s.d_state, s.ssd_heads, s.headdim
    # inputs read once (x, dy, B, C, dt), gradients written once (dx, ddt, dB, dC in fp32)
    nbytes = rows * (2 * Hs * P * e + 2 * G * N * e + Hs * 4) + rows * (Hs * P * 4 + Hs * 4 + 2 * G * N * 4)
    out = {"kernel": "ma_bwd", "workload": CONFIG_NOTES[args.config], "steps": args.steps,
           "bwd_ms": round(bwd_ms, 4), "fwd_ms": round(fwd_ms, 4), "bwd_over_fwd": round(bwd_ms / fwd_ms, 2),
           "compulsory_bytes": nbytes, "compulsory_GB/s": round(nbytes / bwd_ms / 1e6, 1),
           "workspace_GiB": round(mate.lingen_ma_bwd_workspace_bytes(s) / 2 ** 30, 2),
           "saved": {"fwd_ms": round(fwd_saved_ms, 4), "bwd_ms": round(bwd_saved_ms, 4),
                     "bwd_over_fwd": round(bwd_saved_ms / fwd_saved_ms, 2),
                     "saved_GiB": round(saved[0].numel() / 2 ** 30, 2),
                     "workspace_GiB": round(ws_s.numel() / 2 ** 30, 2)}}
    print(json.dumps(out), flush=True)
    return 0


def dense_compare(args, mate, torch):
    """The quadratic mixer MATE replaces, at the workload's L, heads and head
    size: dense softmax attention over all tokens (lingen_dense_attn_fwd)
    against the MATE forward (lingen_mate_fwd, layer_idx cycling 0..3), both
    timed with events on the launch stream in one run; prints their
    latencies, the dense kernel's MFMA rate and the latency and FLOP ratios."""
    from mate_inputs import CONFIGS, CONFIG_NOTES, make_inputs

    s = CONFIGS[args.config]
    if s.dtype != "bf16" or s.attn_headdim != 64:
        print("--dense needs a bf16 workload with 64-wide attention heads", file=sys.stderr)
        return 2
    print(f"[bench] dense comparison: generating inputs, {s.L} tokens", file=sys.stderr, flush=True)
    inp = make_inputs(s, args.config, threads=16)
    d = {n: inp.torch(n, "cuda") for n in ("x", "dt", "A", "B", "C", "D", "q", "k", "v")}
    del inp
    mate_args = [d[n] for n in ("x", "dt", "A", "B", "C", "D", "q", "k", "v")]
    ws = torch.empty(mate.lingen_mate_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    y = torch.empty((1, s.L, s.d_inner), dtype=torch.bfloat16, device="cuda")
    qkv = [d[n].view(1, s.L, s.attn_heads, s.attn_headdim) for n in ("q", "k", "v")]
    o = torch.empty_like(qkv[0])

    def timed(fn, steps, warmup):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(steps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    dense_steps = max(1, min(args.steps, 10))
    print(f"[bench] dense attention: {dense_steps} launches", file=sys.stderr, flush=True)
    dense_ms = timed(lambda i: mate.lingen_dense_attn_fwd(*qkv, out=o), dense_steps, 1)
    print(f"[bench] MATE forward: {args.steps} steps", file=sys.stderr, flush=True)
    mate_ms = timed(lambda i: mate.lingen_mate_fwd(*mate_args, i % 4, s, out=y, workspace=ws), args.steps,
                    args.warmup)
    dense_flops = 4 * s.L * s.L * s.attn_headdim * s.attn_heads
    library = None
    if args.sdpa:
        library = library_attention(torch, qkv, dense_steps, dense_flops, timed)
    work = kernel_work(s)
    mate_flops = sum(w["flops"] for w in work.values())
    tflops = dense_flops / (dense_ms / 1e3) / 1e12
    out = {
        "comparison": "dense softmax attention vs MATE forward, same tokens / heads / head size",
        "workload": CONFIG_NOTES[args.config],
        "tokens": s.L,
        "attention": {"heads": s.attn_heads, "d": s.attn_headdim},
        "dense_attn": {"ms": round(dense_ms, 3), "launches": dense_steps, "flops": dense_flops,
                       "TFLOP/s": round(tflops, 1), "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4)},
        "mate_fwd": {"ms": round(mate_ms, 4), "steps": args.steps, "flops": mate_flops},
        "library_dense_attn": library,
        "latency_ratio_dense_over_mate": round(dense_ms / mate_ms, 2),
        "flop_ratio_dense_over_mate": round(dense_flops / mate_flops, 2),
    }
    print(json.dumps(out), flush=True)
    return 0


# ---------------------------------------------------------------------------

def timed_forward(mate, args_t, s, y, ws, K, W, stream, ev):
    """W warmup and K timed lingen_mate_fwd steps (layer_idx = step mod 4)
    bracketed by HIP events on the launch stream; ms per step."""
    for i in range(W):
        mate.lingen_mate_fwd(*args_t, i % 4, s, out=y, workspace=ws)
    a, b = ev.create(), ev.create()
    import torch
    torch.cuda.synchronize()
    ev.record(a, stream)
    for k in range(K):
        mate.lingen_mate_fwd(*args_t, k % 4, s, out=y, workspace=ws)
    ev.record(b, stream)
    torch.cuda.synchronize()
    return ev.ms(a, b) / K


def roofline_of(work, kernel, ms, workload):
    """Roofline line of one kernel: its bound is the one its arithmetic
    intensity (algorithmic flop per algorithmic byte) puts it under, against
    the ridge of MI355X's dense bf16 MFMA peak over its HBM peak; both
    fractions are reported."""
    t = ms / 1e3
    nbytes, flops = work[kernel]["bytes"], work[kernel]["flops"]
    gbs, tflops = nbytes / t / 1e9, flops / t / 1e12
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    intensity = flops / nbytes
    hbm = {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}
    mfma = {"achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}
    bound = "mfma" if intensity > ridge else "hbm"
    main, other = (mfma, hbm) if bound == "mfma" else (hbm, mfma)
    return {"kernel": kernel, "bound": bound, **main,
            "traffic": traffic_for(kernel, workload) if bound == "hbm" else None,
            "algorithmic_bytes_per_launch": nbytes, "algorithmic_flops_per_launch": flops,
            "flop_per_byte": round(intensity, 1), "ridge_flop_per_byte": round(ridge, 1),
            "other_bound": {"bound": "hbm" if bound == "mfma" else "mfma", **other},
            "avg_launch_ms": round(ms, 4)}


def run_config_child(config_id, steps, warmup):
    """The benchmark line of one workload, from a child process (this
    process never touches the GPU, so each workload gets a fresh one)."""
    import subprocess

    cmd = [sys.executable, os.path.abspath(__file__), "--config", str(config_id), "--steps", str(steps),
           "--warmup", str(warmup), "--no-cpu-baseline", "--no-scaling"]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"bench.py --config {config_id} exited with {res.returncode}")
    lines = [ln for ln in res.stdout.splitlines() if ln.startswith("{")]
    if not lines:
        raise RuntimeError(f"bench.py --config {config_id} printed no result line")
    return json.loads(lines[-1])


def sweep(path, n_configs, run):
    """One benchmark line per workload appended to `path` (JSON lines, each
    tagged with its config id).  Workloads already in the file are skipped,
    so a sweep that was cut short resumes where it stopped; a line that does
    not parse (a run killed mid-write) counts as not done."""
    done = set()
    if os.path.exists(path):
        with open(path) as f:
            for line in f:
                try:
                    done.add(int(json.loads(line)["config_id"]))
                except (ValueError, KeyError, TypeError):
                    continue
    for cid in range(n_configs):
        if cid in done:
            print(f"[bench] sweep: config {cid} already in {path}", file=sys.stderr, flush=True)
            continue
        print(f"[bench] sweep: config {cid}", file=sys.stderr, flush=True)
        rec = dict(run(cid))
        rec["config_id"] = cid
        with open(path, "a+") as f:
            # after a line cut short, start a fresh one
            if f.tell() > 0:
                f.seek(f.tell() - 1)
                if f.read(1) != "\n":
                    f.write("\n")
            f.write(json.dumps(rec) + "\n")
            f.flush()
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="processes for the CPU baseline (default: the host cores this process may use, "
                         f"at most {MAX_CPU_WORKERS})")
    ap.add_argument("--no-scaling", action="store_true",
                    help="skip the linear-scaling leg (the forward on the first quarter of the frames)")
    ap.add_argument("--sweep", metavar="FILE",
                    help="run the benchmark line of every workload, each in a child process (no oracle leg, "
                         "no scaling leg), appending one JSON line per workload to FILE; workloads already "
                         "in FILE are skipped")
    ap.add_argument("--record-traffic", nargs=4, metavar=("MIX_FETCH", "MIX_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="add the --config workload's record to profiles/hbm_traffic.json from rocprofv3 --pmc "
                         "FETCH_SIZE / WRITE_SIZE CSVs of this benchmark and of the --copy-gib calibration run, "
                         "then exit")
    ap.add_argument("--copy-gib", type=float, default=0.0,
                    help="instead of the mixer, time a plain device copy of this many GiB (the RMS gather "
                         "kernel in scan mode 0) and print its bandwidth: the HBM calibration point")
    ap.add_argument("--gather", action="store_true",
                    help="instead of the mixer, time the scan-order gather of x-sized rows in each of the "
                         "four scan orders on the workload's grid")
    ap.add_argument("--sdpa", action="store_true",
                    help="with --dense, also time torch's fused scaled_dot_product_attention on the same "
                         "tensors, as context for the dense kernel")
    ap.add_argument("--te-bwd", action="store_true",
                    help="instead of the benchmark line, time the TE branch's backward pass against its forward")
    ap.add_argument("--block", action="store_true",
                    help="instead of the benchmark line, time the steps either side of the scan (convolution + "
                         "SiLU + softplus, gated RMS norm) and the per-direction scan they feed")
    ap.add_argument("--mate-block", action="store_true",
                    help="instead of the benchmark line, time the whole MATE block (projections around the "
                         "mixer) and the library's own steps inside it")
    ap.add_argument("--ma-bwd", action="store_true",
                    help="instead of the benchmark line, time the MA branch's backward pass against its forward")
    ap.add_argument("--dense", action="store_true",
                    help="instead of the benchmark line, time dense softmax attention over all tokens (the "
                         "quadratic mixer MATE replaces) against the MATE forward on the workload")
    args = ap.parse_args(argv)

    if args.sweep:
        from mate_inputs import CONFIGS

        return sweep(args.sweep, len(CONFIGS), lambda cid: run_config_child(cid, args.steps, args.warmup))
    if args.record_traffic:
        return record_traffic(*args.record_traffic, config=args.config)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the mixer is built and measured on a single MI355X "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        return 2

    side = (args.copy_gib > 0 or args.gather or args.dense or args.te_bwd or args.block or args.mate_block
            or args.ma_bwd)
    inp = None
    cpu = None
    if not side:
        from mate_inputs import CONFIGS, CONFIG_NOTES, make_inputs

        s = CONFIGS[args.config]
        workload = CONFIG_NOTES[args.config]
        print(f"[bench] generating inputs: {workload}, {s.L} tokens", file=sys.stderr, flush=True)
        inp = make_inputs(s, args.config, threads=16)
        if not args.no_cpu_baseline:
            nw = cpu_workers(args.cpu_workers)
            print(f"[bench] timing the oracle on the host ({nw} processes, bounded sample)", file=sys.stderr,
                  flush=True)
            cpu = cpu_baseline(s, inp, nw)
            print(f"[bench] oracle done: {cpu['value']:.1f} tokens/s", file=sys.stderr, flush=True)

    import torch

    import linear_complexity_video_mate_amd as mate

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    mate.lib()
    if args.copy_gib > 0:
        return copy_calibration(args, mate, torch)
    if args.gather:
        return gather_modes(args, mate, torch)
    if args.dense:
        return dense_compare(args, mate, torch)
    if args.te_bwd:
        return te_backward(args, mate, torch)
    if args.block:
        return block_steps(args, mate, torch)
    if args.mate_block:
        return mate_block(args, mate, torch)
    if args.ma_bwd:
        return ma_backward(args, mate, torch)
    d = {n: inp.torch(n, "cuda") for n in ("x", "dt", "A", "B", "C", "D", "q", "k", "v")}
    del inp
    args_t = [d[n] for n in ("x", "dt", "A", "B", "C", "D", "q", "k", "v")]
    ws = torch.empty(mate.lingen_mate_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    y = torch.empty((1, s.L, s.d_inner), dtype=torch.bfloat16 if s.dtype == "bf16" else torch.float32,
                    device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents()
    K, W = args.steps, args.warmup
    step_events = [[ev.create() for _ in range(6)] for _ in range(K)]
    warm_events = [ev.create() for _ in range(6)]
    t_start, t_end = ev.create(), ev.create()

    print(f"[bench] warmup {W} steps", file=sys.stderr, flush=True)
    for i in range(W):
        mate.lingen_mate_fwd_events(*args_t, i % 4, s, warm_events, out=y, workspace=ws)
    torch.cuda.synchronize()

    print(f"[bench] timing {K} steps", file=sys.stderr, flush=True)
    wall0 = time.perf_counter()
    ev.record(t_start, stream)
    for k in range(K):
        mate.lingen_mate_fwd_events(*args_t, k % 4, s, step_events[k], out=y, workspace=ws)
    ev.record(t_end, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = ev.ms(t_start, t_end)
    ms_step = total_ms / K

    stage_ms = {name: 0.0 for name in STAGES}
    per_layer = [0.0] * 4
    per_layer_stage = [{name: 0.0 for name in STAGES} for _ in range(4)]
    for k in range(K):
        e = step_events[k]
        for i, name in enumerate(STAGES):
            t = ev.ms(e[i], e[i + 1])
            stage_ms[name] += t / K
            per_layer_stage[k % 4][name] += t / (K / 4)
        per_layer[k % 4] += ev.ms(e[0], e[5]) / (K / 4)

    work = kernel_work(s)
    stages = {}
    for name in STAGES:
        if name not in work:
            continue
        t = stage_ms[name] / 1e3
        stages[name] = {
            "ms": round(stage_ms[name], 4),
            "GB/s": round(work[name]["bytes"] / t / 1e9, 1),
            "hbm_frac": round(work[name]["bytes"] / t / 1e9 / HBM_PEAK_GBS, 4),
            "TFLOP/s": round(work[name]["flops"] / t / 1e12, 2),
            "mfma_frac": round(work[name]["flops"] / t / 1e12 / BF16_PEAK_TFLOPS, 4),
        }
    dom = max((n for n in stages), key=lambda n: stage_ms[n])
    roofline = roofline_of(work, dom, stage_ms[dom], workload)

    # Linear scaling in T: the same forward on the first quarter of the
    # frames (a T/4 x H x W grid, a prefix of every canonical-order tensor),
    # timed the same way in this run.
    scaling = None
    if not args.no_scaling and s.T % 4 == 0 and s.n_review == 0 and s.batch == 1:
        small = s.with_(T=s.T // 4)
        Ls = small.L
        sub = [d[n][:Ls] if n not in ("A", "D") else d[n] for n in ("x", "dt", "A", "B", "C", "D", "q", "k", "v")]
        sws = ws[:mate.lingen_mate_workspace_bytes(small)]
        sy = y[:, :Ls]
        print(f"[bench] linear-scaling leg: {Ls} tokens, {K} steps", file=sys.stderr, flush=True)
        ms_small = timed_forward(mate, sub, small, sy, sws, K, W, stream, ev)
        wk_small = kernel_work(small)
        f_big = sum(w["flops"] for w in work.values())
        f_small = sum(w["flops"] for w in wk_small.values())
        scaling = {
            "small_grid_THW": [small.T, small.H, small.W],
            "small_tokens": Ls,
            "small_ms_per_step": round(ms_small, 4),
            "tokens_ratio": round(s.L / Ls, 3),
            "flop_ratio": round(f_big / f_small, 3),
            "bytes_ratio": round(sum(w["bytes"] for w in work.values())
                                 / sum(w["bytes"] for w in wk_small.values()), 3),
            "time_ratio": round(ms_step / ms_small, 3),
            "band": [3.6, 4.4],
        }
    ev.close()

    comp = compulsory_bytes(s)
    out = {
        "metric": METRIC,
        "value": round(s.L / (ms_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": workload,
            "tokens": s.L,
            "grid_THW": [s.T, s.H, s.W],
            "ssd": {"heads": s.ssd_heads, "P": s.headdim, "N": s.d_state, "chunk": s.chunk},
            "attention": {"heads": s.attn_heads, "d": s.attn_headdim, "window": list(s.win)},
            "review_tokens": s.n_review,
            "layer_idx": "step k uses k mod 4",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "linear_scaling": scaling,
        "stages": stages,
        "per_layer_ms": [round(v, 4) for v in per_layer],
        "per_layer_stage_ms": [{n: round(v, 4) for n, v in d.items() if n in stages} for d in per_layer_stage],
        "path_vs_compulsory_hbm": round(comp / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "wall_s_timed_region": round(wall, 3),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
