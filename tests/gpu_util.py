"""Helpers shared by the GPU tests (upload of seeded inputs, oracle per head,
error metrics).  Every GPU test prints the case it is about to run, flushed,
before it touches the GPU."""
from __future__ import annotations

import numpy as np
import pytest

from mate_inputs import f32_from_bf16_bits

NAMES = ("x", "dt", "A", "B", "C", "D", "q", "k", "v")


def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_complexity_video_mate_amd as mate

    mate.lib()          # raises if the library is missing: no fallback
    return torch, mate


def say(msg: str) -> None:
    print(msg, flush=True)


def upload(inp, names=NAMES):
    return {n: inp.torch(n, "cuda") for n in names if n in inp.store}


def f64_all(inp, names=NAMES):
    return {n: inp.f64(n) for n in names if n in inp.store}


def head_f64(inp, name: str, h: int) -> np.ndarray:
    """One head of a per-head tensor as float64 with the head axis kept."""
    a = inp.store[name]
    if name in ("A", "D"):
        sl = a[[h]]
    else:
        sl = a[:, [h]]
    return (f32_from_bf16_bits(sl) if sl.dtype == np.uint16 else sl).astype(np.float64)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def to_np(t) -> np.ndarray:
    return t.detach().double().cpu().numpy()


def tol(shape) -> float:
    """Relative L2 bound: 1e-5 for fp32 storage, 2e-2 for bf16 storage."""
    return 1e-5 if shape.dtype == "f32" else 2e-2


def review_of(shape):
    return (shape.rpool, shape.rgrid) if shape.n_review else None
