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


def row_tol(shape) -> float:
    """Bound on the relative L2 error of every single (token, head) row of y:
    5e-2 with bf16 storage, 1e-4 with fp32 storage, so that a wrong chunk,
    window or head cannot hide inside a whole-tensor norm."""
    return 1e-4 if shape.dtype == "f32" else 5e-2


ROW_FLOOR = 0.1


def check_rows(got, ref, width: int, shape, what: str = "y") -> None:
    """Assert the whole-tensor bound (tol) and the per-row bound (row_tol) on
    rows of `width` consecutive elements (one head's slice of one token).
    A row's error is taken relative to its own norm, floored at ROW_FLOOR of
    the mean row norm: the arithmetic's error is relative to the size of the
    terms that add up to a row (the state read-out, the skip term, the
    attention output), and in rare rows those terms cancel to a small
    fraction of that size (seen: 0.5% of the mean row norm, the read-out
    cancelling the skip term), where a bound relative to the row alone would
    ask for more than bf16 storage carries.  A wrong chunk, window or head
    leaves errors of the order of the mean row norm, far above the floor."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, width)
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, width)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    den = np.maximum(den, ROW_FLOOR * max(float(den.mean()), 1e-300))
    rows = num / den
    e = rel_l2(got, ref)
    worst = int(np.argmax(rows))
    say(f"  {what}: rel L2 {e:.3e}, worst row {rows[worst]:.3e} (row {worst})")
    assert e <= tol(shape), f"{what}: relative L2 {e:.3e} > {tol(shape)}"
    assert rows[worst] <= row_tol(shape), f"{what}: row {worst} relative error {rows[worst]:.3e} > {row_tol(shape)}"
