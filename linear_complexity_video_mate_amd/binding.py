"""ctypes binding of liblingen_mate.so (include/lingen_mate.h).

Argument marshalling only: these functions check tensor dtypes, devices and
sizes, allocate outputs and workspaces with torch when the caller passes
none, and call the C entry point of the same name on torch's current HIP
stream.  Every step of the mixer runs in the library's HIP kernels; if the
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# LINGEN_LIB_PATH selects another build of the same library (the host-ASan
# variant the CPU tests run against); there is no other library and no
# fallback.
LIB_PATH = os.environ.get("LINGEN_LIB_PATH") or os.path.join(_PKG, "liblingen_mate.so")

LINGEN_OK = 0
STATUS_NAMES = {
    0: "LINGEN_OK",
    -1: "LINGEN_ERR_NULL",
    -2: "LINGEN_ERR_SHAPE",
    -3: "LINGEN_ERR_DTYPE",
    -4: "LINGEN_ERR_ALIGN",
    -5: "LINGEN_ERR_WORKSPACE",
    -6: "LINGEN_ERR_HIP",
    -7: "LINGEN_ERR_UNSUPPORTED",
    -8: "LINGEN_ERR_SCRATCH",
}
LINGEN_F32, LINGEN_BF16 = 0, 1

EXPORTS = (
    "lingen_status_str",
    "lingen_mate_validate",
    "lingen_mate_workspace_bytes",
    "lingen_rms_index",
    "lingen_rms_index_device",
    "lingen_rms_gather",
    "lingen_ssd_chunk_states",
    "lingen_ma_fwd",
    "lingen_ma_fwd_dirs",
    "lingen_te_fwd",
    "lingen_te_fwd_shift",
    "lingen_te_bwd",
    "lingen_te_fwd_saved",
    "lingen_te_bwd_saved",
    "lingen_mate_fwd",
    "lingen_mate_fwd_events",
    "lingen_mate_fwd_noalloc",
    "lingen_dense_attn_fwd",
    "lingen_ma_prep",
    "lingen_ma_fwd_dirs_conv",
    "lingen_gated_rmsnorm",
    "lingen_mate_block_workspace_bytes",
    "lingen_mate_block_fwd",
    "lingen_ma_bwd_workspace_bytes",
    "lingen_ma_bwd",
    "lingen_ma_saved_bytes",
    "lingen_ma_fwd_saved",
    "lingen_ma_bwd_saved_workspace_bytes",
    "lingen_ma_bwd_saved",
)

BLOCK_WEIGHTS = ("w_z", "w_xbc", "w_dt", "conv_w_f", "conv_b_f", "conv_w_b", "conv_b_b", "dt_bias", "A_f", "D_f",
                 "A_b", "D_b", "norm_w", "w_out_ma", "w_q", "w_k", "w_v", "w_o")


class LingenError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(code, code)} ({status_str(code)})")


class lingen_mate_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "T", "H", "W", "ssd_heads", "headdim", "d_state", "ngroups", "chunk",
        "attn_heads", "attn_headdim", "win_t", "win_h", "win_w", "dtype", "n_review",
        "rpool_t", "rpool_h", "rpool_w", "rgrid_t", "rgrid_h", "rgrid_w")]


class lingen_mate_block_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BLOCK_WEIGHTS]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m linear_complexity_video_mate_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    SP = ctypes.POINTER(lingen_mate_shape)
    sig = {
        "lingen_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "lingen_mate_validate": ([SP], ctypes.c_int),
        "lingen_mate_workspace_bytes": ([SP, ctypes.POINTER(SZ)], ctypes.c_int),
        "lingen_rms_index": ([I32, I32, I32, I32, P, P], ctypes.c_int),
        "lingen_rms_index_device": ([I32, I32, I32, I32, P, P], ctypes.c_int),
        "lingen_rms_gather": ([P, I64, I32, I32, I32, I32, P, P], ctypes.c_int),
        "lingen_ssd_chunk_states": ([P, P, P, P, I32, SP, P, P, P, SZ, P], ctypes.c_int),
        "lingen_ma_fwd": ([P, P, P, P, P, P, I32, SP, P, P, SZ, P], ctypes.c_int),
        "lingen_ma_fwd_dirs": ([P] * 12 + [I32, SP, P, P, SZ, P], ctypes.c_int),
        "lingen_te_fwd": ([P, P, P, I32, SP, P, P], ctypes.c_int),
        "lingen_te_fwd_shift": ([P, P, P, I32, I32, I32, I32, SP, P, P], ctypes.c_int),
        "lingen_te_bwd": ([P, P, P, P, I32, I32, I32, I32, SP, P, P, P, P], ctypes.c_int),
        "lingen_te_fwd_saved": ([P, P, P, I32, I32, I32, I32, SP, P, P, P], ctypes.c_int),
        "lingen_te_bwd_saved": ([P] * 6 + [I32, I32, I32, I32, SP, P, P, P, P], ctypes.c_int),
        "lingen_mate_fwd": ([P, P, P, P, P, P, P, P, P, I32, SP, P, P, SZ, P], ctypes.c_int),
        "lingen_mate_fwd_events": ([P, P, P, P, P, P, P, P, P, I32, SP, P, P, SZ, P, P], ctypes.c_int),
        "lingen_mate_fwd_noalloc": ([P, P, P, P, P, P, P, P, P, I32, SP, P, P], ctypes.c_int),
        "lingen_dense_attn_fwd": ([P, P, P, P, I32, I32, I32, I32, I32, P], ctypes.c_int),
        "lingen_ma_prep": ([P] * 7 + [I32, I32, SP] + [P] * 7 + [P], ctypes.c_int),
        "lingen_ma_fwd_dirs_conv": ([P, P, P, I32] + [P] * 8 + [I32, SP, P, P, SZ, P], ctypes.c_int),
        "lingen_gated_rmsnorm": ([P, P, P, ctypes.c_float, I64, I32, I32, I32, P, P], ctypes.c_int),
        "lingen_mate_block_workspace_bytes": ([SP, I32, ctypes.POINTER(SZ)], ctypes.c_int),
        "lingen_ma_bwd_workspace_bytes": ([SP, ctypes.POINTER(SZ)], ctypes.c_int),
        "lingen_ma_bwd": ([P] * 7 + [I32, SP] + [P] * 7 + [SZ, P], ctypes.c_int),
        "lingen_ma_saved_bytes": ([SP, ctypes.POINTER(SZ)], ctypes.c_int),
        "lingen_ma_fwd_saved": ([P] * 6 + [I32, SP, P, P, SZ, P], ctypes.c_int),
        "lingen_ma_bwd_saved_workspace_bytes": ([SP, ctypes.POINTER(SZ)], ctypes.c_int),
        "lingen_ma_bwd_saved": ([P] * 8 + [SZ, I32, SP] + [P] * 7 + [SZ, P], ctypes.c_int),
        "lingen_mate_block_fwd": ([P, ctypes.POINTER(lingen_mate_block_weights), I32, I32, ctypes.c_float, I32, SP,
                                   P, P, SZ, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def status_str(code: int) -> str:
    return lib().lingen_status_str(int(code)).decode()


def _check(fn: str, rc: int) -> None:
    if rc != LINGEN_OK:
        raise LingenError(fn, rc)


def to_c_shape(s) -> lingen_mate_shape:
    """Build the C struct from any object with the MateShape attribute names."""
    dtype = s.dtype
    if isinstance(dtype, str):
        dtype = {"f32": LINGEN_F32, "bf16": LINGEN_BF16}.get(dtype, 99)
    rpool = getattr(s, "rpool", (1, 1, 1))
    rgrid = getattr(s, "rgrid", (1, 1, 1))
    return lingen_mate_shape(
        s.batch, s.T, s.H, s.W, s.ssd_heads, s.headdim, s.d_state, s.ngroups, s.chunk,
        s.attn_heads, s.attn_headdim, s.win[0], s.win[1], s.win[2], dtype,
        getattr(s, "n_review", 0), rpool[0], rpool[1], rpool[2], rgrid[0], rgrid[1], rgrid[2])


def lingen_mate_validate(shape) -> int:
    """Status code of the host-side shape check (no exception)."""
    cs = to_c_shape(shape)
    return lib().lingen_mate_validate(ctypes.byref(cs))


def lingen_mate_workspace_bytes(shape) -> int:
    cs = to_c_shape(shape)
    n = ctypes.c_size_t(0)
    _check("lingen_mate_workspace_bytes", lib().lingen_mate_workspace_bytes(ctypes.byref(cs), ctypes.byref(n)))
    return int(n.value)


def lingen_rms_index(mode: int, T: int, H: int, W: int) -> Tuple[np.ndarray, np.ndarray]:
    L = T * H * W
    perm = np.empty(L, dtype=np.int32)
    inv = np.empty(L, dtype=np.int32)
    _check("lingen_rms_index", lib().lingen_rms_index(mode, T, H, W, perm.ctypes.data, inv.ctypes.data))
    return perm, inv


# ---------------------------------------------------------------------------
# Device entry points (torch tensors on the GPU)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _tdtype(shape):
    torch = _torch()
    return torch.bfloat16 if shape.dtype in ("bf16", LINGEN_BF16) else torch.float32


def _need(t, name: str, dtype, numel: int):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _sizes(s):
    L = s.T * s.H * s.W
    return dict(
        x=s.batch * L * s.ssd_heads * s.headdim,
        dt=s.batch * L * s.ssd_heads,
        A=s.ssd_heads,
        B=s.batch * L * s.ngroups * s.d_state,
        D=s.ssd_heads,
        q=s.batch * L * s.attn_heads * s.attn_headdim,
        y=s.batch * L * s.ssd_heads * s.headdim,
        states=s.batch * (L // s.chunk) * s.ssd_heads * s.headdim * s.d_state,
    )


def _workspace(shape, workspace):
    torch = _torch()
    need = lingen_mate_workspace_bytes(shape)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    return workspace, ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(nbytes)


def lingen_rms_index_device(mode: int, T: int, H: int, W: int, out=None):
    torch = _torch()
    L = T * H * W
    if out is None:
        out = torch.empty(L, dtype=torch.int32, device="cuda")
    p = _need(out, "out", torch.int32, L)
    _check("lingen_rms_index_device", lib().lingen_rms_index_device(mode, T, H, W, p, _stream()))
    return out


def lingen_rms_gather(src, mode: int, T: int, H: int, W: int, out=None):
    """Scan-order copy of a [T*H*W, ...] GPU tensor (rows = leading dim)."""
    torch = _torch()
    L = T * H * W
    if src.shape[0] != L or not src.is_contiguous() or src.device.type != "cuda":
        raise ValueError("src must be a contiguous GPU tensor with T*H*W rows")
    row_bytes = src.numel() // L * src.element_size()
    if out is None:
        out = torch.empty_like(src)
    _need(out, "out", src.dtype, src.numel())
    _check("lingen_rms_gather", lib().lingen_rms_gather(
        ctypes.c_void_p(src.data_ptr()), row_bytes, mode, T, H, W, ctypes.c_void_p(out.data_ptr()), _stream()))
    return out


def lingen_ssd_chunk_states(x, dt, A, B, mode: int, shape, workspace=None):
    """(h_fwd, h_bwd): scan states entering every chunk, [batch, L/Q, Hs, P, N] fp32."""
    torch = _torch()
    n = _sizes(shape)
    td = _tdtype(shape)
    cs = to_c_shape(shape)
    px = _need(x, "x", td, n["x"])
    pdt = _need(dt, "dt", torch.float32, n["dt"])
    pA = _need(A, "A", torch.float32, n["A"])
    pB = _need(B, "B", td, n["B"])
    L = shape.T * shape.H * shape.W
    hshape = (shape.batch, L // shape.chunk, shape.ssd_heads, shape.headdim, shape.d_state)
    hf = torch.empty(hshape, dtype=torch.float32, device="cuda")
    hb = torch.empty(hshape, dtype=torch.float32, device="cuda")
    workspace, pw, nw = _workspace(shape, workspace)
    _check("lingen_ssd_chunk_states", lib().lingen_ssd_chunk_states(
        px, pdt, pA, pB, mode, ctypes.byref(cs), ctypes.c_void_p(hf.data_ptr()), ctypes.c_void_p(hb.data_ptr()),
        pw, nw, _stream()))
    return hf, hb


def lingen_ma_fwd(x, dt, A, B, C, D, mode: int, shape, out=None, workspace=None):
    """MA branch alone; returns y_ma [batch, L, Hs*P]."""
    torch = _torch()
    n = _sizes(shape)
    td = _tdtype(shape)
    cs = to_c_shape(shape)
    L = shape.T * shape.H * shape.W
    if out is None:
        out = torch.empty((shape.batch, L, shape.ssd_heads * shape.headdim), dtype=td, device="cuda")
    args = [_need(x, "x", td, n["x"]), _need(dt, "dt", torch.float32, n["dt"]),
            _need(A, "A", torch.float32, n["A"]), _need(B, "B", td, n["B"]), _need(C, "C", td, n["B"]),
            _need(D, "D", torch.float32, n["D"])]
    py = _need(out, "out", td, n["y"])
    workspace, pw, nw = _workspace(shape, workspace)
    _check("lingen_ma_fwd", lib().lingen_ma_fwd(*args, mode, ctypes.byref(cs), py, pw, nw, _stream()))
    return out


def lingen_ma_fwd_dirs(fwd, bwd, mode: int, shape, out=None, workspace=None):
    """MA branch with a parameter set per direction: ``fwd`` and ``bwd`` are
    (x, dt, A, B, C, D) tuples; returns y_ma [batch, L, Hs*P]."""
    torch = _torch()
    n = _sizes(shape)
    td = _tdtype(shape)
    cs = to_c_shape(shape)
    L = shape.T * shape.H * shape.W
    if out is None:
        out = torch.empty((shape.batch, L, shape.ssd_heads * shape.headdim), dtype=td, device="cuda")
    args = []
    for tag, (x, dt, A, B, C, D) in (("f", fwd), ("b", bwd)):
        args += [_need(x, "x_" + tag, td, n["x"]), _need(dt, "dt_" + tag, torch.float32, n["dt"]),
                 _need(A, "A_" + tag, torch.float32, n["A"]), _need(B, "B_" + tag, td, n["B"]),
                 _need(C, "C_" + tag, td, n["B"]), _need(D, "D_" + tag, torch.float32, n["D"])]
    py = _need(out, "out", td, n["y"])
    workspace, pw, nw = _workspace(shape, workspace)
    _check("lingen_ma_fwd_dirs", lib().lingen_ma_fwd_dirs(*args, mode, ctypes.byref(cs), py, pw, nw, _stream()))
    return out


def lingen_te_fwd(q, k, v, shifted: int, shape, out=None):
    """TE branch alone; returns y_te [batch, L, Ha*d]."""
    n = _sizes(shape)
    td = _tdtype(shape)
    cs = to_c_shape(shape)
    torch = _torch()
    L = shape.T * shape.H * shape.W
    if out is None:
        out = torch.empty((shape.batch, L, shape.attn_heads * shape.attn_headdim), dtype=td, device="cuda")
    args = [_need(q, "q", td, n["q"]), _need(k, "k", td, n["q"]), _need(v, "v", td, n["q"])]
    py = _need(out, "out", td, n["y"])
    _check("lingen_te_fwd", lib().lingen_te_fwd(*args, int(shifted), ctypes.byref(cs), py, _stream()))
    return out


def lingen_te_fwd_shift(q, k, v, shift, masked: int, shape, out=None):
    """TE branch with window-grid offset ``shift`` = (st, sh, sw) and
    ``masked`` = 1 (border pieces are windows of their own) or 0 (cyclic
    windows); returns y_te [batch, L, Ha*d]."""
    n = _sizes(shape)
    td = _tdtype(shape)
    cs = to_c_shape(shape)
    torch = _torch()
    L = shape.T * shape.H * shape.W
    if out is None:
        out = torch.empty((shape.batch, L, shape.attn_heads * shape.attn_headdim), dtype=td, device="cuda")
    args = [_need(q, "q", td, n["q"]), _need(k, "k", td, n["q"]), _need(v, "v", td, n["q"])]
    py = _need(out, "out", td, n["y"])
    st, sh, sw = (int(a) for a in shift)
    _check("lingen_te_fwd_shift", lib().lingen_te_fwd_shift(*args, st, sh, sw, int(masked), ctypes.byref(cs), py,
                                                            _stream()))
    return out


def lingen_te_bwd(q, k, v, d_out, shift, masked: int, shape, dq=None, dk=None, dv=None):
    """Gradients (dq, dk, dv) of the TE branch for the upstream gradient
    ``d_out`` of its output; window offset ``shift`` and ``masked`` as in
    lingen_te_fwd_shift."""
    n = _sizes(shape)
    td = _tdtype(shape)
    cs = to_c_shape(shape)
    torch = _torch()
    outs = [t if t is not None else torch.empty_like(q) for t in (dq, dk, dv)]
    args = [_need(q, "q", td, n["q"]), _need(k, "k", td, n["q"]), _need(v, "v", td, n["q"]),
            _need(d_out, "d_out", td, n["q"])]
    pouts = [_need(t, name, td, n["q"]) for t, name in zip(outs, ("dq", "dk", "dv"))]
    st, sh, sw = (int(a) for a in shift)
    _check("lingen_te_bwd", lib().lingen_te_bwd(*args, st, sh, sw, int(masked), ctypes.byref(cs), *pouts, _stream()))
    return tuple(outs)


def lingen_te_fwd_saved(q, k, v, shift, masked: int, shape, out=None, lse=None):
    """lingen_te_fwd_shift that also keeps each query's log2 softmax
    denominator; returns (y_te, lse [batch, L, Ha] fp32)."""
    n = _sizes(shape)
    td = _tdtype(shape)
    cs = to_c_shape(shape)
    torch = _torch()
    L = shape.T * shape.H * shape.W
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((shape.batch, L, shape.attn_heads), dtype=torch.float32, device="cuda")
    args = [_need(q, "q", td, n["q"]), _need(k, "k", td, n["q"]), _need(v, "v", td, n["q"])]
    po = _need(out, "out", td, n["q"])
    pl = _need(lse, "lse", torch.float32, shape.batch * L * shape.attn_heads)
    st, sh, sw = (int(a) for a in shift)
    _check("lingen_te_fwd_saved", lib().lingen_te_fwd_saved(*args, st, sh, sw, int(masked), ctypes.byref(cs), po, pl,
                                                            _stream()))
    return out, lse


def lingen_te_bwd_saved(q, k, v, o, d_out, lse, shift, masked: int, shape, dq=None, dk=None, dv=None):
    """lingen_te_bwd from the output ``o`` and statistics ``lse`` that
    lingen_te_fwd_saved returned for the same inputs and offsets."""
    n = _sizes(shape)
    td = _tdtype(shape)
    cs = to_c_shape(shape)
    torch = _torch()
    L = shape.T * shape.H * shape.W
    outs = [t if t is not None else torch.empty_like(q) for t in (dq, dk, dv)]
    args = [_need(q, "q", td, n["q"]), _need(k, "k", td, n["q"]), _need(v, "v", td, n["q"]),
            _need(o, "o", td, n["q"]), _need(d_out, "d_out", td, n["q"]),
            _need(lse, "lse", torch.float32, shape.batch * L * shape.attn_heads)]
    pouts = [_need(t, name, td, n["q"]) for t, name in zip(outs, ("dq", "dk", "dv"))]
    st, sh, sw = (int(a) for a in shift)
    _check("lingen_te_bwd_saved", lib().lingen_te_bwd_saved(*args, st, sh, sw, int(masked), ctypes.byref(cs), *pouts,
                                                            _stream()))
    return tuple(outs)


def lingen_mate_fwd(x, dt, A, B, C, D, q, k, v, layer_idx: int, shape, out=None, workspace=None):
    """The MATE mixer; returns y [batch, L, Hs*P]."""
    torch = _torch()
    n = _sizes(shape)
    td = _tdtype(shape)
    cs = to_c_shape(shape)
    L = shape.T * shape.H * shape.W
    if out is None:
        out = torch.empty((shape.batch, L, shape.ssd_heads * shape.headdim), dtype=td, device="cuda")
    args = [_need(x, "x", td, n["x"]), _need(dt, "dt", torch.float32, n["dt"]),
            _need(A, "A", torch.float32, n["A"]), _need(B, "B", td, n["B"]), _need(C, "C", td, n["B"]),
            _need(D, "D", torch.float32, n["D"]), _need(q, "q", td, n["q"]), _need(k, "k", td, n["q"]),
            _need(v, "v", td, n["q"])]
    py = _need(out, "out", td, n["y"])
    workspace, pw, nw = _workspace(shape, workspace)
    _check("lingen_mate_fwd", lib().lingen_mate_fwd(*args, int(layer_idx), ctypes.byref(cs), py, pw, nw, _stream()))
    return out


def lingen_mate_fwd_noalloc(x, dt, A, B, C, D, q, k, v, layer_idx: int, shape, out=None):
    """The MATE mixer with the library's fixed device scratch array as its
    workspace (no allocation inside the call); returns y [batch, L, Hs*P]."""
    torch = _torch()
    n = _sizes(shape)
    td = _tdtype(shape)
    cs = to_c_shape(shape)
    L = shape.T * shape.H * shape.W
    if out is None:
        out = torch.empty((shape.batch, L, shape.ssd_heads * shape.headdim), dtype=td, device="cuda")
    args = [_need(x, "x", td, n["x"]), _need(dt, "dt", torch.float32, n["dt"]),
            _need(A, "A", torch.float32, n["A"]), _need(B, "B", td, n["B"]), _need(C, "C", td, n["B"]),
            _need(D, "D", torch.float32, n["D"]), _need(q, "q", td, n["q"]), _need(k, "k", td, n["q"]),
            _need(v, "v", td, n["q"])]
    py = _need(out, "out", td, n["y"])
    _check("lingen_mate_fwd_noalloc", lib().lingen_mate_fwd_noalloc(*args, int(layer_idx), ctypes.byref(cs), py,
                                                                    _stream()))
    return out


def lingen_mate_fwd_events(x, dt, A, B, C, D, q, k, v, layer_idx: int, shape, events, out=None, workspace=None):
    """lingen_mate_fwd plus six caller-created HIP events (raw hipEvent_t
    handles as ints) recorded at the stage boundaries; returns y."""
    torch = _torch()
    n = _sizes(shape)
    td = _tdtype(shape)
    cs = to_c_shape(shape)
    L = shape.T * shape.H * shape.W
    if len(events) != 6:
        raise ValueError("events must hold 6 hipEvent_t handles")
    if out is None:
        out = torch.empty((shape.batch, L, shape.ssd_heads * shape.headdim), dtype=td, device="cuda")
    args = [_need(x, "x", td, n["x"]), _need(dt, "dt", torch.float32, n["dt"]),
            _need(A, "A", torch.float32, n["A"]), _need(B, "B", td, n["B"]), _need(C, "C", td, n["B"]),
            _need(D, "D", torch.float32, n["D"]), _need(q, "q", td, n["q"]), _need(k, "k", td, n["q"]),
            _need(v, "v", td, n["q"])]
    py = _need(out, "out", td, n["y"])
    workspace, pw, nw = _workspace(shape, workspace)
    ev = (ctypes.c_void_p * 6)(*[ctypes.c_void_p(int(e)) for e in events])
    _check("lingen_mate_fwd_events", lib().lingen_mate_fwd_events(
        *args, int(layer_idx), ctypes.byref(cs), py, pw, nw, _stream(), ctypes.cast(ev, ctypes.c_void_p)))
    return out


def lingen_dense_attn_fwd(q, k, v, out=None):
    """Dense softmax attention over all tokens; q, k, v [batch, L, heads, d]
    GPU tensors (bf16 or fp32); returns o of the same shape."""
    torch = _torch()
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must be [batch, L, heads, d] tensors of one shape")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"q must be bfloat16 or float32 (got {q.dtype})")
    batch, L, heads, d = (int(n) for n in q.shape)
    code = LINGEN_BF16 if q.dtype == torch.bfloat16 else LINGEN_F32
    if out is None:
        out = torch.empty_like(q)
    args = [_need(t, name, q.dtype, q.numel()) for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out"))]
    _check("lingen_dense_attn_fwd", lib().lingen_dense_attn_fwd(*args, batch, L, heads, d, code, _stream()))
    return out


def lingen_ma_prep(xbc, dt_raw, conv_f, conv_b, dt_bias, mode: int, shape, outs=None):
    """The steps before the scan: ``xbc`` [batch, L, Hs*P + 2*G*N] (x, B, C
    channels, canonical token order) is convolved along the scan order of
    ``mode`` and along its reverse with the (weight [Ch, K], bias [Ch]) pairs
    ``conv_f`` and ``conv_b``, then SiLU; dt = softplus(dt_raw + dt_bias).
    Returns (x_f, B_f, C_f, x_b, B_b, C_b, dt) shaped for lingen_ma_fwd_dirs."""
    torch = _torch()
    n = _sizes(shape)
    td = _tdtype(shape)
    cs = to_c_shape(shape)
    L = shape.T * shape.H * shape.W
    d, gn = shape.ssd_heads * shape.headdim, shape.ngroups * shape.d_state
    ch = d + 2 * gn
    (wf, bf), (wb, bb) = conv_f, conv_b
    if wf.dim() != 2 or wf.shape[0] != ch or wb.shape != wf.shape:
        raise ValueError(f"convolution weights must be [{ch}, K] tensors of one shape")
    K = int(wf.shape[1])
    if outs is None:
        outs = tuple(torch.empty((shape.batch, L, w), dtype=td, device="cuda") for w in (d, gn, gn, d, gn, gn)) + (
            torch.empty((shape.batch, L, shape.ssd_heads), dtype=torch.float32, device="cuda"),)
    f32 = torch.float32
    args = [_need(xbc, "xbc", td, shape.batch * L * ch), _need(dt_raw, "dt_raw", f32, n["dt"]),
            _need(wf, "conv_w_f", f32, ch * K), _need(bf, "conv_b_f", f32, ch),
            _need(wb, "conv_w_b", f32, ch * K), _need(bb, "conv_b_b", f32, ch),
            _need(dt_bias, "dt_bias", f32, shape.ssd_heads)]
    names = ("x_f", "B_f", "C_f", "x_b", "B_b", "C_b")
    sizes = (n["x"], n["B"], n["B"], n["x"], n["B"], n["B"])
    po = [_need(t, nm, td, sz) for t, nm, sz in zip(outs[:6], names, sizes)]
    po.append(_need(outs[6], "dt", f32, n["dt"]))
    _check("lingen_ma_prep", lib().lingen_ma_prep(*args, K, int(mode), ctypes.byref(cs), *po, _stream()))
    return tuple(outs)


def lingen_ma_fwd_dirs_conv(xbc, dt_raw, conv_f, conv_b, dt_bias, A_f, D_f, A_b, D_b, mode: int, shape, out=None,
                            workspace=None):
    """lingen_ma_prep and lingen_ma_fwd_dirs in one pass per direction (the
    convolution, SiLU and softplus taken inside the scan kernels): arguments
    as those two calls; returns y_ma [batch, L, Hs*P]."""
    torch = _torch()
    n = _sizes(shape)
    td = _tdtype(shape)
    cs = to_c_shape(shape)
    L = shape.T * shape.H * shape.W
    d, gn = shape.ssd_heads * shape.headdim, shape.ngroups * shape.d_state
    ch = d + 2 * gn
    (wf, bf), (wb, bb) = conv_f, conv_b
    if wf.dim() != 2 or wf.shape[0] != ch or wb.shape != wf.shape:
        raise ValueError(f"convolution weights must be [{ch}, K] tensors of one shape")
    K = int(wf.shape[1])
    if out is None:
        out = torch.empty((shape.batch, L, d), dtype=td, device="cuda")
    f32 = torch.float32
    args = [_need(xbc, "xbc", td, shape.batch * L * ch), _need(dt_raw, "dt_raw", f32, n["dt"]),
            _need(dt_bias, "dt_bias", f32, shape.ssd_heads), K,
            _need(wf, "conv_w_f", f32, ch * K), _need(bf, "conv_b_f", f32, ch),
            _need(A_f, "A_f", f32, n["A"]), _need(D_f, "D_f", f32, n["D"]),
            _need(wb, "conv_w_b", f32, ch * K), _need(bb, "conv_b_b", f32, ch),
            _need(A_b, "A_b", f32, n["A"]), _need(D_b, "D_b", f32, n["D"])]
    py = _need(out, "out", td, n["y"])
    workspace, pw, nw = _workspace(shape, workspace)
    _check("lingen_ma_fwd_dirs_conv",
           lib().lingen_ma_fwd_dirs_conv(*args, int(mode), ctypes.byref(cs), py, pw, nw, _stream()))
    return out


def lingen_gated_rmsnorm(y, z, weight, eps: float, group: int, out=None):
    """Gated RMS norm after the scan: for y, z [..., dim] (bf16 or fp32, one
    dtype) and weight [dim] fp32, g = y * silu(z) and each group of ``group``
    channels is divided by sqrt(mean(g^2) + eps) and multiplied by the
    weight.  Returns a tensor shaped like y."""
    torch = _torch()
    if z.shape != y.shape or y.dim() < 1:
        raise ValueError("y and z must be tensors of one shape")
    if y.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"y must be bfloat16 or float32 (got {y.dtype})")
    dim = int(y.shape[-1])
    rows = y.numel() // dim if dim else 0
    code = LINGEN_BF16 if y.dtype == torch.bfloat16 else LINGEN_F32
    if out is None:
        out = torch.empty_like(y)
    py, pz, po = (_need(t, nm, y.dtype, y.numel()) for t, nm in ((y, "y"), (z, "z"), (out, "out")))
    pw = _need(weight, "weight", torch.float32, dim)
    _check("lingen_gated_rmsnorm", lib().lingen_gated_rmsnorm(py, pz, pw, float(eps), rows, dim, int(group), code, po,
                                                              _stream()))
    return out


def lingen_mate_block_workspace_bytes(shape, d_model: int) -> int:
    n = ctypes.c_size_t(0)
    _check("lingen_mate_block_workspace_bytes",
           lib().lingen_mate_block_workspace_bytes(ctypes.byref(to_c_shape(shape)), int(d_model), ctypes.byref(n)))
    return n.value


def block_weight_sizes(shape, d_model: int, conv_k: int = 4):
    """Element counts of every block weight (see lingen_mate_block_weights)."""
    d = shape.ssd_heads * shape.headdim
    ch = d + 2 * shape.ngroups * shape.d_state
    hs = shape.ssd_heads
    return dict(w_z=d * d_model, w_xbc=ch * d_model, w_dt=hs * d_model, conv_w_f=ch * conv_k, conv_b_f=ch,
                conv_w_b=ch * conv_k, conv_b_b=ch, dt_bias=hs, A_f=hs, D_f=hs, A_b=hs, D_b=hs, norm_w=d,
                w_out_ma=d_model * d, w_q=d * d_model, w_k=d * d_model, w_v=d * d_model, w_o=d_model * d)


def lingen_mate_block_fwd(u, weights, layer_idx: int, shape, conv_k: int = 4, norm_eps: float = 1e-5, out=None,
                          workspace=None):
    """The whole MATE block on u [batch, L, d_model]: ``weights`` maps every
    name of BLOCK_WEIGHTS to a GPU tensor (projections in the shape dtype,
    the rest fp32).  Returns out [batch, L, d_model]."""
    torch = _torch()
    td = _tdtype(shape)
    cs = to_c_shape(shape)
    L = shape.T * shape.H * shape.W
    if u.dim() != 3 or u.shape[0] != shape.batch or u.shape[1] != L:
        raise ValueError(f"u must be [{shape.batch}, {L}, d_model]")
    d_model = int(u.shape[2])
    sizes = block_weight_sizes(shape, d_model, conv_k)
    w = lingen_mate_block_weights()
    for name in BLOCK_WEIGHTS:
        dtype = td if name.startswith("w_") else torch.float32
        setattr(w, name, _need(weights[name], name, dtype, sizes[name]).value)
    if out is None:
        out = torch.empty_like(u)
    pu = _need(u, "u", td, u.numel())
    po = _need(out, "out", td, u.numel())
    need = lingen_mate_block_workspace_bytes(shape, d_model)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    pw = ctypes.c_void_p(workspace.data_ptr())
    nw = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    _check("lingen_mate_block_fwd", lib().lingen_mate_block_fwd(pu, ctypes.byref(w), d_model, int(conv_k),
                                                                float(norm_eps), int(layer_idx), ctypes.byref(cs),
                                                                po, pw, nw, _stream()))
    return out


def lingen_ma_bwd_workspace_bytes(shape) -> int:
    n = ctypes.c_size_t(0)
    _check("lingen_ma_bwd_workspace_bytes",
           lib().lingen_ma_bwd_workspace_bytes(ctypes.byref(to_c_shape(shape)), ctypes.byref(n)))
    return n.value


def _ma_grads(shape, grads):
    torch = _torch()
    n = _sizes(shape)
    L = shape.T * shape.H * shape.W
    f32 = torch.float32
    if grads is None:
        dev = "cuda"
        grads = (torch.empty((shape.batch, L, shape.ssd_heads, shape.headdim), dtype=f32, device=dev),
                 torch.empty((shape.batch, L, shape.ssd_heads), dtype=f32, device=dev),
                 torch.empty(shape.ssd_heads, dtype=f32, device=dev),
                 torch.empty((shape.batch, L, shape.ngroups, shape.d_state), dtype=f32, device=dev),
                 torch.empty((shape.batch, L, shape.ngroups, shape.d_state), dtype=f32, device=dev),
                 torch.empty(shape.ssd_heads, dtype=f32, device=dev))
    sizes = (n["x"], n["dt"], n["A"], n["B"], n["B"], n["D"])
    pg = [_need(g, name, f32, sz) for g, name, sz in zip(grads, ("dx", "ddt", "dA", "dB", "dC", "dD"), sizes)]
    return grads, pg


def _ma_bwd_inputs(shape, x, dt, A, B, C, D, dy):
    torch = _torch()
    n = _sizes(shape)
    td = _tdtype(shape)
    f32 = torch.float32
    return [_need(x, "x", td, n["x"]), _need(dt, "dt", f32, n["dt"]), _need(A, "A", f32, n["A"]),
            _need(B, "B", td, n["B"]), _need(C, "C", td, n["B"]), _need(D, "D", f32, n["D"]),
            _need(dy, "dy", td, n["y"])]


def _device_buffer(need, buf):
    torch = _torch()
    if buf is None:
        buf = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    return buf, ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(buf.numel() * buf.element_size())


def lingen_ma_bwd(x, dt, A, B, C, D, dy, mode: int, shape, grads=None, workspace=None):
    """Gradients (dx, ddt, dA, dB, dC, dD) of sum(dy * y_ma) for the MA
    branch of lingen_ma_fwd, all fp32 GPU tensors."""
    args = _ma_bwd_inputs(shape, x, dt, A, B, C, D, dy)
    grads, pg = _ma_grads(shape, grads)
    workspace, pw, nw = _device_buffer(lingen_ma_bwd_workspace_bytes(shape), workspace)
    cs = to_c_shape(shape)
    _check("lingen_ma_bwd", lib().lingen_ma_bwd(*args, int(mode), ctypes.byref(cs), *pg, pw, nw, _stream()))
    return grads


def lingen_ma_saved_bytes(shape) -> int:
    n = ctypes.c_size_t(0)
    _check("lingen_ma_saved_bytes", lib().lingen_ma_saved_bytes(ctypes.byref(to_c_shape(shape)), ctypes.byref(n)))
    return n.value


def lingen_ma_bwd_saved_workspace_bytes(shape) -> int:
    n = ctypes.c_size_t(0)
    _check("lingen_ma_bwd_saved_workspace_bytes",
           lib().lingen_ma_bwd_saved_workspace_bytes(ctypes.byref(to_c_shape(shape)), ctypes.byref(n)))
    return n.value


def lingen_ma_fwd_saved(x, dt, A, B, C, D, mode: int, shape, out=None, saved=None):
    """lingen_ma_fwd that keeps its scan states for lingen_ma_bwd_saved;
    returns (y_ma [batch, L, Hs*P], saved uint8 buffer)."""
    torch = _torch()
    n = _sizes(shape)
    td = _tdtype(shape)
    L = shape.T * shape.H * shape.W
    if out is None:
        out = torch.empty((shape.batch, L, shape.ssd_heads * shape.headdim), dtype=td, device="cuda")
    args = [_need(x, "x", td, n["x"]), _need(dt, "dt", torch.float32, n["dt"]),
            _need(A, "A", torch.float32, n["A"]), _need(B, "B", td, n["B"]), _need(C, "C", td, n["B"]),
            _need(D, "D", torch.float32, n["D"])]
    py = _need(out, "out", td, n["y"])
    saved, ps, ns = _device_buffer(lingen_ma_saved_bytes(shape), saved)
    cs = to_c_shape(shape)
    _check("lingen_ma_fwd_saved", lib().lingen_ma_fwd_saved(*args, int(mode), ctypes.byref(cs), py, ps, ns, _stream()))
    return out, saved


def lingen_ma_bwd_saved(x, dt, A, B, C, D, dy, saved, mode: int, shape, grads=None, workspace=None):
    """lingen_ma_bwd from the scan states lingen_ma_fwd_saved left in
    ``saved`` (same inputs and mode); the same gradients."""
    args = _ma_bwd_inputs(shape, x, dt, A, B, C, D, dy)
    grads, pg = _ma_grads(shape, grads)
    _, ps, ns = _device_buffer(0, saved)
    workspace, pw, nw = _device_buffer(lingen_ma_bwd_saved_workspace_bytes(shape), workspace)
    cs = to_c_shape(shape)
    _check("lingen_ma_bwd_saved", lib().lingen_ma_bwd_saved(*args, ps, ns, int(mode), ctypes.byref(cs), *pg, pw, nw,
                                                            _stream()))
    return grads
