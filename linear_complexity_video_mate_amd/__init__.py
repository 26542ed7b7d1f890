"""MI355X-native (gfx950) MATE token mixer of LinGen: Python binding.

The mixer itself lives in ``liblingen_mate.so`` (hand-written HIP kernels
behind the C ABI of ``include/lingen_mate.h``); this package only loads it and
marshals torch tensors into it.  Build the library with
``python -m linear_complexity_video_mate_amd.build``.
"""
from .binding import (
    EXPORTS,
    LIB_PATH,
    LINGEN_BF16,
    LINGEN_F32,
    LingenError,
    STATUS_NAMES,
    lib,
    lingen_dense_attn_fwd,
    lingen_ma_prep,
    lingen_gated_rmsnorm,
    lingen_ma_fwd,
    lingen_ma_fwd_dirs,
    lingen_mate_fwd,
    lingen_mate_fwd_events,
    lingen_mate_validate,
    lingen_mate_workspace_bytes,
    lingen_rms_gather,
    lingen_rms_index,
    lingen_rms_index_device,
    lingen_ssd_chunk_states,
    lingen_te_fwd,
    lingen_te_bwd,
    lingen_te_fwd_shift,
    status_str,
    to_c_shape,
)

__all__ = [
    "EXPORTS",
    "LIB_PATH",
    "LINGEN_BF16",
    "LINGEN_F32",
    "LingenError",
    "STATUS_NAMES",
    "lib",
    "lingen_dense_attn_fwd",
    "lingen_ma_prep",
    "lingen_gated_rmsnorm",
    "lingen_ma_fwd",
    "lingen_ma_fwd_dirs",
    "lingen_mate_fwd",
    "lingen_mate_fwd_events",
    "lingen_mate_validate",
    "lingen_mate_workspace_bytes",
    "lingen_rms_gather",
    "lingen_rms_index",
    "lingen_rms_index_device",
    "lingen_ssd_chunk_states",
    "lingen_te_fwd",
    "lingen_te_bwd",
    "lingen_te_fwd_shift",
    "status_str",
    "to_c_shape",
]
