"""Plain fp64 CPU oracle for the LinGen MATE token mixer (forward pass).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the smoke check and the benchmark's CPU
baseline use it.  It shares no code with the HIP library (the two meet only in
the seeded inputs of ``mate_inputs``).

Sources (cited by page title and section throughout):
  [ABS]  "Towards High-Resolution Minute-Length Text-to-Video Generation with
         Linear Computational Complexity" -- the English abstract (原文摘要).
  [ART]  "视频生成模子太贵太慢如何办？" (QbitAI article) -- section
         "要领：线性复杂度的 MATE 模块" (method) and "评估" (evaluation).
  [ZH]   "LinGen：基于Mamba机制的线性复杂度高清长视频生成框架" -- sections
         "功能特色", "技术细节" and "关键算法创新".
  [SSD]  Mamba2's selective state-space recurrence in its scalar-A form
         (Dao & Gu, "Transformers are SSMs", 2024), which the pages name as the
         MA branch's building block ([ABS]; [ART] 要领).

Every function here is pinned by the tests in ``tests/test_oracle_*.py``
against hand-derived fixtures, closed forms, textbook special cases and brute
force on tiny inputs.  Whether LinGen itself used exactly these conventions is
not something the pages settle (they print no values): parity unpinned with
respect to the original model, pinned with respect to the readings listed in
each docstring.
"""
from .mate_oracle import (
    rms_mode,
    tesa_shift,
    rms_scan_order,
    rms_inverse,
    ssd_scan,
    ssd_bidir,
    ssd_dirs,
    ssd_scan_backward,
    ssd_bidir_backward,
    review_tokens,
    review_state,
    tesa_window_keys,
    tesa,
    tesa_for_queries,
    tesa_backward,
    tesa_lse,
    dense_attention,
    scan_conv_silu,
    ma_prep,
    gated_rmsnorm,
    silu,
    softplus,
    dense_attention_for_queries,
    mate_fwd,
    ma_fwd,
    ma_bwd,
    mate_block,
)

__all__ = [
    "rms_mode",
    "tesa_shift",
    "rms_scan_order",
    "rms_inverse",
    "ssd_scan",
    "ssd_bidir",
    "ssd_dirs",
    "ssd_scan_backward",
    "ssd_bidir_backward",
    "review_tokens",
    "review_state",
    "tesa_window_keys",
    "tesa",
    "tesa_for_queries",
    "tesa_backward",
    "tesa_lse",
    "dense_attention",
    "scan_conv_silu",
    "ma_prep",
    "gated_rmsnorm",
    "silu",
    "softplus",
    "dense_attention_for_queries",
    "mate_fwd",
    "mate_block",
    "ma_fwd",
    "ma_bwd",
]
