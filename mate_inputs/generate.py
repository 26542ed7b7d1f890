"""Seeded input generator.

Every tensor is drawn from its own stream, ``SeedSequence([seed, cfg_id,
tensor_id, head])``, so one head of a large configuration can be regenerated on
its own (the full-size parity tests check sampled heads against the oracle).

Distributions (the same for every configuration):
  x ~ N(0,1); dt = softplus(z), z ~ N(-3,1); A = -exp(u), u ~ U(0, ln 16) per
  head; B, C ~ N(0, sd = 1/sqrt(N)); D ~ N(0,1) per head; q, k, v ~ N(0,1).

bf16 configurations round x, B, C, q, k, v to bfloat16 (round to nearest even)
here, on the host; dt, A and D stay fp32.  The arrays are stored as raw bf16 bit
patterns (uint16) or float32, and ``f64`` gives the exact values as float64.
"""
from __future__ import annotations

import concurrent.futures as _fut
import math
from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence

import numpy as np

from .configs import MateShape

TENSOR_IDS = {"x": 0, "dt": 1, "A": 2, "B": 3, "C": 4, "D": 5, "q": 6, "k": 7, "v": 8}
# Tensors of the steps around the scan (make_block_inputs).
BLOCK_TENSOR_IDS = {"xbc": 9, "dt_raw": 10, "dt_bias": 11, "conv_w_f": 12, "conv_b_f": 13, "conv_w_b": 14,
                    "conv_b_b": 15, "z": 16, "y": 17, "norm_w": 18, "u": 19, "w_z": 20, "w_xbc": 21, "w_dt": 22,
                    "w_out_ma": 23, "w_q": 24, "w_k": 25, "w_v": 26, "w_o": 27, "A_f": 28, "A_b": 29, "D_f": 30,
                    "D_b": 31}
DEFAULT_SEED = 20241212


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest, ties to even.

    NaN/Inf do not occur in generated data; they are not special-cased.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, cfg_id: int, tensor: str, head: int) -> np.random.Generator:
    tid = TENSOR_IDS[tensor] if tensor in TENSOR_IDS else BLOCK_TENSOR_IDS[tensor]
    ss = np.random.SeedSequence([seed, cfg_id, tid, head])
    return np.random.Generator(np.random.PCG64(ss))


def _normal(seed, cfg_id, tensor, head, n, scale=1.0) -> np.ndarray:
    z = _rng(seed, cfg_id, tensor, head).standard_normal(n, dtype=np.float32)
    if scale != 1.0:
        z *= np.float32(scale)
    return z


@dataclass
class MateInputs:
    """Inputs of one batch element in storage form.

    ``store[name]`` is uint16 (bf16 bits) for x, B, C, q, k, v in bf16
    configurations and float32 otherwise.  Layouts: x [L, Hs', P], dt [L, Hs'],
    A [Hs'], B and C [L, N] ([L, G, N] with G > 1 groups), D [Hs'],
    q, k, v [L, Ha', d]; Hs' and Ha' count
    only the generated heads (``heads``), which default to all.
    """

    shape: MateShape
    cfg_id: int
    seed: int
    heads: Sequence[int]
    store: Dict[str, np.ndarray] = field(default_factory=dict)

    def is_bf16(self, name: str) -> bool:
        return self.store[name].dtype == np.uint16

    def f32(self, name: str) -> np.ndarray:
        a = self.store[name]
        return f32_from_bf16_bits(a) if a.dtype == np.uint16 else a

    def f64(self, name: str) -> np.ndarray:
        return self.f32(name).astype(np.float64)

    def torch(self, name: str, device="cuda"):
        import torch  # local import: the oracle tests do not need torch

        a = self.store[name]
        if a.dtype == np.uint16:
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(a)
        return t.to(device)


def make_inputs(shape: MateShape, cfg_id: int, seed: int = DEFAULT_SEED,
                heads: Optional[Sequence[int]] = None, threads: int = 8,
                tensors: Optional[Sequence[str]] = None) -> MateInputs:
    """Generate the inputs of one batch element.

    ``heads`` restricts x, dt, A, D (SSD heads) and q, k, v (attention heads)
    to the listed head indices; values for a head do not depend on which other
    heads are generated.  ``tensors`` restricts which tensors are produced.
    """
    L, P, N, d = shape.L, shape.headdim, shape.d_state, shape.attn_headdim
    Hs, Ha = shape.ssd_heads, shape.attn_heads
    if heads is None:
        hs_list = list(range(Hs))
        ha_list = list(range(Ha))
    else:
        hs_list = [h for h in heads if h < Hs]
        ha_list = [h for h in heads if h < Ha]
    want = set(tensors) if tensors is not None else set(TENSOR_IDS)
    bf16 = shape.dtype == "bf16"
    sdt = np.uint16 if bf16 else np.float32

    def finish(a32: np.ndarray) -> np.ndarray:
        return bf16_bits_from_f32(a32) if bf16 else a32

    out = MateInputs(shape=shape, cfg_id=cfg_id, seed=seed, heads=list(heads) if heads is not None else list(range(max(Hs, Ha))))
    jobs = []

    def per_head(name, hl, width):
        arr = np.empty((L, len(hl), width), dtype=sdt)
        out.store[name] = arr

        def fill(j, h):
            arr[:, j, :] = finish(_normal(seed, cfg_id, name, h, L * width).reshape(L, width))

        for j, h in enumerate(hl):
            jobs.append((fill, j, h))

    if "x" in want:
        per_head("x", hs_list, P)
    for name in ("q", "k", "v"):
        if name in want:
            per_head(name, ha_list, d)

    if "dt" in want:
        dt = np.empty((L, len(hs_list)), dtype=np.float32)
        out.store["dt"] = dt

        def fill_dt(j, h):
            z = _rng(seed, cfg_id, "dt", h).standard_normal(L).astype(np.float64) - 3.0
            # softplus(z) = log(1 + e^z), evaluated stably
            sp = np.where(z > 20.0, z, np.log1p(np.exp(np.minimum(z, 20.0))))
            dt[:, j] = sp.astype(np.float32)

        for j, h in enumerate(hs_list):
            jobs.append((fill_dt, j, h))

    if "A" in want:
        u = _rng(seed, cfg_id, "A", 0).uniform(0.0, math.log(16.0), Hs)
        out.store["A"] = (-np.exp(u)).astype(np.float32)[hs_list]
    if "D" in want:
        out.store["D"] = _rng(seed, cfg_id, "D", 0).standard_normal(Hs).astype(np.float32)[hs_list]
    G = shape.ngroups
    for name in ("B", "C"):
        if name in want:
            # group g draws from stream g (the head slot of the seed), so the
            # single-group tensors are those of group 0; layout [L, N] for one
            # group, [L, G, N] for several
            groups = [_normal(seed, cfg_id, name, g, L * N, 1.0 / math.sqrt(N)).reshape(L, N) for g in range(G)]
            out.store[name] = finish(groups[0] if G == 1 else np.stack(groups, axis=1))

    if threads > 1 and len(jobs) > 1:
        with _fut.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda j: j[0](j[1], j[2]), jobs))
    else:
        for f, j, h in jobs:
            f(j, h)
    return out


def make_block_inputs(shape: MateShape, cfg_id: int, seed: int = DEFAULT_SEED, conv_k: int = 4,
                      rows: Optional[int] = None, tensors: Optional[Sequence[str]] = None) -> MateInputs:
    """Inputs of the steps either side of the scan, for one batch element,
    following the Mamba-2 block's initialisation:
      xbc [L, Hs*P + 2*G*N] ~ N(0, 1) (the projected x, B, C channels);
      conv_w_f, conv_w_b [Ch, K], conv_b_f, conv_b_b [Ch] ~ U(-1/sqrt(K), 1/sqrt(K))
        (a depthwise convolution's default fan-in bound);
      dt_raw [L, Hs] ~ N(0, 0.5^2); dt_bias [Hs] = log(expm1(dt0)), dt0
        log-uniform in [1e-3, 1e-1] (the inverse softplus of Mamba's dt range);
      y, z [rows, Hs*P] ~ N(0, 1) (scan output and gate; rows defaults to L);
      norm_w [Hs*P] ~ 1 + 0.1 N(0, 1).
    xbc, y, z are rounded to bf16 in bf16 configurations; the rest is fp32.
    Each tensor draws from its own stream; ``tensors`` restricts which are
    produced.
    """
    L, Hs = shape.L, shape.ssd_heads
    d = Hs * shape.headdim
    ch = d + 2 * shape.ngroups * shape.d_state
    rows = L if rows is None else rows
    bf16 = shape.dtype == "bf16"

    def finish(a32):
        return bf16_bits_from_f32(a32) if bf16 else a32

    out = MateInputs(shape=shape, cfg_id=cfg_id, seed=seed, heads=list(range(Hs)))
    st = out.store
    want = set(tensors) if tensors is not None else set(BLOCK_TENSOR_IDS)
    if "xbc" in want:
        st["xbc"] = finish(_normal(seed, cfg_id, "xbc", 0, L * ch).reshape(L, ch))
    bound = 1.0 / math.sqrt(conv_k)
    for name, n in (("conv_w_f", ch * conv_k), ("conv_b_f", ch), ("conv_w_b", ch * conv_k), ("conv_b_b", ch)):
        if name in want:
            a = _rng(seed, cfg_id, name, 0).uniform(-bound, bound, n).astype(np.float32)
            st[name] = a.reshape(ch, conv_k) if name.startswith("conv_w") else a
    if "dt_raw" in want:
        st["dt_raw"] = _normal(seed, cfg_id, "dt_raw", 0, L * Hs, 0.5).reshape(L, Hs)
    if "dt_bias" in want:
        dt0 = np.exp(_rng(seed, cfg_id, "dt_bias", 0).uniform(math.log(1e-3), math.log(1e-1), Hs))
        st["dt_bias"] = np.log(np.expm1(dt0)).astype(np.float32)
    for name in ("y", "z"):
        if name in want:
            st[name] = finish(_normal(seed, cfg_id, name, 0, rows * d).reshape(rows, d))
    if "norm_w" in want:
        st["norm_w"] = (1.0 + 0.1 * _normal(seed, cfg_id, "norm_w", 0, d)).astype(np.float32)
    return out


def make_block_weights(shape: MateShape, cfg_id: int, d_model: int, seed: int = DEFAULT_SEED,
                       conv_k: int = 4) -> MateInputs:
    """Input u [L, d_model] and every weight of one MATE block (the names of
    the library's block weights):
      u ~ N(0, 1);
      projections w_z [d, Dm], w_xbc [d + 2GN, Dm], w_dt [Hs, Dm],
        w_out_ma [Dm, d], w_q, w_k, w_v [d, Dm], w_o [Dm, d] ~ U(-1/sqrt(in),
        1/sqrt(in)) (a linear layer's default bound, no bias);
      A_f, A_b = -exp(U(0, ln 16)) per head; D_f, D_b ~ 1 + 0.1 N(0, 1);
      conv weights and biases, dt_bias and norm_w as in make_block_inputs.
    u and the projections are rounded to bf16 in bf16 configurations.
    """
    d = shape.ssd_heads * shape.headdim
    ch = d + 2 * shape.ngroups * shape.d_state
    hs = shape.ssd_heads
    bf16 = shape.dtype == "bf16"

    def finish(a32):
        return bf16_bits_from_f32(a32) if bf16 else a32

    out = make_block_inputs(shape, cfg_id, seed, conv_k,
                            tensors=("conv_w_f", "conv_b_f", "conv_w_b", "conv_b_b", "dt_bias", "norm_w"))
    st = out.store
    st["u"] = finish(_normal(seed, cfg_id, "u", 0, shape.L * d_model).reshape(shape.L, d_model))
    for name, rows, cols in (("w_z", d, d_model), ("w_xbc", ch, d_model), ("w_dt", hs, d_model),
                             ("w_out_ma", d_model, d), ("w_q", d, d_model), ("w_k", d, d_model),
                             ("w_v", d, d_model), ("w_o", d_model, d)):
        bound = 1.0 / math.sqrt(cols)
        a = _rng(seed, cfg_id, name, 0).uniform(-bound, bound, rows * cols).astype(np.float32)
        st[name] = finish(a.reshape(rows, cols))
    for name in ("A_f", "A_b"):
        st[name] = (-np.exp(_rng(seed, cfg_id, name, 0).uniform(0.0, math.log(16.0), hs))).astype(np.float32)
    for name in ("D_f", "D_b"):
        st[name] = (1.0 + 0.1 * _normal(seed, cfg_id, name, 0, hs)).astype(np.float32)
    return out
