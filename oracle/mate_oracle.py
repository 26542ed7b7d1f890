"""fp64 reference implementation of the MATE token mixer.

TEST INFRASTRUCTURE ONLY (see the package docstring for the source legend
[ABS], [ART], [ZH], [SSD] and for who may use this module).

Tensor conventions (one batch element; canonical token order is (t, h, w)
row-major, token index c = (t*H + h)*W + w):
  x  [L, Hs, P]   SSD input, one P-vector per (token, head)
  dt [L, Hs]      positive step sizes (already passed through softplus)
  A  [Hs]         negative scalar decay rate per head
  B, C [L, N]     input / output projections, shared by all heads (one group)
  D  [Hs]         skip weight per head
  q, k, v [L, Ha, d]
All arithmetic is float64.  Inputs may be any float dtype; they are upcast.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------
# Layer schedule: which scan order and which window phase a layer uses.
# --------------------------------------------------------------------------


def rms_mode(layer_idx: int) -> int:
    """Scan mode of a layer.

    [ART] 要领 and [ZH] 关键算法创新 (Rotary Major Scan): four scan orders are
    used in turn on adjacent layers.  Reading taken: mode = layer_idx mod 4,
    in the order the four modes are listed on [ZH].
    """
    if layer_idx < 0:
        raise ValueError("layer_idx must be >= 0")
    return layer_idx % 4


def tesa_shift(layer_idx: int, win: Tuple[int, int, int]) -> Tuple[int, int, int]:
    """Window-grid offset of a layer.

    [ZH] 技术细节 / 关键算法创新 (TEmporal Swin Attention): plain and shifted
    window partitions alternate between adjacent layers.  Reading taken:
    odd layers are shifted, by half a window (floored) along each axis, as in
    Swin attention; even layers are not shifted.
    """
    if layer_idx < 0:
        raise ValueError("layer_idx must be >= 0")
    if layer_idx % 2 == 1:
        return tuple(w // 2 for w in win)
    return (0, 0, 0)


# --------------------------------------------------------------------------
# Rotary Major Scan: the four token orders.
# --------------------------------------------------------------------------

# For each mode, the order of the (T, H, W) axes from slowest to fastest.
# "First priority" in the pages is the axis unfolded first, i.e. the one that
# varies fastest along the scan.
#   mode 0  spatial row-major:     W fastest, then H, then T
#   mode 1  spatial column-major:  H fastest, then W, then T
#   mode 2  temporal row-major:    T fastest, then W, then H
#   mode 3  temporal column-major: T fastest, then H, then W
_RMS_AXES = {0: (0, 1, 2), 1: (0, 2, 1), 2: (1, 2, 0), 3: (2, 1, 0)}


def rms_scan_order(mode: int, T: int, H: int, W: int) -> np.ndarray:
    """perm[s] = canonical index of the token visited at scan position s.

    [ART] 要领: W, H and T carry the first, second and third unfolding
    priority in the default order, and swapping the priorities gives the other
    scans, which need nothing beyond reshaping the token tensor.  [ZH]
    关键算法创新 names the four modes (spatial row-major with W highest,
    spatial column-major with H highest, temporal row-major and temporal
    column-major with T highest).  Written, as the pages say, as a reshape and
    an axis permutation of the (T, H, W) index grid.
    """
    if mode not in _RMS_AXES:
        raise ValueError(f"RMS mode must be 0..3, got {mode}")
    grid = np.arange(T * H * W, dtype=np.int64).reshape(T, H, W)
    return grid.transpose(_RMS_AXES[mode]).ravel()


def rms_inverse(perm: np.ndarray) -> np.ndarray:
    """inv[c] = scan position of canonical token c."""
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=perm.dtype)
    return inv


# --------------------------------------------------------------------------
# Selective SSM scan (MA branch).
# --------------------------------------------------------------------------


def _per_head(M, Hs: int) -> np.ndarray:
    """B or C as [L, Hs, N]: from [L, N] (one group, shared by every head) or
    [L, G, N] (G groups; head h uses group h // (Hs // G), Mamba2's grouping
    of heads)."""
    M = np.asarray(M, dtype=np.float64)
    if M.ndim == 2:
        return np.broadcast_to(M[:, None, :], (M.shape[0], Hs, M.shape[1]))
    G = M.shape[1]
    if Hs % G:
        raise ValueError("the number of groups must divide the number of heads")
    return np.repeat(M, Hs // G, axis=1)


def ssd_scan(x, dt, A, B, C, D, order: Sequence[int], h0=None,
             record_after: Iterable[int] = (), stats: Optional[Dict] = None):
    """Run the scalar-A selective SSM recurrence over tokens in ``order``.

    [SSD]: per head, with state h in R^{P x N} (h = h0, zero by default),
    for each visited token c:
        h <- exp(dt_c * A) * h + dt_c * (x_c outer B_c)
        y_c = h C_c + D * x_c
    The decay applied when a token is absorbed uses that token's own dt.
    B and C are [L, N] (shared by all heads) or [L, G, N] (see ``_per_head``).

    Returns (y, h_final, recorded) where y[c] is set for every visited c (zero
    elsewhere) and recorded[k] is the state after the first k visited tokens,
    for each k in ``record_after``.
    """
    x = np.asarray(x, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = _per_head(B, x.shape[1])
    C = _per_head(C, x.shape[1])
    D = np.asarray(D, dtype=np.float64)
    Hs, P = x.shape[1], x.shape[2]
    N = B.shape[2]
    h = np.zeros((Hs, P, N)) if h0 is None else np.array(h0, dtype=np.float64, copy=True)
    y = np.zeros(x.shape, dtype=np.float64)
    want = set(int(k) for k in record_after)
    recorded = {}
    if 0 in want:
        recorded[0] = h.copy()
    step = 0
    for c in order:
        decay = np.exp(dt[c] * A)                         # [Hs]
        u = dt[c][:, None] * x[c]                         # [Hs, P]
        h = decay[:, None, None] * h + u[:, :, None] * B[c][:, None, :]
        y[c] = np.matmul(h, C[c][:, :, None])[:, :, 0] + D[:, None] * x[c]
        step += 1
        if step in want:
            recorded[step] = h.copy()
    if stats is not None:
        stats["ssd_steps"] = stats.get("ssd_steps", 0) + step
    return y, h, recorded


def ssd_bidir(x, dt, A, B, C, D, perm: np.ndarray, h0=None, stats=None):
    """Bidirectional scan: the forward scan along ``perm`` plus the same scan
    along the reversed order, summed per token in canonical order.

    [ABS]: the MA branch is a bidirectional Mamba2 block.  Readings taken:
    both directions share x, dt, A, B, C, D; the backward direction is the
    plain scan over the reversed sequence ("flip, run, flip back"); each
    direction carries its own D skip, so the sum holds 2*D*x; a review-token
    state h0, when present, is the initial state of both directions.
    """
    perm = np.asarray(perm)
    y_f, _, _ = ssd_scan(x, dt, A, B, C, D, perm, h0=h0, stats=stats)
    y_b, _, _ = ssd_scan(x, dt, A, B, C, D, perm[::-1], h0=h0, stats=stats)
    return y_f + y_b


def _fold_groups(d_per_head, like) -> np.ndarray:
    """Sum a per-head gradient [L, Hs, N] over the heads of each group, into
    the layout of ``like`` ([L, N] for one group, [L, G, N] for several)."""
    like = np.asarray(like)
    L, Hs, N = d_per_head.shape
    if like.ndim == 2:
        return d_per_head.sum(axis=1)
    G = like.shape[1]
    return d_per_head.reshape(L, G, Hs // G, N).sum(axis=2)


def ssd_scan_backward(x, dt, A, B, C, D, dy, order: Sequence[int], h0=None, segment: int = 64,
                      g_final=None, return_dh0: bool = False):
    """Gradients of sum(dy * y) for y = ssd_scan(x, dt, A, B, C, D, order)[0]
    with respect to x, dt, A, B, C, D: (dx, ddt, dA, dB, dC, dD), each in
    the layout of its input.

    The adjoint of the recurrence in ``ssd_scan``, walked backwards over the
    visited tokens: with g the adjoint of the state after token c (g <- dy_c
    C_c^T + exp(dt_next A) g_next),
        dx_c  = dt_c g B_c + D dy_c          dB_c = dt_c g^T x_c
        dC_c  = h_c^T dy_c                   dD  += dy_c . x_c
        ddt_c = x_c^T g B_c + A exp(dt_c A) <h_prev, g>
        dA   += dt_c exp(dt_c A) <h_prev, g>
    per head (dB, dC summed over the heads of a group).  The states h are
    kept every ``segment`` tokens and recomputed within a segment.

    ``g_final`` [Hs, P, N]: the adjoint of the state after the last visited
    token (the scan's final state feeds something else: the review tokens'
    state feeds the main scan), zero by default.  With ``return_dh0`` the
    adjoint of the initial state h0, i.e. g after the walk has passed the
    first token, is returned as a seventh value.
    """
    x = np.asarray(x, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    Hs, P = x.shape[1], x.shape[2]
    Bh = _per_head(B, Hs)
    Ch = _per_head(C, Hs)
    N = Bh.shape[2]
    order = np.asarray(order)
    n = len(order)

    def absorb(h, c):
        a = np.exp(dt[c] * A)
        return a[:, None, None] * h + (dt[c][:, None] * x[c])[:, :, None] * Bh[c][:, None, :]

    h = np.zeros((Hs, P, N)) if h0 is None else np.array(h0, dtype=np.float64, copy=True)
    ckpt = {}
    for i, c in enumerate(order):
        if i % segment == 0:
            ckpt[i] = h.copy()                  # state before token i
        h = absorb(h, c)

    dx = np.zeros_like(x)
    ddt = np.zeros_like(dt)
    dA = np.zeros(Hs)
    dBh = np.zeros((x.shape[0], Hs, N))
    dCh = np.zeros((x.shape[0], Hs, N))
    dD = np.zeros(Hs)
    # adjoint of the state after the token being visited
    g = np.zeros((Hs, P, N)) if g_final is None else np.array(g_final, dtype=np.float64, copy=True)
    for start in reversed(range(0, n, segment)):
        idx = order[start:start + segment]
        states = []
        h = ckpt[start].copy()
        for c in idx:
            h = absorb(h, c)
            states.append(h)
        for j in reversed(range(len(idx))):
            c = idx[j]
            h_t = states[j]
            h_prev = states[j - 1] if j > 0 else ckpt[start]
            g = g + dy[c][:, :, None] * Ch[c][:, None, :]
            dCh[c] += np.einsum("hpn,hp->hn", h_t, dy[c])
            dx[c] += D[:, None] * dy[c]
            dD += np.sum(dy[c] * x[c], axis=1)
            a = np.exp(dt[c] * A)
            gB = np.einsum("hpn,hn->hp", g, Bh[c])
            dx[c] += dt[c][:, None] * gB
            dBh[c] += dt[c][:, None] * np.einsum("hpn,hp->hn", g, x[c])
            cross = np.sum(g * h_prev, axis=(1, 2))
            ddt[c] += np.sum(x[c] * gB, axis=1) + A * a * cross
            dA += dt[c] * a * cross
            g = a[:, None, None] * g
    grads = (dx, ddt, dA, _fold_groups(dBh, B), _fold_groups(dCh, C), dD)
    return grads + (g,) if return_dh0 else grads


def ssd_bidir_backward(x, dt, A, B, C, D, dy, perm: np.ndarray):
    """Gradients of sum(dy * y) for the shared-parameter bidirectional scan
    ``ssd_bidir`` (no review state): the two directions' gradients summed."""
    perm = np.asarray(perm)
    f = ssd_scan_backward(x, dt, A, B, C, D, dy, perm)
    b = ssd_scan_backward(x, dt, A, B, C, D, dy, perm[::-1])
    return tuple(u + v for u, v in zip(f, b))


def ma_bwd(x, dt, A, B, C, D, dy, mode: int, T: int, H: int, W: int, review=None):
    """Gradients of sum(dy * y_MA) for y_MA = ``ma_fwd(x, dt, A, B, C, D,
    mode, T, H, W, review)``: (dx, ddt, dA, dB, dC, dD) in the layouts of
    the inputs.

    Without review tokens this is ``ssd_bidir_backward``.  With them, the
    review state h_R starts both directions, so the adjoints that reach the
    initial state of the two directions add up to dh_R; h_R is the final
    state of the scan over the review tokens, whose outputs are discarded, so
    that scan is walked backwards from dh_R with no output adjoint, giving
    the gradients of the pooled review x, dt and B and a share of dA; each
    pooled value is a block mean, so its gradient is spread evenly over the
    tokens of its pooling block (``review_tokens``).
    """
    perm = rms_scan_order(mode, T, H, W)
    if review is None:
        return ssd_bidir_backward(x, dt, A, B, C, D, dy, perm)
    rpool, rgrid = review
    h0 = review_state(x, dt, A, B, C, T, H, W, rpool, rgrid)
    f = ssd_scan_backward(x, dt, A, B, C, D, dy, perm, h0=h0, return_dh0=True)
    b = ssd_scan_backward(x, dt, A, B, C, D, dy, perm[::-1], h0=h0, return_dh0=True)
    dx, ddt, dA, dB, dC, dD = (u + v for u, v in zip(f[:6], b[:6]))
    dhR = f[6] + b[6]
    xr, dtr, Br, Cr = review_tokens(x, dt, B, C, T, H, W, rpool, rgrid)
    R = xr.shape[0]
    zero_D = np.zeros(np.shape(A))
    rg = ssd_scan_backward(xr, dtr, A, Br, Cr, zero_D, np.zeros(xr.shape), np.arange(R), g_final=dhR)
    dxr, ddtr, dAr, dBr = rg[0], rg[1], rg[2], rg[3]
    dA = dA + dAr
    # spread each review token's gradient over its pooling block
    pt, ph, pw = rpool
    gt, gh, gw = T // pt, H // ph, W // pw
    rt, rh, rw = rgrid
    st, sh, sw = gt // rt, gh // rh, gw // rw
    cnt = pt * ph * pw
    grid_views = [a.reshape((T, H, W) + a.shape[1:]) for a in (dx, ddt, dB)]
    r = 0
    for i in range(rt):
        for j in range(rh):
            for k in range(rw):
                t0, h0_, w0 = i * st * pt, j * sh * ph, k * sw * pw
                blk = (slice(t0, t0 + pt), slice(h0_, h0_ + ph), slice(w0, w0 + pw))
                for view, g in zip(grid_views, (dxr, ddtr, dBr)):
                    view[blk] += g[r] / cnt
                r += 1
    return dx, ddt, dA, dB, dC, dD


def ssd_dirs(fwd, bwd, perm: np.ndarray, review=None, grid=None):
    """Bidirectional scan with a parameter set per direction: the scan of
    ``fwd`` = (x, dt, A, B, C, D) along ``perm`` plus the scan of ``bwd`` along
    the reversed order, summed per token; each direction carries its own D
    skip.

    [ABS] names a bidirectional Mamba2 block without saying whether the two
    directions share weights; this is the reading in which they do not (the
    mixer's default, ``ssd_bidir``, shares them).

    ``review`` = (rpool, rgrid) with ``grid`` = (T, H, W): review tokens
    ([ART] 要领).  Reading taken with a parameter set per direction: each
    direction forms its review tokens from its own inputs (its x, dt, B, C)
    and scans them with its own A, so each direction starts from the state
    its own review tokens leave (``review_state``).
    """
    perm = np.asarray(perm)
    h0_f = h0_b = None
    if review is not None:
        rpool, rgrid = review
        T, H, W = grid
        xf, dtf, Af, Bf, Cf, _ = fwd
        xb, dtb, Ab, Bb, Cb, _ = bwd
        h0_f = review_state(xf, dtf, Af, Bf, Cf, T, H, W, rpool, rgrid)
        h0_b = review_state(xb, dtb, Ab, Bb, Cb, T, H, W, rpool, rgrid)
    y_f, _, _ = ssd_scan(*fwd, perm, h0=h0_f)
    y_b, _, _ = ssd_scan(*bwd, perm[::-1], h0=h0_b)
    return y_f + y_b


# --------------------------------------------------------------------------
# Review tokens.
# --------------------------------------------------------------------------


def review_tokens(x, dt, B, C, T: int, H: int, W: int,
                  rpool: Tuple[int, int, int], rgrid: Tuple[int, int, int]):
    """Build the review tokens from the token tensor.

    [ART] 要领 / [ZH] 功能特色: review tokens give the Mamba hidden state an
    overview of the whole video tensor before the scan starts.  The pages do
    not say how the overview is formed.  Reading taken: mean-pool x, dt, B and
    C over non-overlapping rpool blocks, giving a (T/pt, H/ph, W/pw) grid, then
    keep rgrid points per axis at a regular stride starting from 0, listed in
    canonical (t, h, w) order.
    """
    pt, ph, pw = rpool
    gt, gh, gw = T // pt, H // ph, W // pw
    rt, rh, rw = rgrid
    st, sh, sw = gt // rt, gh // rh, gw // rw

    def pool(a):
        a = np.asarray(a, dtype=np.float64)
        feat = a.shape[1:]
        g = a.reshape((gt, pt, gh, ph, gw, pw) + feat).mean(axis=(1, 3, 5))
        s = g[::st, ::sh, ::sw][:rt, :rh, :rw]
        return s.reshape((rt * rh * rw,) + feat)

    return pool(x), pool(dt), pool(B), pool(C)


def review_state(x, dt, A, B, C, T, H, W, rpool, rgrid):
    """State after scanning the review tokens from a zero state, [Hs, P, N].

    Reading taken: the review tokens are scanned once, in canonical order, and
    their outputs are discarded; only the state they leave is kept and handed
    to both scan directions of the main sequence.
    """
    xr, dtr, Br, Cr = review_tokens(x, dt, B, C, T, H, W, rpool, rgrid)
    R = xr.shape[0]
    zeroD = np.zeros(np.asarray(A).shape)
    _, h, _ = ssd_scan(xr, dtr, A, Br, Cr, zeroD, np.arange(R))
    return h


# --------------------------------------------------------------------------
# TEmporal Swin Attention (TE branch).
# --------------------------------------------------------------------------


def tesa_window_keys(T: int, H: int, W: int, win, shift, cyclic: bool = False) -> np.ndarray:
    """Window key of every token, [L, 3] (canonical order).

    [ART] 要领 / [ZH] 关键算法创新: TESA attends inside small 3D windows whose
    size is fixed regardless of resolution and length, and whose placement
    moves between layers.  Reading taken (Swin's shifted windows): the window
    grid is offset by ``shift``; a token (t, h, w) belongs to window
    (floor((t-st)/wt), floor((h-sh)/wh), floor((w-sw)/ww)).  Tokens cut off at
    the borders form smaller windows of their own; nothing wraps around.

    ``cyclic=True`` is the other reading of a shifted partition, not the one
    the mixer uses: the offset grid wraps around each axis, window
    (floor(((t-st) mod T)/wt), ...), so every window is whole (the axis
    lengths must be multiples of the window).
    """
    wt, wh, ww = win
    st, sh, sw = shift
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    if cyclic:
        if T % wt or H % wh or W % ww:
            raise ValueError("cyclic windows need axis lengths that are multiples of the window")
        keys = np.stack([((t - st) % T) // wt, ((h - sh) % H) // wh, ((w - sw) % W) // ww], axis=-1)
    else:
        keys = np.stack([(t - st) // wt, (h - sh) // wh, (w - sw) // ww], axis=-1)
    return keys.reshape(-1, 3)


def _attend(qg, kg, vg):
    """Softmax attention of one token set, all heads: [n, Ha, d] each."""
    d = qg.shape[-1]
    qh = qg.transpose(1, 0, 2)
    kh = kg.transpose(1, 0, 2)
    vh = vg.transpose(1, 0, 2)
    s = (qh @ kh.transpose(0, 2, 1)) / math.sqrt(d)      # [Ha, n, n]
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return (p @ vh).transpose(1, 0, 2)


def _groups(keys: np.ndarray):
    _, gid = np.unique(keys, axis=0, return_inverse=True)
    gid = np.asarray(gid).ravel()
    order = np.argsort(gid, kind="stable")
    counts = np.bincount(gid)
    return gid, order, counts


def tesa(q, k, v, T: int, H: int, W: int, win, shift, stats: Optional[Dict] = None, cyclic: bool = False):
    """o_i = sum_j softmax_j(q_i . k_j / sqrt(d)) v_j over the tokens j in the
    same window as token i, per head; returns [L, Ha, d].

    Readings taken: scale 1/sqrt(d); no positional bias, no causal mask; the
    window partition is ``tesa_window_keys`` (with ``cyclic`` passed on).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    keys = tesa_window_keys(T, H, W, win, shift, cyclic)
    _, order, counts = _groups(keys)
    o = np.empty(q.shape, dtype=np.float64)
    start = 0
    pairs = 0
    for n in counts:
        idx = order[start:start + n]
        start += n
        o[idx] = _attend(q[idx], k[idx], v[idx])
        pairs += int(n) * int(n)
    if stats is not None:
        stats["tesa_pairs"] = stats.get("tesa_pairs", 0) + pairs * q.shape[1]
    return o


def tesa_lse(q, k, T: int, H: int, W: int, win, shift, cyclic: bool = False) -> np.ndarray:
    """Per query and head, the base-2 log of the softmax denominator of its
    window, lse_i = log2 sum_j exp(q_i . k_j / sqrt(d)) over the tokens j in
    i's window (``tesa_window_keys``); returns [L, Ha].  The softmax weights
    of ``tesa`` are then 2^(q_i . k_j log2(e) / sqrt(d) - lse_i), the
    statistic the backward pass reuses instead of forming it again."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = q.shape[-1]
    keys = tesa_window_keys(T, H, W, win, shift, cyclic)
    _, order, counts = _groups(keys)
    lse = np.empty(q.shape[:2], dtype=np.float64)
    start = 0
    for n in counts:
        idx = order[start:start + n]
        start += n
        qh = q[idx].transpose(1, 0, 2)
        kh = k[idx].transpose(1, 0, 2)
        s = (qh @ kh.transpose(0, 2, 1)) / math.sqrt(d)     # [Ha, n, n]
        mx = s.max(axis=-1, keepdims=True)
        ln = mx[..., 0] + np.log(np.exp(s - mx).sum(axis=-1))
        lse[idx] = (ln / math.log(2.0)).T
    return lse


def tesa_backward(q, k, v, dO, T: int, H: int, W: int, win, shift, cyclic: bool = False):
    """Gradients of TESA, (dq, dk, dv), each [L, Ha, d], for an upstream
    gradient dO of the output: the chain rule through o = softmax(q k^T /
    sqrt(d)) v inside every window, per head.  With P the softmax weights of
    a window and s = 1/sqrt(d):
        dv = P^T dO
        dP = dO v^T
        dS = P * (dP - rowsum(dP * P))     (elementwise; the softmax Jacobian)
        dq = s dS k,   dk = s dS^T q
    Needed for training the mixer (the pages train LinGen progressively, [ART]
    要领 and [ZH] 技术细节); the partition is ``tesa_window_keys``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    sc = 1.0 / math.sqrt(q.shape[-1])
    keys = tesa_window_keys(T, H, W, win, shift, cyclic)
    _, order, counts = _groups(keys)
    dq, dk, dv = np.empty(q.shape), np.empty(k.shape), np.empty(v.shape)
    start = 0
    for n in counts:
        idx = order[start:start + n]
        start += n
        qh, kh, vh, gh = (a[idx].transpose(1, 0, 2) for a in (q, k, v, dO))      # [Ha, n, d]
        S = (qh @ kh.transpose(0, 2, 1)) * sc
        S -= S.max(axis=-1, keepdims=True)
        P = np.exp(S)
        P /= P.sum(axis=-1, keepdims=True)
        dP = gh @ vh.transpose(0, 2, 1)
        dS = P * (dP - (dP * P).sum(axis=-1, keepdims=True))
        dq[idx] = ((dS @ kh) * sc).transpose(1, 0, 2)
        dk[idx] = ((dS.transpose(0, 2, 1) @ qh) * sc).transpose(1, 0, 2)
        dv[idx] = (P.transpose(0, 2, 1) @ gh).transpose(1, 0, 2)
    return dq, dk, dv


def tesa_for_queries(q, k, v, T: int, H: int, W: int, win, shift,
                     query_idx: Sequence[int], cyclic: bool = False) -> np.ndarray:
    """TESA output for selected query tokens only, [len(query_idx), Ha, d].

    Same definition as ``tesa``; each query attends over its own window.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    query_idx = np.asarray(query_idx)
    keys = tesa_window_keys(T, H, W, win, shift, cyclic)
    gid, order, counts = _groups(keys)
    starts = np.concatenate([[0], np.cumsum(counts)])
    out = np.empty((query_idx.size, q.shape[1], q.shape[2]), dtype=np.float64)
    for g in np.unique(gid[query_idx]):
        members = order[starts[g]:starts[g + 1]]
        sel = np.nonzero(gid[query_idx] == g)[0]
        qi = query_idx[sel]
        d = q.shape[-1]
        qh = q[qi].transpose(1, 0, 2)
        kh = k[members].transpose(1, 0, 2)
        vh = v[members].transpose(1, 0, 2)
        s = (qh @ kh.transpose(0, 2, 1)) / math.sqrt(d)
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        out[sel] = (p @ vh).transpose(1, 0, 2)
    return out


# --------------------------------------------------------------------------
# Dense attention: the quadratic mixer MATE replaces.
# --------------------------------------------------------------------------


def dense_attention_for_queries(q, k, v, query_idx: Sequence[int],
                                head_block: int = 4) -> np.ndarray:
    """Softmax attention of the selected queries over ALL L tokens, per head:
    o_i = sum_j softmax_j(q_i . k_j / sqrt(d)) v_j, j = 0..L-1; returns
    [len(query_idx), Ha, d].

    [ABS] (MATE replaces DiT's self-attention, whose cost is quadratic in the
    token count) and [ART] 评估 (latency and FLOPs measured against the
    attention model).  Readings taken: the same scale, no mask and no bias as
    TESA, i.e. TESA with one window holding every token.  Heads are processed
    ``head_block`` at a time to bound memory.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    query_idx = np.asarray(query_idx, dtype=np.int64)
    d = q.shape[-1]
    Ha = q.shape[1]
    out = np.empty((query_idx.size, Ha, d), dtype=np.float64)
    for h0 in range(0, Ha, head_block):
        hs = slice(h0, min(Ha, h0 + head_block))
        qh = q[query_idx, hs].transpose(1, 0, 2)           # [hb, nq, d]
        kh = k[:, hs].transpose(1, 2, 0)                   # [hb, d, L]
        vh = v[:, hs].transpose(1, 0, 2)                   # [hb, L, d]
        s = (qh @ kh) / math.sqrt(d)                        # [hb, nq, L]
        s -= s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=-1, keepdims=True)
        out[:, hs] = (p @ vh).transpose(1, 0, 2)
    return out


def dense_attention(q, k, v) -> np.ndarray:
    """Dense softmax attention of every token over every token, per head,
    [L, Ha, d]; the definition of ``dense_attention_for_queries`` applied to
    all queries."""
    L = np.asarray(q).shape[0]
    return dense_attention_for_queries(q, k, v, np.arange(L))


# --------------------------------------------------------------------------
# Steps either side of the scan (Mamba2 block conventions).
# --------------------------------------------------------------------------


def silu(a):
    a = np.asarray(a, dtype=np.float64)
    return a / (1.0 + np.exp(-a))


def softplus(a):
    a = np.asarray(a, dtype=np.float64)
    return np.maximum(a, 0.0) + np.log1p(np.exp(-np.abs(a)))


def scan_conv_silu(u, w, b, order: Sequence[int]):
    """Depthwise causal convolution along a scan order, then SiLU.

    [SSD] (Mamba2 block): the x, B, C channels pass a short depthwise causal
    convolution and SiLU before the scan.  Reading taken for a scanned video
    tensor: causal along the order the scan visits the tokens.  u [L, Ch]
    (canonical rows), w [Ch, K], b [Ch]; for the token at scan position s,
        out[order[s], c] = silu(b[c] + sum_k w[c, k] u[order[s - K + 1 + k], c]),
    with u taken as 0 before the first position.
    """
    u = np.asarray(u, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    order = np.asarray(order)
    L, K = u.shape[0], w.shape[1]
    us = np.concatenate([np.zeros((K - 1, u.shape[1])), u[order]], axis=0)   # scan order, zero padded
    acc = np.broadcast_to(b, (L, u.shape[1])).copy()
    for k in range(K):
        acc += w[:, k] * us[k:k + L]
    out = np.empty_like(u)
    out[order] = silu(acc)
    return out


def ma_prep(xbc, dt_raw, w_f, b_f, w_b, b_b, dt_bias, order: Sequence[int], Hs: int, P: int, G: int, N: int):
    """The steps between the input projection and the scan, for a parameter
    set per scan direction: the xBC channels (x: Hs*P, then B: G*N, then C:
    G*N, Mamba2's split) convolved along the scan order (forward direction)
    and along the reversed order (backward direction), each with its own
    kernel and bias, then SiLU; and dt = softplus(dt_raw + dt_bias), shared.

    Returns (x_f, B_f, C_f, x_b, B_b, C_b, dt) with x [L, Hs, P], B and C
    [L, G, N], dt [L, Hs].
    """
    order = np.asarray(order)
    L = np.asarray(xbc).shape[0]
    outs = []
    for w, b, o in ((w_f, b_f, order), (w_b, b_b, order[::-1])):
        c = scan_conv_silu(xbc, w, b, o)
        d = Hs * P
        outs += [c[:, :d].reshape(L, Hs, P), c[:, d:d + G * N].reshape(L, G, N), c[:, d + G * N:].reshape(L, G, N)]
    dt = softplus(np.asarray(dt_raw, dtype=np.float64) + np.asarray(dt_bias, dtype=np.float64))
    return tuple(outs) + (dt,)


def gated_rmsnorm(y, z, w, eps: float, group: int):
    """Mamba2's gated RMS norm after the scan: g = y * silu(z), then every
    row's channels in groups of ``group`` are divided by their root mean
    square (plus eps inside the root) and multiplied by the weight w.
    y, z [rows, dim]; w [dim]."""
    g = np.asarray(y, dtype=np.float64) * silu(z)
    rows, dim = g.shape
    gg = g.reshape(rows, dim // group, group)
    r = np.sqrt((gg * gg).mean(axis=-1, keepdims=True) + eps)
    return (gg / r).reshape(rows, dim) * np.asarray(w, dtype=np.float64)


# --------------------------------------------------------------------------
# The whole mixer.
# --------------------------------------------------------------------------


def ma_fwd(x, dt, A, B, C, D, mode: int, T: int, H: int, W: int,
           review=None, stats=None):
    """MA branch: RMS order ``mode``, bidirectional scan, optional review state.

    ``review`` is None or (rpool, rgrid).  Returns y_MA [L, Hs, P].
    """
    perm = rms_scan_order(mode, T, H, W)
    h0 = None
    if review is not None:
        rpool, rgrid = review
        h0 = review_state(x, dt, A, B, C, T, H, W, rpool, rgrid)
    return ssd_bidir(x, dt, A, B, C, D, perm, h0=h0, stats=stats)


def mate_fwd(x, dt, A, B, C, D, q, k, v, layer_idx: int, T: int, H: int, W: int,
             win, review=None, stats=None):
    """MATE mixer: y = y_MA + o, both viewed as [L, Hs*P] (= [L, Ha*d]).

    [ABS]: MATE consists of an MA branch and a TE branch.  The pages do not
    say how the branch outputs are combined; reading taken: a plain sum with
    no weights, SSD head i and attention head i sharing columns i*P..i*P+P-1.
    """
    mode = rms_mode(layer_idx)
    shift = tesa_shift(layer_idx, win)
    y_ma = ma_fwd(x, dt, A, B, C, D, mode, T, H, W, review=review, stats=stats)
    o = tesa(q, k, v, T, H, W, win, shift, stats=stats)
    L = T * H * W
    return y_ma.reshape(L, -1) + o.reshape(L, -1)


# --------------------------------------------------------------------------
# The whole block around the mixer.
# --------------------------------------------------------------------------


def mate_block(u, w, layer_idx: int, T: int, H: int, W: int, Hs: int, P: int, G: int, N: int, Ha: int,
               win, eps: float = 1e-5, review=None):
    """The MATE block on u [L, Dm] (canonical token order): the MA branch
    and the TE branch, each with its projections, outputs summed.

    [ART] 要领: the block is an MA branch plus a TE branch in place of the
    self-attention.  Readings for what the pages leave open (the same as the
    library's): the MA branch follows the Mamba-2 block layout of [SSD]
    (section 7) -- z, xBC and dt_raw are projections of u, then ``ma_prep``,
    the per-direction scan ``ssd_dirs``, ``gated_rmsnorm`` with one group per
    B/C group, and an output projection; the TE branch projects q, k, v,
    applies ``tesa`` and projects its output.  No projection has a bias.
    ``w`` maps names to arrays: w_z [d, Dm], w_xbc [d + 2GN, Dm], w_dt
    [Hs, Dm], conv_w_f, conv_w_b [Ch, K], conv_b_f, conv_b_b [Ch], dt_bias,
    A_f, D_f, A_b, D_b [Hs], norm_w [d], w_out_ma [Dm, d], w_q, w_k, w_v
    [d, Dm], w_o [Dm, d], with d = Hs*P = Ha*(attention head size).
    ``review`` = (rpool, rgrid): review tokens in the MA branch, formed by
    ``ssd_dirs`` from each direction's scan inputs (after the convolution).
    """
    f = {k: np.asarray(v, dtype=np.float64) for k, v in w.items()}
    u = np.asarray(u, dtype=np.float64)
    L = T * H * W
    d = Hs * P
    mode = rms_mode(layer_idx)
    order = rms_scan_order(mode, T, H, W)
    z = u @ f["w_z"].T
    xbc = u @ f["w_xbc"].T
    dt_raw = u @ f["w_dt"].T
    xf, Bf, Cf, xb, Bb, Cb, dt = ma_prep(xbc, dt_raw, f["conv_w_f"], f["conv_b_f"], f["conv_w_b"], f["conv_b_b"],
                                         f["dt_bias"], order, Hs, P, G, N)
    y = ssd_dirs((xf, dt, f["A_f"], Bf, Cf, f["D_f"]), (xb, dt, f["A_b"], Bb, Cb, f["D_b"]), order,
                 review=review, grid=(T, H, W))
    yn = gated_rmsnorm(y.reshape(L, d), z, f["norm_w"], eps, d // G)
    out = yn @ f["w_out_ma"].T
    dh = d // Ha
    q, k, v = ((u @ f[n].T).reshape(L, Ha, dh) for n in ("w_q", "w_k", "w_v"))
    o = tesa(q, k, v, T, H, W, win, tesa_shift(layer_idx, win))
    return out + o.reshape(L, d) @ f["w_o"].T
