"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host-side checks return the documented status codes before any GPU work.
No call in this file reaches a kernel launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from mate_inputs import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lingen_mate.h")

mate = pytest.importorskip("linear_complexity_video_mate_amd")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mate.LIB_PATH):
        pytest.fail("liblingen_mate.so is not built (run __graft_entry__.build())")
    return mate.lib()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lingen_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 10
    assert sorted(mate.EXPORTS) == names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in range(-8, 1):
        assert mate.status_str(code) and mate.status_str(code) != "unknown status"
    assert mate.status_str(5) == "unknown status"


@pytest.mark.parametrize("cfg", range(len(CONFIGS)))
def test_configs_validate(L, cfg):
    assert mate.lingen_mate_validate(CONFIGS[cfg]) == 0


BAD = [
    ("batch", dict(batch=0), -2),
    ("T", dict(T=0), -2),
    ("chunk_not_dividing", dict(chunk=48), -2),
    ("groups_not_dividing", dict(ngroups=3), -2),
    ("groups_zero", dict(ngroups=0), -2),
    ("heads_mismatch", dict(attn_heads=8), -2),
    ("window_not_dividing", dict(win=(3, 8, 8)), -2),
    ("dtype", dict(dtype="f16"), -3),
    ("unsupported_state", dict(d_state=32, chunk=64), -7),
    ("unsupported_window", dict(win=(2, 8, 8)), -7),
    ("review_count", dict(n_review=63, rpool=(2, 8, 8), rgrid=(4, 4, 4)), -2),
    ("review_pool", dict(n_review=64, rpool=(3, 8, 8), rgrid=(4, 4, 4)), -2),
    ("review_grid", dict(n_review=27, rpool=(2, 8, 8), rgrid=(3, 3, 3)), -2),
    ("negative_review", dict(n_review=-1), -2),
    ("huge", dict(T=2 ** 20, H=2 ** 10, W=2 ** 10), -2),
]


@pytest.mark.parametrize("name,kw,code", BAD, ids=[b[0] for b in BAD])
def test_invalid_shapes(L, name, kw, code):
    s = CONFIGS[1].with_(**kw)
    assert mate.lingen_mate_validate(s) == code
    with pytest.raises(mate.LingenError) as e:
        mate.lingen_mate_workspace_bytes(s)
    assert e.value.code == code


def test_grouped_shapes_valid(L):
    for G in (1, 2, 4, 16):
        assert mate.lingen_mate_validate(CONFIGS[1].with_(ngroups=G)) == 0


def test_review_shape_valid(L):
    s = CONFIGS[1].with_(n_review=64, rpool=(2, 4, 4), rgrid=(4, 4, 4))   # pooled 8x8x8
    assert mate.lingen_mate_validate(s) == 0


@pytest.mark.parametrize("cfg", range(len(CONFIGS)))
def test_workspace_formula(L, cfg):
    s = CONFIGS[cfg]
    al = lambda v: (v + 255) // 256 * 256
    nc = s.L // s.chunk
    # chunk states in the input element type, then fp32 chunk decays
    want = al(2 * nc * s.ssd_heads * s.headdim * s.d_state * s.elem_bytes) + al(nc * s.ssd_heads * 4)
    R = s.n_review
    if R:
        want += al(s.ssd_heads * s.headdim * s.d_state * 4) + al(R * s.ssd_heads * s.headdim * 4) \
            + al(R * s.ssd_heads * 4) + al(R * s.ngroups * s.d_state * 4)
    assert mate.lingen_mate_workspace_bytes(s) == want
    if R:   # pooled review B rows are kept per group
        g4 = s.with_(ngroups=4)
        assert mate.lingen_mate_workspace_bytes(g4) == want - al(R * s.d_state * 4) + al(R * 4 * s.d_state * 4)


@pytest.mark.parametrize("mode", range(4))
@pytest.mark.parametrize("cfg", range(len(CONFIGS)))
def test_host_rms_index_bitexact(L, mode, cfg):
    s = CONFIGS[cfg]
    perm, inv = mate.lingen_rms_index(mode, s.T, s.H, s.W)
    ref = oracle.rms_scan_order(mode, s.T, s.H, s.W)
    np.testing.assert_array_equal(perm, ref.astype(np.int32))
    np.testing.assert_array_equal(inv, oracle.rms_inverse(ref).astype(np.int32))


def test_host_rms_index_errors(L):
    buf = np.empty(8, dtype=np.int32)
    assert L.lingen_rms_index(4, 2, 2, 2, buf.ctypes.data, None) == -2
    assert L.lingen_rms_index(0, 0, 2, 2, buf.ctypes.data, None) == -2
    assert L.lingen_rms_index(0, 2 ** 12, 2 ** 12, 2 ** 8, None, None) == -2


# -- entry points reject bad arguments before touching the GPU ---------------

FAKE = 0x1000          # 16-byte aligned, never dereferenced
MISALIGNED = 0x1008


def _mate_call(L, shape, ptrs=None, layer=0, ws=FAKE, ws_bytes=None):
    cs = mate.to_c_shape(shape)
    if ws_bytes is None:
        ws_bytes = mate.lingen_mate_workspace_bytes(shape) if mate.lingen_mate_validate(shape) == 0 else 0
    p = [FAKE] * 10 if ptrs is None else ptrs
    return L.lingen_mate_fwd(*[ctypes.c_void_p(v) for v in p[:9]], layer, ctypes.byref(cs), ctypes.c_void_p(p[9]),
                             ctypes.c_void_p(ws), ws_bytes, None)


def test_mate_fwd_rejects_before_launch(L):
    s = CONFIGS[1]
    for i in range(10):
        p = [FAKE] * 10
        p[i] = 0
        assert _mate_call(L, s, p) == -1, i
        p[i] = MISALIGNED
        assert _mate_call(L, s, p) == -4, i
    assert _mate_call(L, s, layer=-1) == -2
    assert _mate_call(L, s, ws=0) == -1
    need = mate.lingen_mate_workspace_bytes(s)
    assert _mate_call(L, s, ws_bytes=need - 1) == -5
    assert _mate_call(L, s.with_(T=3)) == -2
    cs = None
    assert L.lingen_mate_fwd(*[ctypes.c_void_p(FAKE)] * 9, 0, cs, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                             need, None) == -1


def test_branch_entry_points_reject_before_launch(L):
    s = CONFIGS[0]
    cs = mate.to_c_shape(s)
    F = ctypes.c_void_p(FAKE)
    Z = ctypes.c_void_p(0)
    need = mate.lingen_mate_workspace_bytes(s)
    assert L.lingen_ma_fwd(F, F, F, F, F, F, 4, ctypes.byref(cs), F, F, need, None) == -2
    assert L.lingen_ma_fwd(F, F, F, F, F, Z, 0, ctypes.byref(cs), F, F, need, None) == -1
    assert L.lingen_ma_fwd(F, F, F, F, F, F, 0, ctypes.byref(cs), F, F, need - 256, None) == -5
    assert L.lingen_te_fwd(F, Z, F, 0, ctypes.byref(cs), F, None) == -1
    assert L.lingen_te_fwd(F, F, F, 0, None, F, None) == -1
    assert L.lingen_ssd_chunk_states(F, F, F, F, -1, ctypes.byref(cs), F, F, F, need, None) == -2
    assert L.lingen_ssd_chunk_states(F, F, F, F, 0, ctypes.byref(cs), F, Z, F, need, None) == -1
    assert L.lingen_rms_gather(F, 24, 0, 2, 2, 2, F, None) == -2
    assert L.lingen_rms_gather(F, 32, 0, 2, 2, 2, Z, None) == -1
    assert L.lingen_rms_index_device(5, 2, 2, 2, F, None) == -2
    assert L.lingen_rms_index_device(0, 2, 2, 2, ctypes.c_void_p(MISALIGNED), None) == -4


def test_te_shift_rejects_before_launch(L):
    s = CONFIGS[0]
    cs = mate.to_c_shape(s)
    F = ctypes.c_void_p(FAKE)
    call = L.lingen_te_fwd_shift
    for st, sh, sw, masked in ((2, 0, 0, 1), (-1, 0, 0, 1), (0, 4, 0, 0), (0, 0, 4, 1), (0, 0, 0, 2), (0, 0, 0, -1)):
        assert call(F, F, F, st, sh, sw, masked, ctypes.byref(cs), F, None) == -2
    assert call(F, F, F, 1, 3, 3, 1, None, F, None) == -1
    assert call(F, F, F, 1, 3, 3, 1, ctypes.byref(cs), ctypes.c_void_p(0), None) == -1
    assert call(F, F, F, 1, 3, 3, 0, ctypes.byref(cs), ctypes.c_void_p(MISALIGNED), None) == -4


def test_te_bwd_rejects_before_launch(L):
    F = ctypes.c_void_p(FAKE)
    Z = ctypes.c_void_p(0)
    call = L.lingen_te_bwd
    cs1 = mate.to_c_shape(CONFIGS[1])
    for st, sh, sw, masked in ((4, 0, 0, 1), (0, -1, 0, 1), (0, 0, 8, 0), (0, 0, 0, 3)):
        assert call(F, F, F, F, st, sh, sw, masked, ctypes.byref(cs1), F, F, F, None) == -2
    for i in range(7):
        p = [F] * 7
        p[i] = Z
        assert call(*p[:4], 2, 4, 4, 1, ctypes.byref(cs1), *p[4:], None) == -1, i
        p[i] = ctypes.c_void_p(MISALIGNED)
        assert call(*p[:4], 2, 4, 4, 1, ctypes.byref(cs1), *p[4:], None) == -4, i
    # the backward has the forward's families; a window no family covers
    # (bf16, d 64, 2x4x4 windows) is refused before anything is launched
    csn = mate.to_c_shape(CONFIGS[1].with_(win=(2, 4, 4)))
    assert call(F, F, F, F, 1, 2, 2, 1, ctypes.byref(csn), F, F, F, None) == -7
    assert call(F, F, F, F, 1, 2, 2, 1, None, F, F, F, None) == -1


def test_te_saved_rejects_before_launch(L):
    F = ctypes.c_void_p(FAKE)
    Z = ctypes.c_void_p(0)
    M = ctypes.c_void_p(MISALIGNED)
    fwd, bwd = L.lingen_te_fwd_saved, L.lingen_te_bwd_saved
    cs1 = mate.to_c_shape(CONFIGS[1])
    for st, sh, sw, masked in ((4, 0, 0, 1), (0, -1, 0, 1), (0, 0, 8, 0), (0, 0, 0, 3)):
        assert fwd(F, F, F, st, sh, sw, masked, ctypes.byref(cs1), F, F, None) == -2
        assert bwd(*[F] * 6, st, sh, sw, masked, ctypes.byref(cs1), F, F, F, None) == -2
    for i in range(5):   # q, k, v, y_te, lse
        p = [F] * 5
        p[i] = Z
        assert fwd(*p[:3], 2, 4, 4, 1, ctypes.byref(cs1), *p[3:], None) == -1, i
        p[i] = M
        assert fwd(*p[:3], 2, 4, 4, 1, ctypes.byref(cs1), *p[3:], None) == -4, i
    for i in range(9):   # q, k, v, o, d_out, lse, dq, dk, dv
        p = [F] * 9
        p[i] = Z
        assert bwd(*p[:6], 2, 4, 4, 1, ctypes.byref(cs1), *p[6:], None) == -1, i
        p[i] = M
        assert bwd(*p[:6], 2, 4, 4, 1, ctypes.byref(cs1), *p[6:], None) == -4, i
    # only the 256-token bf16 windows, and for the forward an even head count
    # (its kernel takes two heads per item)
    c = mate.to_c_shape(CONFIGS[0])
    assert fwd(F, F, F, 0, 0, 0, 1, ctypes.byref(c), F, F, None) == -7
    assert bwd(*[F] * 6, 0, 0, 0, 1, ctypes.byref(c), F, F, F, None) == -7
    c = mate.to_c_shape(CONFIGS[1].with_(ssd_heads=15, attn_heads=15))
    assert L.lingen_mate_validate(ctypes.byref(c)) == 0
    assert fwd(F, F, F, 0, 0, 0, 1, ctypes.byref(c), F, F, None) == -7
    assert fwd(F, F, F, 0, 0, 0, 1, None, F, F, None) == -1


def test_odd_window_shapes_validate(L):
    for T in (12, 24):
        s = CONFIGS[1].with_(T=T, H=T, W=T, win=(3, 3, 3))
        assert mate.lingen_mate_validate(s) == 0
    # 27-token windows are compiled for bf16 with d = 64 only
    assert mate.lingen_mate_validate(CONFIGS[0].with_(T=6, H=6, W=12, win=(3, 3, 3))) == -7


def test_dense_attention_rejects_before_launch(L):
    F = ctypes.c_void_p(FAKE)
    Z = ctypes.c_void_p(0)
    M = ctypes.c_void_p(MISALIGNED)
    call = L.lingen_dense_attn_fwd
    assert call(F, F, F, F, 1, 64, 2, 64, 7, None) == -3
    assert call(F, F, F, F, 1, -1, 2, 64, 1, None) == -2
    assert call(F, F, F, F, 1, 64, 2, 0, 1, None) == -2
    assert call(F, F, F, F, 1, 64, 70000, 64, 1, None) == -2
    assert call(F, F, F, F, 1 << 20, 1 << 20, 2, 64, 1, None) == -2
    assert call(F, F, F, F, 1, 64, 2, 32, 1, None) == -7
    assert call(F, F, F, F, 1, 64, 2, 64, 0, None) == -7
    for i in range(4):
        p = [F] * 4
        p[i] = Z
        assert call(*p, 1, 64, 2, 64, 1, None) == -1, i
        p[i] = M
        assert call(*p, 1, 64, 2, 64, 1, None) == -4, i
    # empty problems are valid no-ops (nothing is launched, pointers unused)
    assert call(F, F, F, F, 1, 0, 2, 64, 1, None) == 0
    assert call(Z, Z, Z, Z, 1, 0, 2, 64, 1, None) == 0
    assert call(F, F, F, F, 0, 64, 2, 64, 1, None) == 0
    assert call(F, F, F, F, 1, 64, 0, 64, 1, None) == 0


def test_ma_prep_rejects_before_launch(L):
    F = ctypes.c_void_p(FAKE)
    Z = ctypes.c_void_p(0)
    M = ctypes.c_void_p(MISALIGNED)
    call = L.lingen_ma_prep
    for cfg in (CONFIGS[0], CONFIGS[1]):
        cs = mate.to_c_shape(cfg)
        for K, mode in ((0, 0), (5, 0), (4, -1), (4, 4)):
            assert call(*[F] * 7, K, mode, ctypes.byref(cs), *[F] * 7, None) == -2, (K, mode)
        for i in range(14):
            p = [F] * 14
            p[i] = Z
            assert call(*p[:7], 4, 1, ctypes.byref(cs), *p[7:], None) == -1, i
            p[i] = M
            assert call(*p[:7], 4, 1, ctypes.byref(cs), *p[7:], None) == -4, i
    assert call(*[F] * 7, 4, 0, None, *[F] * 7, None) == -1
    bad = mate.to_c_shape(CONFIGS[1].with_(dtype=5))
    assert call(*[F] * 7, 4, 0, ctypes.byref(bad), *[F] * 7, None) == -3


def test_gated_rmsnorm_rejects_before_launch(L):
    F = ctypes.c_void_p(FAKE)
    Z = ctypes.c_void_p(0)
    M = ctypes.c_void_p(MISALIGNED)
    call = L.lingen_gated_rmsnorm
    assert call(F, F, F, 1e-5, 4, 64, 64, 2, F, None) == -3
    for rows, dim, group, dt, eps in ((-1, 64, 64, 1, 1e-5), (1 << 31, 64, 64, 1, 1e-5), (4, 0, 8, 1, 1e-5),
                                      (4, 64, 0, 1, 1e-5), (4, 64, 48, 1, 1e-5), (4, 64, 4, 1, 1e-5),
                                      (4, 64, 2, 0, 1e-5), (4, 8200, 8, 1, 1e-5), (4, 4100, 4, 0, 1e-5),
                                      (4, 64, 64, 1, -1.0), (4, 64, 64, 1, float("nan"))):
        assert call(F, F, F, eps, rows, dim, group, dt, F, None) == -2, (rows, dim, group, dt, eps)
    for i in range(4):
        p = [F] * 4
        p[i] = Z
        assert call(*p[:3], 1e-5, 4, 64, 64, 1, p[3], None) == -1, i
        p[i] = M
        assert call(*p[:3], 1e-5, 4, 64, 64, 1, p[3], None) == -4, i
    # the largest compiled rows are accepted; zero rows is a no-op
    assert call(Z, Z, Z, 1e-5, 0, 8192, 8192, 1, Z, None) == 0
    assert call(Z, Z, Z, 1e-5, 0, 4096, 64, 0, Z, None) == 0


def test_mate_block_rejects_before_launch(L):
    F = ctypes.c_void_p(FAKE)
    Z = ctypes.c_void_p(0)
    M = ctypes.c_void_p(MISALIGNED)
    call = L.lingen_mate_block_fwd
    cs = mate.to_c_shape(CONFIGS[1])
    n = mate.lingen_mate_block_workspace_bytes(CONFIGS[1], 1024)
    W = mate.binding.lingen_mate_block_weights

    def weights(bad=None, value=None):
        w = W()
        for name in mate.BLOCK_WEIGHTS:
            setattr(w, name, FAKE)
        if bad is not None:
            setattr(w, bad, value)
        return w

    good = weights()   # every call below is rejected before anything is enqueued
    for dm, k, eps, layer in ((0, 4, 1e-5, 0), (70000, 4, 1e-5, 0), (1024, 0, 1e-5, 0), (1024, 5, 1e-5, 0),
                              (1024, 4, -1.0, 0), (1024, 4, 1e-5, -1)):
        assert call(F, ctypes.byref(good), dm, k, eps, layer, ctypes.byref(cs), F, F, n, None) == -2, (dm, k, eps)
    for name in mate.BLOCK_WEIGHTS:
        for value, code in ((0, -1), (MISALIGNED, -4)):
            w = weights(name, value)
            assert call(F, ctypes.byref(w), 1024, 4, 1e-5, 0, ctypes.byref(cs), F, F, n, None) == code, name
    assert call(F, None, 1024, 4, 1e-5, 0, ctypes.byref(cs), F, F, n, None) == -1
    for i in range(3):
        p = [F, F, F]
        p[i] = Z
        assert call(p[0], ctypes.byref(good), 1024, 4, 1e-5, 0, ctypes.byref(cs), p[1], p[2], n, None) == -1
        p[i] = M
        assert call(p[0], ctypes.byref(good), 1024, 4, 1e-5, 0, ctypes.byref(cs), p[1], p[2], n, None) == -4
    assert call(F, ctypes.byref(good), 1024, 4, 1e-5, 0, ctypes.byref(cs), F, F, n - 1, None) == -5
    # review tokens: the per-direction scan the block uses takes them; the
    # workspace grows by the scan's review buffers
    rs = CONFIGS[1].with_(n_review=64, rpool=(2, 4, 4), rgrid=(4, 4, 4))
    rv = mate.to_c_shape(rs)
    size = ctypes.c_size_t(0)
    assert L.lingen_mate_block_workspace_bytes(ctypes.byref(rv), 1024, ctypes.byref(size)) == 0
    assert size.value - int(n) == mate.lingen_mate_workspace_bytes(rs) - mate.lingen_mate_workspace_bytes(CONFIGS[1])
    assert call(F, ctypes.byref(good), 1024, 4, 1e-5, 0, ctypes.byref(rv), F, F, n, None) == -5
    assert L.lingen_mate_block_workspace_bytes(ctypes.byref(cs), 1024, None) == -1
    assert L.lingen_mate_block_workspace_bytes(None, 1024, ctypes.byref(size)) == -1


def test_mate_block_workspace_formula():
    """Workspace = the block's intermediates (aligned to 256 bytes) plus the
    scan's own workspace."""
    for cfg, dm in ((CONFIGS[0], 96), (CONFIGS[1], 1024), (CONFIGS[2], 2048)):
        rows, e = cfg.batch * cfg.L, cfg.elem_bytes
        d, gn, hs = cfg.ssd_heads * cfg.headdim, cfg.ngroups * cfg.d_state, cfg.ssd_heads
        al = lambda b: (b + 255) // 256 * 256
        parts = [rows * d * e, rows * (d + 2 * gn) * e, rows * hs * 4, rows * d * e, rows * gn * e, rows * gn * e,
                 rows * d * e, rows * gn * e, rows * gn * e, rows * hs * 4, rows * d * e, rows * d * e, rows * d * e,
                 rows * d * e, mate.lingen_mate_workspace_bytes(cfg)]
        assert mate.lingen_mate_block_workspace_bytes(cfg, dm) == sum(al(b) for b in parts)


def test_ma_bwd_rejects_before_launch(L):
    F = ctypes.c_void_p(FAKE)
    Z = ctypes.c_void_p(0)
    M = ctypes.c_void_p(MISALIGNED)
    call = L.lingen_ma_bwd
    cs = mate.to_c_shape(CONFIGS[1])
    n = mate.lingen_ma_bwd_workspace_bytes(CONFIGS[1])
    for bad in (-1, 4):
        assert call(*[F] * 7, bad, ctypes.byref(cs), *[F] * 7, n, None) == -2
    for i in range(14):
        p = [F] * 14
        p[i] = Z
        assert call(*p[:7], 0, ctypes.byref(cs), *p[7:], n, None) == -1, i
        p[i] = M
        assert call(*p[:7], 0, ctypes.byref(cs), *p[7:], n, None) == -4, i
    assert call(*[F] * 7, 0, ctypes.byref(cs), *[F] * 7, n - 1, None) == -5
    # the fp32 family (head size 32): two scan workspaces, the crossing sums
    # and the transposed outputs in fp32
    s0 = CONFIGS[0]
    c = mate.to_c_shape(s0)
    size = ctypes.c_size_t(0)
    assert L.lingen_ma_bwd_workspace_bytes(ctypes.byref(c), ctypes.byref(size)) == 0
    al0 = lambda b: (b + 255) // 256 * 256
    rows0 = s0.batch * s0.L
    assert size.value == (2 * al0(mate.lingen_mate_workspace_bytes(s0)) + al0(rows0 * s0.ssd_heads * 4)
                          + al0(rows0 * s0.ssd_heads * s0.headdim * 4))
    # review tokens: supported; the workspace grows by the review buffers of
    # both scan workspaces, the adjoint states' final carries and the
    # pooled tokens' gradients
    rs = CONFIGS[1].with_(n_review=64, rpool=(2, 4, 4), rgrid=(4, 4, 4))
    R, Hs, P, N, G = 64, rs.ssd_heads, rs.headdim, rs.d_state, rs.ngroups
    al = lambda b: (b + 255) // 256 * 256
    grow = (2 * (mate.lingen_mate_workspace_bytes(rs) - mate.lingen_mate_workspace_bytes(CONFIGS[1]))
            + al(2 * Hs * P * N * 4) + al(R * Hs * P * 4) + al(R * Hs * 4) + al(R * G * N * 4))
    assert mate.lingen_ma_bwd_workspace_bytes(rs) == n + grow
    c = mate.to_c_shape(rs)
    assert call(*[F] * 7, 0, ctypes.byref(c), *[F] * 7, n + grow - 1, None) == -5
    assert call(*[F] * 7, 0, None, *[F] * 7, n, None) == -1
    assert L.lingen_ma_bwd_workspace_bytes(ctypes.byref(cs), None) == -1


def test_ma_saved_rejects_before_launch(L):
    """The saved-state forward and backward: sizes and the checks that
    return before any launch."""
    F = ctypes.c_void_p(FAKE)
    Z = ctypes.c_void_p(0)
    M = ctypes.c_void_p(MISALIGNED)
    al = lambda b: (b + 255) // 256 * 256
    for s in (CONFIGS[0], CONFIGS[1], CONFIGS[1].with_(batch=3),
              CONFIGS[1].with_(n_review=64, rpool=(2, 4, 4), rgrid=(4, 4, 4))):
        # per batch element one scan workspace of the forward
        assert mate.lingen_ma_saved_bytes(s) == s.batch * al(mate.lingen_mate_workspace_bytes(s))
        # the backward's workspace without its first scan workspace
        assert (mate.lingen_ma_bwd_saved_workspace_bytes(s)
                == mate.lingen_ma_bwd_workspace_bytes(s) - al(mate.lingen_mate_workspace_bytes(s)))
    s = CONFIGS[1].with_(batch=2)
    cs = mate.to_c_shape(s)
    ns = mate.lingen_ma_saved_bytes(s)
    nw = mate.lingen_ma_bwd_saved_workspace_bytes(s)
    fwd, bwd = L.lingen_ma_fwd_saved, L.lingen_ma_bwd_saved
    for bad in (-1, 4):
        assert fwd(*[F] * 6, bad, ctypes.byref(cs), F, F, ns, None) == -2
        assert bwd(*[F] * 8, ns, bad, ctypes.byref(cs), *[F] * 7, nw, None) == -2
    for i in range(8):   # x, dt, A, B, C, D, y_ma, saved
        p = [F] * 8
        p[i] = Z
        assert fwd(*p[:6], 0, ctypes.byref(cs), p[6], p[7], ns, None) == -1, i
        p[i] = M
        assert fwd(*p[:6], 0, ctypes.byref(cs), p[6], p[7], ns, None) == -4, i
    for i in range(15):   # x, dt, A, B, C, D, dy, saved, six gradients, workspace
        p = [F] * 15
        p[i] = Z
        assert bwd(*p[:8], ns, 0, ctypes.byref(cs), *p[8:], nw, None) == -1, i
        p[i] = M
        assert bwd(*p[:8], ns, 0, ctypes.byref(cs), *p[8:], nw, None) == -4, i
    assert fwd(*[F] * 6, 0, ctypes.byref(cs), F, F, ns - 1, None) == -5
    assert bwd(*[F] * 8, ns - 1, 0, ctypes.byref(cs), *[F] * 7, nw, None) == -5
    assert bwd(*[F] * 8, ns, 0, ctypes.byref(cs), *[F] * 7, nw - 1, None) == -5
    # a scan with no compiled kernels
    c = mate.to_c_shape(CONFIGS[1].with_(d_state=32))
    size = ctypes.c_size_t(0)
    assert L.lingen_ma_saved_bytes(ctypes.byref(c), ctypes.byref(size)) == -7
    assert fwd(*[F] * 6, 0, ctypes.byref(c), F, F, ns, None) == -7
    assert L.lingen_ma_saved_bytes(ctypes.byref(cs), None) == -1
    assert L.lingen_ma_bwd_saved_workspace_bytes(ctypes.byref(cs), None) == -1


def test_missing_library_fails_loudly(monkeypatch):
    import linear_complexity_video_mate_amd.binding as b
    monkeypatch.setattr(b, "_lib", None)
    monkeypatch.setattr(b, "LIB_PATH", "/nonexistent/liblingen_mate.so")
    with pytest.raises(RuntimeError, match="missing"):
        b.lib()
