"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and validates arguments before launching anything."""
import ctypes
import os
import re

import pytest

from hybrid_linear_temporal_amd import hlta as H
from hybrid_linear_temporal_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "hlta.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hlta_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(H.LIB_PATH):
        pytest.fail("libhlta.so is not built (run __graft_entry__.build())")
    return H.load_library()


def test_library_exports_every_header_symbol(lib):
    names = _header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(H.EXPORTS)
    assert lib.hlta_abi_version() == 2


def test_struct_layout_matches_header():
    # 16 int32 fields + 2 floats = 72 bytes; stream state: 3 pointers, int32, int64
    assert ctypes.sizeof(H.hlta_config) == 18 * 4
    assert ctypes.sizeof(H.hlta_stream_state) == 8 * 3 + 8 + 8


def _cfg(**kw):
    return H.make_config(I.P480_T31, **kw)


def test_valid_configs(lib):
    for wl in I.WORKLOADS.values():
        H.hlta_validate_config(H.make_config(wl))


@pytest.mark.parametrize("field,value,status", [
    ("B", 0, 2), ("H", 0, 2), ("T", -1, 2), ("P", 0, 2), ("d", 96, 4), ("swa_frames", -1, 2),
    ("dswa_dilation", 0, 2), ("dswa_taps", -2, 2), ("gdn_chunk", 48, 4), ("in_dtype", 7, 3),
    ("impl", 9, 2), ("softmax_scale", float("inf"), 2), ("gdn_l2norm_qk", 2, 2), ("gate_logits", 3, 2)])
def test_invalid_config_codes(lib, field, value, status):
    cfg = _cfg()
    setattr(cfg, field, value)
    with pytest.raises(H.HLTAError) as e:
        H.hlta_validate_config(cfg)
    assert e.value.status == status
    assert field.split("_")[0].lower() in str(e.value).lower() or str(e.value)


def test_f32_in_bf16_out_rejected(lib):
    cfg = H.make_config(I.TINY_F32, out_dtype="bf16")
    with pytest.raises(H.HLTAError) as e:
        H.hlta_validate_config(cfg)
    assert e.value.status == 3


def test_overflow_rejected(lib):
    cfg = _cfg(T=1 << 20, P=1 << 12)
    with pytest.raises(H.HLTAError):
        H.hlta_validate_config(cfg)


def test_workspace_sizes(lib):
    cfg = _cfg()
    ws = H.hlta_fwd_workspace_bytes(cfg)
    assert ws > 0
    # bf16, d = 128, chunk 64: a 13056-byte record per chunk, then the memory's
    # segment maps, 2G - 1 fp32 d x d matrices per (batch row, head) for G
    # segments side by side
    chunks = -(-cfg.T * cfg.P // cfg.gdn_chunk)
    maps = ws - cfg.B * cfg.H * chunks * 13056
    per = cfg.B * cfg.H * cfg.d * cfg.d * 4
    assert maps > 0 and maps % per == 0 and (maps // per) % 2 == 1
    # float32: the generic kernels' per-chunk records
    f32 = H.make_config(I.TINY_F32)
    chunks = -(-f32.T * f32.P // f32.gdn_chunk)
    assert H.hlta_fwd_workspace_bytes(f32) % (f32.B * f32.H * chunks) == 0
    bad = _cfg(d=96)
    assert H.hlta_fwd_workspace_bytes(bad) == 0
    assert H.hlta_step_workspace_bytes(cfg) > 0
    assert H.hlta_stream_ring_bytes(cfg, 16) == cfg.B * 16 * cfg.P * cfg.H * cfg.d * 2
    assert H.hlta_stream_ring_bytes(cfg, 0) == 0


def test_mfma_impl_needs_supported_shape(lib):
    cfg = H.make_config(I.TINY_F32, impl=H.HLTA_IMPL_MFMA)
    assert H.hlta_fwd_workspace_bytes(cfg) == 0
    assert b"MFMA" in lib.hlta_last_error()


def test_fwd_argument_errors_before_launch(lib):
    cfg = _cfg()
    ws = H.hlta_fwd_workspace_bytes(cfg)
    # pointers are never dereferenced on the host; validation fails first
    fake = ctypes.c_void_p(1 << 20)
    mis = ctypes.c_void_p((1 << 20) + 8)
    args = [fake] * 6 + [None] + [fake] * 4 + [None, fake]
    # NULL q
    a2 = list(args)
    a2[0] = None
    assert lib.hlta_fwd(ctypes.byref(cfg), *a2, ws, None) == 1
    # misaligned k
    a2 = list(args)
    a2[1] = mis
    assert lib.hlta_fwd(ctypes.byref(cfg), *a2, ws, None) == 6
    # small workspace
    assert lib.hlta_fwd(ctypes.byref(cfg), *args, ws - 1, None) == 5
    # NULL workspace
    a2 = list(args)
    a2[12] = None
    assert lib.hlta_fwd(ctypes.byref(cfg), *a2, ws, None) == 1
    # NULL config
    assert lib.hlta_fwd(None, *args, ws, None) == 1
    assert b"NULL" in lib.hlta_last_error()


def test_stream_argument_errors(lib):
    cfg = H.make_config(I.STREAM_P480)
    fake = 1 << 20
    st = H.hlta_stream_state(fake, fake, fake, 8, 0)       # ring too short for dil*taps = 16
    assert lib.hlta_stream_load_prefix(ctypes.byref(cfg), ctypes.byref(st), None, None, 0, None, None) == 7
    st = H.hlta_stream_state(None, fake, fake, 16, 0)
    assert lib.hlta_stream_load_prefix(ctypes.byref(cfg), ctypes.byref(st), None, None, 0, None, None) == 1
    st = H.hlta_stream_state(fake, fake, fake, 16, -1)
    p = ctypes.c_void_p(fake)
    assert lib.hlta_step_frame(ctypes.byref(cfg), ctypes.byref(st), p, p, p, p, p, p, p, p, p, p, 1, p,
                               1 << 40, None) == 7
    st = H.hlta_stream_state(fake, fake, fake, 16, 0)
    assert lib.hlta_stream_load_prefix(ctypes.byref(cfg), ctypes.byref(st), None, None, 3, None, None) == 1


def test_step_rollouts_argument_errors(lib):
    """Per-rollout positions: NULL frames, an entry below -1 and more than 64
    rollouts fail before any launch; a step every rollout sits out is a no-op."""
    import numpy as np
    cfg = H.make_config(I.STREAM_P480)
    fake = 1 << 20
    st = H.hlta_stream_state(fake, fake, fake, 16, 0)
    p = ctypes.c_void_p(fake)
    ws = 1 << 40

    def call(c, frames):
        fp = None if frames is None else frames.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        return lib.hlta_step_frame_rollouts(ctypes.byref(c), ctypes.byref(st), fp, p, p, p, p, p, p, p, p, p, p,
                                            1, p, ws, None)

    assert call(cfg, None) == 1
    frames = np.full(cfg.B, 20, dtype=np.int64)
    frames[3] = -2
    assert call(cfg, frames) == 7
    assert b"frames[3]" in lib.hlta_last_error()
    skip_all = np.full(cfg.B, -1, dtype=np.int64)
    assert call(cfg, skip_all) == 0 and np.all(skip_all == -1)
    big = H.make_config(I.STREAM_P480)
    big.B = 65
    assert call(big, np.zeros(65, dtype=np.int64)) == 4


def test_rope_config_checks(lib):
    """The rotary embedding needs a frame grid of exactly P tokens and a finite
    theta >= 0; it adds two rotated copies of q, k to the workspaces."""
    base = _cfg()
    ws0 = H.hlta_fwd_workspace_bytes(base)
    good = _cfg(rope_theta=10000.0, rope_grid=(30, 52))
    H.hlta_validate_config(good)
    n = good.B * good.T * good.P * good.H * good.d * 2
    assert H.hlta_fwd_workspace_bytes(good) >= ws0 + 2 * n
    assert H.hlta_step_workspace_bytes(good) > H.hlta_step_workspace_bytes(base)
    for theta, grid in ((10000.0, (30, 51)), (10000.0, (0, 1560)), (-1.0, (30, 52)), (float("nan"), (30, 52))):
        with pytest.raises(H.HLTAError) as e:
            H.hlta_validate_config(_cfg(rope_theta=theta, rope_grid=grid))
        assert e.value.status == 2 and b"rope" in lib.hlta_last_error()
    # hlta_attn_fwd has no workspace for the rotated copies
    fake = ctypes.c_void_p(1 << 20)
    assert lib.hlta_attn_fwd(ctypes.byref(good), *([fake] * 9)) == 4
    assert b"workspace" in lib.hlta_last_error()


def test_bwd_workspace_and_argument_errors(lib):
    """Backward: workspace = two [2, B, L, H] fp32 statistics, five d x d
    matrices per chunk, one slot per chunk for the memory's per-chunk
    kernels (sixteen 64 x d and eight 64 x 64 fp32 matrices each) and the
    mix-weight partial sums; argument errors fail before any launch."""
    cfg = _cfg()
    L = cfg.T * cfg.P
    chunks = -(-L // cfg.gdn_chunk)

    def up(x):
        return -(-x // 256) * 256

    bh, dd = cfg.B * cfg.H, cfg.d * cfg.d * 4
    slots = bh * chunks
    slot = (16 * 64 * cfg.d + 8 * 64 * 64) * 4
    want = 2 * up(bh * L * 2 * 4) + 5 * up(bh * chunks * dd) + up(slots * slot) + up(cfg.H * 128 * 3 * 4)
    ws = H.hlta_bwd_workspace_bytes(cfg)
    assert ws == want
    assert H.hlta_bwd_workspace_bytes(_cfg(d=96)) == 0
    fake = ctypes.c_void_p(1 << 20)
    args = [fake] * 6 + [None] + [fake] * 10 + [None, fake]   # S0 and dS0 NULL

    def call(c, a, nbytes=ws):
        return lib.hlta_bwd(ctypes.byref(c), *a, nbytes, None)

    for i, name in ((0, b"q"), (9, b"o_gdn"), (10, b"d_mix"), (15, b"db"), (16, b"dmix_w")):
        a2 = list(args)
        a2[i] = None
        assert call(cfg, a2) == 1 and name + b" is NULL" in lib.hlta_last_error()
    assert call(cfg, args, ws - 1) == 5
    a2 = list(args)
    a2[18] = None
    assert call(cfg, a2) == 1
    a2 = list(args)
    a2[3] = ctypes.c_void_p((1 << 20) + 4)
    assert call(cfg, a2) == 6
    assert call(_cfg(gate_logits=1), args) == 4
    rope = _cfg(rope_theta=10000.0, rope_grid=(30, 52))
    assert call(rope, args) == 4
    # hlta_bwd_lse: the same checks, and the statistics themselves are required
    args_lse = args[:11] + [fake] + args[11:]   # lse after d_mix

    def call_lse(c, a, nbytes=ws):
        return lib.hlta_bwd_lse(ctypes.byref(c), *a, nbytes, None)

    a2 = list(args_lse)
    a2[11] = None
    assert call_lse(cfg, a2) == 1 and b"lse is NULL" in lib.hlta_last_error()
    a2 = list(args_lse)
    a2[0] = None
    assert call_lse(cfg, a2) == 1 and b"q is NULL" in lib.hlta_last_error()
    assert call_lse(cfg, args_lse, ws - 1) == 5


def test_attn_fwd_lse_argument_errors(lib):
    """hlta_attn_fwd_lse checks what hlta_attn_fwd checks, and its lse output."""
    cfg = _cfg()
    fake = ctypes.c_void_p(1 << 20)
    args = [fake] * 8   # q, k, v, mix_w, o_gdn, o_swa, o_dswa, o_mix
    assert lib.hlta_attn_fwd_lse(ctypes.byref(cfg), *args, None, None) == 1
    assert b"lse is NULL" in lib.hlta_last_error()
    a2 = list(args)
    a2[0] = None
    assert lib.hlta_attn_fwd_lse(ctypes.byref(cfg), *a2, fake, None) == 1
    assert lib.hlta_attn_fwd_lse(ctypes.byref(cfg), *args, ctypes.c_void_p((1 << 20) + 4), None) == 6
    rope = _cfg(rope_theta=10000.0, rope_grid=(30, 52))
    assert lib.hlta_attn_fwd_lse(ctypes.byref(rope), *args, fake, None) == 4


def test_split_entry_points_argument_errors(lib):
    """hlta_attn_branches and hlta_gdn_mix_fwd check their arguments before any
    launch: NULL and misaligned pointers, the workspace size, and the rotary
    embedding for hlta_attn_branches (which has no workspace for it)."""
    cfg = _cfg()
    fake = ctypes.c_void_p(1 << 20)
    br = [fake] * 5   # q, k, v, o_swa, o_dswa
    for i, name in ((0, b"q"), (3, b"o_swa"), (4, b"o_dswa")):
        a2 = list(br)
        a2[i] = None
        assert lib.hlta_attn_branches(ctypes.byref(cfg), *a2, None) == 1
        assert name + b" is NULL" in lib.hlta_last_error()
    a2 = list(br)
    a2[3] = ctypes.c_void_p((1 << 20) + 4)
    assert lib.hlta_attn_branches(ctypes.byref(cfg), *a2, None) == 6
    rope = _cfg(rope_theta=10000.0, rope_grid=(30, 52))
    assert lib.hlta_attn_branches(ctypes.byref(rope), *br, None) == 4
    ws = H.hlta_fwd_workspace_bytes(cfg)
    # q, k, v, a, b, mix_w, S0 (NULL), o_swa, o_dswa, o_gdn, o_mix, S_out (NULL), workspace
    gm = [fake] * 6 + [None] + [fake] * 4 + [None, fake]

    def call(a, nbytes=ws):
        return lib.hlta_gdn_mix_fwd(ctypes.byref(cfg), *a, nbytes, None)

    for i, name in ((0, b"q"), (5, b"mix_w"), (7, b"o_swa"), (8, b"o_dswa"), (9, b"o_gdn"), (10, b"o_mix")):
        a2 = list(gm)
        a2[i] = None
        assert call(a2) == 1 and name + b" is NULL" in lib.hlta_last_error()
    a2 = list(gm)
    a2[8] = ctypes.c_void_p((1 << 20) + 4)
    assert call(a2) == 6
    assert call(gm, ws - 1) == 5
