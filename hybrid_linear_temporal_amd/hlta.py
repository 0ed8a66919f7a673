"""Python binding of libhlta.so (ctypes): argument marshalling only.

Each function has the name of the C entry point it calls (include/hlta.h).
PyTorch supplies device memory and the current HIP stream; every step of the
operator runs in the library's HIP kernels. There is no fallback: if the
library is not built, loading raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import inputs as _inputs

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhlta.so")

HLTA_OK = 0
HLTA_F32, HLTA_BF16 = 0, 1
HLTA_IMPL_AUTO, HLTA_IMPL_GENERIC, HLTA_IMPL_MFMA = 0, 1, 2
STATUS = {0: "HLTA_OK", 1: "HLTA_E_NULL", 2: "HLTA_E_SHAPE", 3: "HLTA_E_DTYPE", 4: "HLTA_E_UNSUPPORTED",
          5: "HLTA_E_WORKSPACE", 6: "HLTA_E_ALIGN", 7: "HLTA_E_STATE", 8: "HLTA_E_HIP"}

# every symbol include/hlta.h declares
EXPORTS = ("hlta_abi_version", "hlta_status_string", "hlta_last_error", "hlta_validate_config",
           "hlta_fwd_workspace_bytes", "hlta_fwd", "hlta_gdn_fwd", "hlta_attn_fwd", "hlta_stream_ring_bytes",
           "hlta_stream_load_prefix", "hlta_step_workspace_bytes", "hlta_step_frame",
           "hlta_step_frame_rollouts", "hlta_quantize_fp8", "hlta_attn_fwd_fp8", "hlta_bwd_workspace_bytes",
           "hlta_bwd", "hlta_fwd_noalloc", "hlta_ceiling_mfma_bf16", "hlta_ceiling_copy", "hlta_attn_fwd_lse",
           "hlta_bwd_lse", "hlta_attn_branches", "hlta_gdn_mix_fwd")


class hlta_config(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32), ("P", ctypes.c_int32),
                ("d", ctypes.c_int32), ("swa_frames", ctypes.c_int32), ("dswa_dilation", ctypes.c_int32),
                ("dswa_taps", ctypes.c_int32), ("gdn_chunk", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("gdn_l2norm_qk", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("impl", ctypes.c_int32), ("rope_theta", ctypes.c_float), ("rope_grid_h", ctypes.c_int32),
                ("rope_grid_w", ctypes.c_int32), ("gate_logits", ctypes.c_int32)]


class hlta_stream_state(ctypes.Structure):
    _fields_ = [("S", ctypes.c_void_p), ("ring_k", ctypes.c_void_p), ("ring_v", ctypes.c_void_p),
                ("ring_frames", ctypes.c_int32), ("frames_done", ctypes.c_int64)]


class HLTAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libhlta.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() or "
                          "python -m hybrid_linear_temporal_amd.build")
    lib = ctypes.CDLL(path)
    P, S, I32, I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    cfgp = ctypes.POINTER(hlta_config)
    stp = ctypes.POINTER(hlta_stream_state)
    sig = {
        "hlta_abi_version": (I32, []),
        "hlta_status_string": (ctypes.c_char_p, [I32]),
        "hlta_last_error": (ctypes.c_char_p, []),
        "hlta_validate_config": (I32, [cfgp]),
        "hlta_fwd_workspace_bytes": (S, [cfgp]),
        "hlta_fwd": (I32, [cfgp, P, P, P, P, P, P, P, P, P, P, P, P, P, S, P]),
        "hlta_fwd_noalloc": (I32, [cfgp, P, P, P, P, P, P, P, P, P, P, P, P, P]),
        "hlta_gdn_fwd": (I32, [cfgp, P, P, P, P, P, P, P, P, P, S, P]),
        "hlta_attn_fwd": (I32, [cfgp, P, P, P, P, P, P, P, P, P]),
        "hlta_attn_branches": (I32, [cfgp, P, P, P, P, P, P]),
        "hlta_gdn_mix_fwd": (I32, [cfgp] + [P] * 13 + [S, P]),
        "hlta_attn_fwd_lse": (I32, [cfgp, P, P, P, P, P, P, P, P, P, P]),
        "hlta_stream_ring_bytes": (S, [cfgp, I32]),
        "hlta_stream_load_prefix": (I32, [cfgp, stp, P, P, I32, P, P]),
        "hlta_step_workspace_bytes": (S, [cfgp]),
        "hlta_step_frame": (I32, [cfgp, stp, P, P, P, P, P, P, P, P, P, P, I32, P, S, P]),
        "hlta_step_frame_rollouts": (I32, [cfgp, stp, ctypes.POINTER(I64), P, P, P, P, P, P, P, P, P, P, I32, P,
                                           S, P]),
        "hlta_quantize_fp8": (I32, [cfgp, P, P, P, P, P, P, P, P]),
        "hlta_attn_fwd_fp8": (I32, [cfgp, P, P, P, P, P, P, P, P, P, P]),
        "hlta_bwd_workspace_bytes": (S, [cfgp]),
        "hlta_bwd": (I32, [cfgp] + [P] * 18 + [P, S, P]),
        "hlta_bwd_lse": (I32, [cfgp] + [P] * 19 + [P, S, P]),
        "hlta_ceiling_mfma_bf16": (I32, [P, P, I32, I32, P]),
        "hlta_ceiling_copy": (I32, [P, P, S, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != HLTA_OK:
        raise HLTAError(status, load_library().hlta_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _tdtype(dt: int):
    return torch.bfloat16 if dt == HLTA_BF16 else torch.float32


def make_config(wl: _inputs.Workload | None = None, *, impl: int = HLTA_IMPL_AUTO, out_dtype: str | None = None,
                softmax_scale: float = 0.0, l2norm: bool = True, rope_theta: float = 0.0, rope_grid=(0, 0),
                gate_logits: bool = False, **over) -> hlta_config:
    """hlta_config from a Workload (fields can be overridden by keyword).
    rope_theta > 0 with rope_grid = (rows, columns) of a frame turns on the
    rotary embedding of the softmax branches."""
    f = dict(B=wl.B, H=wl.H, T=wl.T, P=wl.P, d=wl.d, swa_frames=wl.swa_frames, dswa_dilation=wl.dswa_dilation,
             dswa_taps=wl.dswa_taps, gdn_chunk=wl.gdn_chunk, dtype=wl.dtype) if wl is not None else {}
    f.update(over)
    in_dt = HLTA_BF16 if f["dtype"] == "bf16" else HLTA_F32
    out_dt = in_dt if out_dtype is None else (HLTA_BF16 if out_dtype == "bf16" else HLTA_F32)
    return hlta_config(f["B"], f["H"], f["T"], f["P"], f["d"], f["swa_frames"], f["dswa_dilation"],
                       f["dswa_taps"], f["gdn_chunk"], softmax_scale, int(l2norm), in_dt, out_dt, impl,
                       float(rope_theta), int(rope_grid[0]), int(rope_grid[1]), int(bool(gate_logits)))


def hlta_validate_config(cfg: hlta_config) -> None:
    _check(load_library().hlta_validate_config(ctypes.byref(cfg)))


def hlta_fwd_workspace_bytes(cfg: hlta_config) -> int:
    return int(load_library().hlta_fwd_workspace_bytes(ctypes.byref(cfg)))


def hlta_step_workspace_bytes(cfg: hlta_config) -> int:
    return int(load_library().hlta_step_workspace_bytes(ctypes.byref(cfg)))


def hlta_stream_ring_bytes(cfg: hlta_config, ring_frames: int) -> int:
    return int(load_library().hlta_stream_ring_bytes(ctypes.byref(cfg), ring_frames))


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def alloc_outputs(cfg: hlta_config, tokens: int, device="cuda") -> dict:
    shape = (cfg.B, tokens, cfg.H, cfg.d)
    dt = _tdtype(cfg.out_dtype)
    return {n: torch.empty(shape, dtype=dt, device=device) for n in ("o_swa", "o_dswa", "o_gdn", "o_mix")}


def hlta_fwd(cfg: hlta_config, q, k, v, a, b, mix_w, S0=None, out=None, S_out=None, workspace=None,
             stream=None) -> dict:
    """HLTA forward (C: hlta_fwd). Tensors on the GPU, [B, L, H, d] / [B, L, H] / [H, 3].

    Returns dict of the four outputs (allocated when out is None) and S_out.
    """
    lib = load_library()
    L = cfg.T * cfg.P
    if out is None:
        out = alloc_outputs(cfg, L, q.device)
    if workspace is None:
        workspace = alloc_workspace(hlta_fwd_workspace_bytes(cfg), q.device)
    _check(lib.hlta_fwd(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(mix_w), _ptr(S0),
                        _ptr(out["o_swa"]), _ptr(out["o_dswa"]), _ptr(out["o_gdn"]), _ptr(out["o_mix"]),
                        _ptr(S_out), _ptr(workspace), workspace.numel(), _stream(stream)))
    res = dict(out)
    res["S_out"] = S_out
    return res


NOALLOC_SCRATCH_BYTES = 64 << 20   # HLTA_NOALLOC_SCRATCH_BYTES


def hlta_fwd_noalloc(cfg: hlta_config, q, k, v, a, b, mix_w, out: dict, S0=None, S_out=None, stream=None) -> dict:
    """HLTA forward on the library's fixed per-GPU scratch (C: hlta_fwd_noalloc);
    out holds the four preallocated outputs."""
    _check(load_library().hlta_fwd_noalloc(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                           _ptr(mix_w), _ptr(S0), _ptr(out["o_swa"]), _ptr(out["o_dswa"]),
                                           _ptr(out["o_gdn"]), _ptr(out["o_mix"]), _ptr(S_out), _stream(stream)))
    res = dict(out)
    res["S_out"] = S_out
    return res


def hlta_gdn_fwd(cfg: hlta_config, q, k, v, a, b, o_gdn, S0=None, S_out=None, workspace=None, stream=None):
    """Memory branch alone (C: hlta_gdn_fwd)."""
    if workspace is None:
        workspace = alloc_workspace(hlta_fwd_workspace_bytes(cfg), q.device)
    _check(load_library().hlta_gdn_fwd(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(S0),
                                       _ptr(o_gdn), _ptr(S_out), _ptr(workspace), workspace.numel(),
                                       _stream(stream)))


def hlta_attn_fwd(cfg: hlta_config, q, k, v, mix_w, o_gdn, out: dict, stream=None):
    """Softmax branches and the mix (C: hlta_attn_fwd); out holds o_swa, o_dswa, o_mix."""
    _check(load_library().hlta_attn_fwd(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(mix_w), _ptr(o_gdn),
                                        _ptr(out["o_swa"]), _ptr(out["o_dswa"]), _ptr(out["o_mix"]),
                                        _stream(stream)))


def hlta_attn_branches(cfg: hlta_config, q, k, v, out: dict, stream=None):
    """Softmax branches alone (C: hlta_attn_branches); out holds o_swa, o_dswa."""
    _check(load_library().hlta_attn_branches(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(out["o_swa"]),
                                             _ptr(out["o_dswa"]), _stream(stream)))


def hlta_gdn_mix_fwd(cfg: hlta_config, q, k, v, a, b, mix_w, out: dict, S0=None, S_out=None, workspace=None,
                     stream=None):
    """Memory branch and the mix (C: hlta_gdn_mix_fwd) from out's o_swa, o_dswa;
    writes out's o_gdn, o_mix."""
    if workspace is None:
        workspace = alloc_workspace(hlta_fwd_workspace_bytes(cfg), q.device)
    _check(load_library().hlta_gdn_mix_fwd(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                           _ptr(mix_w), _ptr(S0), _ptr(out["o_swa"]), _ptr(out["o_dswa"]),
                                           _ptr(out["o_gdn"]), _ptr(out["o_mix"]), _ptr(S_out),
                                           _ptr(workspace), workspace.numel(), _stream(stream)))


def hlta_bwd_workspace_bytes(cfg: hlta_config) -> int:
    return int(load_library().hlta_bwd_workspace_bytes(ctypes.byref(cfg)))


def hlta_attn_fwd_lse(cfg: hlta_config, q, k, v, mix_w, o_gdn, out: dict, lse=None, stream=None):
    """hlta_attn_fwd that also writes the softmax row statistics (C:
    hlta_attn_fwd_lse); returns lse [2, B, H, L] float32 (allocated when None)."""
    if lse is None:
        lse = torch.empty((2, cfg.B, cfg.H, q.shape[1]), dtype=torch.float32, device=q.device)
    _check(load_library().hlta_attn_fwd_lse(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(mix_w), _ptr(o_gdn),
                                            _ptr(out["o_swa"]), _ptr(out["o_dswa"]), _ptr(out["o_mix"]), _ptr(lse),
                                            _stream(stream)))
    return lse


def hlta_bwd(cfg: hlta_config, q, k, v, a, b, mix_w, fwd: dict, d_mix, S0=None, want_dS0: bool = True,
             workspace=None, stream=None, lse=None) -> dict:
    """Gradients of <d_mix, o_mix> (C: hlta_bwd, or hlta_bwd_lse when the
    forward's softmax statistics lse are given). fwd holds the forward's
    o_swa, o_dswa, o_gdn. Returns float32 dq, dk, dv [B, L, H, d], da, db
    [B, L, H], dmix_w [H, 3] and dS0 [B, H, d, d] (None unless want_dS0)."""
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    g = {n: torch.empty(q.shape, **f32) for n in ("dq", "dk", "dv")}
    g["da"] = torch.empty(a.shape, **f32)
    g["db"] = torch.empty(b.shape, **f32)
    g["dmix_w"] = torch.empty((cfg.H, 3), **f32)
    g["dS0"] = torch.empty((cfg.B, cfg.H, cfg.d, cfg.d), **f32) if want_dS0 else None
    if workspace is None:
        workspace = alloc_workspace(hlta_bwd_workspace_bytes(cfg), dev)
    lib = load_library()
    head = [ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(mix_w), _ptr(S0),
            _ptr(fwd["o_swa"]), _ptr(fwd["o_dswa"]), _ptr(fwd["o_gdn"]), _ptr(d_mix)]
    tail = [_ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["da"]), _ptr(g["db"]), _ptr(g["dmix_w"]),
            _ptr(g["dS0"]), _ptr(workspace), workspace.numel(), _stream(stream)]
    if lse is None:
        _check(lib.hlta_bwd(*head, *tail))
    else:
        _check(lib.hlta_bwd_lse(*head, _ptr(lse), *tail))
    return g


def hlta_quantize_fp8(cfg: hlta_config, q, k, v, stream=None) -> dict:
    """e4m3 codes (uint8 tensors) of q, k, v and their [B, H, 3] float32 scales
    (C: hlta_quantize_fp8)."""
    q8 = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
    k8, v8 = torch.empty_like(q8), torch.empty_like(q8)
    scales = torch.empty((cfg.B, cfg.H, 3), dtype=torch.float32, device=q.device)
    _check(load_library().hlta_quantize_fp8(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(q8), _ptr(k8),
                                            _ptr(v8), _ptr(scales), _stream(stream)))
    return {"q8": q8, "k8": k8, "v8": v8, "scales": scales}


def hlta_attn_fwd_fp8(cfg: hlta_config, fp8: dict, mix_w, o_gdn, out: dict, stream=None):
    """Softmax branches on e4m3 codes and the mix (C: hlta_attn_fwd_fp8)."""
    _check(load_library().hlta_attn_fwd_fp8(ctypes.byref(cfg), _ptr(fp8["q8"]), _ptr(fp8["k8"]), _ptr(fp8["v8"]),
                                            _ptr(fp8["scales"]), _ptr(mix_w), _ptr(o_gdn), _ptr(out["o_swa"]),
                                            _ptr(out["o_dswa"]), _ptr(out["o_mix"]), _stream(stream)))
    return out


class Stream:
    """Device buffers of one stream (state S and the K/V rings) plus the C state struct."""

    def __init__(self, cfg: hlta_config, ring_frames: int, device="cuda"):
        self.cfg = cfg
        dt = _tdtype(cfg.in_dtype)
        self.S = torch.zeros((cfg.B, cfg.H, cfg.d, cfg.d), dtype=torch.float32, device=device)
        shape = (cfg.B, ring_frames, cfg.P, cfg.H, cfg.d)
        self.ring_k = torch.zeros(shape, dtype=dt, device=device)
        self.ring_v = torch.zeros(shape, dtype=dt, device=device)
        self.state = hlta_stream_state(self.S.data_ptr(), self.ring_k.data_ptr(), self.ring_v.data_ptr(),
                                       ring_frames, 0)
        self.workspace = alloc_workspace(hlta_step_workspace_bytes(cfg), device)

    @property
    def frames_done(self) -> int:
        return int(self.state.frames_done)


def hlta_stream_load_prefix(st: Stream, k_prefix, v_prefix, prefix_frames: int, S_prefix=None, stream=None):
    _check(load_library().hlta_stream_load_prefix(ctypes.byref(st.cfg), ctypes.byref(st.state), _ptr(k_prefix),
                                                  _ptr(v_prefix), prefix_frames, _ptr(S_prefix), _stream(stream)))


def hlta_step_frame(st: Stream, q_f, k_f, v_f, a_f, b_f, mix_w, out=None, commit: bool = True,
                    stream=None) -> dict:
    """Append one latent frame to every rollout (C: hlta_step_frame)."""
    cfg = st.cfg
    if out is None:
        out = alloc_outputs(cfg, cfg.P, q_f.device)
    _check(load_library().hlta_step_frame(
        ctypes.byref(cfg), ctypes.byref(st.state), _ptr(q_f), _ptr(k_f), _ptr(v_f), _ptr(a_f), _ptr(b_f),
        _ptr(mix_w), _ptr(out["o_swa"]), _ptr(out["o_dswa"]), _ptr(out["o_gdn"]), _ptr(out["o_mix"]),
        int(bool(commit)), _ptr(st.workspace), st.workspace.numel(), _stream(stream)))
    return out


def hlta_step_frame_rollouts(st: Stream, frames, q_f, k_f, v_f, a_f, b_f, mix_w, out=None, commit: bool = True,
                             stream=None) -> dict:
    """One step with a position per rollout (C: hlta_step_frame_rollouts).
    frames: int64 numpy array [B], frame each rollout appends or -1; advanced
    in place on commit."""
    import numpy as np
    cfg = st.cfg
    if not (isinstance(frames, np.ndarray) and frames.dtype == np.int64 and frames.flags.c_contiguous
            and frames.shape == (cfg.B,)):
        raise TypeError("frames must be a contiguous int64 numpy array of B entries")
    if out is None:
        out = alloc_outputs(cfg, cfg.P, q_f.device)
    _check(load_library().hlta_step_frame_rollouts(
        ctypes.byref(cfg), ctypes.byref(st.state), frames.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        _ptr(q_f), _ptr(k_f), _ptr(v_f), _ptr(a_f), _ptr(b_f), _ptr(mix_w), _ptr(out["o_swa"]),
        _ptr(out["o_dswa"]), _ptr(out["o_gdn"]), _ptr(out["o_mix"]), int(bool(commit)), _ptr(st.workspace),
        st.workspace.numel(), _stream(stream)))
    return out


MFMA_CEILING_FLOP_PER_WAVE_ITER = 8 * 32 * 32 * 16 * 2


def hlta_ceiling_mfma_bf16(sink, clocks, workgroups: int, iters: int, stream=None):
    """Dense bf16 MFMA loop, workgroups * 4 * iters * 8 * 32768 flop
    (C: hlta_ceiling_mfma_bf16). sink: float32 [workgroups * 256]; clocks:
    int64 [2] or None."""
    _check(load_library().hlta_ceiling_mfma_bf16(_ptr(sink), _ptr(clocks), int(workgroups), int(iters),
                                                 _stream(stream)))


def hlta_ceiling_copy(src, dst, stream=None):
    """dst = src with 16-byte loads and stores (C: hlta_ceiling_copy)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    _check(load_library().hlta_ceiling_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def measure_ceilings(reps: int = 5, copy_bytes: int = 2 << 30, device="cuda") -> dict:
    """Best of `reps` timed calls of each ceiling microbenchmark (after one
    untimed call), with HIP events on the launch stream: bf16 MFMA TFLOP/s at
    two workgroups per compute unit, the clock held meanwhile, and streaming
    copy GB/s (read + write bytes over time)."""
    props = torch.cuda.get_device_properties(device)
    wgs, iters = 2 * props.multi_processor_count, 4096
    sink = torch.empty(wgs * 256, dtype=torch.float32, device=device)
    clocks = torch.zeros(2, dtype=torch.int64, device=device)
    stream = torch.cuda.current_stream(device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flop = wgs * 4 * iters * MFMA_CEILING_FLOP_PER_WAVE_ITER
    best_mfma, ghz = 0.0, None
    for r in range(reps + 1):
        e0.record(stream)
        hlta_ceiling_mfma_bf16(sink, clocks, wgs, iters, stream)
        e1.record(stream)
        e1.synchronize()
        if r:
            tf = flop / (e0.elapsed_time(e1) * 1e-3) / 1e12
            if tf > best_mfma:
                best_mfma = tf
                c = clocks.cpu().tolist()
                ghz = c[0] / c[1] * 0.1 if c[1] > 0 else None
    src = torch.empty(copy_bytes // 4, dtype=torch.float32, device=device).fill_(1.0)
    dst = torch.empty_like(src)
    best_copy = 0.0
    for r in range(reps + 1):
        e0.record(stream)
        hlta_ceiling_copy(src, dst, stream)
        e1.record(stream)
        e1.synchronize()
        if r:
            best_copy = max(best_copy, 2 * copy_bytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    return {"mfma_bf16_tflops": best_mfma, "mfma_clock_ghz": ghz, "mfma_workgroups": wgs, "mfma_iters": iters,
            "hbm_copy_gbs": best_copy, "copy_bytes": copy_bytes, "reps": reps}


def to_device(x: dict, dtype: str, device="cuda") -> dict:
    """Move generator output (float32 numpy holding dtype values) to the GPU:
    q, k, v in the workload dtype (exact conversion), gates and weights float32."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for n, arr in x.items():
        t = torch.from_numpy(arr)
        out[n] = t.to(device=device, dtype=tdt if n in ("q", "k", "v") else torch.float32).contiguous()
    return out
