"""Seeded synthetic inputs for HLTA workloads.

This module is the only code shared by the float64 oracle and the GPU path.
It draws random numbers and casts them; it holds none of the operator's
arithmetic.

Workloads stand in for VAE latents of Kairos clips, which are not available:
latent grids of 30x52 (480P) and 45x80 (720P) tokens per latent frame, 31 and
61 latent frames (the 1 -> 241 frame clip-length ladder of the Kairos summary
page, section on the native world-model stack, at 4x temporal compression).

Recipe (per batch row b and head h, each tensor from its own PCG64 stream):
  q, k ~ N(0, 1), then L2-normalised per (token, head) over d, in float64;
  v ~ N(0, 1);
  a ~ U[0.9, 0.999]   (decay gate, float32);
  b = sigmoid(N(0, 1)) (write strength, float32);
  w ~ U[0.1, 1.0] per (head, branch) (mix weights, float32, not normalised);
then q, k, v are rounded once, round-to-nearest-even, from float64 straight to
the workload dtype (bfloat16 or float32).
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# field ids inside one stream
F_Q, F_K, F_V, F_A, F_B, F_W, F_DO = 0, 1, 2, 3, 4, 5, 6
# stream ids: 0 = the clip, 1 = the streaming prefix, 2 + s = streaming step s
S_CLIP, S_PREFIX, S_STEP0 = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    """Sizes of one HLTA workload (mirrors hlta_config in include/hlta.h)."""
    name: str
    B: int
    H: int
    T: int            # latent frames
    P: int            # tokens per latent frame
    d: int            # head dim (d_k = d_v)
    swa_frames: int   # W: frames in the sliding window, counting the current one
    dswa_dilation: int
    dswa_taps: int
    gdn_chunk: int
    dtype: str        # "f32" or "bf16" (inputs and outputs)
    seed: int
    # streaming only
    rollouts: int = 0
    prefix_frames: int = 0
    steps: int = 0
    ring_frames: int = 0

    @property
    def L(self) -> int:
        return self.T * self.P


TINY_F32 = Workload("tiny_f32_T8_P16", B=1, H=2, T=8, P=16, d=32, swa_frames=2,
                    dswa_dilation=2, dswa_taps=2, gdn_chunk=16, dtype="f32", seed=1000)
P480_T31 = Workload("p480_T31_bf16", B=1, H=24, T=31, P=1560, d=128, swa_frames=3,
                    dswa_dilation=4, dswa_taps=4, gdn_chunk=64, dtype="bf16", seed=1001)
P480_T61 = dataclasses.replace(P480_T31, name="p480_T61_bf16", T=61, seed=1002)
P720_T61 = Workload("p720_T61_bf16", B=1, H=24, T=61, P=3600, d=128, swa_frames=3,
                    dswa_dilation=4, dswa_taps=4, gdn_chunk=64, dtype="bf16", seed=1003)
# 8 rollouts stepping one 480P latent frame at a time, after a 16-frame prefix
STREAM_P480 = Workload("stream_p480_x8_bf16", B=8, H=24, T=1, P=1560, d=128, swa_frames=3,
                       dswa_dilation=4, dswa_taps=4, gdn_chunk=64, dtype="bf16", seed=1004,
                       rollouts=8, prefix_frames=16, steps=64, ring_frames=16)

WORKLOADS = {w.name: w for w in (TINY_F32, P480_T31, P480_T61, P720_T61, STREAM_P480)}


def rng(seed: int, stream: int, field: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, field, b, h])))


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to bfloat16, nearest-even, in one step.

    Returns float32 values (bfloat16 is a subset of float32, so the result is
    exact in float32). Handles bfloat16 subnormals; inputs must be finite and
    below the bfloat16 overflow threshold.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # below 2**-126 the quantum is fixed: 2**-133
    r = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)
    if not np.all(np.abs(r) < 3.3895313892515355e38):
        raise OverflowError("value outside the bfloat16 range")
    return r.astype(np.float32)


def cast(x, dtype: str) -> np.ndarray:
    """float64 -> workload dtype values, stored as float32 (exact)."""
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    # distribution recipe: directions uniform on the sphere
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def head_qkv(seed: int, stream: int, b: int, h: int, n: int, d: int, dtype: str,
             q_scale: float = 1.0):
    """q, k, v of one (b, h) head, n tokens: float32 arrays [n, d] of dtype values."""
    q = _unit_rows(rng(seed, stream, F_Q, b, h).standard_normal((n, d))) * q_scale
    k = _unit_rows(rng(seed, stream, F_K, b, h).standard_normal((n, d)))
    v = rng(seed, stream, F_V, b, h).standard_normal((n, d))
    return cast(q, dtype), cast(k, dtype), cast(v, dtype)


def head_gates(seed: int, stream: int, b: int, h: int, n: int,
               a_range=(0.9, 0.999)):
    """a, b gates of one (b, h) head: float32 arrays [n]."""
    a = rng(seed, stream, F_A, b, h).uniform(a_range[0], a_range[1], n).astype(np.float32)
    z = rng(seed, stream, F_B, b, h).standard_normal(n)
    bb = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    return a, bb


def mix_weights(seed: int, H: int) -> np.ndarray:
    """w [H, 3] float32 ~ U[0.1, 1.0]."""
    return rng(seed, S_CLIP, F_W, 0, 0).uniform(0.1, 1.0, (H, 3)).astype(np.float32)


def make_clip(wl: Workload, stream: int = S_CLIP, T: int | None = None, B: int | None = None,
              q_scale: float = 1.0, a_range=(0.9, 0.999), threads: int = 8):
    """Full-clip inputs as float32 numpy arrays.

    Returns dict with q, k, v [B, L, H, d] and a, b [B, L, H], w [H, 3].
    """
    T = wl.T if T is None else T
    B = wl.B if B is None else B
    L = T * wl.P
    q = np.empty((B, L, wl.H, wl.d), np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)
    a = np.empty((B, L, wl.H), np.float32)
    bb = np.empty_like(a)

    def one(bh):
        b, h = bh
        q[b, :, h], k[b, :, h], v[b, :, h] = head_qkv(wl.seed, stream, b, h, L, wl.d, wl.dtype, q_scale)
        a[b, :, h], bb[b, :, h] = head_gates(wl.seed, stream, b, h, L, a_range)

    jobs = [(b, h) for b in range(B) for h in range(wl.H)]
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, jobs))
    return dict(q=q, k=k, v=v, a=a, b=bb, w=mix_weights(wl.seed, wl.H))


def stream_step_inputs(wl: Workload, s: int, threads: int = 8):
    """Inputs of streaming step s: one latent frame per rollout, [B, P, H, d]."""
    step_wl = dataclasses.replace(wl, T=1)
    return make_clip(step_wl, stream=S_STEP0 + s, T=1, threads=threads)


def upstream_grad(wl: Workload, dtype: str, T: int | None = None, seed_offset: int = 0) -> np.ndarray:
    """dL/do_mix for the backward: standard normal [B, L, H, d] values of dtype
    (stored as float32), one generator per (b, h) as for the inputs."""
    T = wl.T if T is None else T
    L = T * wl.P
    g = np.empty((wl.B, L, wl.H, wl.d), np.float32)
    for b in range(wl.B):
        for h in range(wl.H):
            g[b, :, h] = cast(rng(wl.seed + seed_offset, S_CLIP, F_DO, b, h).standard_normal((L, wl.d)), dtype)
    return g
