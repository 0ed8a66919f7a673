"""Shared helpers of the GPU parity tests: run the library through the C ABI and
the float64 oracle on the same seeded inputs, and compare per branch."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from hybrid_linear_temporal_amd import hlta as H
from hybrid_linear_temporal_amd import inputs as I
from oracle import hlta_oracle as O

BRANCHES = ("o_swa", "o_dswa", "o_gdn", "o_mix")
# tolerances on relative L2 per branch: float32 inputs / bf16 inputs with fp32 accumulation
TOL = {"f32": 1e-4, "bf16": 1e-2}


def small(name, **kw) -> I.Workload:
    base = dict(B=1, H=2, T=8, P=16, d=32, swa_frames=2, dswa_dilation=2, dswa_taps=2, gdn_chunk=16,
                dtype="f32", seed=2000)
    base.update(kw)
    return I.Workload(name, **base)


def run_gpu(wl: I.Workload, x: dict, impl=H.HLTA_IMPL_AUTO, out_dtype=None, S0=None, want_state=True,
            **cfg_over):
    cfg = H.make_config(wl, impl=impl, out_dtype=out_dtype, **cfg_over)
    dev = H.to_device(x, wl.dtype)
    S_out = torch.empty((cfg.B, cfg.H, cfg.d, cfg.d), dtype=torch.float32, device="cuda") if want_state else None
    S0_t = None if S0 is None else torch.from_numpy(np.asarray(S0, np.float32)).cuda()
    res = H.hlta_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], S0=S0_t, S_out=S_out)
    torch.cuda.synchronize()
    return res


def to64(t) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def run_oracle(wl: I.Workload, x: dict, S0=None, heads=None, gdn="chunked", **over):
    T = over.get("T", wl.T)
    return O.hlta_forward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], T, wl.P,
                          over.get("swa_frames", wl.swa_frames), over.get("dswa_dilation", wl.dswa_dilation),
                          over.get("dswa_taps", wl.dswa_taps), over.get("gdn_chunk", wl.gdn_chunk),
                          S0=S0, gdn=gdn, heads=heads, rope_cfg=over.get("rope_cfg"),
                          gate_logits=over.get("gate_logits", False))


def frame_diagnostics(g: np.ndarray, r: np.ndarray, P: int) -> tuple[int, float, float]:
    """Worst latent frame of one branch ([B, L, H, d], L = T P): its index, its
    rel-L2 and the largest absolute difference anywhere (diagnostics only)."""
    T = g.shape[1] // P
    per = [O.rel_l2(g[:, f * P:(f + 1) * P], r[:, f * P:(f + 1) * P]) for f in range(T)]
    worst = int(np.argmax(per)) if per else 0
    return worst, (per[worst] if per else 0.0), float(np.max(np.abs(g - r))) if g.size else 0.0


def compare(gpu: dict, ref, tol: float, heads=None, label="", P=None):
    """rel-L2 per branch (and state) over the given heads; asserts <= tol.
    With P (tokens per frame) it also prints, per branch, the worst frame's
    rel-L2 and the largest absolute difference (not asserted)."""
    errs = {}
    diag = {}
    for i, n in enumerate(BRANCHES):
        g = to64(gpu[n])
        r = ref[i]
        if heads is not None:
            g = np.stack([g[b, :, h] for b, h in heads])
            r = np.stack([r[b, :, h] for b, h in heads])
        errs[n] = O.rel_l2(g, r)
        if P and heads is None and g.shape[1] % P == 0:
            f, e, m = frame_diagnostics(g, r, P)
            diag[n] = f"frame {f}: {e:.2e}, max-abs {m:.2e}"
    if gpu.get("S_out") is not None:
        g = to64(gpu["S_out"])
        r = ref[4]
        if heads is not None:
            g = np.stack([g[b, h] for b, h in heads])
            r = np.stack([r[b, h] for b, h in heads])
        errs["S_out"] = O.rel_l2(g, r)
    print(label, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    if diag:
        print(label, "worst frame per branch:", diag, flush=True)
    for n, e in errs.items():
        assert e <= tol, f"{label} {n}: rel-L2 {e:.3e} > {tol:.0e}"
    return errs


def replace(wl, **kw):
    return dataclasses.replace(wl, **kw)


def rescale_qk(x: dict, dtype: str, seed: int, lo: float = 0.3, hi: float = 3.0) -> dict:
    """Copy of x with every (token, head) row of q and k multiplied by its own
    factor ~ U[lo, hi], rounded once to dtype: keys and queries of non-unit
    norm, so the memory's in-op L2 normalisation changes the result."""
    rng = np.random.default_rng(seed)
    y = dict(x)
    for n in ("q", "k"):
        s = rng.uniform(lo, hi, x[n].shape[:-1])[..., None]
        y[n] = I.cast(x[n].astype(np.float64) * s, dtype)
    return y
