#!/usr/bin/env python3
"""HLTA forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one whole HLTA forward (gated-delta-rule memory, SWA, DSWA and the
mix) over one synthetic clip that is already resident in HBM. Prints one JSON
line: tokens/s over the timed steps, the roofline of the dominant kernel (the
softmax-branch kernel, priced against the bf16 MFMA peak) measured with HIP
events on the stream the library launches on, and the float64 CPU oracle timed
on a bounded sample of the same workload. Extra legs (reported beside, never in
`value`): the FP8 softmax branches, the rotary embedding, the backward
(hlta_bwd) and the streaming frame step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HLTA fwd tokens/s at 480P 31 latent frames (1 MI355X); % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA


def valid_pairs(T, P, W, dil, taps):
    """(SWA pairs, DSWA pairs) per (batch row, head): queries x keys of the frame sets."""
    swa = dsw = 0
    for f in range(T):
        swa += min(W, f + 1) * P * P
        dsw += min(taps, f // dil) * P * P
    return swa, dsw


def work(wl):
    """Algorithmic work of one forward: flops of the softmax branches (4*d per
    valid query-key pair: QK^T and PV), and compulsory HBM bytes of the memory
    branch (q, k, v read, a and b read, o_gdn written, per token-head, plus S out)."""
    swa, dsw = valid_pairs(wl.T, wl.P, wl.swa_frames, wl.dswa_dilation, wl.dswa_taps)
    heads = wl.B * wl.H
    attn_flops = 4 * wl.d * (swa + dsw) * heads
    el = 2 if wl.dtype == "bf16" else 4
    per_token_head = 3 * wl.d * el + 8 + wl.d * el
    gdn_bytes = per_token_head * wl.L * heads + heads * wl.d * wl.d * 4
    return attn_flops, gdn_bytes, per_token_head


def source_digest(*names):
    """Digest of kernel sources (plus the shared device header)."""
    h = hashlib.sha256()
    for n in (*names, "hlta_device.h"):
        with open(os.path.join(ROOT, "hybrid_linear_temporal_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_file, digest):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", kernel_file)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_digest") != digest or "bytes_per_launch" not in kv:
        return None
    return float(kv["bytes_per_launch"])


def cpu_baseline(wl, budget_s=12.0):
    """The float64 oracle (as it stands) on whole heads of the same workload,
    until the time budget is spent; scaled to whole-workload tokens/s."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from hybrid_linear_temporal_amd import inputs as I
    from oracle import hlta_oracle as O

    w = I.mix_weights(wl.seed, wl.H)
    done = []
    t_total = 0.0
    cpu0 = os.times()
    for b in range(wl.B):
        for h in range(wl.H):
            q, k, v = I.head_qkv(wl.seed, I.S_CLIP, b, h, wl.L, wl.d, wl.dtype)
            a, bb = I.head_gates(wl.seed, I.S_CLIP, b, h, wl.L)
            t0 = time.perf_counter()
            O.hlta_head(q, k, v, a, bb, w[h], wl.T, wl.P, wl.swa_frames, wl.dswa_dilation, wl.dswa_taps,
                        wl.gdn_chunk)
            t_total += time.perf_counter() - t0
            done.append((b, h))
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    cpu1 = os.times()
    frac = len(done) / (wl.B * wl.H)
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    host = host_cpu()
    busy = ((cpu1.user - cpu0.user) + (cpu1.system - cpu0.system)) / t_total
    return {"value": wl.B * wl.L * frac / t_total, "unit": "tokens/s", "cores": host["cores"],
            "kind": "oracle",
            "sample": f"float64 oracle (SWA, DSWA, chunked GDN, mix) on {len(done)} of {wl.B * wl.H} "
                      f"(batch, head) pairs of {wl.name}, {t_total:.1f} s; tokens/s scaled by that fraction",
            "cpu_model": host["model"], "logical_cpus": host["logical"],
            "blas_threads": int(max(blas) if blas else 1), "busy_cores_avg": round(busy, 2)}


def host_cpu():
    """The host CPUs this process may run on: model name, physical cores
    (distinct (package, core) pairs) and logical CPUs, from /proc/cpuinfo."""
    allowed = os.sched_getaffinity(0)
    model, cores, cpu, phys, core = "unknown", set(), None, None, None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f.read().splitlines() + [""]:
                if not line.strip():
                    if cpu in allowed:
                        cores.add((phys, core if core is not None else cpu))
                    cpu, phys, core = None, None, None
                    continue
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "processor":
                    cpu = int(v)
                elif k == "physical id":
                    phys = v
                elif k == "core id":
                    core = v
                elif k == "model name" and model == "unknown":
                    model = v
    except OSError:
        pass
    return {"model": model, "cores": len(cores) or len(allowed), "logical": len(allowed)}


def torch_recipe(shape, dtype, gen, device="cuda"):
    """q, k, v, a, b drawn on the GPU with the same recipe as the numpy
    generator (for timing-only runs: L2-normalised q, k; v ~ N(0,1);
    a ~ U[0.9, 0.999]; b = sigmoid(N(0,1)))."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B, L, Hh, d = shape
    q = torch.nn.functional.normalize(torch.randn(shape, generator=gen, device=device), dim=-1).to(tdt)
    k = torch.nn.functional.normalize(torch.randn(shape, generator=gen, device=device), dim=-1).to(tdt)
    v = torch.randn(shape, generator=gen, device=device).to(tdt)
    a = torch.rand((B, L, Hh), generator=gen, device=device) * 0.099 + 0.9
    b = torch.sigmoid(torch.randn((B, L, Hh), generator=gen, device=device))
    return q, k, v, a, b


def stream_leg(steps, warmup=4, distinct=4):
    """Streaming frame steps on the 8-rollout 480P workload: 16-frame prefix
    through hlta_fwd, then `steps` timed hlta_step_frame calls (inputs cycle
    over `distinct` pre-drawn frames). Returns a dict for the JSON line."""
    import torch
    from hybrid_linear_temporal_amd import hlta as H
    from hybrid_linear_temporal_amd import inputs as I

    wl = I.STREAM_P480
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed)
    P, R, prefix = wl.P, wl.ring_frames, wl.prefix_frames
    w = torch.from_numpy(I.mix_weights(wl.seed, wl.H)).cuda()
    q, k, v, a, b = torch_recipe((wl.B, prefix * P, wl.H, wl.d), wl.dtype, gen)
    cfg_pre = H.make_config(wl, T=prefix)
    S_pre = torch.empty((wl.B, wl.H, wl.d, wl.d), dtype=torch.float32, device="cuda")
    H.hlta_fwd(cfg_pre, q, k, v, a, b, w, S_out=S_pre)
    cfg = H.make_config(wl, T=1)
    st = H.Stream(cfg, R)
    H.hlta_stream_load_prefix(st, k, v, prefix, S_pre)
    del q, k, v, a, b
    frames = [torch_recipe((wl.B, P, wl.H, wl.d), wl.dtype, gen) for _ in range(distinct)]
    out = H.alloc_outputs(cfg, P)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fq, fk, fv, fa, fb = frames[i % distinct]
        H.hlta_step_frame(st, fq, fk, fv, fa, fb, w, out=out, stream=stream)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(stream)
    for i in range(steps):
        fq, fk, fv, fa, fb = frames[i % distinct]
        H.hlta_step_frame(st, fq, fk, fv, fa, fb, w, out=out, stream=stream)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    total = sum(per_step)
    pairs = (wl.swa_frames + wl.dswa_taps) * P * P * wl.B * wl.H   # every tap is valid after the prefix
    res = {"workload": wl.name, "steps": steps, "tokens_per_step": wl.B * P,
           "tokens_per_s": wl.B * P * steps / (total * 1e-3), "ms_per_step": total / steps,
           "ms_per_step_first8": sum(per_step[:8]) / min(8, steps),
           "ms_per_step_last8": sum(per_step[-8:]) / min(8, steps),
           "attn_tflops_per_step": 4 * wl.d * pairs / 1e12,
           "inputs": "torch-seeded GPU draws, same recipe; 4 distinct frames cycled"}
    res["rollouts"] = rollouts_leg(H, st, frames, w, out, max(2, steps // 2))
    return res


def rollouts_leg(H, st, frames, w, out, steps):
    """hlta_step_frame_rollouts on the same stream: first the rollouts are
    spread out (rollout b ends b frames ahead of rollout 0), then `steps`
    timed steps with every rollout at its own position, then `steps` with
    alternate rollouts sitting out (half the tokens per step)."""
    import numpy as np
    import torch
    B, P = st.cfg.B, st.cfg.P
    pos = np.full(B, st.frames_done, dtype=np.int64)
    stream = torch.cuda.current_stream()
    for j in range(B - 1):            # step j advances the rollouts b > j
        call = np.where(np.arange(B) > j, pos, -1).astype(np.int64)
        fq, fk, fv, fa, fb = frames[j % len(frames)]
        H.hlta_step_frame_rollouts(st, call, fq, fk, fv, fa, fb, w, out=out, stream=stream)
        pos = np.where(call >= 0, call, pos)
    spread = (pos - pos[0]).tolist()

    def timed(active):
        nonlocal pos
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        tokens = 0
        e0.record(stream)
        for i in range(steps):
            mask = active(i)
            call = np.where(mask, pos, -1).astype(np.int64)
            fq, fk, fv, fa, fb = frames[i % len(frames)]
            H.hlta_step_frame_rollouts(st, call, fq, fk, fv, fa, fb, w, out=out, stream=stream)
            pos = np.where(call >= 0, call, pos)
            tokens += int(mask.sum()) * P
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        return ms / steps, tokens / (ms * 1e-3)

    every = np.ones(B, dtype=bool)
    ms_all, tps_all = timed(lambda i: every)
    ms_half, tps_half = timed(lambda i: (np.arange(B) % 2) == (i % 2))
    return {"steps": steps, "frames_ahead_of_rollout0": spread,
            "ms_per_step": ms_all, "tokens_per_s": tps_all,
            "half_sitting_out_ms_per_step": ms_half, "half_sitting_out_tokens_per_s": tps_half}


# latent token grid of a frame (rows x columns) for the rotary-embedding leg
LATENT_GRID = {1560: (30, 52), 3600: (45, 80)}


def rope_leg(H, wl, dev, out, S_out, steps, impl):
    """hlta_fwd with the rotary embedding of the softmax branches on (theta
    10000, the frame's latent grid) against the same call without it, in the
    same process: whole-forward time per step for both."""
    import torch
    stream = torch.cuda.current_stream()
    res = {"grid": list(LATENT_GRID[wl.P]), "theta": 10000.0, "steps": steps}
    for tag, kw in (("with", dict(rope_theta=10000.0, rope_grid=LATENT_GRID[wl.P])), ("without", {})):
        cfg = H.make_config(wl, impl=impl, **kw)
        ws = H.alloc_workspace(H.hlta_fwd_workspace_bytes(cfg))

        def fwd():
            H.hlta_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], out=out, S_out=S_out,
                       workspace=ws, stream=stream)
        fwd()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fwd()
        e1.record(stream)
        torch.cuda.synchronize()
        res[f"ms_per_step_{tag}"] = e0.elapsed_time(e1) / steps
        del ws
    res["tokens_per_s_with"] = wl.B * wl.L / (res["ms_per_step_with"] * 1e-3)
    res["extra_ms"] = res["ms_per_step_with"] - res["ms_per_step_without"]
    return res


def fp8_leg(H, wl, dev, out, steps, impl):
    """The FP8 variant of the softmax branches on the same clip: quantisation
    (per (batch row, head) e4m3 codes and scales) and the attention kernel with
    the mix, each timed with HIP events, against the bf16 attention with the
    mix (hlta_attn_fwd) timed in the same loop."""
    import torch
    stream = torch.cuda.current_stream()
    cfg = H.make_config(wl, impl=impl)
    fp8 = H.hlta_quantize_fp8(cfg, dev["q"], dev["k"], dev["v"], stream=stream)
    H.hlta_attn_fwd_fp8(cfg, fp8, dev["w"], out["o_gdn"], out, stream=stream)
    H.hlta_attn_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["w"], out["o_gdn"], out, stream=stream)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        H.hlta_quantize_fp8(cfg, dev["q"], dev["k"], dev["v"], stream=stream)
        e[1].record(stream)
        H.hlta_attn_fwd_fp8(cfg, fp8, dev["w"], out["o_gdn"], out, stream=stream)
        e[2].record(stream)
        H.hlta_attn_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["w"], out["o_gdn"], out, stream=stream)
        e[3].record(stream)
    torch.cuda.synchronize()
    q_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    a_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    b_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / steps
    flops = work(wl)[0]
    tf = flops / (a_ms * 1e-3) / 1e12
    return {"steps": steps, "quantize_ms": q_ms, "attn_ms": a_ms, "attn_tflops": tf,
            "frac_of_fp8_peak": tf / PEAK_FP8_TFLOPS, "attn_ms_bf16": b_ms,
            "attn_speedup_vs_bf16": b_ms / a_ms,
            "note": "attn_ms and attn_ms_bf16 both include the mix kernel (hlta_attn_fwd_fp8, hlta_attn_fwd)"}


def bwd_leg(H, wl, dev, out, S_out, steps, impl):
    """The backward (hlta_bwd) on the same clip with a standard-normal upstream
    gradient in the output dtype: whole-call time per step with HIP events, and
    the softmax-branch part priced at the algorithmic backward flops (2.5x the
    forward's: QK^T, dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q)."""
    import torch
    stream = torch.cuda.current_stream()
    cfg = H.make_config(wl, impl=impl)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed + 7)
    d_mix = torch.randn(out["o_mix"].shape, generator=gen, device="cuda").to(out["o_mix"].dtype)
    ws = H.alloc_workspace(H.hlta_bwd_workspace_bytes(cfg))
    S0 = torch.zeros_like(S_out)

    def bwd():
        return H.hlta_bwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], out, d_mix, S0=S0,
                          workspace=ws, stream=stream)
    g = bwd()
    torch.cuda.synchronize()
    finite = all(bool(torch.isfinite(t).all()) for t in g.values() if t is not None)
    del g
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        bwd()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # the same with the forward's softmax statistics handed over (hlta_attn_fwd_lse
    # then hlta_bwd_lse, as a training step would call them)
    lse = H.hlta_attn_fwd_lse(cfg, dev["q"], dev["k"], dev["v"], dev["w"], out["o_gdn"], out, stream=stream)
    torch.cuda.synchronize()

    def bwd_lse():
        return H.hlta_bwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], out, d_mix, S0=S0,
                          workspace=ws, stream=stream, lse=lse)
    bwd_lse()
    e0.record(stream)
    for _ in range(steps):
        bwd_lse()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_lse = e0.elapsed_time(e1) / steps
    attn_flops = 2.5 * work(wl)[0]
    return {"steps": steps, "ms_per_step": ms, "tokens_per_s": wl.B * wl.L / (ms * 1e-3),
            "ms_per_step_lse_given": ms_lse, "tokens_per_s_lse_given": wl.B * wl.L / (ms_lse * 1e-3),
            "attn_bwd_flops": attn_flops, "workspace_bytes": ws.numel(), "grads_finite": finite,
            "note": "softmax branches on bf16 MFMA (fp32 gradients), memory on split-bf16 MFMA (fp32 "
                    "accumulation); _lse_given: the forward's softmax statistics passed in (hlta_bwd_lse); "
                    "per-kernel times in profiles/kernels_bwd_p480_T31_bf16.md"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="p480_T31_bf16")
    ap.add_argument("--impl", type=int, default=0, help="0 auto, 1 generic, 2 mfma")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stream-steps", type=int, default=64, help="streaming frame steps to time (0: skip)")
    ap.add_argument("--fp8-steps", type=int, default=5,
                    help="steps of the FP8 softmax branches timed (0: skip)")
    ap.add_argument("--rope-steps", type=int, default=5,
                    help="hlta_fwd steps timed with and without the rotary embedding (0: skip)")
    ap.add_argument("--bwd-steps", type=int, default=3,
                    help="steps of the backward (hlta_bwd) timed on the same clip (0: skip)")
    ap.add_argument("--ceiling-reps", type=int, default=5,
                    help="timed calls of each measured-ceiling microbenchmark (dense bf16 MFMA loop, HBM copy); "
                         "0: skip")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the library's streaming copy over 1 GiB (1 GiB read + 1 GiB written, 3 "
                         "launches), to scale rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1 (heads and rollouts shard across GPUs with no exchange, but no multi-GPU path is built)"}))
        sys.exit(2)

    import torch
    from hybrid_linear_temporal_amd import hlta as H
    from hybrid_linear_temporal_amd import inputs as I

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            H.hlta_ceiling_copy(src, dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"read_bytes": src.numel() * 4, "write_bytes": dst.numel() * 4,
                                               "launches": 3}}))
        return

    wl = I.WORKLOADS[args.workload]
    if wl.rollouts:
        raise SystemExit("use a whole-clip workload (the streaming workload has its own driver)")
    torch.cuda.set_device(0)
    H.load_library()
    print(f"# generating {wl.name} inputs", file=sys.stderr, flush=True)
    x = I.make_clip(wl, threads=16)
    dev = H.to_device(x, wl.dtype)
    del x
    cfg = H.make_config(wl, impl=args.impl)
    out = H.alloc_outputs(cfg, wl.L)
    ws = H.alloc_workspace(H.hlta_fwd_workspace_bytes(cfg))
    S_out = torch.empty((wl.B, wl.H, wl.d, wl.d), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    # one step = hlta_fwd as its two halves (hlta_attn_branches, then
    # hlta_gdn_mix_fwd: the memory branch with the mix), so that HIP events
    # bracket the attention kernel alone
    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        H.hlta_attn_branches(cfg, dev["q"], dev["k"], dev["v"], out, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        H.hlta_gdn_mix_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], out, S_out=S_out,
                           workspace=ws, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    print(f"# warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    print(f"# timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    attn_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    gdn_mix_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    ms = elapsed * 1e3 / args.steps
    # the memory branch alone (hlta_gdn_fwd: the step's second half without the
    # mix kernel), timed the same way right after the steps
    gev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    gev[0].record(stream)
    for i in range(args.steps):
        H.hlta_gdn_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], out["o_gdn"], S_out=S_out,
                       workspace=ws, stream=stream)
        gev[i + 1].record(stream)
    torch.cuda.synchronize()
    gdn_ms = gev[0].elapsed_time(gev[-1]) / args.steps
    tokens = wl.B * wl.L
    attn_flops, gdn_bytes, per_th = work(wl)
    attn_tflops = attn_flops / (attn_ms * 1e-3) / 1e12
    gdn_gbs = gdn_bytes / (gdn_ms * 1e-3) / 1e9
    mfma = cfg.impl != H.HLTA_IMPL_GENERIC and wl.dtype == "bf16" and wl.d == 128
    attn_src = "attn_mfma.hip" if mfma else "attn_generic.hip"
    srcs = (attn_src, "attn_mfma_tiles.h") if mfma else (attn_src,)
    traffic = read_traffic(f"traffic_{attn_src.split('.')[0]}_{wl.name}.txt", source_digest(*srcs))
    res = {
        "metric": METRIC, "value": tokens * args.steps / elapsed, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "P": wl.P, "d": wl.d,
                   "swa_frames": wl.swa_frames, "dswa_dilation": wl.dswa_dilation, "dswa_taps": wl.dswa_taps,
                   "gdn_chunk": wl.gdn_chunk, "tokens": tokens, "impl": ["auto", "generic", "mfma"][args.impl]},
        "roofline": {"bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "kernel": attn_src.split(".")[0], "flops_per_launch": attn_flops,
                     "avg_launch_ms": attn_ms},
        "gdn_roofline": {"bound": "hbm", "achieved": gdn_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gdn_gbs / PEAK_HBM_GBS, "bytes_per_launch": gdn_bytes,
                         "bytes_per_token_head": per_th, "avg_ms": gdn_ms,
                         "covers": "memory branch (4 kernels), hlta_gdn_fwd timed after the steps"},
        "step_split_ms": {"hlta_attn_branches": attn_ms, "hlta_gdn_mix_fwd": gdn_mix_ms},
        "device": torch.cuda.get_device_name(0),
    }
    if args.ceiling_reps > 0:
        print("# measured ceilings (bf16 MFMA loop, HBM copy)", file=sys.stderr, flush=True)
        ceil = H.measure_ceilings(reps=args.ceiling_reps)
        res["ceilings"] = ceil
        res["roofline"]["frac_of_measured"] = attn_tflops / ceil["mfma_bf16_tflops"]
        res["gdn_roofline"]["frac_of_measured"] = gdn_gbs / ceil["hbm_copy_gbs"]
    if args.fp8_steps > 0 and wl.d == 128 and wl.P >= 64:
        print(f"# FP8 leg, {args.fp8_steps} steps", file=sys.stderr, flush=True)
        res["fp8"] = fp8_leg(H, wl, dev, out, args.fp8_steps, args.impl)
    if args.rope_steps > 0 and wl.P in LATENT_GRID:
        print(f"# rotary-embedding leg, {args.rope_steps} steps", file=sys.stderr, flush=True)
        res["rope"] = rope_leg(H, wl, dev, out, S_out, args.rope_steps, args.impl)
    if args.bwd_steps > 0:
        print(f"# backward leg, {args.bwd_steps} steps", file=sys.stderr, flush=True)
        res["bwd"] = bwd_leg(H, wl, dev, out, S_out, args.bwd_steps, args.impl)
    if args.stream_steps > 0:
        del dev, out, ws
        torch.cuda.empty_cache()
        print(f"# streaming leg, {args.stream_steps} frame steps", file=sys.stderr, flush=True)
        res["stream"] = stream_leg(args.stream_steps)
    if not args.no_cpu_baseline:
        print("# cpu baseline (float64 oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
