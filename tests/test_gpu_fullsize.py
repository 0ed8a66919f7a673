"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (all heads, whole clips), checked on sampled outputs the float64 oracle
computes one by one: the whole memory branch and final state of sampled heads,
and the softmax branches and mix on sampled query frames of those heads.
Tolerance: relative L2 1e-2 (bf16 inputs, fp32 accumulation)."""
import numpy as np
import pytest
import torch

from hybrid_linear_temporal_amd import hlta as H
from hybrid_linear_temporal_amd import inputs as I
from oracle import hlta_oracle as O
from tests.helpers import BRANCHES as BRANCH_NAMES, TOL, to64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    H.load_library()


def _check_head(wl, x, res, b, h, frames, label):
    q, k, v = x["q"][b, :, h], x["k"][b, :, h], x["v"][b, :, h]
    o_gdn, S = O.gdn_chunked(q, k, v, x["a"][b, :, h], x["b"][b, :, h], wl.gdn_chunk)
    e = O.rel_l2(to64(res["o_gdn"][b, :, h]), o_gdn)
    eS = O.rel_l2(to64(res["S_out"][b, h]), S)
    print(f"{label} (b={b}, h={h}) o_gdn {e:.2e} S_out {eS:.2e}", flush=True)
    assert e <= TOL["bf16"] and eS <= TOL["bf16"]
    w3 = x["w"][h].astype(np.float64)
    P = wl.P
    for f in frames:
        sl = slice(f * P, (f + 1) * P)
        swa = O.attend_rows(q[sl], k, v, P, O.swa_frames(f, wl.swa_frames))
        dsw = O.attend_rows(q[sl], k, v, P, O.dswa_frames(f, wl.dswa_dilation, wl.dswa_taps))
        mix = w3[0] * swa + w3[1] * dsw + w3[2] * o_gdn[sl]
        for name, ref in (("o_swa", swa), ("o_dswa", dsw), ("o_mix", mix)):
            got = to64(res[name][b, sl, h])
            err = O.rel_l2(got, ref)
            print(f"{label} (b={b}, h={h}) frame {f} {name} {err:.2e}", flush=True)
            assert err <= TOL["bf16"], f"{label} frame {f} {name}: {err:.3e}"


@pytest.mark.parametrize("wl", [I.P480_T31, I.P480_T61, I.P720_T61], ids=lambda w: w.name)
def test_full_size_sampled(wl):
    print(f"generating {wl.name}", flush=True)
    x = I.make_clip(wl, threads=16)
    dev = H.to_device(x, wl.dtype)
    cfg = H.make_config(wl)
    S_out = torch.empty((wl.B, wl.H, wl.d, wl.d), dtype=torch.float32, device="cuda")
    res = H.hlta_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], S_out=S_out)
    torch.cuda.synchronize()
    del dev
    # frames: first (no DSWA key frame), one with a partial DSWA set, middle, last
    frames = sorted({0, 5, wl.T // 2, wl.T - 1})
    for b, h in ((0, 0), (wl.B - 1, wl.H - 1)):
        _check_head(wl, x, res, b, h, frames, wl.name)


def _fill_sampled(wl, T, stream, pairs, gen):
    """Device inputs [B, T*P, H, d] of a streaming workload: the sampled (rollout,
    head) pairs from the seeded NumPy generator (returned too, for the oracle),
    every other pair from torch's seeded GPU generator with the same recipe.
    Rollouts and heads are independent, so the others only have to fill the
    launch configuration."""
    B, L, Hh, d = wl.B, T * wl.P, wl.H, wl.d
    dev = {}
    for n in ("q", "k"):
        x = torch.randn((B, L, Hh, d), generator=gen, device="cuda")
        dev[n] = (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    dev["v"] = torch.randn((B, L, Hh, d), generator=gen, device="cuda").to(torch.bfloat16)
    dev["a"] = 0.9 + 0.099 * torch.rand((B, L, Hh), generator=gen, device="cuda")
    dev["b"] = torch.sigmoid(torch.randn((B, L, Hh), generator=gen, device="cuda"))
    dev["w"] = torch.from_numpy(I.mix_weights(wl.seed, Hh)).cuda()
    host = {}
    for b, h in pairs:
        q, k, v = I.head_qkv(wl.seed, stream, b, h, L, d, wl.dtype)
        a, bb = I.head_gates(wl.seed, stream, b, h, L)
        host[b, h] = dict(q=q, k=k, v=v, a=a, b=bb)
        for n, arr in host[b, h].items():
            t = torch.from_numpy(arr).cuda()
            dev[n][b, :, h] = t.to(dev[n].dtype)
    return dev, host


def test_stream_full_size_all_steps():
    """8 rollouts of 480P frames, the whole 64-step rollout: a 16-frame prefix
    through hlta_fwd, then 64 committed frame steps at full size (all 8
    rollouts, all 24 heads). Three sampled (rollout, head) pairs follow a
    float64 stream each: o_gdn on every step, all four outputs on every 8th
    step and the last, and the carried state after step 64."""
    wl = I.STREAM_P480
    P, R, prefix, steps = wl.P, wl.ring_frames, wl.prefix_frames, wl.steps
    pairs = ((0, 0), (3, 11), (wl.B - 1, wl.H - 1))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed)
    pre_wl = I.Workload("stream_prefix", B=wl.B, H=wl.H, T=prefix, P=P, d=wl.d, swa_frames=wl.swa_frames,
                        dswa_dilation=wl.dswa_dilation, dswa_taps=wl.dswa_taps, gdn_chunk=wl.gdn_chunk,
                        dtype=wl.dtype, seed=wl.seed)
    print("stream prefix (16 frames, 8 rollouts) through hlta_fwd", flush=True)
    dev, host = _fill_sampled(wl, prefix, I.S_PREFIX, pairs, gen)
    S_pre = torch.empty((wl.B, wl.H, wl.d, wl.d), dtype=torch.float32, device="cuda")
    H.hlta_fwd(H.make_config(pre_wl), dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], S_out=S_pre)
    st = H.Stream(H.make_config(wl), R)
    H.hlta_stream_load_prefix(st, dev["k"], dev["v"], prefix, S_pre)
    torch.cuda.synchronize()
    del dev
    w = I.mix_weights(wl.seed, wl.H)
    ost = {}
    for b, h in pairs:
        x = host[b, h]
        _, Sp = O.gdn_chunked(x["q"], x["k"], x["v"], x["a"], x["b"], wl.gdn_chunk)
        s = O.StreamHead(P, wl.swa_frames, wl.dswa_dilation, wl.dswa_taps, wl.gdn_chunk)
        s.load_prefix(x["k"], x["v"], prefix, Sp)
        ost[b, h] = s
    for s_i in range(steps):
        dev, host = _fill_sampled(wl, 1, I.S_STEP0 + s_i, pairs, gen)
        got = H.hlta_step_frame(st, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"])
        torch.cuda.synchronize()
        full_check = s_i % 8 == 0 or s_i == steps - 1
        for b, h in pairs:
            x, s = host[b, h], ost[b, h]
            f = s.f
            if full_check:
                refs = s.step(x["q"], x["k"], x["v"], x["a"], x["b"], w[h])
                names = BRANCH_NAMES
            else:
                # the memory only: advance the float64 stream exactly as its
                # step does (the keys of frame f join its store unrotated)
                o_gdn, S = O.gdn_chunked(x["q"], x["k"], x["v"], x["a"], x["b"], wl.gdn_chunk, s.S0)
                s.k[f], s.v[f] = np.asarray(x["k"], np.float64), np.asarray(x["v"], np.float64)
                s.S0, s.f = S, f + 1
                refs, names = (o_gdn,), ("o_gdn",)
            for name, ref in zip(names, refs):
                err = O.rel_l2(to64(got[name][b, :, h]), ref)
                print(f"stream step {s_i} (frame {f}, b={b}, h={h}) {name} {err:.2e}", flush=True)
                assert err <= TOL["bf16"], f"step {s_i} (b={b}, h={h}) {name}: {err:.3e}"
    assert st.frames_done == prefix + steps
    for b, h in pairs:
        err = O.rel_l2(to64(st.S[b, h]), ost[b, h].S0)
        print(f"stream state after {steps} steps (b={b}, h={h}) {err:.2e}", flush=True)
        assert err <= TOL["bf16"], f"stream state (b={b}, h={h}) {err:.3e}"


def test_full_size_rope_and_fp8_sampled():
    """480P / 31 frames at full size: the rotary embedding (the 30 x 52 latent
    grid) on sampled query frames of two heads against the float64 oracle; the
    FP8 softmax branches against exact attention over the dequantised inputs
    and the quantiser's codes bit for bit on those heads."""
    wl = I.P480_T31
    grid, theta = (30, 52), 10000.0
    x = I.make_clip(wl, threads=16)
    dev = H.to_device(x, wl.dtype)
    P = wl.P
    frames = (0, 5, wl.T - 1)
    heads = ((0, 0), (0, wl.H - 1))
    # rotary embedding
    cfg = H.make_config(wl, rope_theta=theta, rope_grid=grid)
    res = H.hlta_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"])
    torch.cuda.synchronize()
    pos = O.rope_positions(wl.T, P, grid[1])
    for b, h in heads:
        qr, kr = O.rope(x["q"][b, :, h], pos, theta), O.rope(x["k"][b, :, h], pos, theta)
        v = x["v"][b, :, h]
        for f in frames:
            sl = slice(f * P, (f + 1) * P)
            for name, fr in (("o_swa", O.swa_frames(f, wl.swa_frames)),
                             ("o_dswa", O.dswa_frames(f, wl.dswa_dilation, wl.dswa_taps))):
                err = O.rel_l2(to64(res[name][b, sl, h]), O.attend_rows(qr[sl], kr, v, P, fr))
                print(f"rope (b={b}, h={h}) frame {f} {name} {err:.2e}", flush=True)
                assert err <= TOL["bf16"], (b, h, f, name, err)
    del res
    # FP8 variant
    cfg = H.make_config(wl)
    fp8 = H.hlta_quantize_fp8(cfg, dev["q"], dev["k"], dev["v"])
    out = H.alloc_outputs(cfg, wl.L)
    out["o_gdn"].zero_()
    H.hlta_attn_fwd_fp8(cfg, fp8, dev["w"], out["o_gdn"], out)
    torch.cuda.synchronize()
    scales = fp8["scales"].cpu().numpy()
    for b, h in heads:
        deq = {}
        for i, n in enumerate("qkv"):
            code, s = O.quantize_e4m3(x[n][b:b + 1, :, h:h + 1])
            assert np.array_equal(fp8[n + "8"][b, :, h].cpu().numpy(), code[0, :, 0]), (n, b, h)
            assert scales[b, h, i] == s[0, 0], (n, b, h)
            deq[n] = O.dequantize_e4m3(code, s)[0, :, 0]
        for f in frames:
            sl = slice(f * P, (f + 1) * P)
            for name, fr in (("o_swa", O.swa_frames(f, wl.swa_frames)),
                             ("o_dswa", O.dswa_frames(f, wl.dswa_dilation, wl.dswa_taps))):
                ref = O.attend_rows(deq["q"][sl], deq["k"], deq["v"], P, fr)
                err = O.rel_l2(to64(out[name][b, sl, h]), ref)
                print(f"fp8 (b={b}, h={h}) frame {f} {name} {err:.2e}", flush=True)
                assert err <= 3e-2, (b, h, f, name, err)


def test_full_size_backward_one_head():
    """hlta_bwd at 480P / 31 frames (all 24 heads, the launch configuration
    bench.py times) against the float64 oracle's gradients of one whole head:
    its dq, dk, dv over all 48360 tokens (sums of the three branches), its gate
    gradients, its start-state gradient, and its mix-weight gradient (B = 1, so
    dw[h] is a sum over this head alone). Bar: relative L2 1e-2 (bf16 inputs
    and outputs; the softmax branches round P and dS to bf16 for their products)."""
    wl = I.P480_T31
    print(f"generating {wl.name} and its upstream gradient", flush=True)
    x = I.make_clip(wl, threads=16)
    g = I.upstream_grad(wl, "bf16")
    dev = H.to_device(x, wl.dtype)
    cfg = H.make_config(wl)
    S0 = (0.1 * np.random.default_rng(wl.seed).standard_normal((wl.B, wl.H, wl.d, wl.d))).astype(np.float32)
    S0_t = torch.from_numpy(S0).cuda()
    fwd = H.hlta_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], S0=S0_t)
    g_t = torch.from_numpy(g).cuda().to(torch.bfloat16)
    got = H.hlta_bwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], fwd, g_t, S0=S0_t)
    torch.cuda.synchronize()
    print("GPU backward done; oracle on one head", flush=True)
    b, h = 0, 7
    q, k, v = x["q"][b, :, h], x["k"][b, :, h], x["v"][b, :, h]
    a, bb = x["a"][b, :, h], x["b"][b, :, h]
    gh = g[b, :, h].astype(np.float64)
    w3 = x["w"][h].astype(np.float64)
    P, T = wl.P, wl.T
    dq = np.zeros(q.shape)
    dk = np.zeros(q.shape)
    dv = np.zeros(q.shape)
    frame_sets = ((w3[0], lambda f: O.swa_frames(f, wl.swa_frames)),
                  (w3[1], lambda f: O.dswa_frames(f, wl.dswa_dilation, wl.dswa_taps)))
    for wi, fo in frame_sets:
        gq, gk, gv = O.attention_backward(q, k, v, wi * gh, T, P, fo)
        dq += gq
        dk += gk
        dv += gv
    gq, gk, gv, ga, gb, gS = O.gdn_recurrent_backward(q, k, v, a, bb, w3[2] * gh, S0[b, h])
    dq += gq
    dk += gk
    dv += gv
    o_swa = O.swa(q, k, v, T, P, wl.swa_frames)
    o_dswa = O.dswa(q, k, v, T, P, wl.dswa_dilation, wl.dswa_taps)
    o_gdn, _ = O.gdn_recurrent(q, k, v, a, bb, S0[b, h])
    dw = np.array([np.sum(gh * o_swa), np.sum(gh * o_dswa), np.sum(gh * o_gdn)])
    checks = (("dq", to64(got["dq"][b, :, h]), dq), ("dk", to64(got["dk"][b, :, h]), dk),
              ("dv", to64(got["dv"][b, :, h]), dv), ("da", to64(got["da"][b, :, h]), ga),
              ("db", to64(got["db"][b, :, h]), gb), ("dS0", to64(got["dS0"][b, h]), gS),
              ("dmix_w", to64(got["dmix_w"][h]), dw))
    for name, gv_, rv in checks:
        err = O.rel_l2(gv_, rv)
        print(f"{wl.name} backward (b={b}, h={h}) {name} {err:.2e}", flush=True)
        assert err <= TOL["bf16"], f"{name}: {err:.3e}"
