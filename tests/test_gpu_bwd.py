"""Backward parity: hlta_bwd (through the C ABI) against the float64 oracle's
gradients (oracle.hlta_backward, itself pinned by central differences of the
pinned forward) on the same seeded inputs, upstream gradient and start state.

Cases span several row and key tiles of the softmax kernels with ragged tails
(P not a multiple of 64 or 32), ragged last chunks of the memory's
checkpoints, batch rows > 1, every dtype pair, and the empty clip."""
import numpy as np
import pytest
import torch

from hybrid_linear_temporal_amd import hlta as H
from hybrid_linear_temporal_amd import inputs as I
from oracle import hlta_oracle as O
from tests.helpers import TOL, small, to64

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "da", "db", "dmix_w", "dS0")

GEN, AUTO = H.HLTA_IMPL_GENERIC, H.HLTA_IMPL_AUTO
_BF16 = small("bwd_bf16", B=1, H=2, T=5, P=72, d=128, swa_frames=3, dswa_dilation=2, dswa_taps=2, gdn_chunk=64,
              dtype="bf16", seed=2102)
CASES = [
    # name, workload, out dtype, impl
    ("tiny_f32", small("bwd_tiny"), "f32", AUTO),
    ("ragged_f32_d64", small("bwd_ragged", B=2, H=2, T=7, P=40, d=64, swa_frames=3, dswa_dilation=2,
                             dswa_taps=3, gdn_chunk=32, seed=2101), "f32", AUTO),
    # bf16 in and out, d = 128, P >= 64: the softmax branches on the MFMA kernels
    ("bf16_d128_mfma", _BF16, "bf16", AUTO),
    ("bf16_d128_generic", _BF16, "bf16", GEN),
    ("bf16_mfma_B2_P100", small("bwd_bf16b", B=2, H=2, T=9, P=100, d=128, swa_frames=3, dswa_dilation=2,
                                dswa_taps=3, gdn_chunk=64, dtype="bf16", seed=2104), "bf16", AUTO),
    ("bf16_in_f32_out", small("bwd_bf16f", B=1, H=1, T=6, P=24, d=128, swa_frames=2, dswa_dilation=3,
                              dswa_taps=2, gdn_chunk=16, dtype="bf16", seed=2103), "f32", AUTO),
    # 16 heads x 35 chunks (the last one ragged): more chunk jobs than the
    # memory's persistent grid of 512 workgroups, so some walk a second chunk
    # and its slot; the forward runs 7 segments of 5 chunks
    ("bf16_mfma_560_chunks", small("bwd_bf16w", B=1, H=16, T=10, P=220, d=128, swa_frames=3, dswa_dilation=2,
                                   dswa_taps=3, gdn_chunk=64, dtype="bf16", seed=2105), "bf16", AUTO),
]


def _mfma(wl, out_dt, impl):
    return impl != GEN and wl.dtype == "bf16" and out_dt == "bf16" and wl.d == 128 and wl.P >= 64


def _start_state(wl):
    return (0.1 * np.random.default_rng(wl.seed).standard_normal((wl.B, wl.H, wl.d, wl.d))).astype(np.float32)


def _run(wl, out_dt, impl=AUTO, with_S0=True):
    x = I.make_clip(wl)
    cfg = H.make_config(wl, out_dtype=out_dt, impl=impl)
    dev = H.to_device(x, wl.dtype)
    S0 = _start_state(wl) if with_S0 else None
    S0_t = None if S0 is None else torch.from_numpy(S0).cuda()
    fwd = H.hlta_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], S0=S0_t)
    g = I.upstream_grad(wl, out_dt)
    g_t = torch.from_numpy(g).cuda().to(torch.bfloat16 if out_dt == "bf16" else torch.float32)
    got = H.hlta_bwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], fwd, g_t, S0=S0_t)
    torch.cuda.synchronize()
    ref = O.hlta_backward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], g, wl.T, wl.P, wl.swa_frames,
                          wl.dswa_dilation, wl.dswa_taps, S0=S0)
    return got, dict(zip(GRADS, ref))


@pytest.mark.parametrize("name,wl,out_dt,impl", CASES, ids=[c[0] for c in CASES])
def test_bwd_matches_oracle(name, wl, out_dt, impl):
    print(f"case {name}: B={wl.B} H={wl.H} T={wl.T} P={wl.P} d={wl.d} C={wl.gdn_chunk} {wl.dtype}->{out_dt} "
          f"impl={impl}", flush=True)
    got, ref = _run(wl, out_dt, impl)
    # The generic kernels evaluate every gradient in fp32 from the same
    # (dtype-exact) inputs, so the fp32 bar holds whatever the dtypes. The
    # bf16 bar applies to (a) the mix-weight gradient with bf16 outputs (it
    # reads the branch outputs as stored, rounded to bf16, where the oracle
    # takes exact ones) and (b) dq, dk, dv on the MFMA kernels, which round P
    # and dS to bf16 for their products and take D from the stored outputs.
    # da, db and dS0 come from the memory alone (fp32) on every path.
    mfma = _mfma(wl, out_dt, impl)
    errs = {n: O.rel_l2(to64(got[n]), ref[n]) for n in GRADS}
    print(name, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n, e in errs.items():
        loose = (n == "dmix_w" and out_dt == "bf16") or (mfma and n in ("dq", "dk", "dv"))
        tol = TOL["bf16"] if loose else TOL["f32"]
        assert e <= tol, f"{name} {n}: rel-L2 {e:.3e} > {tol:.0e}"


LSE_CASES = [("bf16_mfma_B2_P100", CASES[4][1], "bf16", AUTO), ("tiny_f32", CASES[0][1], "f32", AUTO)]


@pytest.mark.parametrize("name,wl,out_dt,impl", LSE_CASES, ids=[c[0] for c in LSE_CASES])
def test_forward_statistics_and_backward_with_them(name, wl, out_dt, impl):
    """hlta_attn_fwd_lse leaves the outputs of hlta_attn_fwd unchanged (bit for
    bit) and writes each row's log-sum-exp (log2 units) as the oracle's
    frame_softmax_lse2 gives it, 0 for rows without keys; hlta_bwd_lse with
    those statistics gives hlta_bwd's gradients (to the rounding of the
    statistics) and the oracle's, to the same bar as test_bwd_matches_oracle."""
    print(f"case {name} with forward statistics", flush=True)
    x = I.make_clip(wl)
    cfg = H.make_config(wl, out_dtype=out_dt, impl=impl)
    dev = H.to_device(x, wl.dtype)
    S0 = _start_state(wl)
    S0_t = torch.from_numpy(S0).cuda()
    fwd = H.hlta_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], S0=S0_t)
    out2 = H.alloc_outputs(cfg, wl.L)
    lse = H.hlta_attn_fwd_lse(cfg, dev["q"], dev["k"], dev["v"], dev["w"], fwd["o_gdn"], out2)
    torch.cuda.synchronize()
    for n in ("o_swa", "o_dswa", "o_mix"):
        assert torch.equal(out2[n], fwd[n]), n
    got_lse = lse.double().cpu().numpy()
    worst = 0.0
    for b in range(wl.B):
        for h in range(wl.H):
            qb, kb = x["q"][b, :, h].astype(np.float64), x["k"][b, :, h].astype(np.float64)
            sets = (lambda f: O.swa_frames(f, wl.swa_frames),
                    lambda f: O.dswa_frames(f, wl.dswa_dilation, wl.dswa_taps))
            for br, frames_of in enumerate(sets):
                ref = O.frame_softmax_lse2(qb, kb, wl.T, wl.P, frames_of)
                worst = max(worst, float(np.abs(got_lse[br, b, h] - ref).max()))
    print(f"{name} lse max abs error (log2 units) {worst:.2e}", flush=True)
    assert worst <= (1e-3 if out_dt == "bf16" else 1e-5)
    g = I.upstream_grad(wl, out_dt)
    g_t = torch.from_numpy(g).cuda().to(torch.bfloat16 if out_dt == "bf16" else torch.float32)
    plain = H.hlta_bwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], fwd, g_t, S0=S0_t)
    given = H.hlta_bwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], fwd, g_t, S0=S0_t,
                       lse=lse)
    torch.cuda.synchronize()
    ref = dict(zip(GRADS, O.hlta_backward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], g, wl.T, wl.P,
                                          wl.swa_frames, wl.dswa_dilation, wl.dswa_taps, S0=S0)))
    mfma = _mfma(wl, out_dt, impl)
    for n in GRADS:
        same = O.rel_l2(to64(given[n]), to64(plain[n]))
        e = O.rel_l2(to64(given[n]), ref[n])
        print(f"{name} {n}: vs hlta_bwd {same:.1e}, vs oracle {e:.2e}", flush=True)
        # the generic kernels recompute the statistics, so they match exactly
        assert same <= (1e-3 if mfma else 0.0), n
        loose = (n == "dmix_w" and out_dt == "bf16") or (mfma and n in ("dq", "dk", "dv"))
        assert e <= (TOL["bf16"] if loose else TOL["f32"]), n


def test_bwd_without_start_state_gradient():
    """dS0 = NULL is allowed; the other gradients are unchanged, and a NULL S0
    means the zero start state."""
    wl = CASES[0][1]
    print("case tiny_f32 without S0 / dS0", flush=True)
    x = I.make_clip(wl)
    cfg = H.make_config(wl)
    dev = H.to_device(x, wl.dtype)
    fwd = H.hlta_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"])
    g = I.upstream_grad(wl, "f32")
    g_t = torch.from_numpy(g).cuda()
    got = H.hlta_bwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], fwd, g_t, want_dS0=False)
    torch.cuda.synchronize()
    assert got["dS0"] is None
    ref = O.hlta_backward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], g, wl.T, wl.P, wl.swa_frames,
                          wl.dswa_dilation, wl.dswa_taps)
    for n, r in zip(GRADS[:-1], ref[:-1]):
        assert O.rel_l2(to64(got[n]), r) <= TOL["f32"], n


def test_bwd_empty_clip():
    """T = 0: the mix-weight and start-state gradients are zero, nothing else is touched."""
    wl = small("bwd_empty", T=0)
    print("case empty clip", flush=True)
    cfg = H.make_config(wl)
    z = torch.zeros((wl.B, 0, wl.H, wl.d), device="cuda")
    zg = torch.zeros((wl.B, 0, wl.H), device="cuda")
    w = torch.ones((wl.H, 3), device="cuda")
    fwd = {"o_swa": z, "o_dswa": z, "o_gdn": z}
    got = H.hlta_bwd(cfg, z, z, z, zg, zg, w, fwd, z)
    torch.cuda.synchronize()
    assert torch.count_nonzero(got["dmix_w"]).item() == 0
    assert torch.count_nonzero(got["dS0"]).item() == 0


def test_bwd_deterministic():
    """Two backward calls on the same inputs give bit-identical gradients (no
    atomics; every reduction runs in a fixed order), on the MFMA path."""
    wl = CASES[4][1]
    print(f"case {CASES[4][0]} twice", flush=True)
    x = I.make_clip(wl)
    cfg = H.make_config(wl)
    dev = H.to_device(x, wl.dtype)
    fwd = H.hlta_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"])
    g_t = torch.from_numpy(I.upstream_grad(wl, "bf16")).cuda().to(torch.bfloat16)
    r1 = H.hlta_bwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], fwd, g_t)
    r2 = H.hlta_bwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], fwd, g_t)
    torch.cuda.synchronize()
    for n in GRADS:
        assert torch.equal(r1[n], r2[n]), n


def test_bwd_graph_replays_match_eager():
    """hlta_bwd captured in a HIP graph (MFMA path): every replay, with eager
    work and synchronisation in between, equals the eager call bit for bit."""
    wl = CASES[4][1]
    print(f"case {CASES[4][0]} captured", flush=True)
    x = I.make_clip(wl)
    cfg = H.make_config(wl)
    dev = H.to_device(x, wl.dtype)
    fwd = H.hlta_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"])
    g_t = torch.from_numpy(I.upstream_grad(wl, "bf16")).cuda().to(torch.bfloat16)
    ws = H.alloc_workspace(H.hlta_bwd_workspace_bytes(cfg))

    def call():
        return H.hlta_bwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], fwd, g_t, workspace=ws)

    ref = call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            out = call()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for t in out.values():
            t.fill_(float("nan"))
        ws.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in GRADS:
            assert torch.equal(out[n], ref[n]), (rep, n)


def _oracle_grads(wl, x, g, S0, l2norm):
    """Gradients of every head from the oracle's per-branch functions, with the
    memory's L2 normalisation on or off (hlta_backward takes the default)."""
    B, Lt, Hh, d = x["q"].shape
    out = {n: np.zeros((B, Lt, Hh, d)) for n in ("dq", "dk", "dv")}
    out["da"], out["db"] = np.zeros((B, Lt, Hh)), np.zeros((B, Lt, Hh))
    out["dmix_w"], out["dS0"] = np.zeros((Hh, 3)), np.zeros((B, Hh, d, d))
    for b in range(B):
        for h in range(Hh):
            q, k, v = x["q"][b, :, h], x["k"][b, :, h], x["v"][b, :, h]
            a, bb = x["a"][b, :, h], x["b"][b, :, h]
            gh = g[b, :, h].astype(np.float64)
            w3 = x["w"][h].astype(np.float64)
            s0 = None if S0 is None else S0[b, h]
            for i, fo in ((0, lambda f: O.swa_frames(f, wl.swa_frames)),
                          (1, lambda f: O.dswa_frames(f, wl.dswa_dilation, wl.dswa_taps))):
                gq, gk, gv = O.attention_backward(q, k, v, w3[i] * gh, wl.T, wl.P, fo)
                out["dq"][b, :, h] += gq
                out["dk"][b, :, h] += gk
                out["dv"][b, :, h] += gv
            gq, gk, gv, ga, gb, gS = O.gdn_recurrent_backward(q, k, v, a, bb, w3[2] * gh, s0, l2norm=l2norm)
            out["dq"][b, :, h] += gq
            out["dk"][b, :, h] += gk
            out["dv"][b, :, h] += gv
            out["da"][b, :, h], out["db"][b, :, h], out["dS0"][b, h] = ga, gb, gS
            o_gdn, _ = O.gdn_recurrent(q, k, v, a, bb, s0, l2norm=l2norm)
            out["dmix_w"][h] += [np.sum(gh * O.swa(q, k, v, wl.T, wl.P, wl.swa_frames)),
                                 np.sum(gh * O.dswa(q, k, v, wl.T, wl.P, wl.dswa_dilation, wl.dswa_taps)),
                                 np.sum(gh * o_gdn)]
    return out


@pytest.mark.parametrize("name,wl,out_dt,l2norm", [
    ("f32_no_l2norm", small("bwd_nol2", B=1, H=2, T=6, P=20, d=32, swa_frames=2, dswa_dilation=2, dswa_taps=2,
                            gdn_chunk=16, seed=2105), "f32", False),
    ("bf16_mfma_chunk32", small("bwd_c32", B=1, H=2, T=5, P=72, d=128, swa_frames=3, dswa_dilation=2,
                                dswa_taps=2, gdn_chunk=32, dtype="bf16", seed=2106), "bf16", True),
], ids=["f32_no_l2norm", "bf16_mfma_chunk32"])
def test_bwd_options(name, wl, out_dt, l2norm):
    """The memory's L2 normalisation off (q and k halved, so it matters), with
    the forward's memory output checked too; and the MFMA softmax-branch
    kernels beside a 32-token memory chunk."""
    print(f"case {name}", flush=True)
    x = I.make_clip(wl)
    x["q"] = (x["q"] * 0.5).astype(np.float32)   # exact in every dtype
    x["k"] = (x["k"] * 0.5).astype(np.float32)
    cfg = H.make_config(wl, out_dtype=out_dt, l2norm=l2norm)
    dev = H.to_device(x, wl.dtype)
    S0 = _start_state(wl)
    S0_t = torch.from_numpy(S0).cuda()
    fwd = H.hlta_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], S0=S0_t)
    g = I.upstream_grad(wl, out_dt)
    g_t = torch.from_numpy(g).cuda().to(torch.bfloat16 if out_dt == "bf16" else torch.float32)
    got = H.hlta_bwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], fwd, g_t, S0=S0_t)
    torch.cuda.synchronize()
    tol = TOL[out_dt]
    for b in range(wl.B):
        for h in range(wl.H):
            o_ref, _ = O.gdn_recurrent(x["q"][b, :, h], x["k"][b, :, h], x["v"][b, :, h], x["a"][b, :, h],
                                       x["b"][b, :, h], S0[b, h], l2norm=l2norm)
            e = O.rel_l2(to64(fwd["o_gdn"][b, :, h]), o_ref)
            print(f"{name} forward o_gdn (b={b}, h={h}) {e:.2e}", flush=True)
            assert e <= tol
    ref = _oracle_grads(wl, x, g, S0, l2norm)
    mfma = _mfma(wl, out_dt, AUTO)
    for n in GRADS:
        e = O.rel_l2(to64(got[n]), ref[n])
        print(f"{name} {n} {e:.2e}", flush=True)
        loose = (n == "dmix_w" and out_dt == "bf16") or (mfma and n in ("dq", "dk", "dv"))
        assert e <= (TOL["bf16"] if loose else TOL["f32"]), f"{name} {n}: {e:.3e}"


@pytest.mark.parametrize("name,wl,out_dt", [
    ("f32_scale", small("scale_f32", B=1, H=2, T=6, P=20, d=32, swa_frames=2, dswa_dilation=2, dswa_taps=2,
                        gdn_chunk=16, seed=2108), "f32"),
    ("bf16_mfma_scale", small("scale_bf16", B=1, H=1, T=5, P=72, d=128, swa_frames=3, dswa_dilation=2,
                              dswa_taps=2, gdn_chunk=64, dtype="bf16", seed=2109), "bf16"),
], ids=["f32", "bf16_mfma"])
def test_softmax_scale_forward_and_backward(name, wl, out_dt):
    """A caller-set softmax scale (0.3 instead of 1/sqrt(d)) reaches both
    softmax branches of the forward and their gradients."""
    scale = 0.3
    print(f"case {name} scale {scale}", flush=True)
    x = I.make_clip(wl, q_scale=4.0)   # peaked enough that the scale matters
    cfg = H.make_config(wl, out_dtype=out_dt, softmax_scale=scale)
    dev = H.to_device(x, wl.dtype)
    fwd = H.hlta_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"])
    g = I.upstream_grad(wl, out_dt)
    g_t = torch.from_numpy(g).cuda().to(torch.bfloat16 if out_dt == "bf16" else torch.float32)
    got = H.hlta_bwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], fwd, g_t)
    torch.cuda.synchronize()
    tol = TOL[out_dt]
    for h in range(wl.H):
        q, k, v = x["q"][0, :, h], x["k"][0, :, h], x["v"][0, :, h]
        for name_o, ref in (("o_swa", O.swa(q, k, v, wl.T, wl.P, wl.swa_frames, scale)),
                            ("o_dswa", O.dswa(q, k, v, wl.T, wl.P, wl.dswa_dilation, wl.dswa_taps, scale))):
            e = O.rel_l2(to64(fwd[name_o][0, :, h]), ref)
            print(f"{name} {name_o} h={h} {e:.2e}", flush=True)
            assert e <= tol
    ref = O.hlta_backward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], g, wl.T, wl.P, wl.swa_frames,
                          wl.dswa_dilation, wl.dswa_taps, scale=scale)
    mfma = _mfma(wl, out_dt, AUTO)
    for n, r in zip(GRADS, ref):
        e = O.rel_l2(to64(got[n]), r)
        print(f"{name} {n} {e:.2e}", flush=True)
        loose = (n == "dmix_w" and out_dt == "bf16") or (mfma and n in ("dq", "dk", "dv"))
        assert e <= (TOL["bf16"] if loose else TOL["f32"]), f"{name} {n}: {e:.3e}"


# ---------------------------------------------------------------------------
# softmax-branch gradients alone: the memory's mix weight is 0, so dq, dk, dv
# come from the SWA/DSWA backward kernels only and nothing else can hide an
# error in them
# ---------------------------------------------------------------------------

def _softmax_only_weights(Hh):
    """Per head: SWA alone, DSWA alone, then both (memory weight 0 everywhere)."""
    pattern = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 0.0], [0.7, 0.4, 0.0]], np.float32)
    return pattern[np.arange(Hh) % 3]


def _softmax_oracle_grads(wl, x, g, scale=None):
    """dq, dk, dv of w0 * SWA + w1 * DSWA per (row, head), float64."""
    out = {n: np.zeros(x["q"].shape) for n in ("dq", "dk", "dv")}
    for b in range(wl.B):
        for h in range(wl.H):
            q, k, v = x["q"][b, :, h], x["k"][b, :, h], x["v"][b, :, h]
            gh = g[b, :, h].astype(np.float64)
            for i, fo in ((0, lambda f: O.swa_frames(f, wl.swa_frames)),
                          (1, lambda f: O.dswa_frames(f, wl.dswa_dilation, wl.dswa_taps))):
                wi = float(x["w"][h, i])
                if wi == 0.0:
                    continue
                gq, gk, gv = O.attention_backward(q, k, v, wi * gh, wl.T, wl.P, fo, scale)
                out["dq"][b, :, h] += gq
                out["dk"][b, :, h] += gk
                out["dv"][b, :, h] += gv
    return out


SOFTMAX_ONLY_CASES = [
    # name, workload, out dtype, impl. P >= 64 and not a multiple of 64 (ragged
    # row and key tiles); T below dil * taps, so early frames have partial DSWA
    # tap sets and frame 0 none; three heads: SWA only, DSWA only, both.
    ("mfma_P72", small("smx_mfma", B=1, H=3, T=6, P=72, d=128, swa_frames=3, dswa_dilation=2, dswa_taps=3,
                       gdn_chunk=64, dtype="bf16", seed=2110), "bf16", AUTO),
    ("mfma_B2_P100", small("smx_mfma_b2", B=2, H=3, T=9, P=100, d=128, swa_frames=3, dswa_dilation=2,
                           dswa_taps=3, gdn_chunk=64, dtype="bf16", seed=2111), "bf16", AUTO),
    ("generic_bf16_P72", small("smx_gen", B=1, H=3, T=6, P=72, d=128, swa_frames=3, dswa_dilation=2,
                               dswa_taps=3, gdn_chunk=64, dtype="bf16", seed=2112), "bf16", GEN),
    ("generic_f32_d64", small("smx_f32", B=2, H=3, T=7, P=40, d=64, swa_frames=2, dswa_dilation=2, dswa_taps=3,
                              gdn_chunk=32, seed=2113), "f32", AUTO),
]


@pytest.mark.parametrize("name,wl,out_dt,impl", SOFTMAX_ONLY_CASES, ids=[c[0] for c in SOFTMAX_ONLY_CASES])
def test_bwd_softmax_branches_alone(name, wl, out_dt, impl):
    """With the memory's mix weight 0 and peaked queries (q x 8, so the
    softmax Jacobian term dS carries weight), dq, dk and dv each come only from
    the softmax-branch backward and are compared with the float64 gradient of
    exact attention; the memory's own gradients (da, db, dS0) are exactly 0."""
    print(f"case {name}: B={wl.B} H={wl.H} T={wl.T} P={wl.P} d={wl.d} {wl.dtype}->{out_dt} impl={impl}",
          flush=True)
    x = I.make_clip(wl, q_scale=8.0)
    x["w"] = _softmax_only_weights(wl.H)
    cfg = H.make_config(wl, out_dtype=out_dt, impl=impl)
    dev = H.to_device(x, wl.dtype)
    S0_t = torch.from_numpy(_start_state(wl)).cuda()
    fwd = H.hlta_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], S0=S0_t)
    g = I.upstream_grad(wl, out_dt)
    g_t = torch.from_numpy(g).cuda().to(torch.bfloat16 if out_dt == "bf16" else torch.float32)
    got = H.hlta_bwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], fwd, g_t, S0=S0_t)
    torch.cuda.synchronize()
    ref = _softmax_oracle_grads(wl, x, g)
    mfma = _mfma(wl, out_dt, impl)
    tol = TOL["bf16"] if mfma else TOL["f32"]
    for n in ("dq", "dk", "dv"):
        gv_ = to64(got[n])
        for h in range(wl.H):
            e = O.rel_l2(gv_[:, :, h], ref[n][:, :, h])
            print(f"{name} {n} head {h} (w = {x['w'][h].tolist()}) {e:.2e}", flush=True)
            assert e <= tol, f"{name} {n} head {h}: rel-L2 {e:.3e} > {tol:.0e}"
    for n in ("da", "db", "dS0"):
        assert torch.count_nonzero(got[n]).item() == 0, n


@pytest.mark.slow
def test_full_size_backward_softmax_branches_alone():
    """hlta_bwd at 480P / 31 frames (all 24 heads) with the memory's mix weight
    0 and SWA, DSWA weighted (1, 1): dq, dk, dv of one whole head against the
    float64 gradient of exact attention over both branches."""
    wl = I.P480_T31
    print(f"generating {wl.name}, memory weight 0", flush=True)
    x = I.make_clip(wl, q_scale=8.0, threads=16)
    x["w"] = np.tile(np.array([[1.0, 1.0, 0.0]], np.float32), (wl.H, 1))
    g = I.upstream_grad(wl, "bf16")
    dev = H.to_device(x, wl.dtype)
    cfg = H.make_config(wl)
    fwd = H.hlta_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"])
    g_t = torch.from_numpy(g).cuda().to(torch.bfloat16)
    got = H.hlta_bwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], fwd, g_t)
    torch.cuda.synchronize()
    print("GPU backward done; oracle on one head", flush=True)
    b, h = 0, 11
    q, k, v = x["q"][b, :, h], x["k"][b, :, h], x["v"][b, :, h]
    gh = g[b, :, h].astype(np.float64)
    ref = {n: np.zeros(q.shape) for n in ("dq", "dk", "dv")}
    for fo in (lambda f: O.swa_frames(f, wl.swa_frames), lambda f: O.dswa_frames(f, wl.dswa_dilation, wl.dswa_taps)):
        for n, r in zip(("dq", "dk", "dv"), O.attention_backward(q, k, v, gh, wl.T, wl.P, fo)):
            ref[n] += r
    for n in ("dq", "dk", "dv"):
        err = O.rel_l2(to64(got[n][b, :, h]), ref[n])
        print(f"{wl.name} softmax-only backward (b={b}, h={h}) {n} {err:.2e}", flush=True)
        assert err <= TOL["bf16"], f"{n}: {err:.3e}"
