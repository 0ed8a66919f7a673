"""GPU streaming parity: hlta_step_frame against the float64 streaming oracle,
and against hlta_fwd over the whole clip."""
import numpy as np
import pytest
import torch

from hybrid_linear_temporal_amd import hlta as H
from hybrid_linear_temporal_amd import inputs as I
from oracle import hlta_oracle as O
from tests.helpers import BRANCHES, TOL, small, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    H.load_library()


def _frames(x, f0, f1, P):
    return {n: (arr[:, f0 * P:f1 * P] if n != "w" else arr) for n, arr in x.items()}


STREAM_CASES = [
    (small("stream_bf16", B=2, H=2, T=22, P=70, d=128, swa_frames=3, dswa_dilation=4, dswa_taps=4,
           gdn_chunk=64, dtype="bf16", seed=3000), 16, 16),
    (small("stream_f32", B=2, H=2, T=14, P=20, d=32, swa_frames=2, dswa_dilation=2, dswa_taps=2,
           gdn_chunk=16, dtype="f32", seed=3001), 3, 5),
]


@pytest.mark.parametrize("wl,prefix,R", STREAM_CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_stream_steps_match_oracle_and_full_forward(wl, prefix, R):
    """Prefix through hlta_fwd, then one hlta_step_frame per remaining frame
    (with an uncommitted evaluation before each committed one)."""
    x = I.make_clip(wl)
    P = wl.P
    tol = TOL[wl.dtype]
    dev = H.to_device(x, wl.dtype)
    cfg_full = H.make_config(wl)
    full = H.hlta_fwd(cfg_full, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"])
    # prefix
    cfg_pre = H.make_config(wl, T=prefix)
    pre = {n: t[:, :prefix * P].contiguous() if n != "w" else t for n, t in dev.items()}
    S_pre = torch.empty((wl.B, wl.H, wl.d, wl.d), dtype=torch.float32, device="cuda")
    H.hlta_fwd(cfg_pre, pre["q"], pre["k"], pre["v"], pre["a"], pre["b"], pre["w"], S_out=S_pre)
    st = H.Stream(H.make_config(wl, T=1), R)
    H.hlta_stream_load_prefix(st, pre["k"], pre["v"], prefix, S_pre)
    # oracle streams, one per (b, h)
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    ost = {}
    for b, h in heads:
        _, Sp = O.gdn_recurrent(x["q"][b, :prefix * P, h], x["k"][b, :prefix * P, h], x["v"][b, :prefix * P, h],
                                x["a"][b, :prefix * P, h], x["b"][b, :prefix * P, h])
        s = O.StreamHead(P, wl.swa_frames, wl.dswa_dilation, wl.dswa_taps, wl.gdn_chunk)
        s.load_prefix(x["k"][b, :, h], x["v"][b, :, h], prefix, Sp)
        ost[b, h] = s
    for f in range(prefix, wl.T):
        fr = {n: t[:, f * P:(f + 1) * P].contiguous() if n != "w" else t for n, t in dev.items()}
        # an uncommitted evaluation with different inputs must leave the stream unchanged
        H.hlta_step_frame(st, fr["q"] * 2, fr["k"], fr["v"] * 3, fr["a"], fr["b"], fr["w"], commit=False)
        assert st.frames_done == f
        got = H.hlta_step_frame(st, fr["q"], fr["k"], fr["v"], fr["a"], fr["b"], fr["w"])
        torch.cuda.synchronize()
        assert st.frames_done == f + 1
        refs = {n: np.zeros((wl.B, P, wl.H, wl.d)) for n in BRANCHES}
        for b, h in heads:
            sl = slice(f * P, (f + 1) * P)
            outs = ost[b, h].step(x["q"][b, sl, h], x["k"][b, sl, h], x["v"][b, sl, h], x["a"][b, sl, h],
                                  x["b"][b, sl, h], x["w"][h])
            for n, o in zip(BRANCHES, outs):
                refs[n][b, :, h] = o
        for n in BRANCHES:
            e = O.rel_l2(to64(got[n]), refs[n])
            e_full = O.rel_l2(to64(got[n]), to64(full[n][:, f * P:(f + 1) * P]))
            assert e <= tol, f"frame {f} {n}: {e:.2e}"
            assert e_full <= tol, f"frame {f} {n} vs full: {e_full:.2e}"
    Sref = np.stack([np.stack([ost[b, h].S0 for h in range(wl.H)]) for b in range(wl.B)])
    assert O.rel_l2(to64(st.S), Sref) <= tol


def test_stream_resume_is_bitwise():
    """Saving (S, rings, frames_done) and restoring it reproduces the run."""
    wl, prefix, R = STREAM_CASES[0]
    x = I.make_clip(wl)
    P = wl.P
    dev = H.to_device(x, wl.dtype)
    cfg = H.make_config(wl, T=1)
    st = H.Stream(cfg, R)
    pre = {n: t[:, :prefix * P].contiguous() if n != "w" else t for n, t in dev.items()}
    H.hlta_stream_load_prefix(st, pre["k"], pre["v"], prefix, None)

    def step(s, f):
        fr = {n: t[:, f * P:(f + 1) * P].contiguous() if n != "w" else t for n, t in dev.items()}
        return H.hlta_step_frame(s, fr["q"], fr["k"], fr["v"], fr["a"], fr["b"], fr["w"])

    step(st, prefix)
    snap = (st.S.clone(), st.ring_k.clone(), st.ring_v.clone(), st.frames_done)
    a1 = step(st, prefix + 1)
    a2 = step(st, prefix + 2)
    st2 = H.Stream(cfg, R)
    st2.S.copy_(snap[0])
    st2.ring_k.copy_(snap[1])
    st2.ring_v.copy_(snap[2])
    st2.state.frames_done = snap[3]
    b1 = step(st2, prefix + 1)
    b2 = step(st2, prefix + 2)
    torch.cuda.synchronize()
    for n in BRANCHES:
        assert torch.equal(a1[n], b1[n]) and torch.equal(a2[n], b2[n]), n
    assert torch.equal(st.S, st2.S)
