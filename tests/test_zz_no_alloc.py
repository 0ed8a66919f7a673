"""hlta_fwd_noalloc (through the C ABI) against hlta_fwd with a caller
workspace: two calls in a row on the library's fixed scratch, the second on a
smaller clip (the scratch still holds the first call's contents), each equal
to hlta_fwd bit for bit; a call needing more scratch than the array holds is
refused before anything runs."""
import numpy as np
import pytest
import torch

from hybrid_linear_temporal_amd import hlta as H
from hybrid_linear_temporal_amd import inputs as I
from oracle import hlta_oracle as O
from tests.helpers import BRANCHES, TOL, small, to64

pytestmark = pytest.mark.gpu

FIRST_SECOND = [
    # bf16, d = 128, chunk 64: the MFMA kernels; the second clip is smaller in every dimension
    (small("noalloc_bf16_big", B=2, H=3, T=18, P=70, d=128, swa_frames=3, dswa_dilation=4, dswa_taps=4,
           gdn_chunk=64, dtype="bf16", seed=2200),
     small("noalloc_bf16_small", B=1, H=2, T=7, P=66, d=128, swa_frames=3, dswa_dilation=2, dswa_taps=3,
           gdn_chunk=64, dtype="bf16", seed=2201)),
    # float32: the generic kernels
    (small("noalloc_f32_big", B=2, H=2, T=10, P=50, d=64, swa_frames=3, dswa_dilation=3, dswa_taps=2,
           gdn_chunk=32, seed=2202),
     small("noalloc_f32_small", B=1, H=2, T=6, P=20, d=32, swa_frames=2, dswa_dilation=2, dswa_taps=2,
           gdn_chunk=16, seed=2203)),
]


def _both(wl, x, S0):
    cfg = H.make_config(wl)
    dev = H.to_device(x, wl.dtype)
    S0_t = torch.from_numpy(S0).cuda()
    ref = H.hlta_fwd(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], S0=S0_t,
                     S_out=torch.empty_like(S0_t))
    out = {n: torch.full_like(t, float("nan")) for n, t in ref.items() if n in BRANCHES}
    S_out = torch.full_like(S0_t, float("nan"))
    got = H.hlta_fwd_noalloc(cfg, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["w"], out, S0=S0_t,
                             S_out=S_out)
    torch.cuda.synchronize()
    return got, ref


@pytest.mark.parametrize("big,smaller", FIRST_SECOND, ids=["bf16_mfma", "f32_generic"])
def test_noalloc_equals_fwd_on_two_calls(big, smaller):
    for i, wl in enumerate((big, smaller)):
        print(f"call {i}: {wl.name} B={wl.B} H={wl.H} T={wl.T} P={wl.P} d={wl.d} {wl.dtype}", flush=True)
        assert H.hlta_fwd_workspace_bytes(H.make_config(wl)) <= H.NOALLOC_SCRATCH_BYTES
        x = I.make_clip(wl)
        S0 = (0.1 * np.random.default_rng(wl.seed).standard_normal((wl.B, wl.H, wl.d, wl.d))).astype(np.float32)
        got, ref = _both(wl, x, S0)
        for n in BRANCHES + ("S_out",):
            assert torch.equal(got[n], ref[n]), (wl.name, n)
        oracle = O.hlta_forward(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], wl.T, wl.P, wl.swa_frames,
                                wl.dswa_dilation, wl.dswa_taps, wl.gdn_chunk, S0=S0)
        for j, n in enumerate(BRANCHES + ("S_out",)):
            e = O.rel_l2(to64(got[n]), oracle[j])
            print(f"{wl.name} {n} vs oracle {e:.2e}", flush=True)
            assert e <= TOL[wl.dtype], (wl.name, n, e)


def test_noalloc_refuses_more_scratch_than_it_holds():
    """480P / 61 frames with the rotary embedding needs far more scratch than
    the fixed array: HLTA_E_WORKSPACE, checked on the host, nothing launched."""
    wl = I.P480_T61
    cfg = H.make_config(wl, rope_theta=10000.0, rope_grid=(30, 52))
    need = H.hlta_fwd_workspace_bytes(cfg)
    assert need > H.NOALLOC_SCRATCH_BYTES
    t = torch.empty((16,), dtype=torch.bfloat16, device="cuda")
    out = {n: t for n in BRANCHES}
    with pytest.raises(H.HLTAError) as err:
        H.hlta_fwd_noalloc(cfg, t, t, t, t, t, t, out)
    assert err.value.status == 5 and str(need) in str(err.value)
