"""The measured-ceiling microbenchmarks (hlta_ceiling_mfma_bf16,
hlta_ceiling_copy) do the work their flop and byte counts claim: the copy is
exact over sizes with ragged tails, and the MFMA loop's products sum to
4 chains x 2 iters x (sum over i, j, k of A[i][k] B[k][j]) for its register
operands, for two iteration counts, so every counted MFMA ran."""
import numpy as np
import pytest
import torch

from hybrid_linear_temporal_amd import hlta as H

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16", [1, 3, 1000, 262147])
def test_copy_is_exact(n16):
    g = torch.Generator(device="cuda")
    g.manual_seed(n16)
    src = torch.randint(-2**31, 2**31 - 1, (4 * n16,), dtype=torch.int32, device="cuda", generator=g)
    dst = torch.zeros(4 * n16 + 4, dtype=torch.int32, device="cuda")
    H.hlta_ceiling_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst[:4 * n16], src)
    assert int(dst[4 * n16:].abs().sum()) == 0   # nothing past the end


def _operand_total():
    """sum_{i,j,k} A[i][k] B[k][j] for the loop's operands: lane l holds row
    (A) / column (B) l % 32 and reduction indices 8 (l // 32) .. +7 of both."""
    total = 0.0
    for half in range(2):
        for e in range(8):
            sa = sum(0.0078125 * ((l + e) & 15) for l in range(64) if l // 32 == half)
            sb = sum(0.0078125 * ((l * 3 + e) & 15) - 0.0625 for l in range(64) if l // 32 == half)
            total += sa * sb
    return total


@pytest.mark.parametrize("iters", [1, 3])
def test_mfma_loop_sums(iters):
    wgs = 4
    sink = torch.full((wgs * 256,), float("nan"), dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    H.hlta_ceiling_mfma_bf16(sink, clocks, wgs, iters)
    torch.cuda.synchronize()
    per_wave = sink.double().cpu().numpy().reshape(wgs * 4, 64).sum(axis=1)
    want = 4 * 2 * iters * _operand_total()
    np.testing.assert_allclose(per_wave, want, rtol=0, atol=1e-9)
    c = clocks.cpu().tolist()
    assert c[0] > 0 and c[1] > 0
    print(f"iters {iters}: core ticks {c[0]}, reference ticks {c[1]}")


def test_ceiling_arguments_refused():
    sink = torch.empty(256, dtype=torch.float32, device="cuda")
    with pytest.raises(H.HLTAError, match="HLTA_E_SHAPE"):
        H.hlta_ceiling_mfma_bf16(sink, None, 0, 1)
    with pytest.raises(H.HLTAError, match="HLTA_E_NULL"):
        H.hlta_ceiling_mfma_bf16(None, None, 1, 1)
    src = torch.empty(6, dtype=torch.int32, device="cuda")
    with pytest.raises(H.HLTAError, match="HLTA_E_SHAPE"):
        H.hlta_ceiling_copy(src, torch.empty_like(src))
