"""fp8b_mfma_loop, the MFMA-only measurement loop the benchmark sets the
GEMMs' rates beside: it must run the products it is given.

Whatever the lane layout, an MFMA takes lane l's A elements and B elements
over the same K slots (slot set fixed by the lane's 16-lane group), so the
sum of one product's outputs over a wave equals, per group, the sum over
the lane's elements e of (sum over the group's lanes of A[e]) times (sum of
B[e]).  One round is checked against that sum in fp64, and two rounds
against twice one round.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def F():
    import fp8_block_scaled_02_amd as F
    assert torch.cuda.is_available()
    return F


def _ops(kind, seed):
    """64 x 64 operand words and the per-lane element values (fp64) of the
    chains' A and B operands."""
    g = torch.Generator().manual_seed(seed)
    if kind == 0:
        v = torch.randn(64, 128, generator=g).to(torch.bfloat16)           # 2 bf16 per word
        words = v.view(torch.int16).view(torch.int32)
        vals = v.double().numpy()                                           # [64, 128]
        a = [vals[:, 16 * c:16 * c + 8] for c in range(2)]
        b = [vals[:, 16 * c + 8:16 * c + 16] for c in range(2)]
    else:
        v = (torch.randn(64, 256, generator=g) * 4).to(torch.float8_e4m3fn)  # 4 E4M3 per word
        words = v.view(torch.uint8).view(torch.int32)
        vals = v.double().numpy()                                           # [64, 256]
        a = [vals[:, 64 * c:64 * c + 32] for c in range(2)]
        b = [vals[:, 64 * c + 32:64 * c + 64] for c in range(2)]
    return words.contiguous().to(DEV), a, b


def _wave_sum_ref(a, b):
    """Sum over a wave of one round's outputs, and the sum of |terms|."""
    s = t = 0.0
    for ac, bc in zip(a, b):
        for grp in range(4):
            sa = ac[16 * grp:16 * grp + 16].sum(axis=0)
            sb = bc[16 * grp:16 * grp + 16].sum(axis=0)
            s += float((sa * sb).sum())
            t += float((np.abs(ac[16 * grp:16 * grp + 16]).sum(axis=0) *
                        np.abs(bc[16 * grp:16 * grp + 16]).sum(axis=0)).sum())
    return s, t


@pytest.mark.parametrize("kind", [0, 1])
def test_mfma_loop_runs_the_given_products(F, kind):
    words, a, b = _ops(kind, seed=11 + kind)
    wg = 3
    out1 = F.fp8b_mfma_loop(kind, words, 1, wg).cpu().numpy().astype(np.float64)
    out2 = F.fp8b_mfma_loop(kind, words, 2, wg).cpu().numpy().astype(np.float64)
    ref, mag = _wave_sum_ref(a, b)
    # every wave of every workgroup computes the same thing
    waves = out1.reshape(wg * 4, 64)
    assert np.all(waves == waves[0])
    # bf16 products are exact and summed in fp32; the FP8 instruction
    # aligns each group of 8 products to 13 fraction bits (measured on
    # Gaussian codes: at most 1.7e-5 of the sum of |products|)
    rel = 1e-5 if kind == 0 else 1e-4
    assert abs(waves[0].sum() - ref) <= rel * mag, (waves[0].sum(), ref, mag)
    # two rounds give twice one round; a lane's own |terms| are bounded by
    # four times the wave average, far below |out1| for these operands
    lane_mag = mag / 16
    assert np.all(np.abs(out2 - 2 * out1) <= rel * lane_mag)
    assert np.median(np.abs(out1)) > 10 * rel * lane_mag

