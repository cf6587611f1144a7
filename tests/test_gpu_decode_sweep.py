"""Every token count from 1 to 130 through the block GEMM on both weight
layouts, against the CPU oracle, element by element.

The launcher picks a kernel from the token count, the weight layout, the
number of K blocks and the number of 128-row weight tiles against the CU
count: up to 64 tokens the register-streamed kernel (packed weights, even K
block count, at most one tile per CU) or the streaming kernel (one to four
16-token subtiles), 33-64 tokens on 64 x 128 tiles (row-major weights),
65-128 tokens on 128 x 128 tiles with or without the K split, and above 128
the prefill tiles.  Two shapes cover both sides of the K-block parity: K 1024
(eight blocks) and K 640 (five).  Token rows are independent, so the oracle
computes the 130-row case once and each launch is checked on its first M
rows.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity import assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def F():
    import fp8_block_scaled_02_amd as F
    assert torch.cuda.is_available()
    return F


@pytest.mark.parametrize("N,K,fmt", [(512, 1024, "ue8m0"), (384, 640, "fp32")])
def test_block_gemm_every_token_count(F, orc, N, K, fmt):
    Mmax = 130
    c = W.prefill_linear(M=Mmax, K=K, N=N, seed=N + K)   # 0.5% outlier channels x50, as at decode
    x = c.x
    fi = {"fp32": 0, "ue8m0": 1}[fmt]
    a, sa = F.fp8_act_quant(x.to(DEV), 128, fmt)
    wq, ws = F.fp8_weight_quant(c.w.to(DEV), fmt)
    wp = F.fp8_weight_pack(wq)
    oa, osa = orc.act_quant(W.bits(x), 128, fi)
    ow, osw = orc.weight_quant(W.bits(c.w), fi)
    yr, bnd = orc.block_gemm(oa, osa, ow, osw)
    for M in range(1, Mmax + 1):
        for name, fn, w in (("row-major", F.fp8_block_gemm, wq), ("packed", F.fp8_block_gemm_packed, wp)):
            y = fn(a[:M], sa[:M], w, ws, torch.bfloat16)
            torch.cuda.synchronize()
            yg = y.float().cpu().numpy().astype(np.float64)
            assert yg.shape == (M, N)
            assert_parity(yg, yr[:M], bnd[:M], True, f"M={M} {name} {N}x{K} {fmt}")


def test_mx_gemm_every_row_count(F, orc):
    """mxfp8_gemm for every M from 1 to 260 (one to three 128-row m-tiles,
    every ragged last tile) on the 128 x 128 tiles, N 256, K 384 (three K
    steps), each launch on the first M rows of one quantised operand,
    against the oracle element by element."""
    Mmax, N, K = 260, 256, 384
    a_bf, b_bf = W.mx_case(M=Mmax, N=N, K=K, seed=7)
    qa, ea = F.fp8_act_quant(a_bf.to(DEV), 32, "e8m0")
    qb, eb = F.fp8_act_quant(b_bf.to(DEV), 32, "e8m0")
    oa, oea = orc.act_quant(W.bits(a_bf), 32, 2)
    ob, oeb = orc.act_quant(W.bits(b_bf), 32, 2)
    yr, bnd = orc.mx_gemm(oa, oea, ob, oeb)
    for M in range(1, Mmax + 1):
        y = F.mxfp8_gemm(qa[:M], ea[:M], qb, eb)
        torch.cuda.synchronize()
        yg = y.cpu().numpy().astype(np.float64)
        assert yg.shape == (M, N)
        assert_parity(yg, yr[:M], bnd[:M], False, f"mx M={M}")
