"""Pins for the oracle's GEMM references (CPU only).

Routes independent of the oracle's C loops: exact rational arithmetic on the
integer block sums (numpy int64 matmul + fractions), an fp64 BLAS route that
is exact for the per-block integer sums (every partial sum stays below
2^53), and special cases that reduce to a plain integer matmul.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch


def _ival(orc, codes):
    """512 * value of each E4M3 code, from torch's decoder (a library routine)."""
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    tab = (t.to(torch.float64) * 512).numpy()
    tab[np.isnan(tab)] = 0
    assert (tab == np.round(tab)).all()
    return tab.astype(np.int64)[codes]


def _quantized_linear(orc, case):
    import workloads as W
    fmt = 0 if case.scale_fmt == "fp32" else 1
    a, sa = orc.act_quant(W.bits(case.x), 128, fmt)
    w, sw = orc.weight_quant(W.bits(case.w), fmt)
    return a, sa, w, sw


def test_block_gemm_exact_rational_tiny(orc):
    """All of the 16x512 -> 256 case against exact rationals."""
    import workloads as W
    a, sa, w, sw = _quantized_linear(orc, W.tiny_linear())
    y, bnd = orc.block_gemm(a, sa, w, sw)
    A, B = _ival(orc, a), _ival(orc, w)
    M, K = a.shape
    N = w.shape[0]
    nkb = K // 128
    P = [A[:, kb * 128:(kb + 1) * 128] @ B[:, kb * 128:(kb + 1) * 128].T for kb in range(nkb)]
    Pa = [np.abs(A[:, kb * 128:(kb + 1) * 128]) @ np.abs(B[:, kb * 128:(kb + 1) * 128]).T
          for kb in range(nkb)]
    assert len(set(sw.reshape(-1).tolist())) > 1 and len(set(sa.reshape(-1).tolist())) > 1
    for m in range(M):
        for n in range(N):
            ex = sum(Fraction(float(sa[m, kb])) * Fraction(float(sw[n // 128, kb]))
                     * int(P[kb][m, n]) for kb in range(nkb)) / 2 ** 18
            exb = sum(abs(Fraction(float(sa[m, kb])) * Fraction(float(sw[n // 128, kb])))
                      * int(Pa[kb][m, n]) for kb in range(nkb)) / 2 ** 18
            assert abs(Fraction(y[m, n]) - ex) <= Fraction(exb) * Fraction(1, 2 ** 50), (m, n)
            assert abs(Fraction(bnd[m, n]) - exb) <= exb * Fraction(1, 2 ** 50)


def test_block_gemm_fp64_blas_route(orc):
    import workloads as W
    c = W.prefill_linear(M=40, K=1024, N=384)
    a, sa, w, sw = _quantized_linear(orc, c)
    y, bnd = orc.block_gemm(a, sa, w, sw)
    A = _ival(orc, a).astype(np.float64)
    B = _ival(orc, w).astype(np.float64)
    ref = np.zeros_like(y)
    for kb in range(8):
        P = A[:, kb * 128:(kb + 1) * 128] @ B[:, kb * 128:(kb + 1) * 128].T   # exact
        s = sa[:, kb].astype(np.float64)[:, None] * np.repeat(
            sw[:, kb].astype(np.float64), 128)[None, :]
        ref += s * P * 2.0 ** -18
    assert np.all(np.abs(y - ref) <= 1e-13 * bnd)


def test_block_gemm_single_kblock_is_one_product(orc):
    rng = np.random.default_rng(1)
    a = rng.integers(0, 0x7E, size=(8, 128), dtype=np.uint8)
    w = rng.integers(0x80, 0xFE, size=(128, 128), dtype=np.uint8)
    sa = rng.uniform(0.5, 2, size=(8, 1)).astype(np.float32)
    sw = rng.uniform(0.5, 2, size=(1, 1)).astype(np.float32)
    y, _ = orc.block_gemm(a, sa, w, sw)
    P = _ival(orc, a) @ _ival(orc, w).T
    ref = (sa.astype(np.float64) * sw.astype(np.float64)[0, 0]) * (P * 2.0 ** -18)
    np.testing.assert_array_equal(y, ref)
    assert (y < 0).all()          # negative codes in w, positive in a


def test_block_gemm_unit_scales_integer_matmul(orc):
    """Codes for the small integers -8..8 with unit scales: y is the integer matmul."""
    ints = list(range(-8, 9))
    code = {v: int(orc.e4m3_encode(np.array([v], np.float32))[0]) for v in ints}
    rng = np.random.default_rng(2)
    ia = rng.choice(ints, size=(16, 256))
    iw = rng.choice(ints, size=(256, 256))
    a = np.vectorize(code.get)(ia).astype(np.uint8)
    w = np.vectorize(code.get)(iw).astype(np.uint8)
    y, bnd = orc.block_gemm(a, np.ones((16, 2), np.float32), w, np.ones((2, 2), np.float32))
    np.testing.assert_array_equal(y, (ia @ iw.T).astype(np.float64))
    np.testing.assert_array_equal(bnd, (np.abs(ia) @ np.abs(iw).T).astype(np.float64))


def test_mx_gemm_unit_scales_is_plain_fp8_gemm(orc):
    import workloads as W
    a_b, b_b = W.mx_case(M=16, N=64, K=256)
    a, _ = orc.act_quant(W.bits(a_b), 32, 2)
    b, _ = orc.act_quant(W.bits(b_b), 32, 2)
    ones_a = np.full((16, 8), 127, np.uint8)
    ones_b = np.full((64, 8), 127, np.uint8)
    y, _ = orc.mx_gemm(a, ones_a, b, ones_b)
    P = _ival(orc, a) @ _ival(orc, b).T                 # exact int64
    np.testing.assert_array_equal(y, P.astype(np.float64) * 2.0 ** -18)


def test_mx_gemm_exact_rational(orc):
    import workloads as W
    a_b, b_b = W.mx_case(M=8, N=32, K=256)
    a, ea = orc.act_quant(W.bits(a_b), 32, 2)
    b, eb = orc.act_quant(W.bits(b_b), 32, 2)
    assert len(set(ea.reshape(-1).tolist())) > 4
    y, bnd = orc.mx_gemm(a, ea, b, eb)
    A, B = _ival(orc, a), _ival(orc, b)
    for m in range(8):
        for n in range(32):
            ex = Fraction(0)
            for kb in range(8):
                p = int(A[m, kb * 32:(kb + 1) * 32] @ B[n, kb * 32:(kb + 1) * 32])
                ex += Fraction(p) * Fraction(2) ** (int(ea[m, kb]) + int(eb[n, kb]) - 254 - 18)
            assert abs(Fraction(y[m, n]) - ex) <= Fraction(bnd[m, n]) * Fraction(1, 2 ** 50)


def _small_moe(orc, T=24, E=5, topk=2, N=256, K=256, s=1.0):
    import workloads as W
    case = W.moe_case(T=T, E=E, topk=topk, N=N, K=K, s=s)
    a, sa = orc.act_quant(W.bits(case.x), 128, 0)
    ws = [orc.weight_quant(W.bits(case.w[e]), 0) for e in range(E)]
    return case, a, sa, ws


def test_grouped_rows_equal_block_gemm_of_gathered_rows(orc):
    case, a, sa, ws = _small_moe(orc)
    ri = case.row_index.numpy()
    offs = case.offs.numpy()
    y, bnd = orc.grouped_gemm(a, sa, ri, offs, [w for w, _ in ws], [s for _, s in ws])
    E = len(offs) - 1
    for e in range(E):
        lo, hi = offs[e], offs[e + 1]
        if hi == lo:
            continue
        rows = ri[lo:hi]
        yb, bb = orc.block_gemm(a[rows], sa[rows], ws[e][0], ws[e][1])
        np.testing.assert_array_equal(y[lo:hi], yb)
        np.testing.assert_array_equal(bnd[lo:hi], bb)


def test_grouped_single_expert_is_block_gemm(orc):
    case, a, sa, ws = _small_moe(orc, T=16, E=1, topk=1)
    ri = case.row_index.numpy()
    assert (ri == np.arange(16)).all()
    y, _ = orc.grouped_gemm(a, sa, ri, case.offs.numpy(), [ws[0][0]], [ws[0][1]])
    yb, _ = orc.block_gemm(a, sa, ws[0][0], ws[0][1])
    np.testing.assert_array_equal(y, yb)


def test_grouped_row_subset_and_missing_experts(orc):
    case, a, sa, ws = _small_moe(orc)
    ri = case.row_index.numpy()
    offs = case.offs.numpy()
    full, _ = orc.grouped_gemm(a, sa, ri, offs, [w for w, _ in ws], [s for _, s in ws])
    rows = np.array([0, 3, len(ri) - 1, 7])
    part, _ = orc.grouped_gemm(a, sa, ri, offs, [w for w, _ in ws], [s for _, s in ws], rows=rows)
    np.testing.assert_array_equal(part, full[rows])
    # an expert given as None leaves its rows untouched (NaN)
    wl = [w for w, _ in ws]
    sl = [s for _, s in ws]
    e0 = int(np.searchsorted(offs, 0, side="right") - 1)
    wl[e0] = None
    sl[e0] = None
    miss, _ = orc.grouped_gemm(a, sa, ri, offs, wl, sl)
    assert np.isnan(miss[offs[e0]:offs[e0 + 1]]).all()
    others = np.ones(len(ri), bool)
    others[offs[e0]:offs[e0 + 1]] = False
    np.testing.assert_array_equal(miss[others], full[others])


def test_routing_invariants():
    import workloads as W
    ri, offs, ex = W.routing(64, 16, 4, 1.0, W.gen(3))
    assert offs[0] == 0 and offs[-1] == 256 and (np.diff(offs.numpy()) >= 0).all()
    # each token appears exactly topk times, each time with a distinct expert
    tok = ri.numpy()
    exn = ex.numpy()
    for t in range(64):
        sel = exn[tok == t]
        assert len(sel) == 4 and len(set(sel.tolist())) == 4
    # rows are sorted by (expert, token)
    key = exn.astype(np.int64) * 64 + tok
    assert (np.diff(key) > 0).all()
