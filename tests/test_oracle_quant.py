"""Pins for the oracle's scale rules, act_quant and weight quant (CPU only).

Independent routes used here: numpy's IEEE float32 division, exact rational
arithmetic (fractions.Fraction), torch's CPU float8 casts, a hand-worked
block (tests/golden/act_quant_block.txt) and invariants that follow from the
format (the block maximum lands on +-448; the dequantisation error bound of
a 3-bit mantissa).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))


def _all_pos_bf16():
    b = np.arange(1, 0x7F80, dtype=np.uint32)          # +subnormals .. max finite
    return (b << 16).astype(np.uint32).view(np.float32)


def test_scale_fp32_exhaustive_vs_numpy(orc):
    a = _all_pos_bf16()
    want = (a / np.float32(448.0)).astype(np.float32)
    got = np.array([orc.scale_fp32(float(v)) for v in a], np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    assert orc.scale_fp32(0.0) == 1.0


def test_scale_pow2_exhaustive_exact(orc):
    """e = smallest integer with amax <= 448 * 2^e (exact rational check)."""
    L = orc.lib()
    for v in _all_pos_bf16():
        v = float(v)
        m, E = math.frexp(v)            # v = m * 2^E, m in [0.5, 1)
        sig, E = m * 2.0, E - 1         # v = sig * 2^E, sig in [1, 2)
        cand = E - 8 + (1 if sig > 1.75 else 0)
        fv = Fraction(v)
        assert fv <= 448 * Fraction(2) ** cand
        assert fv > 448 * Fraction(2) ** (cand - 1)
        want = max(-127, min(127, cand))
        assert L.orc_scale_pow2_exp(v) == want, v
    assert orc.scale_pow2_exp(0.0) == 0


def _brute_act_quant(x_bits, block, fmt):
    """Per-block definition with numpy fp32 division and torch's E4M3 cast."""
    x = (x_bits.astype(np.uint32) << 16).view(np.float32)
    M, K = x.shape
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // block), np.uint8 if fmt == 2 else np.float32)
    for m in range(M):
        for j in range(K // block):
            blk = x[m, j * block:(j + 1) * block]
            amax = np.float32(np.max(np.abs(blk)))
            if fmt == 0:
                d = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(448.0))
            else:
                if amax == 0:
                    e = 0
                else:
                    e = -127
                    while e < 127 and Fraction(float(amax)) > 448 * Fraction(2) ** e:
                        e += 1
                d = np.float32(2.0 ** e)
            t = np.clip((blk / d).astype(np.float32), -448, 448)
            q[m, j * block:(j + 1) * block] = (
                torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
            s[m, j] = (127 + e) if fmt == 2 else d
    return q, s


@pytest.mark.parametrize("block,fmt", [(128, 0), (128, 1), (32, 2), (32, 0)])
def test_act_quant_vs_brute(orc, block, fmt):
    import workloads as W
    c = W.tiny_linear()
    xb = W.bits(c.x)
    q, s = orc.act_quant(xb, block, fmt)
    q2, s2 = _brute_act_quant(xb, block, fmt)
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(s.view(np.uint8), s2.view(np.uint8))


def test_act_quant_mx_operand_vs_brute(orc):
    import workloads as W
    a, _ = W.mx_case(M=8, N=8, K=256)
    xb = W.bits(a)
    for fmt in (2, 1):
        q, s = orc.act_quant(xb, 32, fmt)
        q2, s2 = _brute_act_quant(xb, 32, fmt)
        np.testing.assert_array_equal(q, q2)
        np.testing.assert_array_equal(s.view(np.uint8), s2.view(np.uint8))


def test_act_quant_hand_worked_block(orc):
    xs, codes = [], []
    with open(os.path.join(HERE, "golden", "act_quant_block.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                a, _, c = line.split()[:3]
                xs.append(float(a))
                codes.append(int(c, 16))
    assert len(xs) == 32
    x = torch.tensor(xs, dtype=torch.float32).to(torch.bfloat16)
    assert x.float().tolist() == xs                    # all exactly bf16
    xb = x.view(torch.int16).numpy().view(np.uint16).reshape(1, 32)
    for fmt, scale in ((0, 2.0), (1, 2.0), (2, 128)):
        q, s = orc.act_quant(xb, 32, fmt)
        assert q.reshape(-1).tolist() == codes, fmt
        assert s.reshape(-1)[0] == scale


def test_act_quant_zero_block_and_sign(orc):
    x = np.zeros((2, 128), np.float32)
    x[1, :] = -0.0
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    for fmt in (0, 1):
        q, s = orc.act_quant(xb, 128, fmt)
        assert (q[0] == 0x00).all() and (q[1] == 0x80).all()
        assert (s == 1.0).all()
    q, s = orc.act_quant(xb, 128, 2)
    assert (s == 127).all()


def test_act_quant_invariants(orc):
    import workloads as W
    c = W.prefill_linear(M=64, K=1024, N=128)
    xb = W.bits(c.x)
    x = c.x.float().numpy()
    t4 = orc.e4m3_table()
    for fmt in (0, 1):
        q, s = orc.act_quant(xb, 128, fmt)
        d = np.repeat(s, 128, axis=1).astype(np.float64)
        val = t4[q]
        blocks = np.abs(val).reshape(64, 8, 128).max(axis=2)
        if fmt == 0:
            # the block maximum always lands on +-448
            assert (blocks == 448).all()
        else:
            assert ((blocks >= 224) & (blocks <= 448)).all()
            assert (np.log2(s) == np.round(np.log2(s))).all()
        # dequantisation error x - d*val (page 5: x_hat = s * x_fp8)
        err = np.abs(x - val * d)
        rel = np.abs(x) / d
        normal = rel >= 2.0 ** -6
        assert (err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 2.0 ** -20)).all()
        assert (err[~normal] <= 2.0 ** -10 * d[~normal] * (1 + 2.0 ** -20)).all()


def _brute_weight_quant(w_bits, fmt):
    w = (w_bits.astype(np.uint32) << 16).view(np.float32)
    N, K = w.shape
    q = np.empty((N, K), np.uint8)
    s = np.empty((N // 128, K // 128), np.float32)
    for i in range(N // 128):
        for j in range(K // 128):
            t = w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            amax = np.float32(np.abs(t).max())
            if fmt == 0:
                d = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(448.0))
            else:
                e = 0
                if amax != 0:
                    e = -127
                    while e < 127 and Fraction(float(amax)) > 448 * Fraction(2) ** e:
                        e += 1
                d = np.float32(2.0 ** e)
            c = np.clip((t / d).astype(np.float32), -448, 448)
            q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128] = (
                torch.from_numpy(c).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
            s[i, j] = d
    return q, s


@pytest.mark.parametrize("fmt", [0, 1])
def test_weight_quant_vs_brute(orc, fmt):
    import workloads as W
    g = W.gen(7)
    w = W.weights(256, 384, 0.02, g)
    w[5, 7] = 1.5          # one tile with a large outlier
    wb = W.bits(w)
    q, s = orc.weight_quant(wb, fmt)
    q2, s2 = _brute_weight_quant(wb, fmt)
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(s, s2)
    assert s[0, 0] != s[0, 1]


def test_quant_rejects_bad_shapes(orc):
    xb = np.zeros((2, 100), np.uint16)
    with pytest.raises(ValueError):
        orc.act_quant(xb, 128, 0)
    with pytest.raises(ValueError):
        orc.weight_quant(np.zeros((100, 128), np.uint16), 0)
