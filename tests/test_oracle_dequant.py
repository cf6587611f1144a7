"""Pins of the oracle's weight dequantisation (w = value(code) * block scale,
formed in fp32, stored as bf16).

Sources: the DeepSeek-V3 guide's dispatch snippet, whose bf16 branch calls
weight_dequant(weight, weight.scale) on the FP8 weights with 128x128 block
scales; "量化: FP8 与混合精度推理", section "FP8 也需要 scale": x_hat = s * x_fp8.

The checks use routes independent of the oracle's C code: torch's float8
decoder for code values, exact double products (at most 28 significant
bits), numpy's fp32 rounding and torch's bf16 rounding.
"""
import numpy as np
import pytest
import torch

import oracle as O


def _code_values():
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return codes, vals


def _library_route(vals, d):
    """fp32(value * d) via an exact double product, then bf16 RNE (torch)."""
    p64 = vals.astype(np.float64) * np.float64(np.float32(d))   # exact
    p32 = p64.astype(np.float32)                                 # one RNE rounding
    return torch.from_numpy(p32).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


def _scales():
    rng = np.random.default_rng(7)
    s = [1.0, 0.5, 2.0 ** -20, 2.0 ** 20, 1.0 / 448, 3.0e-3, 7.3e-5, 1.7e30, 3.0e35, 1.0e-38, 1.4e-45]
    s += list(rng.uniform(1e-6, 1e-1, 40)) + list(np.exp(rng.uniform(-80, 80, 40)))
    return np.array(s, np.float32)


def test_every_code_times_scales_matches_library_route():
    codes, vals = _code_values()
    finite = np.isfinite(vals)
    for d in _scales():
        want = _library_route(vals[finite], d)
        got = np.array([O.dequant_one(c, d) for c in codes[finite]], np.uint16)
        bad = np.flatnonzero(got != want)
        assert len(bad) == 0, f"d={d!r}: code {codes[finite][bad[0]]:#x} got {got[bad[0]]:#06x} want {want[bad[0]]:#06x}"


def test_nan_codes_and_signed_zero():
    nan = lambda b: (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0
    assert nan(O.dequant_one(0x7F, 1.0)) and nan(O.dequant_one(0xFF, 1.0))
    assert O.dequant_one(0x00, 3.0) == 0x0000
    assert O.dequant_one(0x80, 3.0) == 0x8000
    # 448 * 1e38 overflows fp32 already: +-Inf
    assert O.dequant_one(0x7E, 1e38) == 0x7F80 and O.dequant_one(0xFE, 1e38) == 0xFF80


def test_power_of_two_scales_are_exact():
    """ue8m0 scales: value * 2^e has at most 4 significant bits, so the bf16
    result is the exact product whenever it is a normal bf16."""
    codes, vals = _code_values()
    for e in (-120, -40, -7, 0, 5, 60, 110):
        d = np.float32(2.0 ** e)
        for c, v in zip(codes, vals):
            if not np.isfinite(v):
                continue
            exact = v * 2.0 ** e
            got = O.dequant_one(int(c), float(d))
            back = np.array([got << 16], np.uint32).view(np.float32)[0]
            if exact == 0 or 2.0 ** -126 <= abs(exact) < 2.0 ** 127:
                assert back == exact, (hex(c), e)


def test_double_rounding_reading():
    """A pair whose exact product lies just above a bf16 tie but whose fp32
    rounding lands on the tie: the reading (fp32 first) rounds the tie to
    even, a single direct rounding would not."""
    v = 1.125                                   # E4M3 code 0x39
    code = int(O.e4m3_encode(np.array([v], np.float32))[0])
    assert code == 0x39
    tie = 1.0 + 2.0 ** -8                       # halfway between bf16 1.0 and 1.0078125
    d0 = np.float32(tie / v)
    found = None
    for k in range(-64, 65):                    # fp32 neighbours of tie / v
        d = d0
        for _ in range(abs(k)):
            d = np.nextafter(d, np.float32(np.inf if k > 0 else -np.inf))
        exact = v * float(d)                    # exact in double
        if exact > tie and np.float32(exact) == np.float32(tie):
            found = d
            break
    assert found is not None
    got = O.dequant_one(code, float(found))
    assert got == 0x3F80   # 1.0: the fp32 product is the tie, which goes to the even mantissa
    # (rounding the exact product once, to bf16, would give 1.0078125 = 0x3F81)


def test_weight_dequant_matrix_layout_and_round_trip():
    """Block layout (scale of block (n/128, k/128)) and the round trip of the
    weight quantiser: |w - dequant(quant(w))| stays within half an E4M3 step
    of the block scale plus the bf16 rounding."""
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    w[5, 300] = 1.5
    wb = torch.from_numpy(w).to(torch.bfloat16)
    bits = wb.view(torch.int16).numpy().astype(np.uint16)
    q, s = O.weight_quant(bits, 0)
    deq = O.weight_dequant(q, s)
    _, vals = _code_values()
    for n in (0, 127, 128, 255):
        for k in (0, 127, 128, 383):
            want = _library_route(vals[q[n, k]:q[n, k] + 1], s[n // 128, k // 128])[0]
            assert deq[n, k] == want
    x = wb.to(torch.float64).numpy()
    y = torch.from_numpy(deq.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    dfull = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)
    step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(x) / dfull, 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(x - y) <= 0.5 * step * dfull * (1 + 2 ** -7) + np.abs(y) * 2.0 ** -8)


def test_weight_dequant_rejects_bad_shapes():
    with pytest.raises(ValueError):
        O.weight_dequant(np.zeros((100, 128), np.uint8), np.ones((1, 1), np.float32))
