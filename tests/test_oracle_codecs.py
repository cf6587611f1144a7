"""Pins for the oracle's FP8 codecs and encoders (CPU only).

Each check ties the oracle to something other than itself: the constants the
pages print (tests/golden/format_constants.txt), hand-derived rounding cases
(tests/golden/encoder_cases.txt), torch's CPU float8 decoders/casts (library
routines), and an exhaustive brute-force nearest-value search written
separately in C (tests/brute/nearest.c).
"""
import ctypes
import math
import os
import subprocess

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = os.path.join(HERE, "golden")


def _constants():
    out = {}
    with open(os.path.join(GOLD, "format_constants.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, v = line.split()
                out[k] = float(v)
    return out


def _torch_table(dtype):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(dtype).to(torch.float64).numpy()


def test_page_constants(orc):
    c = _constants()
    t4 = orc.e4m3_table()
    t5 = orc.e5m2_table()
    assert np.nanmax(t4) == c["e4m3_max"] == 448
    assert np.nanmax(t5[np.isfinite(t5)]) == c["e5m2_max"] == 57344
    # bit allocation: 2^mantissa_bits codes per binade, 2^exp_bits binades
    pos4 = t4[:128]
    binade1 = pos4[(pos4 >= 1) & (pos4 < 2)]
    assert len(binade1) == 2 ** c["e4m3_mantissa_bits"]
    pos5 = t5[:128]
    assert len(pos5[(pos5 >= 1) & (pos5 < 2)]) == 2 ** c["e5m2_mantissa_bits"]
    # smallest normal
    assert orc.e4m3_table()[0x08] == 2.0 ** c["e4m3_min_normal_log2"]
    assert orc.e5m2_table()[0x04] == 2.0 ** c["e5m2_min_normal_log2"]
    # sign bit is the top bit
    assert c["e4m3_sign_bits"] == 1
    np.testing.assert_array_equal(t4[128:][~np.isnan(t4[128:])],
                                  -t4[:128][~np.isnan(t4[:128])])


def test_e4m3_table_vs_torch(orc):
    ours = orc.e4m3_table()
    ref = _torch_table(torch.float8_e4m3fn)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert [c for c in range(256) if np.isnan(ours[c])] == [0x7F, 0xFF]
    m = ~np.isnan(ours)
    np.testing.assert_array_equal(ours[m], ref[m])
    # signed zeros
    assert math.copysign(1.0, ours[0x80]) == -1.0
    # monotone over the positive codes, no infinities
    assert np.all(np.diff(ours[:0x7F]) > 0)
    assert not np.any(np.isinf(ours))


def test_e5m2_table_vs_torch(orc):
    ours = orc.e5m2_table()
    ref = _torch_table(torch.float8_e5m2)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    m = ~np.isnan(ours)
    np.testing.assert_array_equal(ours[m], ref[m])
    assert ours[0x7C] == np.inf and ours[0xFC] == -np.inf
    assert ours[0x7B] == 57344.0 and ours[0x01] == 2.0 ** -16
    assert np.all(np.diff(ours[:0x7D]) > 0)


def test_e8m0_table_vs_torch(orc):
    ours = orc.e8m0_table()
    ref = _torch_table(torch.float8_e8m0fnu)
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def test_encoder_golden_cases(orc):
    n = 0
    with open(os.path.join(GOLD, "encoder_cases.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            hx, fmt, code = line.split()[:3]
            v = np.array([int(hx, 16)], np.uint32).view(np.float32)
            enc = orc.e4m3_encode if fmt == "e4m3" else orc.e5m2_encode
            got = int(enc(v)[0])
            assert got == int(code, 16), (line, hex(got))
            n += 1
    assert n >= 25


def test_encoder_roundtrip_all_codes(orc):
    """Every finite code's value encodes back to itself."""
    for table, enc in ((orc.e4m3_table(), orc.e4m3_encode),
                       (orc.e5m2_table(), orc.e5m2_encode)):
        for c in range(256):
            v = table[c]
            if np.isfinite(v):
                assert int(enc(np.array([v], np.float32))[0]) == c, hex(c)


def test_encoder_vs_torch_cast_random(orc):
    """torch's CPU float8 casts (round to nearest even) on clamped inputs."""
    rng = np.random.default_rng(12345)
    u = rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    v = u.view(np.float32)
    v = v[~np.isnan(v)]
    for fmax, enc, dt in ((448.0, orc.e4m3_encode, torch.float8_e4m3fn),
                          (57344.0, orc.e5m2_encode, torch.float8_e5m2)):
        c = np.clip(v, -fmax, fmax)
        ref = torch.from_numpy(c).to(dt).view(torch.uint8).numpy()
        got = enc(c)
        np.testing.assert_array_equal(got, ref)
        # encoding the unclamped value equals encoding the clamped one
        np.testing.assert_array_equal(enc(v), got)


@pytest.fixture(scope="module")
def brute(tmp_path_factory):
    d = tmp_path_factory.mktemp("brute")
    so = str(d / "nearest.so")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", so,
                           os.path.join(HERE, "brute", "nearest.c"), "-lm"])
    L = ctypes.CDLL(so)
    L.count_mismatch.restype = ctypes.c_uint64
    L.count_mismatch.argtypes = [ctypes.c_uint64, ctypes.c_uint64,
                                 ctypes.POINTER(ctypes.c_double), ctypes.c_int,
                                 ctypes.c_double, ctypes.c_void_p,
                                 ctypes.POINTER(ctypes.c_uint32)]
    return L


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_encoder_exhaustive_brute_force(orc, brute, fmt):
    """All 2^32 fp32 bit patterns: oracle encoder == nearest grid value with
    ties to the even code, after clamping to +-Fmax."""
    if fmt == "e4m3":
        tab = _torch_table(torch.float8_e4m3fn)[:0x7F]      # codes 0..0x7E
        fmax = 448.0
        fn = orc.lib().orc_e4m3_encode
    else:
        tab = _torch_table(torch.float8_e5m2)[:0x7C]        # codes 0..0x7B
        fmax = 57344.0
        fn = orc.lib().orc_e5m2_encode
    grid = np.ascontiguousarray(tab, np.float64)
    first = ctypes.c_uint32(0)
    ptr = ctypes.cast(fn, ctypes.c_void_p)
    bad = brute.count_mismatch(0, 1 << 32, grid.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                               len(grid), fmax, ptr, ctypes.byref(first))
    assert bad == 0, f"{bad} mismatches, first at 0x{first.value:08x}"
