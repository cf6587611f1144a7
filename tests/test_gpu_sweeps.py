"""Exhaustive sweeps that the bit-exactness of the quantisers rests on.

* fp8_cast_f32 over every fp32 bit pattern (NaN patterns aside: their codes
  are unspecified), E4M3 and E5M2, against the oracle's encoders.
* The act_quant division in fp32-scale mode (the kernel replaces the IEEE
  quotient x / d with a reciprocal-and-correction sequence): every positive
  finite bf16 amax, each with every bf16 |x| <= amax in the same block, for
  128- and 32-wide blocks, against the oracle's act_quant.
* The same for the KV-cache quantiser (E5M2, d = amax / 57344, one scale per
  row).

Each sweep runs in chunks of about 2^26 elements; every chunk's codes and
scales are compared element by element with the oracle's (stronger than a
hash).  Runtime on MI355X with a 16-thread host: about 10-30 s per test.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"
CHUNK = 1 << 26


@pytest.fixture(scope="module")
def F():
    import fp8_block_scaled_02_amd as F
    assert torch.cuda.is_available()
    return F


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_cast_every_fp32_pattern(F, orc, fmt):
    f, enc = (F.FMT_E4M3, orc.e4m3_encode) if fmt == "e4m3" else (F.FMT_E5M2, orc.e5m2_encode)
    q = torch.empty(CHUNK, dtype=torch.uint8, device=DEV)
    checked = 0
    for c in range((1 << 32) // CHUNK):
        u = np.arange(c * CHUNK, (c + 1) * CHUNK, dtype=np.uint64).astype(np.uint32)
        s0 = c * CHUNK - (1 << 32 if c * CHUNK >= 1 << 31 else 0)    # the same patterns as int32
        xg = torch.arange(s0, s0 + CHUNK, dtype=torch.int32, device=DEV)
        F.fp8_cast_f32(xg.view(torch.float32), f, q)
        got = q.cpu().numpy()
        want = enc(u.view(np.float32))
        nan = ((u >> 23) & 0xFF == 0xFF) & (u & 0x7FFFFF != 0)
        bad = np.flatnonzero((got != want) & ~nan)
        assert len(bad) == 0, (f"{fmt}: {len(bad)} mismatches in chunk {c}, first pattern "
                               f"{u[bad[0]]:#010x}: gpu {got[bad[0]]:#04x} oracle {want[bad[0]]:#04x}")
        checked += int((~nan).sum())
    assert checked == (1 << 32) - 2 * ((1 << 23) - 1)


def _amax_blocks(a_lo, a_hi, width):
    """bf16 bit patterns [rows, width]: for every amax pattern a in
    [a_lo, a_hi) (positive finite bf16), rows [a, x_1 .. x_{width-1}] that
    together hold every pattern 0 .. a (every bf16 magnitude <= amax), the
    last row padded with a; odd magnitudes get a minus sign."""
    a = np.arange(a_lo, a_hi, dtype=np.int64)
    per = width - 1
    nrow = (a + per) // per
    ra = np.repeat(a, nrow)
    j = np.arange(ra.size) - np.repeat(np.cumsum(nrow) - nrow, nrow)
    v = np.minimum(per * j[:, None] + np.arange(per)[None, :], ra[:, None])
    x = np.empty((ra.size, width), np.uint16)
    x[:, 0] = ra
    x[:, 1:] = v | ((v & 1) << 15)
    return x


def _amax_chunks(width):
    """[a_lo, a_hi) ranges of amax patterns (together 1 .. 0x7F7F, every
    positive finite bf16) of about CHUNK elements each."""
    a = np.arange(1, 0x7F80, dtype=np.int64)
    cum = np.cumsum((a + width - 1) // (width - 1) * width)
    idx = [0] + list(np.flatnonzero(np.diff(cum // CHUNK)) + 1) + [len(a)]
    return [(int(a[i]), int(a[j - 1]) + 1) for i, j in zip(idx[:-1], idx[1:])]


def _as_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("block", [128, 32])
def test_act_quant_every_amax_and_magnitude(F, orc, block):
    seen = 0
    for lo, hi in _amax_chunks(block):
        x = _amax_blocks(lo, hi, block)
        q, s = F.fp8_act_quant(_as_bf16(x).to(DEV), block, "fp32")
        qg, sg = q.cpu().numpy(), s.cpu().numpy()
        q2, s2 = orc.act_quant(x, block, 0)
        bad = np.argwhere(qg != q2)
        assert len(bad) == 0, (f"block {block}, amax {x[bad[0][0], 0]:#06x}: {len(bad)} code mismatches, first x "
                               f"{x[tuple(bad[0])]:#06x}: gpu {qg[tuple(bad[0])]:#04x} oracle {q2[tuple(bad[0])]:#04x}")
        assert np.array_equal(sg.view(np.uint32), s2.view(np.uint32)), f"block {block}: scale mismatch"
        seen += hi - lo
    assert seen == 0x7F7F


def test_kv_quant_every_amax_and_magnitude(F, orc):
    seen = 0
    for lo, hi in _amax_chunks(128):
        x = _amax_blocks(lo, hi, 128)
        q, s = F.fp8_kv_quant(_as_bf16(x).to(DEV))
        qg, sg = q.cpu().numpy(), s.cpu().numpy()
        q2, s2 = orc.kv_quant(x)
        bad = np.argwhere(qg != q2)
        assert len(bad) == 0, (f"amax {x[bad[0][0], 0]:#06x}: {len(bad)} code mismatches, first x "
                               f"{x[tuple(bad[0])]:#06x}: gpu {qg[tuple(bad[0])]:#04x} oracle {q2[tuple(bad[0])]:#04x}")
        assert np.array_equal(sg.view(np.uint32), s2.view(np.uint32)), "scale mismatch"
        seen += hi - lo
    assert seen == 0x7F7F
