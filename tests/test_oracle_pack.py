"""Pins of the oracle's packed weight layout (fp8_weight_pack in
include/fp8blk.h): a storage order of the GPU library, not a step of the
method.  The GEMMs on packed weights must compute exactly what they compute
on row-major weights; these tests pin where each code goes.

Independent routes: hand-worked byte offsets (tests/golden), numpy's
reshape/transpose of the matrix, and the per-lane view the kernels rely on
(each 16-byte piece of a chunk is 16 consecutive codes of one row)."""
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "weight_pack_positions.txt")


def _source_index(N, K, G=1):
    """Packed position -> flat source index, recovered from two byte planes."""
    idx = np.arange(G * N * K, dtype=np.int64).reshape(G, N, K)
    planes = [O.weight_pack(((idx >> (8 * i)) & 0xFF).astype(np.uint8)) for i in range(3)]
    return sum(p.astype(np.int64) << (8 * i) for i, p in enumerate(planes)).reshape(-1)


def test_hand_worked_offsets():
    cases = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        N, K, n, k, off = map(int, line.split())
        cases.setdefault((N, K), []).append((n, k, off))
    assert len(cases) == 3
    for (N, K), pts in cases.items():
        src = _source_index(N, K)
        for n, k, off in pts:
            assert src[off] == n * K + k, (N, K, n, k, off, src[off])


def test_is_a_permutation_of_every_matrix():
    G, N, K = 3, 48, 192
    src = _source_index(N, K, G)
    assert np.array_equal(np.sort(src), np.arange(G * N * K))
    # matrix i stays in its own N*K bytes
    assert (src // (N * K) == np.arange(G * N * K) // (N * K)).all()


def test_matches_numpy_transpose():
    rng = np.random.default_rng(0)
    G, N, K = 2, 64, 256
    w = rng.integers(0, 256, size=(G, N, K), dtype=np.uint8)
    # [G][p][r][kc][g][b] -> [G][kc][p][g][r][b]
    want = w.reshape(G, N // 16, 16, K // 64, 4, 16).transpose(0, 3, 1, 4, 2, 5).reshape(G, N, K)
    np.testing.assert_array_equal(O.weight_pack(w), want)


def test_lane_view_of_each_chunk():
    """Lane l = 16g + r reading 16 bytes at 16l of chunk (kc, p) gets codes
    [16p + r][64kc + 16g .. 64kc + 16g + 15]."""
    rng = np.random.default_rng(1)
    N, K = 32, 128
    w = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    flat = O.weight_pack(w).reshape(-1)
    for kc in range(K // 64):
        for p in range(N // 16):
            chunk = flat[(kc * (N // 16) + p) * 1024:][:1024]
            for lane in range(64):
                r, g = lane & 15, lane >> 4
                np.testing.assert_array_equal(chunk[16 * lane:16 * lane + 16],
                                              w[16 * p + r, 64 * kc + 16 * g:64 * kc + 16 * g + 16])


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        O.weight_pack(np.zeros((24, 64), np.uint8))      # N % 16
    with pytest.raises(ValueError):
        O.weight_pack(np.zeros((16, 96), np.uint8))      # K % 64
