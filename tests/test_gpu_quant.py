"""GPU parity of the quantisation kernels against the CPU oracle.

Codes and scales must match bit for bit.  Inputs are the seeded synthetic
workloads (small case, decode, prefill, MX operands) plus hand-made edge
cases; the oracle quantises the same bf16 values on the CPU.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def F():
    import fp8_block_scaled_02_amd as F
    assert torch.cuda.is_available()
    return F


def _np(t):
    return t.detach().cpu().numpy()


def _run_act(F, orc, x, block, fmt):
    fi = {"fp32": 0, "ue8m0": 1, "e8m0": 2}[fmt]
    q, s = F.fp8_act_quant(x.to(DEV), block, fmt)
    torch.cuda.synchronize()
    q2, s2 = orc.act_quant(W.bits(x), block, fi)
    return _np(q), _np(s), q2, s2


def _assert_same(q, s, q2, s2, what):
    bad = np.argwhere(q != q2)
    assert len(bad) == 0, f"{what}: {len(bad)} code mismatches, first at {tuple(bad[0])}: gpu {q[tuple(bad[0])]:#x} oracle {q2[tuple(bad[0])]:#x}"
    sv, sv2 = s.view(np.uint8), s2.view(np.uint8)
    bad = np.argwhere(sv != sv2)
    assert len(bad) == 0, f"{what}: {len(bad)} scale byte mismatches"


@pytest.mark.parametrize("block,fmt", [(128, "fp32"), (128, "ue8m0"), (32, "fp32"), (32, "ue8m0"), (32, "e8m0")])
def test_act_quant_tiny(F, orc, block, fmt):
    x = W.tiny_linear().x
    _assert_same(*_run_act(F, orc, x, block, fmt), f"tiny {block} {fmt}")


def _edge_rows():
    """Rows of 128 bf16 values exercising zero blocks, signed zeros,
    subnormals, ties, saturation of the block maximum and huge values."""
    rows = []
    rows.append(np.zeros(128, np.float32))
    z = np.zeros(128, np.float32); z[::2] = -0.0; rows.append(z)
    rows.append(np.full(128, 2.0 ** -133, np.float32))                      # bf16 subnormals
    t = np.linspace(-1, 1, 128).astype(np.float32) * 2.0 ** -130; rows.append(t)
    rows.append(np.full(128, 3.0e38, np.float32) * np.sign(np.linspace(-1, 1, 128)).astype(np.float32))
    h = np.zeros(128, np.float32)                                           # hand-worked style ties
    vals = [896, -896, 2, -2, 1, 6, 0.0078125, 0.001953125, 0.005859375, 832, 864, 2.25, 2.125, 2.375,
            0.029296875, 0.03125, 640, 12, 0.25, 100, 3, 5, 7, 9]
    h[:len(vals)] = vals; rows.append(h)
    rng = np.random.default_rng(5)
    for scale in (1e-3, 1.0, 1e3, 2.0 ** 100, 2.0 ** -100):
        rows.append((rng.standard_normal(128) * scale).astype(np.float32))
    o = rng.standard_normal(128).astype(np.float32); o[17] = 1e4; rows.append(o)  # one outlier
    x = torch.from_numpy(np.stack(rows)).to(torch.bfloat16)
    return x


@pytest.mark.parametrize("block,fmt", [(128, "fp32"), (128, "ue8m0"), (32, "fp32"), (32, "e8m0")])
def test_act_quant_edge_cases(F, orc, block, fmt):
    x = _edge_rows()
    _assert_same(*_run_act(F, orc, x, block, fmt), f"edge {block} {fmt}")


@pytest.mark.parametrize("M,K", [(1, 128), (3, 256), (5, 7168), (33, 384)])
def test_act_quant_ragged_shapes(F, orc, M, K):
    g = W.gen(11 + M)
    x = W.activations(M, K, 1, 30.0, g)
    _assert_same(*_run_act(F, orc, x, 128, "fp32"), f"{M}x{K}")


def test_act_quant_strided_rows(F, orc):
    """ld_x > K and ld_q > K: only the first K columns are read/written."""
    g = W.gen(3)
    big = W.activations(40, 512, 2, 25.0, g).to(DEV)
    x = big[:, :384]
    q = torch.full((40, 400), 0xAB, dtype=torch.uint8, device=DEV)
    s = torch.empty(40, 3, dtype=torch.float32, device=DEV)
    F.fp8_act_quant(x, 128, "fp32", q=q[:, :384], scales=s)
    torch.cuda.synchronize()
    q2, s2 = orc.act_quant(W.bits(x.cpu()), 128, 0)
    qn = _np(q)
    assert (qn[:, 384:] == 0xAB).all()
    _assert_same(qn[:, :384], _np(s), q2, s2, "strided")


def test_act_quant_decode_full(F, orc):
    c = W.decode_linear(device=DEV)
    for M in (1, 8, 32, 128):
        _assert_same(*_run_act(F, orc, c.x[:M], 128, "ue8m0"), f"decode M={M}")


def test_act_quant_prefill_full(F, orc):
    c = W.prefill_linear(device=DEV)
    _assert_same(*_run_act(F, orc, c.x, 128, "fp32"), "prefill 4096x7168")


def test_act_quant_mx_operand_full(F, orc):
    a, _ = W.mx_case(device=DEV, N=128)
    _assert_same(*_run_act(F, orc, a, 32, "e8m0"), "mx 8192x8192")


def test_act_quant_deterministic(F):
    c = W.prefill_linear(device=DEV, M=512)
    q1, s1 = F.fp8_act_quant(c.x, 128, "fp32")
    q2, s2 = F.fp8_act_quant(c.x, 128, "fp32")
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_weight_quant_tiny_and_outlier(F, orc, fmt):
    g = W.gen(21)
    w = W.weights(384, 512, 0.02, g)
    w[3, 200] = 1.5
    w[300, 7] = -40.0
    wq, ws = F.fp8_weight_quant(w.to(DEV), fmt)
    torch.cuda.synchronize()
    q2, s2 = orc.weight_quant(W.bits(w), {"fp32": 0, "ue8m0": 1}[fmt])
    _assert_same(_np(wq), _np(ws), q2, s2, f"weight {fmt}")


def test_weight_quant_prefill_full(F, orc):
    c = W.prefill_linear(device=DEV)
    wq, ws = F.fp8_weight_quant(c.w, "fp32")
    torch.cuda.synchronize()
    q2, s2 = orc.weight_quant(W.bits(c.w), 0)
    _assert_same(_np(wq), _np(ws), q2, s2, "weight 18432x7168")


def test_weight_quant_decode_sampled(F, orc):
    c = W.decode_linear(device=DEV)
    wq, ws = F.fp8_weight_quant(c.w, "ue8m0")
    torch.cuda.synchronize()
    for r0 in (0, 14336, 28672 - 1024):           # 128-row blocks are independent
        q2, s2 = orc.weight_quant(W.bits(c.w[r0:r0 + 1024]), 1)
        _assert_same(_np(wq[r0:r0 + 1024]), _np(ws[r0 // 128:(r0 + 1024) // 128]), q2, s2, f"weight rows {r0}")


def _cast_inputs():
    """fp32 patterns: every exponent, mantissas at and around every E4M3 and
    E5M2 rounding boundary, both signs, plus random patterns."""
    pats = []
    hi = np.arange(0, 256, dtype=np.uint32)          # sign+exponent byte
    lows = np.array([0, 1, 2, 0x7FFF, 0x8000, 0x8001, 0x7FFFF, 0x80000, 0x80001, 0xFFFFF, 0x100000,
                     0x100001, 0x3FFFFF, 0x400000, 0x400001, 0x7FFFFF], np.uint32)
    top = np.arange(0, 8, dtype=np.uint32) << 20     # the 3 mantissa bits E4M3 keeps
    for h in hi:
        for t in top:
            pats.append((h << 23) | t | lows)
            pats.append(((h | 0x100) << 23) | t | lows)   # negative
    pats.append(np.random.default_rng(9).integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32))
    u = np.concatenate(pats).astype(np.uint32)
    v = u.view(np.float32)
    return v[~np.isnan(v)]


def test_cast_e4m3_e5m2(F, orc):
    v = _cast_inputs()
    x = torch.from_numpy(v).to(DEV)
    for fmt, enc in ((F.FMT_E4M3, orc.e4m3_encode), (F.FMT_E5M2, orc.e5m2_encode)):
        q = _np(F.fp8_cast_f32(x, fmt))
        want = enc(v)
        bad = np.argwhere(q != want)
        assert len(bad) == 0, f"fmt {fmt}: {len(bad)} mismatches, first v={v[bad[0][0]]!r} ({v.view(np.uint32)[bad[0][0]]:#010x}) gpu {q[bad[0][0]]:#x} oracle {want[bad[0][0]]:#x}"


@pytest.mark.parametrize("block", [128, 32])
def test_act_quant_fp32_scales_every_block_magnitude(F, orc, block):
    """One quantisation block per bf16 amax pattern (every exponent incl.
    subnormals, every mantissa): the block holds amax itself, its negation,
    -0, and random in-range values, so the scale division runs over the whole
    fp32 range, including the tiny blocks that take the IEEE-division path."""
    amax_bits = np.arange(1, 0x7F80, dtype=np.uint32)          # every positive finite bf16
    amax = (amax_bits << 16).view(np.float32)
    nb = len(amax)
    rng = np.random.default_rng(17)
    vals = rng.uniform(-1, 1, size=(nb, block)).astype(np.float32) * amax[:, None]
    vals[:, 0] = amax
    vals[:, 1] = -amax
    vals[:, 2] = -0.0
    vals[:, 3] = amax * np.float32(0.5 ** 12)                  # rounds deep in the subnormal codes
    x = torch.from_numpy(vals[: (nb // 4) * 4].reshape(-1, 4 * block)).to(torch.bfloat16)
    assert float(x.abs().max()) <= 3.39e38
    _assert_same(*_run_act(F, orc, x, block, "fp32"), f"every amax block {block}")


# ---- weight dequantisation ---------------------------------------------------
def _deq_check(gpu_bits, want, what):
    g = gpu_bits.astype(np.uint16)
    nan_w = ((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0)
    nan_g = ((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)
    assert (nan_w == nan_g).all(), f"{what}: NaN positions differ"
    bad = np.argwhere((g != want) & ~nan_w)
    assert len(bad) == 0, f"{what}: {len(bad)} mismatches, first at {tuple(bad[0])}: gpu {g[tuple(bad[0])]:#06x} oracle {want[tuple(bad[0])]:#06x}"


def test_weight_dequant_every_code_wide_scales(F, orc):
    """Every code (NaN codes included) against fp32 block scales spread over
    the whole fp32 range, in both signs of magnitude overflow/underflow."""
    rng = np.random.default_rng(31)
    q = rng.integers(0, 256, size=(512, 1024), dtype=np.uint8)
    q[0, :256] = np.arange(256, dtype=np.uint8)
    s = np.exp(rng.uniform(-87, 87, size=(4, 8))).astype(np.float32)   # finite fp32
    s[0, 0], s[1, 1], s[2, 2], s[3, 3] = 1.0, 2.0 ** -140, 3.0e38, 1.0 / 448
    w = F.fp8_weight_dequant(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV))
    torch.cuda.synchronize()
    _deq_check(_np(w.view(torch.int16)).view(np.uint16), orc.weight_dequant(q, s), "wide scales")


def test_weight_dequant_strided(F, orc):
    g = W.gen(6)
    wq, ws = F.fp8_weight_quant(W.weights(256, 384, 0.02, g).to(DEV), "fp32")
    qbig = torch.zeros(256, 400, dtype=torch.uint8, device=DEV)
    qbig[:, :384] = wq
    out = torch.full((256, 392), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    F.fp8_weight_dequant(qbig[:, :384], ws, w=out[:, :384])
    torch.cuda.synchronize()
    o = _np(out.view(torch.int16)).view(np.uint16)
    assert (o[:, 384:] == 0xFFFF).all()
    _deq_check(o[:, :384], orc.weight_dequant(_np(wq), _np(ws)), "strided")


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_weight_dequant_prefill_full(F, orc, fmt):
    c = W.prefill_linear(device=DEV)
    wq, ws = F.fp8_weight_quant(c.w, fmt)
    w = F.fp8_weight_dequant(wq, ws)
    torch.cuda.synchronize()
    _deq_check(_np(w.view(torch.int16)).view(np.uint16), orc.weight_dequant(_np(wq), _np(ws)), f"18432x7168 {fmt}")


# ---- KV cache (E5M2, one scale per row) ----------------------------------------
def _kv_run(F, orc, x, what):
    q, s = F.fp8_kv_quant(x.to(DEV))
    torch.cuda.synchronize()
    q2, s2 = orc.kv_quant(W.bits(x))
    _assert_same(_np(q), _np(s), q2, s2, what)
    return q, s, q2, s2


@pytest.mark.parametrize("T,D", [(1, 16), (7, 128), (5, 576), (9, 1024), (3, 4096), (6, 8192), (2, 16384), (130, 1040)])
def test_kv_quant_shapes(F, orc, T, D):
    g = W.gen(T * 7 + D)
    _kv_run(F, orc, W.kv_rows(T, D, g), f"kv {T}x{D}")


def test_kv_quant_every_row_magnitude(F, orc):
    """One row per bf16 amax pattern (every exponent incl. subnormals): the row
    holds amax, -amax, -0, a value deep in the E5M2 subnormal codes and random
    in-range values, so the scale division spans the whole fp32 range."""
    amax = (np.arange(1, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(19)
    vals = rng.uniform(-1, 1, size=(len(amax), 128)).astype(np.float32) * amax[:, None]
    vals[:, 0], vals[:, 1], vals[:, 2] = amax, -amax, -0.0
    vals[:, 3] = amax * np.float32(2.0 ** -30)
    x = torch.from_numpy(vals).to(torch.bfloat16)
    _kv_run(F, orc, x, "every amax row")


def test_kv_quant_full_and_dequant(F, orc):
    c = W.CONFIGS["kv"]
    x = W.kv_rows(c["T"], c["D"], W.gen(12, DEV))
    q, s, q2, s2 = _kv_run(F, orc, x, "kv 32768x1024")
    out = F.fp8_kv_dequant(q, s)
    torch.cuda.synchronize()
    _deq_check(_np(out.view(torch.int16)).view(np.uint16), orc.kv_dequant(q2, s2), "kv dequant full")


def test_kv_dequant_every_code_and_strides(F, orc):
    rng = np.random.default_rng(23)
    q = rng.integers(0, 256, size=(64, 512), dtype=np.uint8)
    q[0, :256] = np.arange(256, dtype=np.uint8)
    s = np.exp(rng.uniform(-87, 87, size=64)).astype(np.float32)
    s[1], s[2] = 2.0 ** -140, 1.0
    qd = torch.zeros(64, 528, dtype=torch.uint8, device=DEV)
    qd[:, :512] = torch.from_numpy(q).to(DEV)
    out = torch.full((64, 520), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    F.fp8_kv_dequant(qd[:, :512], torch.from_numpy(s).to(DEV), out=out[:, :512])
    torch.cuda.synchronize()
    o = _np(out.view(torch.int16)).view(np.uint16)
    assert (o[:, 512:] == 0xFFFF).all()
    _deq_check(o[:, :512], orc.kv_dequant(q, s), "kv dequant codes")



@pytest.mark.parametrize("T,D", [(77, 16), (9, 16384), (100, 1040), (3, 2048), (16421, 1024), (262151, 16)])
def test_kv_dequant_row_grouping(F, orc, T, D):
    """Every branch of the dequant grid: many rows per workgroup with a
    partial last one (16 codes a row), a row over two segments (16384), a
    row whose 130 groups cannot share a workgroup, one row of 256 groups,
    and shared rows in launches large enough that each lane takes one group
    in each of four rows (1024 and 16 codes a row, partial last workgroup)."""
    rng = np.random.default_rng(T * 7 + D)
    q = rng.integers(0, 256, size=(T, D), dtype=np.uint8)
    s = np.exp(rng.uniform(-20, 20, size=T)).astype(np.float32)
    out = F.fp8_kv_dequant(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV))
    torch.cuda.synchronize()
    _deq_check(_np(out.view(torch.int16)).view(np.uint16), orc.kv_dequant(q, s), f"kv dequant {T}x{D}")


def test_weight_dequant_shared_rows_four_per_lane(F, orc):
    """Weights 4224 x 1024: two 128-group rows per 256 lanes, four row pairs
    per workgroup (the grid's folded form), every element against the
    oracle."""
    g = W.gen(61)
    w = W.weights(4224, 1024, 0.02, g)
    wq, ws = F.fp8_weight_quant(w.to(DEV), "fp32")
    out = F.fp8_weight_dequant(wq, ws)
    torch.cuda.synchronize()
    _deq_check(_np(out.view(torch.int16)).view(np.uint16), orc.weight_dequant(_np(wq), _np(ws)),
               "weight dequant 4224x1024")


def test_weight_dequant_two_segments(F, orc):
    """A 16384-wide weight row spans two segments of the dequant grid."""
    rng = np.random.default_rng(5)
    q = rng.integers(0, 256, size=(256, 16384), dtype=np.uint8)
    sc = np.exp(rng.uniform(-20, 20, size=(2, 128))).astype(np.float32)
    out = F.fp8_weight_dequant(torch.from_numpy(q).to(DEV), torch.from_numpy(sc).to(DEV))
    torch.cuda.synchronize()
    _deq_check(_np(out.view(torch.int16)).view(np.uint16), orc.weight_dequant(q, sc), "weight dequant 256x16384")


# ---- delayed scaling ----------------------------------------------------------
def _delayed_steps(S, n, seed, dev="cpu"):
    g = W.gen(seed, dev)
    mag = torch.exp2(torch.rand(S, 1, generator=g, device=dev) * 12 - 6)
    x = (torch.randn(S, n, generator=g, device=dev) * mag).to(torch.bfloat16)
    x[S // 2] = 0                                        # an all-zero step
    return x


@pytest.mark.parametrize("L,algo", [(3, "max"), (1, "max"), (16, "latest"), (64, "max")])
def test_delayed_scaling_steps(F, orc, L, algo):
    S, n = 10, 64 * 7168
    x = _delayed_steps(S, n, L)
    ds = F.DelayedScaler(L, algo, 400.0)
    xd = x.to(DEV)
    got_q, got_s = [], []
    for s in range(S):
        q, su = ds.quantize(xd[s])
        got_q.append(_np(q)), got_s.append(_np(su)[0])
    q2, s2 = orc.delayed_scaling(W.bits(x), L, 0 if algo == "max" else 1, 400.0)
    np.testing.assert_array_equal(np.array(got_s, np.float32).view(np.uint32), s2.view(np.uint32))
    for s in range(S):
        bad = np.flatnonzero(got_q[s] != q2[s])
        assert len(bad) == 0, f"step {s}: {len(bad)} code mismatches, first {bad[0]}"
    # reset restarts the sequence
    ds.reset()
    q, su = ds.quantize(xd[0])
    assert _np(su)[0] == 1.0 and (_np(q) == q2[0]).all()


@pytest.mark.parametrize("algo", ["max", "latest"])
def test_delayed_scaling_history_128(F, orc, algo):
    """The pitfall section's setting, amax_history_len = 128 with the max
    algorithm (and latest beside it), over 150 steps: the history fills past
    64 entries (the closing wave's strided scan takes a second pass) and then
    wraps.  Step magnitudes fall steadily, so once the window is full every
    step's window maximum is its oldest entry and changes as that entry
    leaves; an all-zero step and a late spike sit inside the run."""
    S, n, L = 150, 8192, 128
    g = W.gen(128 + (algo == "max"))
    mag = torch.exp2(torch.linspace(6.0, -6.0, S)).reshape(S, 1)
    mag[140] = 2.0 ** 8                                   # a late spike (still in the window at the end)
    x = (torch.randn(S, n, generator=g) * mag).to(torch.bfloat16)
    x[70] = 0
    ds = F.DelayedScaler(L, algo, 400.0)
    xd = x.to(DEV)
    outs = [ds.quantize(xd[s]) for s in range(S)]
    torch.cuda.synchronize()
    q2, s2 = orc.delayed_scaling(W.bits(x), L, 0 if algo == "max" else 1, 400.0)
    got_s = np.array([_np(su)[0] for _, su in outs], np.float32)
    np.testing.assert_array_equal(got_s.view(np.uint32), s2.view(np.uint32))
    for s, (q, _) in enumerate(outs):
        bad = np.flatnonzero(_np(q) != q2[s])
        assert len(bad) == 0, f"step {s}: {len(bad)} code mismatches, first {bad[0]}"
    if algo == "max":
        # after the history wrapped, the scale kept falling as the oldest
        # entries left the window, so the wrap itself is exercised
        assert len(set(s2[L + 1:141].tolist())) >= 6


def test_delayed_scaling_full_activation(F, orc):
    S, n = 3, 4096 * 7168
    x = _delayed_steps(S, n, 99, DEV)
    ds = F.DelayedScaler(16, "max", 400.0)
    outs = [ds.quantize(x[s]) for s in range(S)]
    torch.cuda.synchronize()
    q2, s2 = orc.delayed_scaling(W.bits(x), 16, 0, 400.0)
    for s, (q, su) in enumerate(outs):
        assert _np(su)[0] == s2[s], s
        assert (_np(q) == q2[s]).all(), s


@pytest.mark.parametrize("n", [8, 8 * 1000, 8192, 8192 * 3 + 40])
def test_delayed_scaling_ragged_sizes(F, orc, n):
    """One step is one kernel whose last workgroup closes the step: a single
    partial workgroup, a ragged last workgroup, and exactly one full one."""
    S = 6
    x = _delayed_steps(S, n, n)
    ds = F.DelayedScaler(4, "max", 400.0)
    xd = x.to(DEV)
    outs = [ds.quantize(xd[s]) for s in range(S)]
    torch.cuda.synchronize()
    q2, s2 = orc.delayed_scaling(W.bits(x), 4, 0, 400.0)
    for s, (q, su) in enumerate(outs):
        assert _np(su)[0] == s2[s], (n, s)
        assert (_np(q) == q2[s]).all(), (n, s)


def test_delayed_scaling_graph_replays(F, orc):
    """A step captured in a HIP graph and replayed on new inputs, with eager
    work and synchronisations between the replays, follows the oracle's
    scale sequence at every replay."""
    S, n = 6, 64 * 7168
    x = _delayed_steps(S, n, 7).to(DEV)
    ds = F.DelayedScaler(3, "max", 400.0)
    buf = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    q = torch.empty(n, dtype=torch.uint8, device=DEV)
    su = torch.empty(1, dtype=torch.float32, device=DEV)
    buf.copy_(x[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm-up outside the graph, then restart the state
        ds.quantize(buf, q=q, scale_used=su)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ds.reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ds.quantize(buf, q=q, scale_used=su)
    ds.reset()                          # capture does not run the step
    q2, s2 = orc.delayed_scaling(W.bits(x.cpu()), 3, 0, 400.0)
    for s in range(S):
        buf.copy_(x[s])
        g.replay()
        torch.cuda.synchronize()
        assert _np(su)[0] == s2[s], s
        assert (_np(q) == q2[s]).all(), s
        _ = (x[s].float() * 2).sum().item()   # eager work between replays


def test_act_quant_non_finite_blocks_stay_local(F, orc):
    """NaN and +-Inf inside some blocks: those blocks' codes and scales are
    unspecified, but every other block must still match the oracle exactly
    (and nothing faults)."""
    g = W.gen(44)
    x = W.activations(64, 1024, 4, 20.0, g)
    xf = x.float()
    xf[3, 5] = float("nan")
    xf[10, 300] = float("inf")
    xf[20, 1023] = float("-inf")
    x = xf.to(torch.bfloat16)
    bad_blocks = {(3, 0), (10, 2), (20, 7)}
    for fmt, fi in (("fp32", 0), ("ue8m0", 1)):
        q, s = F.fp8_act_quant(x.to(DEV), 128, fmt)
        torch.cuda.synchronize()
        q2, s2 = orc.act_quant(W.bits(x), 128, fi)
        qn, sn = _np(q), _np(s)
        for r in range(64):
            for b in range(8):
                if (r, b) in bad_blocks:
                    continue
                assert (qn[r, 128 * b:128 * (b + 1)] == q2[r, 128 * b:128 * (b + 1)]).all(), (fmt, r, b)
                assert sn[r, b].view(np.uint32) == s2[r, b].view(np.uint32), (fmt, r, b)


def test_act_quant_many_short_rows(F, orc):
    """70000 token rows of 128 channels: the row grid dimension far beyond
    65535 (the y-dimension limit)."""
    g = W.gen(45)
    x = W.activations(70000, 128, 1, 30.0, g)
    _assert_same(*_run_act(F, orc, x, 128, "fp32"), "70000x128")


def test_stream_probe_moves_the_act_quant_bytes(F):
    """The act_quant measurement probe: the copy kind writes each bf16's low
    byte as its code and zero scales (every row, including a partial last
    workgroup of chunks); the empty kind writes nothing."""
    g = W.gen(70)
    x = W.activations(37, 7168, 4, 20.0, g).to(DEV)
    q = torch.full((37, 7168), 0xAB, dtype=torch.uint8, device=DEV)
    sc = torch.full((37, 56), 7.0, dtype=torch.float32, device=DEV)
    F.fp8b_stream_probe(F.PROBE_EMPTY, x, q, sc)
    torch.cuda.synchronize()
    assert (_np(q) == 0xAB).all() and (_np(sc) == 7.0).all()
    F.fp8b_stream_probe(F.PROBE_COPY, x, q, sc)
    torch.cuda.synchronize()
    low = W.bits(x).astype(np.uint16) & 0xFF
    assert np.array_equal(_np(q), low.astype(np.uint8)) and (_np(sc) == 0.0).all()

