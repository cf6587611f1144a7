"""GPU parity of the GEMM kernels (block-scaled, MXFP8, grouped MoE) against
the CPU oracle.

Each side quantises the same seeded bf16 inputs itself (the quantisers are
proven bit-identical in test_gpu_quant.py); the oracle then computes y with
exact block sums and an fp64 combination, and the GPU output must meet the
tolerance in tests/parity.py.  Small cases are compared element by element;
full-size cases on sampled rows (each sampled row covers every column, so
every N tile and both ends of the M range are checked).
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


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _linear_case(F, orc, x, w, fmt, out_dtype, rows=None):
    """Run act_quant + weight quant + block GEMM on the GPU; the oracle
    recomputes everything from the bf16 inputs for the given rows."""
    fi = {"fp32": 0, "ue8m0": 1}[fmt]
    a, sa = F.fp8_act_quant(x.to(DEV), 128, fmt)
    wq, ws = F.fp8_weight_quant(w.to(DEV), fmt)
    y = F.fp8_block_gemm(a, sa, wq, ws, out_dtype)
    torch.cuda.synchronize()
    xs = x if rows is None else x[torch.as_tensor(rows, device=x.device)]
    oa, osa = orc.act_quant(W.bits(xs), 128, fi)
    ow, osw = orc.weight_quant(W.bits(w), fi)
    yr, bnd = orc.block_gemm(oa, osa, ow, osw)
    yg = _np(y) if rows is None else _np(y[torch.as_tensor(rows, device=y.device)])
    return yg, yr, bnd


def test_block_gemm_tiny_fp32(F, orc):
    c = W.tiny_linear()
    yg, yr, bnd = _linear_case(F, orc, c.x, c.w, "fp32", torch.float32)
    worst = assert_parity(yg, yr, bnd, False, "tiny")
    print(f"tiny worst err/allowed {worst:.3g}")


@pytest.mark.parametrize("M,N,K", [(300, 384, 640), (1, 128, 128), (129, 256, 256), (64, 512, 1280)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_block_gemm_ragged(F, orc, M, N, K, out):
    c = W.prefill_linear(M=M, K=K, N=N, seed=M + N + K)
    yg, yr, bnd = _linear_case(F, orc, c.x, c.w, "fp32", out)
    assert_parity(yg, yr, bnd, out == torch.bfloat16, f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 512, 1152), (2, 256, 640), (1, 128, 128), (2, 384, 2176),
                                   (7, 384, 640), (16, 128, 128), (17, 256, 384),
                                   (20, 256, 1152), (32, 640, 2048), (33, 256, 640), (40, 128, 128),
                                   (48, 384, 1152), (49, 256, 384), (64, 640, 2048), (65, 256, 640)])
def test_block_gemm_few_tokens(F, orc, M, N, K):
    """M <= 64 takes the streaming decode kernel: one to four 16-token
    subtiles (2- and 1-deep register rings), K-block counts below, at and
    past the prefetch depth and not a multiple of the K split; M = 65 is the
    first size on 128 x 128 tiles (and 33 .. 64 take 64 x 128 tiles on
    row-major weights)."""
    c = W.decode_linear(K=K, N=N, seed=M + K)
    yg, yr, bnd = _linear_case(F, orc, c.x[:M], c.w, "ue8m0", torch.bfloat16)
    assert_parity(yg, yr, bnd, True, f"{M}x{N}x{K}")
    yg, yr, bnd = _linear_case(F, orc, c.x[:M], c.w, "fp32", torch.float32)
    assert_parity(yg, yr, bnd, False, f"{M}x{N}x{K} f32")


def test_block_gemm_ue8m0_small(F, orc):
    c = W.decode_linear(K=1024, N=512)
    yg, yr, bnd = _linear_case(F, orc, c.x, c.w, "ue8m0", torch.bfloat16)
    assert_parity(yg, yr, bnd, True, "ue8m0 128x512x1024")


@pytest.mark.parametrize("M,K", [(1, 256), (40, 256), (100, 256), (300, 256), (300, 384)])
@pytest.mark.parametrize("scale", ["small", "large"])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_block_gemm_scale_products_near_the_fp32_range_ends(F, orc, M, K, scale, out):
    """Hand-made codes and scales whose per-block products a_scales * w_scales
    lie just above fp32's smallest normal (2^-126 .. 2^-122) or near 2^100,
    on every path (streaming for M <= 64 on packed weights, 64-row tiles for
    M 40 on row-major ones, 128-row tiles with the K split at two K blocks and
    without it at three) and both weight layouts."""
    rng = np.random.default_rng(31 + M + K)
    N = 256

    def codes(rows):
        c = rng.integers(0, 0x7F, size=(rows, K)).astype(np.uint8)   # 0x7F is NaN
        return c | (rng.integers(0, 2, size=(rows, K)).astype(np.uint8) << 7)

    a, w = codes(M), codes(N)
    lo_a, lo_w = (-66, -60) if scale == "small" else (50, 49)
    sa = np.ldexp(rng.uniform(1, 2, size=(M, K // 128)), lo_a).astype(np.float32)
    sw = np.ldexp(rng.uniform(1, 2, size=(N // 128, K // 128)), lo_w).astype(np.float32)
    prod = sa[:, None, :].astype(np.float64) * sw[None, :, :]
    assert prod.min() >= 2.0 ** -126 and prod.max() < 2.0 ** 102
    yr, bnd = orc.block_gemm(a, sa, w, sw)
    assert np.all(np.isfinite(yr)) and bnd.max() < 2.0 ** 127
    ta, tsa, tw, tsw = (torch.from_numpy(v).to(DEV) for v in (a, sa, w, sw))
    for y in (F.fp8_block_gemm(ta, tsa, tw, tsw, out),
              F.fp8_block_gemm_packed(ta, tsa, F.fp8_weight_pack(tw), tsw, out)):
        torch.cuda.synchronize()
        assert_parity(_np(y), yr, bnd, out == torch.bfloat16, f"scale products {scale}, M {M}")


@pytest.mark.parametrize("M,K", [(40, 640), (300, 640), (8, 1024), (40, 1024)])
def test_linear_step_graph_replay_matches_eager(F, M, K):
    """act_quant + block GEMM (packed weights) captured once as a HIP graph
    and replayed on new activations, with eager work between replays: every
    replay equals the eager step bit for bit (no allocation, memset or
    synchronisation is recorded).  K 640 (five K blocks) takes the streaming
    kernel and the tiles, K 1024 the register-streamed kernel."""
    N = 384
    g = torch.Generator(device=DEV).manual_seed(61 + M)
    w = (torch.randn(N, K, device=DEV, generator=g) * 0.02).to(torch.bfloat16)
    wq, ws = F.fp8_weight_quant(w, "fp32")
    wp = F.fp8_weight_pack(wq)
    x = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    a = torch.empty(M, K, dtype=torch.uint8, device=DEV)
    sa = torch.empty(M, K // 128, dtype=torch.float32, device=DEV)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)

    def step():
        F.fp8_act_quant(x, 128, "fp32", q=a, scales=sa)
        F.fp8_block_gemm_packed(a, sa, wp, ws, torch.bfloat16, y=y)

    x.copy_(torch.randn(M, K, device=DEV, generator=g).to(torch.bfloat16))
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        x.copy_((torch.randn(M, K, device=DEV, generator=g) * (1 + r)).to(torch.bfloat16))
        step()
        torch.cuda.synchronize()
        want = y.clone()
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), want.view(torch.int16)), f"replay {r}"


@pytest.mark.parametrize("M", [1, 16, 17, 32])
@pytest.mark.parametrize("fmt,out", [("ue8m0", torch.bfloat16), ("fp32", torch.float32)])
def test_block_gemm_decode_panels_split_evenly(F, orc, M, fmt, out):
    """N = 28672 packed weights: 1792 panels of 16 rows, 7 per CU on 256 CUs,
    so one and two 16-token subtiles run 112-row workgroups (elsewhere 64);
    K 640 (5 K blocks over the 4 waves); every output element."""
    N, K = 28672, 640
    c = W.decode_linear(K=K, N=N, seed=3 * M + 1)
    fi = {"fp32": 0, "ue8m0": 1}[fmt]
    a, sa = F.fp8_act_quant(c.x[:M].to(DEV), 128, fmt)
    wq, ws = F.fp8_weight_quant(c.w.to(DEV), fmt)
    y = F.fp8_block_gemm_packed(a, sa, F.fp8_weight_pack(wq), ws, out)
    torch.cuda.synchronize()
    oa, osa = orc.act_quant(W.bits(c.x[:M]), 128, fi)
    ow, osw = orc.weight_quant(W.bits(c.w), fi)
    yr, bnd = orc.block_gemm(oa, osa, ow, osw)
    assert_parity(_np(y), yr, bnd, out == torch.bfloat16, f"{M}x{N}x{K} {fmt}")


def test_block_gemm_decode_full(F, orc):
    """8192 -> 28672 at every decode size and across the path switches
    (up to 64 tokens the register-streamed kernel on packed weights and the
    streaming kernel or 64 x 128 tiles on row-major ones, then 128 x 128
    tiles), both weight layouts; sampled token rows x every output column."""
    c = W.decode_linear(device=DEV)
    a, sa = F.fp8_act_quant(c.x, 128, "ue8m0")
    wq, ws = F.fp8_weight_quant(c.w, "ue8m0")
    wp = F.fp8_weight_pack(wq)
    ow, osw = orc.weight_quant(W.bits(c.w), 1)
    for M in (1, 8, 32, 48, 64, 65, 100, 128):
        rows = sorted({0, M - 1, M // 2})
        oa, osa = orc.act_quant(W.bits(c.x[rows]), 128, 1)
        yr, bnd = orc.block_gemm(oa, osa, ow, osw)
        for name, y in (("row-major", F.fp8_block_gemm(a[:M], sa[:M], wq, ws, torch.bfloat16)),
                        ("packed", F.fp8_block_gemm_packed(a[:M], sa[:M], wp, ws, torch.bfloat16))):
            torch.cuda.synchronize()
            assert_parity(_np(y[rows]), yr, bnd, True, f"decode M={M} {name}")


@pytest.mark.parametrize("M,N,K", [(65, 128, 256), (128, 256, 768), (100, 384, 1024), (256, 512, 2048),
                                   (128, 256, 384), (97, 40960, 256)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_block_gemm_k_split(F, orc, M, N, K, out):
    """Grids of at most one 128 x 128 tile per CU with an even K-block count
    split K between two wave groups (one, three and four blocks per group;
    two m-tiles); an odd count (K 384) and a grid wider than the CU count
    (97 x 40960, 320 tiles) keep the unsplit kernel.  Both weight layouts,
    sampled rows x every column on the wide case."""
    c = W.prefill_linear(M=M, K=K, N=N, seed=7 * M + K)
    a, sa = F.fp8_act_quant(c.x.to(DEV), 128, "fp32")
    wq, ws = F.fp8_weight_quant(c.w.to(DEV), "fp32")
    rows = list(range(M)) if N * M <= 1 << 17 else sorted({0, 1, M // 2, M - 1})
    oa, osa = orc.act_quant(W.bits(c.x[rows]), 128, 0)
    ow, osw = orc.weight_quant(W.bits(c.w), 0)
    yr, bnd = orc.block_gemm(oa, osa, ow, osw)
    for name, y in (("row-major", F.fp8_block_gemm(a, sa, wq, ws, out)),
                    ("packed", F.fp8_block_gemm_packed(a, sa, F.fp8_weight_pack(wq), ws, out))):
        torch.cuda.synchronize()
        assert_parity(_np(y[rows]), yr, bnd, out == torch.bfloat16, f"{M}x{N}x{K} {name}")


@pytest.mark.parametrize("M,N", [(2000, 2304), (2048, 2176)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_block_gemm_grids_wider_than_the_chip(F, orc, M, N, out):
    """128 x 128 tile grids of more tiles than CUs (288 and 272, so no K
    split), N a multiple of 256 and not; a ragged last m-tile (M 2000);
    both weight layouts; sampled rows across m-tiles x every column."""
    K = 512
    c = W.prefill_linear(M=M, K=K, N=N, seed=M + N)
    a, sa = F.fp8_act_quant(c.x.to(DEV), 128, "fp32")
    wq, ws = F.fp8_weight_quant(c.w.to(DEV), "fp32")
    rows = [0, 1, 127, 128, 1000, M - 2, M - 1]
    oa, osa = orc.act_quant(W.bits(c.x[rows]), 128, 0)
    ow, osw = orc.weight_quant(W.bits(c.w), 0)
    yr, bnd = orc.block_gemm(oa, osa, ow, osw)
    for name, y in (("row-major", F.fp8_block_gemm(a, sa, wq, ws, out)),
                    ("packed", F.fp8_block_gemm_packed(a, sa, F.fp8_weight_pack(wq), ws, out))):
        torch.cuda.synchronize()
        assert_parity(_np(y[rows]), yr, bnd, out == torch.bfloat16, f"{M}x{N}x{K} {name}")


def test_block_gemm_prefill_full_sampled(F, orc):
    c = W.prefill_linear(device=DEV)
    rows = [0, 1, 127, 128, 1000, 2047, 2048, 3071, 4094, 4095]
    yg, yr, bnd = _linear_case(F, orc, c.x, c.w, "fp32", torch.bfloat16, rows=rows)
    worst = assert_parity(yg, yr, bnd, True, "prefill 4096x18432x7168")
    print(f"prefill worst err/allowed {worst:.3g}")


def test_block_gemm_deterministic(F):
    c = W.prefill_linear(device=DEV, M=256, N=1024, K=2048)
    a, sa = F.fp8_act_quant(c.x, 128, "fp32")
    wq, ws = F.fp8_weight_quant(c.w, "fp32")
    y1 = F.fp8_block_gemm(a, sa, wq, ws, torch.bfloat16)
    y2 = F.fp8_block_gemm(a, sa, wq, ws, torch.bfloat16)
    assert torch.equal(y1, y2)


# ---- MXFP8 -------------------------------------------------------------------
def _mx_case(F, orc, a_bf, b_bf, rows=None):
    qa, ea = F.fp8_act_quant(a_bf.to(DEV), 32, "e8m0")
    qb, eb = F.fp8_act_quant(b_bf.to(DEV), 32, "e8m0")
    y = F.mxfp8_gemm(qa, ea, qb, eb)
    torch.cuda.synchronize()
    asel = a_bf if rows is None else a_bf[torch.as_tensor(rows, device=a_bf.device)]
    oa, oea = orc.act_quant(W.bits(asel), 32, 2)
    ob, oeb = orc.act_quant(W.bits(b_bf), 32, 2)
    yr, bnd = orc.mx_gemm(oa, oea, ob, oeb)
    yg = _np(y) if rows is None else _np(y[torch.as_tensor(rows, device=y.device)])
    return yg, yr, bnd


# (2085, 512, 384) and (2048, 256, 128) run on the 256 x 256 tiles (M >= 2048
# and N a multiple of 256): a ragged last m-tile with an odd number of K
# steps, and a single K step; the others on the 128 x 128 tiles.
@pytest.mark.parametrize("M,N,K", [(200, 256, 512), (16, 128, 128), (130, 384, 640), (2085, 512, 384),
                                   (2048, 256, 128)])
def test_mx_gemm_small(F, orc, M, N, K):
    a, b = W.mx_case(M=M, N=N, K=K, seed=M + K)
    yg, yr, bnd = _mx_case(F, orc, a, b)
    worst = assert_parity(yg, yr, bnd, False, f"mx {M}x{N}x{K}")
    print(f"mx {M}x{N}x{K} worst {worst:.3g}")


def test_mx_gemm_unit_scales_equal_plain_products(F, orc):
    """All E8M0 bytes 127: the MX GEMM is a plain FP8 GEMM (exact integer
    sums here: codes of small integers)."""
    ints = np.arange(-6, 7)
    code = {v: int(orc.e4m3_encode(np.array([v], np.float32))[0]) for v in ints}
    rng = np.random.default_rng(4)
    ia = rng.choice(ints, size=(64, 256))
    ib = rng.choice(ints, size=(128, 256))
    qa = torch.from_numpy(np.vectorize(code.get)(ia).astype(np.uint8)).to(DEV)
    qb = torch.from_numpy(np.vectorize(code.get)(ib).astype(np.uint8)).to(DEV)
    ea = torch.full((64, 8), 127, dtype=torch.uint8, device=DEV)
    eb = torch.full((128, 8), 127, dtype=torch.uint8, device=DEV)
    y = F.mxfp8_gemm(qa, ea, qb, eb)
    np.testing.assert_array_equal(_np(y), (ia @ ib.T).astype(np.float64))


def test_mx_gemm_full_sampled(F, orc):
    a, b = W.mx_case(device=DEV)
    rows = [0, 127, 128, 4095, 8190, 8191]
    yg, yr, bnd = _mx_case(F, orc, a, b, rows=rows)
    worst = assert_parity(yg, yr, bnd, False, "mx 8192^3")
    print(f"mx 8192^3 worst {worst:.3g}")


# ---- grouped MoE ---------------------------------------------------------------
def _moe_run(F, orc, case, rows=None):
    x = case.x.to(DEV)
    a, sa = F.fp8_act_quant(x, 128, "fp32")
    E, N, K = case.w.shape
    wq = torch.empty(E, N, K, dtype=torch.uint8, device=DEV)
    ws = torch.empty(E, N // 128, K // 128, dtype=torch.float32, device=DEV)
    for e in range(E):
        F.fp8_weight_quant(case.w[e].to(DEV), "fp32", q=wq[e], scales=ws[e])
    ri = case.row_index.to(DEV)
    offs = case.offs.to(DEV)
    y = F.fp8_grouped_gemm(a, sa, ri, offs, wq, ws, torch.bfloat16)
    torch.cuda.synchronize()
    R = case.row_index.shape[0]
    rows = np.arange(R) if rows is None else np.asarray(rows)
    offs_np = case.offs.numpy()
    experts = sorted({int(np.searchsorted(offs_np, r, side="right") - 1) for r in rows})
    toks = sorted({int(case.row_index[r]) for r in rows})
    # the oracle quantises the tokens and experts it needs from the bf16 inputs
    oa_full = np.zeros((case.x.shape[0], K), np.uint8)
    osa_full = np.ones((case.x.shape[0], K // 128), np.float32)
    oa, osa = orc.act_quant(W.bits(case.x[torch.as_tensor(toks, device=case.x.device)]), 128, 0)
    oa_full[toks] = oa
    osa_full[toks] = osa
    wl, sl = [None] * E, [None] * E
    for e in experts:
        wl[e], sl[e] = orc.weight_quant(W.bits(case.w[e]), 0)
    yr, bnd = orc.grouped_gemm(oa_full, osa_full, case.row_index.numpy(), offs_np, wl, sl, rows=rows)
    return _np(y[torch.as_tensor(rows, device=y.device)]), yr, bnd


def test_grouped_small_full(F, orc):
    case = W.moe_case(T=64, E=8, topk=2, N=256, K=384)
    yg, yr, bnd = _moe_run(F, orc, case)
    assert_parity(yg, yr, bnd, True, "moe small")


def test_grouped_skewed_with_empty_experts(F, orc):
    case = W.moe_case(T=300, E=32, topk=3, N=256, K=256, s=2.0)
    counts = (case.offs[1:] - case.offs[:-1]).numpy()
    assert (counts == 0).any() and counts.max() > 128
    yg, yr, bnd = _moe_run(F, orc, case)
    assert_parity(yg, yr, bnd, True, "moe skewed")


def _moe_counts_case(counts, T, N, K, seed):
    """A routing with the given rows per expert (tokens drawn at random)."""
    counts = np.asarray(counts, np.int64)
    g = W.gen(seed)
    x = W.activations(T, K, max(1, round(0.005 * K)), 50.0, g)
    w = torch.stack([W.weights(N, K, 0.02, g) for _ in counts])
    offs = np.zeros(len(counts) + 1, np.int64)
    offs[1:] = np.cumsum(counts)
    ri = np.random.default_rng(seed).integers(0, T, size=int(offs[-1]))
    experts = np.repeat(np.arange(len(counts)), counts)
    return W.MoeCase(x, w, torch.from_numpy(ri.astype(np.int32)), torch.from_numpy(offs.astype(np.int32)),
                     torch.from_numpy(experts.astype(np.int32)))


def test_grouped_every_tail_kind(F, orc):
    """Expert sizes around every branch of the work map: empty experts,
    short tails on the streaming path (1, 16 / 17, 32 rows: one and two
    16-row subtiles), longer tails padded into a 128-row tile (33, 127),
    whole tiles (128, 256) and whole tiles plus either kind of tail."""
    counts = [0, 1, 16, 17, 32, 33, 127, 128, 129, 144, 160, 161, 256, 300, 0, 5]
    case = _moe_counts_case(counts, T=200, N=256, K=640, seed=41)
    yg, yr, bnd = _moe_run(F, orc, case)
    assert_parity(yg, yr, bnd, True, "moe tails")


@pytest.mark.parametrize("scale", ["small", "large"])
def test_grouped_scale_products_near_the_fp32_range_ends(F, orc, scale):
    """The grouped GEMM with hand-made codes and scale products just above
    2^-126 or near 2^100: experts of 5 rows (streaming items), 40 (a padded
    tile) and 150 (a whole tile and a streaming tail), both weight layouts."""
    rng = np.random.default_rng(51)
    T, E, N, K = 120, 3, 256, 256
    counts = [5, 40, 150]

    def codes(*shape):
        c = rng.integers(0, 0x7F, size=shape).astype(np.uint8)      # 0x7F is NaN
        return c | (rng.integers(0, 2, size=shape).astype(np.uint8) << 7)

    a, w = codes(T, K), codes(E, N, K)
    lo_a, lo_w = (-66, -60) if scale == "small" else (50, 49)
    sa = np.ldexp(rng.uniform(1, 2, size=(T, K // 128)), lo_a).astype(np.float32)
    sw = np.ldexp(rng.uniform(1, 2, size=(E, N // 128, K // 128)), lo_w).astype(np.float32)
    ri = rng.integers(0, T, size=sum(counts)).astype(np.int32)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    yr, bnd = orc.grouped_gemm(a, sa, ri, offs, list(w), list(sw))
    assert np.all(np.isfinite(yr)) and bnd.max() < 2.0 ** 127
    ta, tsa, tw, tsw, tri, tof = (torch.from_numpy(v).to(DEV) for v in (a, sa, w, sw, ri, offs))
    for out in (torch.float32, torch.bfloat16):
        for y in (F.fp8_grouped_gemm(ta, tsa, tri, tof, tw, tsw, out),
                  F.fp8_grouped_gemm_packed(ta, tsa, tri, tof, F.fp8_weight_pack(tw), tsw, out)):
            torch.cuda.synchronize()
            assert_parity(_np(y), yr, bnd, out == torch.bfloat16, f"grouped, scale products {scale}")


@pytest.mark.parametrize("counts", [[200, 150] + [3] * 62,
                                    [600, 500, 400, 300, 2, 5, 9] + [0] * 57])
def test_grouped_two_half_schedule(F, orc, counts):
    """64 experts at N 1024 give a 512-workgroup grid, which splits into a
    tile-first and a stream-first half: stream items outweighing tile items
    (the tile-first half also takes stream items) and the reverse (the
    stream-first half also takes the last tile items); both layouts."""
    case = _moe_counts_case(counts, T=2048, N=1024, K=256, seed=47)
    E, N, K = case.w.shape
    a, sa = F.fp8_act_quant(case.x.to(DEV), 128, "fp32")
    wq = torch.empty(E, N, K, dtype=torch.uint8, device=DEV)
    ws = torch.empty(E, N // 128, K // 128, dtype=torch.float32, device=DEV)
    for e in range(E):
        F.fp8_weight_quant(case.w[e].to(DEV), "fp32", q=wq[e], scales=ws[e])
    ri, offs = case.row_index.to(DEV), case.offs.to(DEV)
    R = case.row_index.shape[0]
    oa, osa = orc.act_quant(W.bits(case.x), 128, 0)
    wl, sl = zip(*(orc.weight_quant(W.bits(case.w[e]), 0) for e in range(E)))
    yr, bnd = orc.grouped_gemm(oa, osa, case.row_index.numpy(), case.offs.numpy(), list(wl), list(sl))
    for name, y in (("row-major", F.fp8_grouped_gemm(a, sa, ri, offs, wq, ws, torch.bfloat16)),
                    ("packed", F.fp8_grouped_gemm_packed(a, sa, ri, offs, F.fp8_weight_pack(wq), ws, torch.bfloat16))):
        torch.cuda.synchronize()
        assert y.shape == (R, N)
        assert_parity(_np(y), yr, bnd, True, f"two halves {name}")


def test_grouped_only_short_experts(F, orc):
    """Every expert below 32 rows: no tile items at all."""
    counts = [3, 0, 31, 7, 1, 0, 20, 16]
    case = _moe_counts_case(counts, T=64, N=384, K=1152, seed=43)
    yg, yr, bnd = _moe_run(F, orc, case)
    assert_parity(yg, yr, bnd, True, "moe short")


def test_grouped_full_sampled(F, orc):
    case = W.moe_case(device=DEV)
    offs = case.offs.numpy()
    counts = offs[1:] - offs[:-1]
    big = int(np.argmax(counts))
    small = [e for e in range(len(counts)) if counts[e] == 1][:3]
    rows = {0, int(offs[-1]) - 1, int(offs[big]), int(offs[big + 1]) - 1, int(offs[big]) + 130}
    rows |= {int(offs[e]) for e in small}
    rows = sorted(rows)
    yg, yr, bnd = _moe_run(F, orc, case, rows=rows)
    worst = assert_parity(yg, yr, bnd, True, "moe 256 experts")
    print(f"moe full worst {worst:.3g}; rows {rows}")


def test_block_gemm_decodes_every_code_exactly(F, orc):
    """W = identity (code for 1.0 on the diagonal), unit scales: y[m][n] is
    the value of a[m][n], for all 254 finite E4M3 codes."""
    tab = orc.e4m3_table()
    codes = np.array([c for c in range(256) if np.isfinite(tab[c])], np.uint8)
    a = np.zeros((2, 128), np.uint8)
    a.reshape(-1)[:len(codes)] = codes
    w = np.zeros((128, 128), np.uint8)
    np.fill_diagonal(w, int(orc.e4m3_encode(np.array([1.0], np.float32))[0]))
    ta, tw = torch.from_numpy(a).to(DEV), torch.from_numpy(w).to(DEV)
    one = torch.ones(2, 1, dtype=torch.float32, device=DEV)
    y = F.fp8_block_gemm(ta, one, tw, torch.ones(1, 1, dtype=torch.float32, device=DEV), torch.float32)
    np.testing.assert_array_equal(_np(y), tab[a])


def test_mx_gemm_applies_block_exponents_exactly(F, orc):
    """Identity B with byte 127; A codes with E8M0 bytes 117..137 per 32-block:
    y = value(a) * 2^(e - 127) exactly."""
    tab = orc.e4m3_table()
    rng = np.random.default_rng(8)
    a = rng.integers(0, 0x7E, size=(8, 128)).astype(np.uint8)
    a[:, ::3] |= 0x80
    ea = rng.integers(117, 138, size=(8, 4)).astype(np.uint8)
    b = np.zeros((128, 128), np.uint8)
    np.fill_diagonal(b, int(orc.e4m3_encode(np.array([1.0], np.float32))[0]))
    eb = np.full((128, 4), 127, np.uint8)
    y = F.mxfp8_gemm(*[torch.from_numpy(v).to(DEV) for v in (a, ea, b, eb)])
    want = tab[a] * np.ldexp(1.0, np.repeat(ea.astype(int) - 127, 32, axis=1))
    np.testing.assert_array_equal(_np(y), want)



@pytest.mark.parametrize("edge", ["low", "high"])
def test_mx_gemm_exact_at_the_scale_byte_range_edges(F, orc, edge):
    """Folding 2^(e - 127) into the widened codes keeps every code a normal
    bf16 for scale bytes 10..246.  One operand takes bytes at an edge of that
    range, the other bytes that keep every product and sum in fp32's normal
    range; checked with each operand in each role."""
    rng = np.random.default_rng(21 if edge == "low" else 22)
    M = N = 128
    K = 256

    def codes(rows):
        c = rng.integers(0, 0x7F, size=(rows, K)).astype(np.uint8)   # 0x7F is NaN
        return c | (rng.integers(0, 2, size=(rows, K)).astype(np.uint8) << 7)

    a, b = codes(M), codes(N)
    if edge == "low":     # 2^-117 * 2^-9 = 2^-126; sums 146..152: products >= 2^-126
        ea = rng.integers(10, 13, size=(M, K // 32)).astype(np.uint8)
        eb = rng.integers(136, 141, size=(N, K // 32)).astype(np.uint8)
    else:                 # 448 * 2^119 < bf16 max; sums <= 346: |y| < 2^118
        ea = rng.integers(244, 247, size=(M, K // 32)).astype(np.uint8)
        eb = rng.integers(96, 101, size=(N, K // 32)).astype(np.uint8)
    for x, ex, w, ew in ((a, ea, b, eb), (b, eb, a, ea)):
        y = F.mxfp8_gemm(*[torch.from_numpy(v).to(DEV) for v in (x, ex, w, ew)])
        torch.cuda.synchronize()
        yr, bnd = orc.mx_gemm(x, ex, w, ew)
        assert np.all(np.isfinite(yr)) and np.all(bnd > 0)
        assert_parity(_np(y), yr, bnd, False, f"mx scale bytes at the {edge} edge")


def _mx_codes(rng, rows, K):
    c = rng.integers(0, 0x7F, size=(rows, K)).astype(np.uint8)      # 0x7F is NaN
    return c | (rng.integers(0, 2, size=(rows, K)).astype(np.uint8) << 7)


@pytest.mark.parametrize("edge", ["low", "high"])
@pytest.mark.parametrize("M,N", [(128, 128), (2048, 256)])
def test_mx_gemm_exact_outside_the_fold_range(F, orc, edge, M, N):
    """Scale bytes 0..9 or 247..254 on one operand (every tile takes the
    exact per-32-block path), the other operand's bytes chosen so every
    product and sum stays in fp32's normal range; each operand in each role,
    on the 128 x 128 and the 256 x 256 tile shapes."""
    rng = np.random.default_rng(31 + (edge == "high") + M)
    K = 256
    a, b = _mx_codes(rng, M, K), _mx_codes(rng, N, K)
    if edge == "low":     # products >= 2^(0 + 146 - 272) = 2^-126
        ea = rng.integers(0, 10, size=(M, K // 32)).astype(np.uint8)
        eb = rng.integers(146, 234, size=(N, K // 32)).astype(np.uint8)
    else:                 # products <= 2^(254 + 100 - 254 + 17.6); sums < 2^126
        ea = rng.integers(247, 255, size=(M, K // 32)).astype(np.uint8)
        eb = rng.integers(26, 101, size=(N, K // 32)).astype(np.uint8)
    cases = [(a, ea, b, eb)] + ([(b, eb, a, ea)] if M == N else [])
    for x, ex, w, ew in cases:
        y = F.mxfp8_gemm(*[torch.from_numpy(v).to(DEV) for v in (x, ex, w, ew)])
        torch.cuda.synchronize()
        yr, bnd = orc.mx_gemm(x, ex, w, ew)
        assert np.all(np.isfinite(yr)) and np.all(bnd > 0)
        assert_parity(_np(y), yr, bnd, False, f"mx scale bytes beyond the {edge} fold edge, {x.shape[0]}x{w.shape[0]}")


def test_mx_gemm_exact_and_folded_tiles_in_one_launch(F, orc):
    """Out-of-range bytes in a few rows and columns only: the tiles holding
    them take the exact path (mixing in-range and out-of-range rows), the
    others the folded path, in the same launch (256 x 256 tiles)."""
    rng = np.random.default_rng(40)
    M, N, K = 2048, 512, 384
    a, b = _mx_codes(rng, M, K), _mx_codes(rng, N, K)
    ea = rng.integers(120, 135, size=(M, K // 32)).astype(np.uint8)
    eb = rng.integers(146, 160, size=(N, K // 32)).astype(np.uint8)
    ea[300:304, 5] = rng.integers(0, 10, size=4)          # tile row 1
    ea[1800, :] = 3                                       # tile row 7
    eb[260, 11] = 8                                       # tile column 1, with in-range A rows
    y = F.mxfp8_gemm(*[torch.from_numpy(v).to(DEV) for v in (a, ea, b, eb)])
    torch.cuda.synchronize()
    yr, bnd = orc.mx_gemm(a, ea, b, eb)
    assert_parity(_np(y), yr, bnd, False, "mx with exact and folded tiles")


# ---- MoE combine ---------------------------------------------------------------
def _combine_check(F, orc, y, tr, gates, out_dtype, what):
    out = F.fp8_moe_combine(y, tr, gates, out_dtype)
    torch.cuda.synchronize()
    ref, bnd = orc.moe_combine(y.view(torch.int16).cpu().numpy().view(np.uint16),
                               tr.cpu().numpy(), gates.cpu().numpy())
    k = tr.shape[1]
    # fp32 accumulation of k exact products: at most k roundings of 2^-24
    return assert_parity(_np(out), ref, bnd, out_dtype == torch.bfloat16, what, rel=k * 2.0 ** -24)


@pytest.mark.parametrize("T,E,k,N", [(64, 8, 4, 256), (1, 4, 1, 8), (37, 16, 8, 136), (300, 64, 6, 1024)])
def test_moe_combine_small(F, orc, T, E, k, N):
    r = W.routing_full(T, E, k, 1.0, W.gen(T + N))
    R = T * k
    y = torch.randn(R, N, generator=W.gen(k), dtype=torch.float32).to(torch.bfloat16).to(DEV)
    tr, g = r["token_rows"].to(DEV), r["gates"].to(DEV)
    _combine_check(F, orc, y, tr, g, torch.float32, f"combine f32 {T}x{k}x{N}")
    _combine_check(F, orc, y, tr, g, torch.bfloat16, f"combine bf16 {T}x{k}x{N}")


def test_moe_forward_full(F, orc):
    """The whole expert projection at 4096 tokens x 256 experts (top-8): the
    routed rows are checked on sampled rows against the oracle's grouped
    GEMM, and every token's combine against the oracle's combine of them."""
    case = W.moe_case(device=DEV)
    r = W.routing_full(4096, 256, 8, 1.0, W.gen(4, "cpu"))
    assert torch.equal(r["row_index"], case.row_index)
    E, N, K = case.w.shape
    wq = torch.empty(E, N, K, dtype=torch.uint8, device=DEV)
    ws = torch.empty(E, N // 128, K // 128, dtype=torch.float32, device=DEV)
    for e in range(E):
        F.fp8_weight_quant(case.w[e], "fp32", q=wq[e], scales=ws[e])
    tr, g = r["token_rows"].to(DEV), r["gates"].to(DEV)
    out, y = F.moe_forward(case.x, case.row_index.to(DEV), case.offs.to(DEV), tr, g, wq, ws)
    torch.cuda.synchronize()
    worst = _combine_check(F, orc, y, tr, g, torch.bfloat16, "moe combine 4096x2048")
    # the routed rows of two tokens, against the oracle GEMM
    rows = sorted(set(r["token_rows"][0].tolist()) | set(r["token_rows"][4095].tolist()))
    offs = case.offs.numpy()
    toks = sorted({int(case.row_index[q]) for q in rows})
    oa_full = np.zeros((case.x.shape[0], K), np.uint8)
    osa_full = np.ones((case.x.shape[0], K // 128), np.float32)
    oa, osa = orc.act_quant(W.bits(case.x[torch.as_tensor(toks, device=case.x.device)]), 128, 0)
    oa_full[toks], osa_full[toks] = oa, osa
    wl, sl = [None] * E, [None] * E
    for e in sorted({int(np.searchsorted(offs, q, side="right") - 1) for q in rows}):
        wl[e], sl[e] = orc.weight_quant(W.bits(case.w[e]), 0)
    yr, bnd = orc.grouped_gemm(oa_full, osa_full, case.row_index.numpy(), offs, wl, sl, rows=np.asarray(rows))
    assert_parity(_np(y[torch.as_tensor(rows, device=DEV)]), yr, bnd, True, "moe routed rows")
    print(f"moe combine worst {worst:.3g}")


def test_grouped_max_experts(F, orc):
    """1024 experts (the entry point's maximum), almost all empty: one large
    expert, a few short ones, the rest with no rows."""
    counts = [0] * 1024
    counts[0], counts[511], counts[512], counts[1023] = 5, 300, 17, 1
    case = _moe_counts_case(counts, T=96, N=128, K=256, seed=46)
    yg, yr, bnd = _moe_run(F, orc, case)
    assert_parity(yg, yr, bnd, True, "moe 1024 experts")


def test_gemms_with_activations_beyond_4gib(F, orc):
    """A 9000-row activation matrix with a 512 KiB row stride (4.7 GB):
    rows past 8192 lie beyond 2^32 bytes from its start, so the tile bases
    must be 64-bit.  Block-scaled and MX GEMMs, rows on both sides checked."""
    M, K, N, ld = 9000, 256, 256, 1 << 19
    g = W.gen(47)
    x = W.activations(M, K, 2, 20.0, g)
    w = W.weights(N, K, 0.02, g)
    big = torch.zeros(M * ld, dtype=torch.uint8, device=DEV)
    qa = big.view(M, ld)[:, :K]
    sa = torch.empty(M, K // 128, dtype=torch.float32, device=DEV)
    F.fp8_act_quant(x.to(DEV), 128, "fp32", q=qa, scales=sa)
    wq, ws = F.fp8_weight_quant(w.to(DEV), "fp32")
    y = F.fp8_block_gemm(qa, sa, wq, ws, torch.float32)
    torch.cuda.synchronize()
    rows = [0, 8191, 8192, 8960, M - 1]
    oa, osa = orc.act_quant(W.bits(x[rows]), 128, 0)
    ow, osw = orc.weight_quant(W.bits(w), 0)
    yr, bnd = orc.block_gemm(oa, osa, ow, osw)
    assert_parity(_np(y[rows]), yr, bnd, False, "block gemm, rows past 4 GiB")
    # MX: the same strided storage for 32-blocks with E8M0 bytes
    ea = torch.empty(M, K // 32, dtype=torch.uint8, device=DEV)
    F.fp8_act_quant(x.to(DEV), 32, "e8m0", q=qa, scales=ea)
    b = W.mx_operand(N, K, g)
    qb, eb = F.fp8_act_quant(b.to(DEV), 32, "e8m0")
    ym = F.mxfp8_gemm(qa, ea, qb, eb)
    torch.cuda.synchronize()
    oa, oea = orc.act_quant(W.bits(x[rows]), 32, 2)
    ob, oeb = orc.act_quant(W.bits(b), 32, 2)
    yr, bnd = orc.mx_gemm(oa, oea, ob, oeb)
    assert_parity(_np(ym[rows]), yr, bnd, False, "mx gemm, rows past 4 GiB")
    del big
    torch.cuda.empty_cache()


# ---- 1 .. 64 tokens on packed weights (weights streamed into registers) ----
@pytest.mark.parametrize("N,K", [(128, 256), (384, 512), (256, 768), (640, 1024), (128, 1280),
                                 (256, 1536), (384, 1792), (128, 2048), (256, 2560),
                                 (896, 768), (1792, 1024), (896, 2560)])
def test_block_gemm_register_streamed_decode(F, orc, N, K):
    """Packed weights with at most 64 tokens, a grid of at most one 128-row
    tile per CU and an even K-block count: one to eight and ten steps per K-split
    group (a main loop of three and a tail of one to four steps), one and
    two 32-token fragments with ragged last fragments, both scale formats
    and output types, grids of one to fourteen tiles; every output against
    the oracle."""
    c = W.decode_linear(K=K, N=N, seed=N + K)
    for fmt, out in (("ue8m0", torch.bfloat16), ("fp32", torch.float32)):
        fi = {"fp32": 0, "ue8m0": 1}[fmt]
        a, sa = F.fp8_act_quant(c.x[:64].to(DEV), 128, fmt)
        wq, ws = F.fp8_weight_quant(c.w.to(DEV), fmt)
        wp = F.fp8_weight_pack(wq)
        oa, osa = orc.act_quant(W.bits(c.x[:64]), 128, fi)
        ow, osw = orc.weight_quant(W.bits(c.w), fi)
        yr, bnd = orc.block_gemm(oa, osa, ow, osw)
        for M in (1, 2, 17, 31, 32, 33, 40, 63, 64):
            y = F.fp8_block_gemm_packed(a[:M], sa[:M], wp, ws, out)
            torch.cuda.synchronize()
            assert_parity(_np(y), yr[:M], bnd[:M], out == torch.bfloat16, f"{M}x{N}x{K} {fmt}")


@pytest.mark.parametrize("N,K", [(256, 1024), (28672, 8192)])
def test_register_streamed_decode_rows_equal_the_tiled_kernel(F, N, K):
    """Rows are independent, so y of M <= 64 tokens (the register-streamed
    kernel) must equal, bit for bit, the first M rows of the same GEMM over
    65 tokens (the 128 x 128 tiles in their K-split form), which compute
    every row with the same MFMA chains and folds."""
    c = W.decode_linear(device=DEV, K=K, N=N, seed=5)
    a, sa = F.fp8_act_quant(c.x[:65], 128, "ue8m0")
    wq, ws = F.fp8_weight_quant(c.w, "ue8m0")
    wp = F.fp8_weight_pack(wq)
    del c
    for out in (torch.bfloat16, torch.float32):
        ref = F.fp8_block_gemm_packed(a, sa, wp, ws, out)
        for M in (1, 8, 32, 33, 64):
            y = F.fp8_block_gemm_packed(a[:M], sa[:M], wp, ws, out)
            torch.cuda.synchronize()
            iv = torch.int16 if out == torch.bfloat16 else torch.int32
            assert torch.equal(y.view(iv), ref[:M].view(iv)), f"M {M} {out} {N}x{K}"


@pytest.mark.parametrize("M", [5, 30, 33, 64])
def test_register_streamed_decode_strided_operands(F, orc, M):
    """The register-streamed kernel on activation rows with a leading
    dimension above K (a column slice of a wider code matrix, whose bytes
    past K hold codes that must never be read) and an output that is a
    column slice of a wider y (bytes past N must stay untouched)."""
    N, K, extra = 384, 1024, 128
    c = W.decode_linear(K=K, N=N, seed=13 * M)
    a, sa = F.fp8_act_quant(c.x[:M].to(DEV), 128, "ue8m0")
    wq, ws = F.fp8_weight_quant(c.w.to(DEV), "ue8m0")
    wp = F.fp8_weight_pack(wq)
    wide = torch.full((M, K + extra), 0x7E, dtype=torch.uint8, device=DEV)
    wide[:, :K] = a
    ywide = torch.full((M, N + 64), -7.0, dtype=torch.bfloat16, device=DEV)
    y = F.fp8_block_gemm_packed(wide[:, :K], sa, wp, ws, torch.bfloat16, y=ywide[:, :N])
    torch.cuda.synchronize()
    assert y.stride(0) == N + 64
    assert torch.all(ywide[:, N:] == -7.0), "bytes past N written"
    oa, osa = orc.act_quant(W.bits(c.x[:M]), 128, 1)
    ow, osw = orc.weight_quant(W.bits(c.w), 1)
    yr, bnd = orc.block_gemm(oa, osa, ow, osw)
    assert_parity(_np(ywide[:, :N]), yr, bnd, True, f"strided M {M}")
    dense = F.fp8_block_gemm_packed(a, sa, wp, ws, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(dense.view(torch.int16), ywide[:, :N].contiguous().view(torch.int16)), f"strided vs dense M {M}"


@pytest.mark.parametrize("extra_tiles", [0, 1])
def test_register_streamed_decode_at_the_cu_count(F, orc, extra_tiles):
    """Packed weights with N / 128 equal to the CU count take the
    register-streamed kernel (one tile per CU); one tile more and the GEMM
    falls back to the streaming kernel.  Both sides against the oracle on
    sampled token rows x every column, 1 and 40 tokens."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N, K = 128 * (cus + extra_tiles), 256
    c = W.decode_linear(K=K, N=N, seed=17 + extra_tiles)
    a, sa = F.fp8_act_quant(c.x[:40].to(DEV), 128, "ue8m0")
    wq, ws = F.fp8_weight_quant(c.w.to(DEV), "ue8m0")
    wp = F.fp8_weight_pack(wq)
    ow, osw = orc.weight_quant(W.bits(c.w), 1)
    for M in (1, 40):
        y = F.fp8_block_gemm_packed(a[:M], sa[:M], wp, ws, torch.bfloat16)
        torch.cuda.synchronize()
        rows = sorted({0, M - 1})
        oa, osa = orc.act_quant(W.bits(c.x[rows]), 128, 1)
        yr, bnd = orc.block_gemm(oa, osa, ow, osw)
        assert_parity(_np(y[rows]), yr, bnd, True, f"M {M} N {N}")


@pytest.mark.parametrize("M,N,K", [(256, 384, 640), (2048, 2304, 1024), (128, 1024, 1024)])
def test_gemm_probe_computes_tile_zero_everywhere(F, M, N, K):
    """fp8b_gemm_probe (a measurement aid): every workgroup reads output tile
    (0, 0)'s operands, so tile (0, 0) of its output is the packed GEMM's own
    tile bit for bit, and every other tile is a copy of it.  The first two
    shapes run the plain 128 x 128 tiles (an odd K-block count; more tiles
    than CUs), the third their K-split form (eight tiles, eight K blocks),
    as the GEMM does."""
    c = W.prefill_linear(device=DEV, M=M, K=K, N=N, seed=M + N)
    a, sa = F.fp8_act_quant(c.x, 128, "fp32")
    wq, ws = F.fp8_weight_quant(c.w, "fp32")
    wp = F.fp8_weight_pack(wq)
    y = F.fp8_block_gemm_packed(a, sa, wp, ws, torch.bfloat16)
    yp = F.fp8b_gemm_probe(F.GEMM_PROBE_TILE0, a, sa, wp, ws)
    torch.cuda.synchronize()
    t0 = y[:128, :128].view(torch.int16)
    tiles = yp.view(torch.int16).reshape(M // 128, 128, N // 128, 128).permute(0, 2, 1, 3)
    assert torch.equal(tiles[0, 0], t0)
    assert torch.equal(tiles, t0.expand_as(tiles))
