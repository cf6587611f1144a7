#!/usr/bin/env python3
"""Benchmark of the W8A8 block-scaled FP8 linear-layer hot path on one MI355X.

Headline ("step"): one prefill-shaped linear layer, 4096 tokens x 7168 ->
18432, i.e. fp8_act_quant (per token, per 128 channels, fp32 scales) on the
bf16 activations followed by fp8_block_gemm_packed against E4M3 weights
with 128x128 fp32 block scales, bf16 output.  Weights are quantised and
put in the packed layout (fp8_weight_pack) once, outside the timed region
(offline in the method; the layout changes no result).  Inputs are seeded
synthetic tensors already resident in HBM.

value = 2*M*N*K / (time per step), i.e. block-scaled FP8 GEMM TFLOP/s
including act_quant.

The same JSON line carries
  roofline      for the dominant kernel (the block GEMM), its average
                launch duration measured with events on its stream;
                and, under measured_ceilings, what torch's bf16 GEMM
                (hipBLASLt) reaches on the same shape, what the library's
                MFMA-only loop reaches (bf16 16x16x32 and FP8 16x16x128),
                and what a 1 GiB device copy reaches on this GPU;
  cpu_baseline  the CPU oracle timed on a bounded sample of the same
                workload (rank 0, one GPU only), on all host threads and on
                one;
  legs          the other rows of the hot path measured the same way:
                the headline GEMM on row-major weights, decode-shaped GEMMs
                (M = 1, 8, 32, 128; K 8192 -> N 28672, ue8m0 scales, weights
                rotated over two copies so the 256 MB last-level cache
                cannot serve them; packed and row-major), the MXFP8 GEMM
                (8192^3), the grouped MoE GEMM (256 experts, 4096 tokens,
                top-8, N 2048, K 7168) with the combine and the whole layer,
                weight dequant, KV-cache quant/dequant and delayed scaling,
                plus act_quant bandwidth.
"""
import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA (the instruction the products run on)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=50,
                   help="untimed steps first; under sustained MFMA load the clock dips for the "
                        "first ~25 ms and settles after ~50 steps")
    p.add_argument("--settle-ms", type=float, default=150.0,
                   help="after the warm-up steps, keep stepping until this much time has passed "
                        "before the timed steps (the clock settles within ~50 ms of MFMA load)")
    p.add_argument("--no-legs", action="store_true", help="time the headline step only")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the measured ceilings (torch bf16 GEMM on the same shape, 1 GiB device copy)")
    p.add_argument("--cpu-rows", type=int, default=0, help="oracle sample rows (0 = auto)")
    p.add_argument("--only", default="", help="run one leg only: prefill|decode|mx|moe|dequant|kv|delayed")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (a kernel of known traffic, for "
                        "scaling profiler byte counters)")
    return p.parse_args()


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace collapsed, so that
    editing a comment does not count as changing a kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_hash():
    """Hash of the kernel sources' code (comments and layout ignored)."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "fp8_block_scaled_02_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(name):
    """HBM bytes of one launch from the committed rocprofv3 counter summary
    (profiles/traffic_<name>.txt, "key: value" lines), or None if it is
    missing or was taken on different kernel sources."""
    path = os.path.join(HERE, "profiles", f"traffic_{name}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_hash") != kernel_hash():
        return None
    try:
        return int(float(rec["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def warm(torch, fn, ms=100.0):
    """Calls fn() until about ms of device work has run.  Under sustained
    MFMA load the chip's clock first overshoots downward (a ~1 ms kernel
    runs ~20% slower around its fifth call) and settles within ~50 ms, so
    millisecond-long kernels are timed only after this."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    once = max(time.perf_counter() - t0, 1e-6)
    for _ in range(max(1, int(ms * 1e-3 / once))):
        fn()
    torch.cuda.synchronize()


def timed(torch, fn, iters, warm_ms=100.0):
    """Average device time of fn() over iters launches (events on the
    current stream, which is where the library enqueues), after warm()."""
    warm(torch, fn, warm_ms)
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(iters):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters * 1e-3


def interleaved(torch, fns, rounds=4, iters=10):
    """Median per-launch device time of each fn over `rounds` alternating
    rounds of `iters` launches (A B A B ...), after a shared warm-up: the
    kernels compared see the same clock state."""
    warm(torch, lambda: [f() for f in fns], 100.0)
    s = torch.cuda.current_stream()
    times = [[] for _ in fns]
    for _ in range(rounds):
        for i, f in enumerate(fns):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(iters):
                f()
            e1.record(s)
            e1.synchronize()
            times[i].append(e0.elapsed_time(e1) / iters * 1e-3)
    return [statistics.median(t) for t in times]


def timed_graph(torch, fn, iters):
    """Average device time of fn() for kernels short enough that host-side
    argument marshalling between launches would leave the GPU idle: iters
    calls are captured into one HIP graph (the library's kernels make no
    allocations, memsets or synchronisations), which is replayed once
    untimed and once between events."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(iters):
            fn()
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    g.replay()
    e1.record(s)
    e1.synchronize()
    t = e0.elapsed_time(e1) / iters * 1e-3
    del g
    return t


def mfma_loop_rates(torch, F, dev):
    """TFLOP/s of the library's MFMA-only loop (fp8b_mfma_loop): seeded
    register operands, four waves per SIMD, ~0.3-0.6 ms per launch, timed
    after the same settling as the step.  bf16 16x16x32 is the instruction
    the GEMMs' products run on; FP8 16x16x128 is shown beside it."""
    g = torch.Generator().manual_seed(5)
    ops = {"bf16": torch.randn(64, 128, generator=g).to(torch.bfloat16).view(torch.int16).view(torch.int32),
           "fp8": (torch.randn(64, 256, generator=g) * 4).to(torch.float8_e4m3fn).view(torch.uint8)
           .view(torch.int32)}
    wg = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(wg, 256, dtype=torch.float32, device=dev)
    rates = {}
    for name, kind, iters in (("bf16", F.MFMA_BF16_16X16X32, 8192), ("fp8", F.MFMA_FP8_16X16X128, 2048)):
        w = ops[name].contiguous().to(dev)
        t = timed(torch, lambda w=w, kind=kind, iters=iters: F.fp8b_mfma_loop(kind, w, iters, wg, out), 20)
        rates[name] = wg * 4 * iters * 2 * F.MFMA_LOOP_FLOPS[kind] / t / 1e12
    return rates


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import fp8_block_scaled_02_amd as F
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    dev = "cuda"
    legs = {}

    # ---- headline: prefill linear ------------------------------------------------
    c = W.prefill_linear(device=dev)
    M, K = c.x.shape
    N = c.w.shape[0]
    wq_rm, ws = F.fp8_weight_quant(c.w, "fp32")
    wq = F.fp8_weight_pack(wq_rm)        # offline, like the quantisation: the packed layout
    del wq_rm
    x = c.x
    a = torch.empty(M, K, dtype=torch.uint8, device=dev)
    sa = torch.empty(M, K // 128, dtype=torch.float32, device=dev)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

    def aq():
        F.fp8_act_quant(x, 128, "fp32", q=a, scales=sa)

    def gemm():
        F.fp8_block_gemm_packed(a, sa, wq, ws, torch.bfloat16, y=y)

    # The step is two plain launches; each GPU step (~1 ms) is far longer
    # than the host's enqueue, so the queue never runs dry (a captured HIP
    # graph of the step measured the same).  In every timed step the block
    # GEMM is bracketed by events on the library's stream, so its average
    # duration comes from the timed region itself.
    def step():
        aq()
        gemm()

    for _ in range(args.warmup):
        step()
    # Then settle on time, not on a step count: under sustained MFMA load the
    # clock dips for the first ~25 ms and settles after ~50 ms, so steps
    # keep running until args.settle_ms of device time has passed (whatever
    # --warmup was), and the timed steps start from the settled clock.
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    settle_steps = 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(10):
            step()
        settle_steps += 10
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for es, e0, e1 in ev:
        es.record(stream)
        aq()
        e0.record(stream)
        gemm()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    flops = 2.0 * M * N * K
    value = flops / (wall / args.steps) / 1e12
    gemm_ms = [e0.elapsed_time(e1) for _, e0, e1 in ev]
    step_ms = [es.elapsed_time(e1) for es, _, e1 in ev]
    t_gemm = sum(gemm_ms) / len(gemm_ms) * 1e-3
    t_gemm_median = statistics.median(gemm_ms) * 1e-3

    # act_quant alone: 17 us, so timed back to back from a captured graph;
    # beside it, the same launch with the arithmetic removed (the same bytes
    # moved) and an empty launch of the same grid (fp8b_stream_probe)
    t_aq = timed_graph(torch, aq, max(args.steps, 10))
    t_copy = timed_graph(torch, lambda: F.fp8b_stream_probe(F.PROBE_COPY, x, a, sa), max(args.steps, 10))
    t_empty = timed_graph(torch, lambda: F.fp8b_stream_probe(F.PROBE_EMPTY, x, a, sa), max(args.steps, 10))
    aq()                                   # restore the step's codes and scales
    # the same GEMM kernel with every tile reading tile (0, 0)'s operands
    # (fp8b_gemm_probe: the same work, operands resident in L2), interleaved
    # with the GEMM itself: what the operand traffic beyond L2 costs
    y_probe = torch.empty_like(y)
    t_g2, t_probe = interleaved(torch, [gemm, lambda: F.fp8b_gemm_probe(F.GEMM_PROBE_TILE0, a, sa, wq, ws,
                                                                         y=y_probe)])
    del y_probe
    gemm_bytes = M * K + N * K + M * (K // 128) * 4 + (N // 128) * (K // 128) * 4 + M * N * 2
    aq_bytes = M * K * 2 + M * K + M * (K // 128) * 4
    achieved = flops / t_gemm / 1e12
    traffic = load_traffic("block_gemm_prefill")
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
                "kernel": "block_gemm_kernel", "avg_launch_us": round(t_gemm * 1e6, 2),
                "median_launch_us": round(t_gemm_median * 1e6, 2),
                "achieved_at_median": round(flops / t_gemm_median / 1e12, 1),
                "algorithmic_bytes": gemm_bytes,
                "frac_of_bf16_dense_peak": round(achieved / PEAK_BF16_TFLOPS, 4)}
    legs["prefill"] = {"act_quant_us": round(t_aq * 1e6, 2),
                       "act_quant_GBps": round(aq_bytes / t_aq / 1e9, 1),
                       "act_quant_hbm_frac": round(aq_bytes / t_aq / 1e9 / PEAK_HBM_GBS, 4),
                       "act_quant_probe": {"copy_us": round(t_copy * 1e6, 2),
                                           "copy_GBps": round(aq_bytes / t_copy / 1e9, 1),
                                           "empty_us": round(t_empty * 1e6, 2),
                                           "act_quant_vs_copy": round(t_copy / t_aq, 4),
                                           "note": "same grid, loads and stores as act_quant: copy moves the "
                                                   "same bytes with no arithmetic, empty returns at once"},
                       "gemm_us": round(t_gemm * 1e6, 2), "gemm_TFLOPs": round(achieved, 1),
                       "gemm_l2_probe": {"gemm_us": round(t_g2 * 1e6, 2), "probe_us": round(t_probe * 1e6, 2),
                                         "probe_vs_gemm": round(t_probe / t_g2, 4),
                                         "note": "interleaved medians: the GEMM, and the same kernel with every "
                                                 "tile reading tile (0, 0)'s operands (no operand traffic "
                                                 "beyond L2)"},
                       "weights": "packed layout (fp8_weight_pack, offline)"}
    del c

    # ---- CPU baseline: the oracle on a bounded sample -----------------------------
    cpu = None
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle as O
        sys.path.insert(0, os.path.join(HERE, "tests"))
        import parity as P
        xb = W.bits(x)
        ow, osw = O.weight_quant(W.bits(W.prefill_linear(device=dev).w), 0)   # offline, untimed
        rows = args.cpu_rows or 32
        t0 = time.perf_counter()
        oa, osa = O.act_quant(xb[:rows], 128, 0)
        O.block_gemm(oa, osa, ow, osw)
        t_cpu = time.perf_counter() - t0
        if not args.cpu_rows and t_cpu < 8.0:      # grow the sample toward ~10-30 s
            rows = int(min(M, max(rows, rows * 12.0 / max(t_cpu, 1e-3))))
            t0 = time.perf_counter()
            oa, osa = O.act_quant(xb[:rows], 128, 0)
            O.block_gemm(oa, osa, ow, osw)
            t_cpu = time.perf_counter() - t0
        cpu = {"value": round(2.0 * rows * N * K / t_cpu / 1e12, 6), "unit": "TFLOP/s",
               "cores": O.num_threads(), "kind": "oracle",
               "sample": f"act_quant + block GEMM of the first {rows} of {M} token rows "
                         f"(all {N} outputs, K {K}), {t_cpu:.1f} s"}
        # the same oracle rows against the timed step's output (outside the
        # timed region): worst |err| / allowed over every sampled output
        yr, bnd = O.block_gemm(oa, osa, ow, osw)
        yg = y[:rows].float().cpu().numpy().astype(np.float64)
        ok, worst = P.check_bf16(yg, yr, bnd)
        cpu["parity_prefill"] = {"worst_err_over_allowed": round(worst, 5), "outputs": int(yg.size),
                                 "all_within": bool(ok.all())}
        del yr, bnd, yg
        # the same oracle on one thread, over a sample sized to a few seconds
        all_threads = O.num_threads()
        rows1 = max(1, min(rows, int(rows * 4.0 / max(t_cpu * all_threads, 1e-3))))
        O.set_num_threads(1)
        try:
            t0 = time.perf_counter()
            oa, osa = O.act_quant(xb[:rows1], 128, 0)
            O.block_gemm(oa, osa, ow, osw)
            t_one = time.perf_counter() - t0
        finally:
            O.set_num_threads(all_threads)
        cpu["single_thread"] = {"value": round(2.0 * rows1 * N * K / t_one / 1e12, 6), "unit": "TFLOP/s",
                                "sample": f"first {rows1} token rows, {t_one:.1f} s"}
        del ow, osw, xb

    # ---- measured ceilings on this GPU, beside the spec peaks ------------------------
    # torch's bf16 GEMM (hipBLASLt) on the same shape: what a tuned library reaches
    # on the MFMA instruction the products run on; and a 1 GiB device copy.
    ceilings = None
    if not args.no_ceilings:
        wb = W.prefill_linear(device=dev).w                            # bf16 [N, K]
        mm = lambda: torch.nn.functional.linear(x, wb)                  # noqa: E731
        t_mm = timed(torch, mm, max(args.steps, 10))    # after the same settling as the step
        del wb
        torch.cuda.empty_cache()
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        t_cp = timed(torch, lambda: dst.copy_(src), 10)
        del src, dst
        torch.cuda.empty_cache()
        copy_gbs = 2.0 * (1 << 30) / t_cp / 1e9
        mm_tflops = flops / t_mm / 1e12
        loops = mfma_loop_rates(torch, F, dev)
        ceilings = {"bf16_gemm_torch_us": round(t_mm * 1e6, 2), "bf16_gemm_torch_TFLOPs": round(mm_tflops, 1),
                    "block_gemm_vs_bf16_gemm_torch": round(achieved / mm_tflops, 4),
                    "mfma_loop_bf16_16x16x32_TFLOPs": round(loops["bf16"], 1),
                    "mfma_loop_fp8_16x16x128_TFLOPs": round(loops["fp8"], 1),
                    "block_gemm_vs_mfma_loop_bf16": round(achieved / loops["bf16"], 4),
                    "device_copy_GBps": round(copy_gbs, 1),
                    "act_quant_vs_device_copy": round(aq_bytes / t_aq / 1e9 / copy_gbs, 4)}
        roofline["measured_ceilings"] = ceilings

    del x, a, sa, y, wq, ws
    torch.cuda.empty_cache()

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    if not args.no_legs:
        legs.update(run_legs(torch, F, W, dev, args.only))

    if cpu is not None and not args.no_legs and not args.only:
        cpu["configs"] = oracle_configs(torch, F, W, O, P, dev)

    out = {
        "metric": "block-scaled FP8 GEMM TFLOPS (incl. act_quant) and % of MI355X FP8 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms_median": round(statistics.median(step_ms), 4),
        "settle": {"ms": round(settle_ms, 1), "steps": settle_steps,
                   "note": "untimed steps after the warm-up, until the clock settled"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "compute": "E4M3 codes widened exactly to bf16 in registers, bf16 MFMA, fp32 accumulation "
                   "and per-128-block fp32 rescale",
        "data": "synthetic",
        "step_launch": "eager (act_quant and GEMM launches; GEMM bracketed by events)",
        "pct_of_fp8_peak": round(100.0 * value / PEAK_FP8_TFLOPS, 2),
        "config": {"workload": "prefill linear: act_quant (per token per 128, fp32 scales) + "
                               "block-scaled FP8 GEMM (128x128 fp32 weight scales, weights in the "
                               "packed layout), bf16 out",
                   "M": M, "K": K, "N": N},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "legs": legs,
    }
    print(json.dumps(out), flush=True)


def oracle_configs(torch, F, W, O, P, dev):
    """The oracle on a bounded sample of every workload, timed on the host
    cores, and compared with the GPU's output for the same sample (run once
    more, outside every timed region): worst |err| / allowed per config
    (1.0 is the edge of the tolerance; codes are compared bit for bit
    separately in the tests).  The prefill case is covered by the headline's
    own sample above."""
    import numpy as np
    res = {}
    cores = O.num_threads()

    def rec(name, yg, yr, bnd, bf16, macs, t, sample):
        ok, worst = (P.check_bf16 if bf16 else P.check_f32)(yg, yr, bnd)
        res[name] = {"worst_err_over_allowed": round(worst, 5), "all_within": bool(ok.all()),
                     "outputs": int(np.asarray(yg).size),
                     "oracle_s": round(t, 3), "oracle_TFLOPs": round(2.0 * macs / max(t, 1e-9) / 1e12, 6),
                     "cores": cores, "sample": sample}

    # tiny linear, 16 x 512 -> 256, fp32 out: the whole output
    c = W.tiny_linear()
    a, sa = F.fp8_act_quant(c.x.to(dev), 128, "fp32")
    wq, ws = F.fp8_weight_quant(c.w.to(dev), "fp32")
    yg = F.fp8_block_gemm(a, sa, wq, ws, torch.float32).cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    oa, osa = O.act_quant(W.bits(c.x), 128, 0)
    ow, osw = O.weight_quant(W.bits(c.w), 0)
    yr, bnd = O.block_gemm(oa, osa, ow, osw)
    rec("tiny", yg, yr, bnd, False, 16 * 512 * 256, time.perf_counter() - t0, "all 16 x 256 outputs")

    # decode, 8192 -> 28672, ue8m0, bf16 out: every token row, weight rows
    # 0..255 and the last 256 (whole 128-row scale blocks)
    c = W.decode_linear(device=dev)
    N, K = c.w.shape
    wq, ws = F.fp8_weight_quant(c.w, "ue8m0")
    wp = F.fp8_weight_pack(wq)
    cols = np.r_[0:256, N - 256:N]
    t0 = time.perf_counter()
    ow, osw = O.weight_quant(W.bits(c.w[torch.as_tensor(cols, device=dev)]), 1)
    t_w = time.perf_counter() - t0
    for M in (1, 8, 32, 128):
        x = c.x[:M].contiguous()
        a, sa = F.fp8_act_quant(x, 128, "ue8m0")
        yg = F.fp8_block_gemm_packed(a, sa, wp, ws, torch.bfloat16)[:, torch.as_tensor(cols, device=dev)]
        yg = yg.float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        oa, osa = O.act_quant(W.bits(x), 128, 1)
        yr, bnd = O.block_gemm(oa, osa, ow, osw)
        rec(f"decode_M{M}", yg, yr, bnd, True, M * len(cols) * K, time.perf_counter() - t0 + t_w,
            f"all {M} token rows x weight rows 0-255 and {N - 256}-{N - 1} (packed weights)")
    del c, wq, ws, wp
    torch.cuda.empty_cache()

    # MXFP8 8192^3, fp32 out: 8 rows spread over A, every column
    A, B = W.mx_case(device=dev)
    M = A.shape[0]
    qa, ea = F.fp8_act_quant(A, 32, "e8m0")
    qb, eb = F.fp8_act_quant(B, 32, "e8m0")
    rows = np.linspace(0, M - 1, 8).astype(np.int64)
    yg = F.mxfp8_gemm(qa, ea, qb, eb)[torch.as_tensor(rows, device=dev)].cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    oa, oea = O.act_quant(W.bits(A[torch.as_tensor(rows, device=dev)]), 32, 2)
    ob, oeb = O.act_quant(W.bits(B), 32, 2)
    yr, bnd = O.mx_gemm(oa, oea, ob, oeb)
    rec("mx_8192", yg, yr, bnd, False, len(rows) * B.shape[0] * A.shape[1], time.perf_counter() - t0,
        f"token rows {rows.tolist()} x all {B.shape[0]} columns (quant of B included)")
    del A, B, qa, ea, qb, eb
    torch.cuda.empty_cache()

    # grouped MoE, 256 experts: routed rows of the largest expert (first,
    # last, one past a tile) and of three single-row experts
    case = W.moe_case(device=dev)
    E, N, K = case.w.shape
    a, sa = F.fp8_act_quant(case.x, 128, "fp32")
    wq = torch.empty(E, N, K, dtype=torch.uint8, device=dev)
    ws = torch.empty(E, N // 128, K // 128, dtype=torch.float32, device=dev)
    for e in range(E):
        F.fp8_weight_quant(case.w[e], "fp32", q=wq[e], scales=ws[e])
    wp = F.fp8_weight_pack(wq)
    del wq
    ri, offs = case.row_index.to(dev), case.offs.to(dev)
    yfull = F.fp8_grouped_gemm_packed(a, sa, ri, offs, wp, ws, torch.bfloat16)
    offs_np = case.offs.numpy()
    counts = offs_np[1:] - offs_np[:-1]
    big = int(np.argmax(counts))
    small = [e for e in range(E) if counts[e] == 1][:3]
    rows = sorted({int(offs_np[big]), int(offs_np[big + 1]) - 1, int(offs_np[big]) + 130}
                  | {int(offs_np[e]) for e in small})
    yg = yfull[torch.as_tensor(rows, device=dev)].float().cpu().numpy().astype(np.float64)
    del yfull, wp, ws, a, sa
    t0 = time.perf_counter()
    experts = sorted({int(np.searchsorted(offs_np, r, side="right") - 1) for r in rows})
    toks = sorted({int(case.row_index[r]) for r in rows})
    oa_full = np.zeros((case.x.shape[0], K), np.uint8)
    osa_full = np.ones((case.x.shape[0], K // 128), np.float32)
    oa, osa = O.act_quant(W.bits(case.x[torch.as_tensor(toks, device=dev)]), 128, 0)
    oa_full[toks], osa_full[toks] = oa, osa
    wl, sl = [None] * E, [None] * E
    for e in experts:
        wl[e], sl[e] = O.weight_quant(W.bits(case.w[e]), 0)
    yr, bnd = O.grouped_gemm(oa_full, osa_full, case.row_index.numpy(), offs_np, wl, sl, rows=rows)
    rec("moe_256x8", yg, yr, bnd, True, len(rows) * N * K, time.perf_counter() - t0,
        f"routed rows {rows} (experts {experts}, weights quantised by the oracle)")
    del case
    torch.cuda.empty_cache()
    return res


def run_legs(torch, F, W, dev, only=""):
    legs = {}
    iters = 20
    if only in ("", "prefill"):
        # the headline GEMM on row-major weight codes, for comparison
        c = W.prefill_linear(device=dev)
        M, K = c.x.shape
        N = c.w.shape[0]
        a, sa = F.fp8_act_quant(c.x, 128, "fp32")
        wq, ws = F.fp8_weight_quant(c.w, "fp32")
        del c
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        t = timed(torch, lambda: F.fp8_block_gemm(a, sa, wq, ws, torch.bfloat16, y=y), iters)
        legs["prefill_row_major_weights"] = {"gemm_us": round(t * 1e6, 2),
                                             "TFLOPs": round(2.0 * M * N * K / t / 1e12, 1)}
        del a, sa, wq, ws, y
        torch.cuda.empty_cache()
    if only in ("", "decode"):
        c = W.decode_linear(device=dev)
        K, N = c.x.shape[1], c.w.shape[0]
        copies = [F.fp8_weight_quant(c.w, "ue8m0") for _ in range(2)]   # > 256 MB together
        packed = [(F.fp8_weight_pack(wq), ws) for wq, ws in copies]
        del c.w
        dec = {}
        for M in (1, 8, 32, 128):
            a, sa = F.fp8_act_quant(c.x[:M].contiguous(), 128, "ue8m0")
            y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            nbytes = N * K + (N // 128) * (K // 128) * 4 + M * K + M * (K // 128) * 4 + M * N * 2
            res = {}
            for layout, ws_list, gemm in (("packed", packed, F.fp8_block_gemm_packed),
                                          ("row_major", copies, F.fp8_block_gemm)):
                st = [0]

                def g():
                    wq, ws = ws_list[st[0] & 1]
                    st[0] += 1
                    gemm(a, sa, wq, ws, torch.bfloat16, y=y)
                for _ in range(4):
                    g()
                res[layout] = timed_graph(torch, g, iters)
            t = res["packed"]
            dec[f"M{M}"] = {"us": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1),
                            "hbm_frac": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4),
                            "TFLOPs": round(2.0 * M * N * K / t / 1e12, 2),
                            "row_major_us": round(res["row_major"] * 1e6, 2),
                            "row_major_GBps": round(nbytes / res["row_major"] / 1e9, 1)}
            if M % 128 == 0:
                # the same tiles with every one reading tile (0, 0)'s operands
                # (fp8b_gemm_probe): what the weight stream from HBM costs
                wq0, ws0 = packed[0]
                yp = torch.empty_like(y)
                t_p = timed_graph(torch, lambda: F.fp8b_gemm_probe(F.GEMM_PROBE_TILE0, a, sa, wq0, ws0, y=yp),
                                  iters)
                dec[f"M{M}"]["l2_probe_us"] = round(t_p * 1e6, 2)
                del yp
        dec["weights"] = "packed layout (fp8_weight_pack); row_major_* = the same GEMM on row-major codes"
        legs["decode"] = dec
        del copies, packed, c
        torch.cuda.empty_cache()
    if only in ("", "mx"):
        A, B = W.mx_case(device=dev)
        M, K = A.shape
        N = B.shape[0]
        qa, ea = F.fp8_act_quant(A, 32, "e8m0")
        qb, eb = F.fp8_act_quant(B, 32, "e8m0")
        y = torch.empty(M, N, dtype=torch.float32, device=dev)
        t_q = timed_graph(torch, lambda: F.fp8_act_quant(A, 32, "e8m0", q=qa, scales=ea), iters)
        t = timed(torch, lambda: F.mxfp8_gemm(qa, ea, qb, eb, y=y), iters)
        qbytes = M * K * 3 + M * K // 32
        legs["mx"] = {"gemm_us": round(t * 1e6, 2), "TFLOPs": round(2.0 * M * N * K / t / 1e12, 1),
                      "frac_fp8_peak": round(2.0 * M * N * K / t / 1e12 / PEAK_FP8_TFLOPS, 4),
                      "act_quant32_us": round(t_q * 1e6, 2), "act_quant32_GBps": round(qbytes / t_q / 1e9, 1)}
        del A, B, qa, ea, qb, eb, y
        torch.cuda.empty_cache()
    if only in ("", "moe"):
        case = W.moe_case(device=dev)
        E, N, K = case.w.shape
        T = case.x.shape[0]
        a, sa = F.fp8_act_quant(case.x, 128, "fp32")
        wq = torch.empty(E, N, K, dtype=torch.uint8, device=dev)
        ws = torch.empty(E, N // 128, K // 128, dtype=torch.float32, device=dev)
        for e in range(E):
            F.fp8_weight_quant(case.w[e], "fp32", q=wq[e], scales=ws[e])
        del case.w
        torch.cuda.empty_cache()
        ri, offs = case.row_index.to(dev), case.offs.to(dev)
        R = ri.shape[0]
        y = torch.empty(R, N, dtype=torch.bfloat16, device=dev)
        t_rm = timed(torch, lambda: F.fp8_grouped_gemm(a, sa, ri, offs, wq, ws, torch.bfloat16, y=y), iters)
        wq = F.fp8_weight_pack(wq)          # the layer runs on packed expert weights
        torch.cuda.empty_cache()
        t = timed(torch, lambda: F.fp8_grouped_gemm_packed(a, sa, ri, offs, wq, ws, torch.bfloat16, y=y), iters)
        counts = (case.offs[1:] - case.offs[:-1])
        active = int((counts > 0).sum())
        nbytes = active * (N * K + (N // 128) * (K // 128) * 4) + T * (K + K // 128 * 4) + R * N * 2
        # the whole projection: act_quant, grouped GEMM, gate-weighted combine
        rt = W.routing_full(T, E, case.row_index.shape[0] // T, 1.0, W.gen(4, "cpu"))
        tr, gt = rt["token_rows"].to(dev), rt["gates"].to(dev)
        out = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
        t_c = timed_graph(torch, lambda: F.fp8_moe_combine(y, tr, gt, torch.bfloat16, out=out), iters)
        t_l = timed(torch, lambda: F.moe_forward(case.x, ri, offs, tr, gt, wq, ws, packed=True), iters)
        cbytes = R * N * 2 + T * N * 2 + R * 8
        legs["moe"] = {"us": round(t * 1e6, 2), "TFLOPs": round(2.0 * R * N * K / t / 1e12, 1),
                       "GBps": round(nbytes / t / 1e9, 1), "hbm_frac": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4),
                       "row_major_us": round(t_rm * 1e6, 2), "weights": "packed layout (fp8_weight_pack)",
                       "active_experts": active, "max_rows": int(counts.max()),
                       "combine_us": round(t_c * 1e6, 2), "combine_GBps": round(cbytes / t_c / 1e9, 1),
                       "layer_us": round(t_l * 1e6, 2), "layer_TFLOPs": round(2.0 * R * N * K / t_l / 1e12, 1)}
        del wq, ws, a, sa, y, out, tr, gt
        torch.cuda.empty_cache()
    if only in ("", "dequant"):
        c = W.prefill_linear(device=dev)
        N, K = c.w.shape
        wq, ws = F.fp8_weight_quant(c.w, "fp32")
        del c
        out = torch.empty(N, K, dtype=torch.bfloat16, device=dev)
        t = timed_graph(torch, lambda: F.fp8_weight_dequant(wq, ws, w=out), iters)
        nbytes = N * K * 3 + (N // 128) * (K // 128) * 4
        legs["weight_dequant"] = {"shape": [N, K], "us": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1),
                                  "hbm_frac": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4)}
        del wq, ws, out
        torch.cuda.empty_cache()
    if only in ("", "kv"):
        c = W.CONFIGS["kv"]
        T, D = c["T"], c["D"]
        x = W.kv_rows(T, D, W.gen(12, dev))
        q, sc = F.fp8_kv_quant(x)
        out = torch.empty(T, D, dtype=torch.bfloat16, device=dev)
        t_q = timed_graph(torch, lambda: F.fp8_kv_quant(x, q=q, scales=sc), iters)
        t_d = timed_graph(torch, lambda: F.fp8_kv_dequant(q, sc, out=out), iters)
        nbytes = T * D * 3 + T * 4
        legs["kv_cache"] = {"shape": [T, D], "quant_us": round(t_q * 1e6, 2), "quant_GBps": round(nbytes / t_q / 1e9, 1),
                            "dequant_us": round(t_d * 1e6, 2), "dequant_GBps": round(nbytes / t_d / 1e9, 1)}
        del x, q, sc, out
        torch.cuda.empty_cache()
    if only in ("", "delayed"):
        c = W.prefill_linear(device=dev)
        x = c.x
        n = x.numel()
        del c
        ds = F.DelayedScaler(128, "max", 400.0, device=dev)   # amax_history_len 128, algo max
        q = torch.empty(n, dtype=torch.uint8, device=dev)
        su = torch.empty(1, dtype=torch.float32, device=dev)
        t = timed_graph(torch, lambda: ds.quantize(x, q=q, scale_used=su), iters)
        nbytes = n * 3
        legs["delayed_scaling"] = {"shape": list(x.shape), "us": round(t * 1e6, 2),
                                   "GBps": round(nbytes / t / 1e9, 1)}
        del x, q, su, ds
        torch.cuda.empty_cache()
    return legs


if __name__ == "__main__":
    main()
