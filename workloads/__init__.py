"""Seeded synthetic inputs for the W8A8 block-scaled FP8 linear layer.

This module is shared by the tests, the benchmark and the smoke check, and
feeds both the HIP path and the CPU oracle.  It holds none of the method's
arithmetic: it only draws random numbers, rounds them to bf16 (round to
nearest even, torch's own cast) and forms the MoE routing that the grouped
GEMM takes as input.

Recipes (the pages' workloads have no public data; these are stand-ins with
their shapes and value structure):

* activations x ~ N(0, 1) with a fixed, seeded set of outlier channels whose
  values are multiplied before the bf16 rounding (the pages describe
  channel outliers of 30-100x in LLM activations);
* weights W ~ N(0, 0.02);
* MXFP8 operands: bf16(z * 2^u) with z ~ N(0, 1) and u ~ U(-8, 8) drawn once
  per (row, 32-element K block);
* MoE routing: logits z ~ N(0, 1) plus a per-expert bias -s*ln(rank) (Zipf
  skew, s = 1 by default), top-k by logit with ties to the lower expert id,
  rows ordered by (expert, token, slot); gate weights for the combine are a
  softmax over each token's chosen logits (the model's gating function is
  an input to the method, not part of it);
* KV-cache rows: bf16(z * 2^u), u ~ U(-8, 8) per token.
"""
from dataclasses import dataclass
import math

import numpy as np
import torch

__all__ = [
    "bits", "gen", "activations", "weights", "mx_operand", "kv_rows", "routing", "routing_full",
    "LinearCase", "tiny_linear", "decode_linear", "prefill_linear",
    "mx_case", "moe_case", "CONFIGS",
]

# Workload sizes.
CONFIGS = {
    "tiny": dict(M=16, K=512, N=256),
    "decode": dict(Ms=(1, 8, 32, 128), K=8192, N=28672),
    "prefill": dict(M=4096, K=7168, N=18432),
    "mx": dict(M=8192, K=8192, N=8192),
    "moe": dict(T=4096, E=256, topk=8, N=2048, K=7168),
    # KV cache of a 32K-token context: 8 KV heads x 128 per token, K or V
    "kv": dict(T=32768, D=1024),
}


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def outlier_channels(K: int, count: int, g: torch.Generator) -> torch.Tensor:
    """`count` distinct channels, a seeded sample without replacement."""
    return torch.randperm(K, generator=g, device=g.device)[:count]


def activations(M: int, K: int, n_outliers: int, mult: float,
                g: torch.Generator) -> torch.Tensor:
    """x ~ N(0,1) [M, K] with n_outliers channels scaled by mult, as bf16."""
    dev = g.device
    x = torch.randn(M, K, generator=g, device=dev, dtype=torch.float32)
    if n_outliers:
        ch = outlier_channels(K, n_outliers, g)
        x[:, ch] *= mult
    return x.to(torch.bfloat16)


def weights(N: int, K: int, std: float, g: torch.Generator) -> torch.Tensor:
    dev = g.device
    w = torch.randn(N, K, generator=g, device=dev, dtype=torch.float32) * std
    return w.to(torch.bfloat16)


def mx_operand(R: int, K: int, g: torch.Generator, block: int = 32,
               lo: float = -8.0, hi: float = 8.0) -> torch.Tensor:
    """bf16(z * 2^u), u ~ U(lo, hi) per (row, block) of K."""
    dev = g.device
    z = torch.randn(R, K, generator=g, device=dev, dtype=torch.float32)
    u = torch.rand(R, K // block, generator=g, device=dev, dtype=torch.float32)
    u = lo + (hi - lo) * u
    z = z.view(R, K // block, block) * torch.exp2(u).unsqueeze(-1)
    return z.view(R, K).to(torch.bfloat16)


def kv_rows(T: int, D: int, g: torch.Generator, lo: float = -8.0, hi: float = 8.0) -> torch.Tensor:
    """K or V cache rows: bf16(z * 2^u), z ~ N(0,1), u ~ U(lo, hi) per token,
    so token magnitudes differ by orders of magnitude along the sequence."""
    dev = g.device
    z = torch.randn(T, D, generator=g, device=dev, dtype=torch.float32)
    u = lo + (hi - lo) * torch.rand(T, 1, generator=g, device=dev, dtype=torch.float32)
    return (z * torch.exp2(u)).to(torch.bfloat16)


def routing_full(T: int, E: int, topk: int, s: float, g: torch.Generator) -> dict:
    """Top-k MoE routing (CPU) with the combine inputs:
    row_index int32 [R]   token of each routed row (rows ordered by
                          (expert, token, slot)),
    offs      int32 [E+1] expert offsets into the routed rows,
    experts   int32 [R]   expert of each routed row,
    token_rows int32 [T, topk] routed row of (token, slot),
    gates     fp32 [T, topk]  gate weight of (token, slot): softmax over the
                          token's chosen logits (fp32)."""
    assert g.device.type == "cpu"
    z = torch.randn(T, E, generator=g, dtype=torch.float32)
    rank = torch.randperm(E, generator=g) + 1            # 1..E
    bias = (-s * torch.log(rank.to(torch.float64))).to(torch.float32)
    logits = z + bias
    # stable descending sort: equal logits keep the lower expert id first
    order = torch.sort(logits, dim=1, descending=True, stable=True).indices
    chosen = order[:, :topk]                             # [T, topk]
    tok = torch.arange(T).unsqueeze(1).expand(T, topk)
    slot = torch.arange(topk).unsqueeze(0).expand(T, topk)
    key = (chosen.to(torch.int64) * T + tok) * topk + slot
    perm = torch.argsort(key.reshape(-1))
    experts = chosen.reshape(-1)[perm].to(torch.int32)
    row_index = tok.reshape(-1)[perm].to(torch.int32)
    counts = torch.bincount(experts.to(torch.int64), minlength=E)
    offs = torch.zeros(E + 1, dtype=torch.int32)
    offs[1:] = torch.cumsum(counts, 0).to(torch.int32)
    token_rows = torch.empty(T * topk, dtype=torch.int32)
    token_rows[perm] = torch.arange(T * topk, dtype=torch.int32)
    gates = torch.softmax(torch.gather(logits, 1, chosen), dim=1)
    return dict(row_index=row_index, offs=offs, experts=experts,
                token_rows=token_rows.view(T, topk), gates=gates.contiguous())


def routing(T: int, E: int, topk: int, s: float, g: torch.Generator):
    """Top-k MoE routing (CPU).  Returns (row_index int32 [T*topk],
    expert_offsets int32 [E+1], per-row expert id int32 [T*topk])."""
    r = routing_full(T, E, topk, s, g)
    return r["row_index"], r["offs"], r["experts"]


@dataclass
class LinearCase:
    x: torch.Tensor        # bf16 [M, K]
    w: torch.Tensor        # bf16 [N, K]
    scale_fmt: str         # "fp32" | "ue8m0"
    out_dtype: str         # "f32" | "bf16"


def tiny_linear(device="cpu", seed=0) -> LinearCase:
    """16 x 512 -> 256: 4 outlier channels x20, fp32 scales, fp32 output."""
    c = CONFIGS["tiny"]
    g = gen(seed, device)
    x = activations(c["M"], c["K"], 4, 20.0, g)
    w = weights(c["N"], c["K"], 0.02, g)
    return LinearCase(x, w, "fp32", "f32")


def decode_linear(device="cpu", seed=1, K=None, N=None) -> LinearCase:
    """128 x 8192 -> 28672 (use the first M rows for M in 1, 8, 32, 128):
    0.5% outlier channels x50, ue8m0 scales, bf16 output."""
    c = CONFIGS["decode"]
    K = K or c["K"]
    N = N or c["N"]
    g = gen(seed, device)
    x = activations(max(c["Ms"]), K, round(0.005 * K), 50.0, g)
    w = weights(N, K, 0.02, g)
    return LinearCase(x, w, "ue8m0", "bf16")


def prefill_linear(device="cpu", seed=2, M=None, K=None, N=None) -> LinearCase:
    """4096 x 7168 -> 18432: 0.5% outlier channels x50, fp32 scales, bf16."""
    c = CONFIGS["prefill"]
    M = M or c["M"]
    K = K or c["K"]
    N = N or c["N"]
    g = gen(seed, device)
    x = activations(M, K, round(0.005 * K), 50.0, g)
    w = weights(N, K, 0.02, g)
    return LinearCase(x, w, "fp32", "bf16")


def mx_case(device="cpu", seed=3, M=None, N=None, K=None):
    """MXFP8 operands A [M, K], B [N, K] (bf16), default 8192^3."""
    c = CONFIGS["mx"]
    M = M or c["M"]
    N = N or c["N"]
    K = K or c["K"]
    g = gen(seed, device)
    a = mx_operand(M, K, g)
    b = mx_operand(N, K, g)
    return a, b


@dataclass
class MoeCase:
    x: torch.Tensor            # bf16 [T, K]
    w: torch.Tensor            # bf16 [E, N, K]
    row_index: torch.Tensor    # int32 [R]  (CPU)
    offs: torch.Tensor         # int32 [E+1] (CPU)
    experts: torch.Tensor      # int32 [R]  (CPU)


def moe_case(device="cpu", seed=4, T=None, E=None, topk=None, N=None, K=None,
             s=1.0) -> MoeCase:
    """Tokens x [T, K] as in the prefill case, per-expert W [E, N, K] ~
    N(0, 0.02), Zipf-skewed top-k routing.  Defaults: 4096 tokens, 256
    experts, top-8, N 2048, K 7168."""
    c = CONFIGS["moe"]
    T = T or c["T"]
    E = E or c["E"]
    topk = topk or c["topk"]
    N = N or c["N"]
    K = K or c["K"]
    gr = gen(seed, "cpu")
    row_index, offs, experts = routing(T, E, topk, s, gr)
    g = gen(seed + 1000, device)
    x = activations(T, K, round(0.005 * K), 50.0, g)
    w = torch.empty(E, N, K, dtype=torch.bfloat16, device=device)
    for e in range(E):   # per expert, to keep the fp32 temporaries small
        w[e] = weights(N, K, 0.02, g)
    return MoeCase(x, w, row_index, offs, experts)


def zipf_histogram(offs: torch.Tensor):
    counts = (offs[1:] - offs[:-1]).tolist()
    nz = [c for c in counts if c > 0]
    return dict(active=len(nz), max=max(counts), median=float(np.median(counts)),
                total=int(sum(counts)))
