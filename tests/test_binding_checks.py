"""The Python binding rejects misuse before anything reaches the kernels
(no GPU needed: every case raises ValueError on the host, before the
library is called).  Layout and dtype checks come before the device check,
so each one can be exercised here with host tensors; tensors that are laid
out correctly but live on the host must fail the device check, since the
kernels would dereference their host addresses as device memory."""
import pytest
import torch

import fp8_block_scaled_02_amd as F

u8, f32, i32, bf16 = torch.uint8, torch.float32, torch.int32, torch.bfloat16


def _raises(match, fn, *a, **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


def test_host_tensors_never_reach_a_kernel():
    M, N, K = 16, 256, 512
    a, w = torch.zeros(M, K, dtype=u8), torch.zeros(N, K, dtype=u8)
    sa, sw = torch.ones(M, K // 128), torch.ones(N // 128, K // 128)
    on = "on a GPU"
    _raises(on, F.fp8_act_quant, torch.zeros(M, K, dtype=bf16))
    _raises(on, F.fp8_weight_quant, torch.zeros(N, K, dtype=bf16))
    _raises(on, F.fp8_block_gemm, a, sa, w, sw)
    _raises(on, F.fp8_block_gemm_packed, a, sa, w, sw)
    _raises(on, F.mxfp8_gemm, a, torch.zeros(M, K // 32, dtype=u8), w, torch.zeros(N, K // 32, dtype=u8))
    _raises(on, F.fp8_weight_dequant, w, sw)
    _raises(on, F.fp8_weight_pack, w)
    _raises(on, F.fp8_kv_quant, torch.zeros(4, 64, dtype=bf16))
    _raises(on, F.fp8_kv_dequant, torch.zeros(4, 64, dtype=u8), torch.ones(4))
    _raises(on, F.fp8_cast_f32, torch.zeros(8))


def test_grouped_gemm_with_host_routing():
    """Routing tensors straight from the workload generator live on the
    host: with everything else laid out correctly the call must still be
    refused."""
    T, E, N, K, R = 8, 4, 128, 256, 16
    args = (torch.zeros(T, K, dtype=u8), torch.ones(T, K // 128), torch.zeros(R, dtype=i32),
            torch.tensor([0, 4, 8, 12, 16], dtype=i32), torch.zeros(E, N, K, dtype=u8),
            torch.ones(E, N // 128, K // 128))
    _raises("on a GPU", F.fp8_grouped_gemm, *args)
    _raises("on a GPU", F.fp8_grouped_gemm_packed, *args)


def test_combine_with_host_routing():
    y = torch.zeros(16, 64, dtype=bf16)
    _raises("on a GPU", F.fp8_moe_combine, y, torch.zeros(2, 8, dtype=i32), torch.ones(2, 8))


def test_block_gemm_scale_layouts():
    M, N, K = 16, 256, 512
    a, w = torch.zeros(M, K, dtype=u8), torch.zeros(N, K, dtype=u8)
    sa, sw = torch.ones(M, K // 128), torch.ones(N // 128, K // 128)
    for fn in (F.fp8_block_gemm, F.fp8_block_gemm_packed):
        _raises("a_scales must have shape", fn, a, torch.ones(M, K // 128 + 1), w, sw)
        _raises("w_scales must have shape", fn, a, sa, w, torch.ones(N // 128, K // 64))
        _raises("contiguous", fn, a, torch.ones(K // 128, M).t(), w, sw)   # column-major scales
        _raises("float32", fn, a, sa.double(), w, sw)
        _raises("uint8", fn, a.to(torch.int8), sa, w, sw)
        _raises("K =", fn, a, sa, torch.zeros(N, K + 128, dtype=u8), sw)
        _raises("y must have shape", fn, a, sa, w, sw, torch.bfloat16, torch.zeros(M, N + 8, dtype=bf16))
        _raises("out_dtype", fn, a, sa, w, sw, torch.float16)
    _raises("rows contiguous", F.fp8_block_gemm, torch.zeros(K, M, dtype=u8).t(), sa, w, sw)


def test_mx_gemm_scale_layouts():
    M, N, K = 16, 256, 512
    a, b = torch.zeros(M, K, dtype=u8), torch.zeros(N, K, dtype=u8)
    ea, eb = torch.zeros(M, K // 32, dtype=u8), torch.zeros(N, K // 32, dtype=u8)
    _raises("a_e8m0 must have shape", F.mxfp8_gemm, a, torch.zeros(M, K // 128, dtype=u8), b, eb)
    _raises("b_e8m0 must be contiguous", F.mxfp8_gemm, a, ea, b, torch.zeros(K // 32, N, dtype=u8).t())
    _raises("b_e8m0 must be contiguous uint8", F.mxfp8_gemm, a, ea, b, eb.float())
    _raises("y must have shape", F.mxfp8_gemm, a, ea, b, eb, torch.zeros(M, N - 128))


def test_grouped_gemm_routing_layouts():
    T, E, N, K, R = 8, 4, 128, 256, 16
    a, sa = torch.zeros(T, K, dtype=u8), torch.ones(T, K // 128)
    ri, offs = torch.zeros(R, dtype=i32), torch.tensor([0, 4, 8, 12, 16], dtype=i32)
    w, sw = torch.zeros(E, N, K, dtype=u8), torch.ones(E, N // 128, K // 128)
    g = F.fp8_grouped_gemm
    _raises("E \\+ 1", g, a, sa, ri, offs[:E], w, sw)                    # E entries: kernel reads OFFS[E]
    _raises("int32", g, a, sa, ri.long(), offs, w, sw)
    _raises("1-D", g, a, sa, ri.view(4, 4), offs, w, sw)
    _raises("a_scales must have shape", g, a, torch.ones(T, K // 64), ri, offs, w, sw)
    _raises("w_scales must have shape", g, a, sa, ri, offs, w, torch.ones(E, N // 128, K // 64))
    _raises("contiguous", g, a, sa, ri, offs, w, torch.ones(E, N // 128, 2 * (K // 128))[:, :, ::2])
    _raises("K =", g, a, sa, ri, offs, torch.zeros(E, N, 2 * K, dtype=u8), sw)


def test_quantiser_output_layouts():
    x = torch.zeros(16, 512, dtype=bf16)
    _raises("scales must have shape", F.fp8_act_quant, x, 128, "fp32", None, torch.ones(16, 8))
    _raises("uint8 for e8m0", F.fp8_act_quant, x, 32, "e8m0", None, torch.ones(16, 16))
    _raises("q must have shape", F.fp8_act_quant, x, 128, "fp32", torch.zeros(16, 256, dtype=u8))
    _raises("scales must have shape", F.fp8_weight_quant, torch.zeros(256, 512, dtype=bf16), "fp32", None,
            torch.ones(2, 2))
    _raises("scales must have shape", F.fp8_kv_quant, torch.zeros(4, 64, dtype=bf16), None, torch.ones(5))
    _raises("one code per element", F.fp8_cast_f32, torch.zeros(8), F.FMT_E4M3, torch.zeros(4, dtype=u8))
