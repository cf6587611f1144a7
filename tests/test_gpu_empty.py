"""Empty inputs through the binding: zero token rows, zero routed rows, an
empty KV cache and an empty cast reach the library as calls with an empty
dimension (which read and write nothing, whatever the empty tensors' data
pointers), and return outputs of the right shapes with no error."""
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def F():
    import fp8_block_scaled_02_amd as F
    assert torch.cuda.is_available()
    return F


def test_zero_token_rows(F):
    K, N = 512, 256
    x = torch.empty(0, K, dtype=torch.bfloat16, device=DEV)
    a, sa = F.fp8_act_quant(x, 128, "fp32")
    assert a.shape == (0, K) and sa.shape == (0, K // 128)
    a32, e32 = F.fp8_act_quant(x, 32, "e8m0")
    assert a32.shape == (0, K) and e32.shape == (0, K // 32)
    w = (torch.randn(N, K, device=DEV) * 0.02).to(torch.bfloat16)
    wq, ws = F.fp8_weight_quant(w, "fp32")
    for out in (torch.float32, torch.bfloat16):
        assert F.fp8_block_gemm(a, sa, wq, ws, out).shape == (0, N)
        assert F.fp8_block_gemm_packed(a, sa, F.fp8_weight_pack(wq), ws, out).shape == (0, N)
    b32, eb32 = F.fp8_act_quant(w, 32, "e8m0")
    assert F.mxfp8_gemm(a32, e32, b32, eb32).shape == (0, N)
    torch.cuda.synchronize()


def test_zero_routed_rows(F):
    T, E, N, K = 8, 4, 256, 256
    x = torch.randn(T, K, device=DEV).to(torch.bfloat16)
    a, sa = F.fp8_act_quant(x, 128, "fp32")
    wq = torch.zeros(E, N, K, dtype=torch.uint8, device=DEV)
    ws = torch.ones(E, N // 128, K // 128, device=DEV)
    ri = torch.empty(0, dtype=torch.int32, device=DEV)
    offs = torch.zeros(E + 1, dtype=torch.int32, device=DEV)
    assert F.fp8_grouped_gemm(a, sa, ri, offs, wq, ws).shape == (0, N)
    assert F.fp8_grouped_gemm_packed(a, sa, ri, offs, F.fp8_weight_pack(wq), ws).shape == (0, N)
    y = torch.empty(0, N, dtype=torch.bfloat16, device=DEV)
    tr = torch.empty(0, 2, dtype=torch.int32, device=DEV)
    g = torch.empty(0, 2, dtype=torch.float32, device=DEV)
    assert F.fp8_moe_combine(y, tr, g).shape == (0, N)
    torch.cuda.synchronize()


def test_empty_kv_cache_and_cast(F):
    x = torch.empty(0, 1024, dtype=torch.bfloat16, device=DEV)
    q, s = F.fp8_kv_quant(x)
    assert q.shape == (0, 1024) and s.shape == (0,)
    assert F.fp8_kv_dequant(q, s).shape == (0, 1024)
    assert F.fp8_cast_f32(torch.empty(0, device=DEV)).shape == (0,)
    torch.cuda.synchronize()
