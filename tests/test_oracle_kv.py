"""Pins of the oracle's KV-cache quantiser: E5M2 codes with one scale per
cache row ("LLM 推理的 FP8 混合精度工程 2026", section 4 and its precision
table: KV cache in E5M2, per-token scale from the real-time amax).

Independent routes: torch's fp32 division and its float8_e5m2 cast (round
to nearest even), torch's float8_e5m2 decoder, exact double products and
torch's bf16 rounding.
"""
import numpy as np
import torch

import oracle as O


def _rows(seed=0, T=96, D=576):
    """Rows whose magnitudes differ by orders of magnitude along the sequence
    (the section's description of K/V), plus zero, tiny and signed-zero rows."""
    rng = np.random.default_rng(seed)
    mag = 2.0 ** rng.uniform(-20, 20, size=(T, 1))
    x = (rng.standard_normal((T, D)) * mag).astype(np.float32)
    x[3] = 0.0
    x[4] = -0.0
    x[5, ::3] = -0.0
    x[6] = rng.standard_normal(D).astype(np.float32) * 2.0 ** -128    # bf16 subnormal range
    x[7, 10] = 3.0e38
    xb = torch.from_numpy(x).to(torch.bfloat16)
    return xb, xb.view(torch.int16).numpy().astype(np.uint16)


def _torch_route(xb):
    x = xb.float()
    amax = x.abs().amax(dim=1, keepdim=True)
    d = torch.where(amax == 0, torch.ones_like(amax), amax / 57344.0)
    q = (x / d).clamp(-57344.0, 57344.0).to(torch.float8_e5m2).view(torch.uint8)
    return q.numpy(), d[:, 0].numpy()


def test_kv_quant_matches_torch_route():
    for seed in range(4):
        xb, bits = _rows(seed)
        q, s = O.kv_quant(bits)
        qt, st = _torch_route(xb)
        np.testing.assert_array_equal(s.view(np.uint32), st.view(np.uint32))
        bad = np.argwhere(q != qt)
        assert len(bad) == 0, f"seed {seed}: {len(bad)} code mismatches, first {tuple(bad[0])}"


def test_kv_row_maximum_maps_to_the_largest_code():
    xb, bits = _rows(1)
    q, s = O.kv_quant(bits)
    x = xb.float().numpy()
    for t in range(x.shape[0]):
        if np.abs(x[t]).max() == 0:
            assert s[t] == 1.0 and (q[t] & 0x7F == 0).all()
            continue
        k = int(np.argmax(np.abs(x[t])))
        assert q[t, k] & 0x7F == 0x7B, (t, hex(q[t, k]))    # +-57344


def test_kv_dequant_matches_torch_route_and_round_trip():
    xb, bits = _rows(2)
    q, s = O.kv_quant(bits)
    out = O.kv_dequant(q, s)
    vals = torch.from_numpy(q).view(torch.float8_e5m2).to(torch.float64).numpy()
    p32 = (vals * s.astype(np.float64)[:, None]).astype(np.float32)       # exact product, one rounding
    want = torch.from_numpy(p32).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    np.testing.assert_array_equal(out, want)
    # round trip: within half an E5M2 step of the row scale, plus the bf16
    # rounding of the output (relative, or half the subnormal spacing 2^-133)
    x = xb.to(torch.float64).numpy()
    y = torch.from_numpy(out.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    d = s.astype(np.float64)[:, None]
    r = np.abs(x) / d
    step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(r, 2.0 ** -14))) - 2), 2.0 ** -16)
    assert np.all(np.abs(x - y) <= 0.5 * step * d * (1 + 2 ** -7) + np.abs(y) * 2.0 ** -8 + 2.0 ** -134)


def test_kv_dequant_special_codes():
    q = np.array([[0x00, 0x80, 0x7C, 0xFC, 0x7D, 0xFF, 0x7B, 0x01] + [0] * 8], np.uint8)
    out = O.kv_dequant(q, np.array([1.0], np.float32))
    assert out[0, 0] == 0x0000 and out[0, 1] == 0x8000
    assert out[0, 2] == 0x7F80 and out[0, 3] == 0xFF80                     # +-Inf codes
    assert (out[0, 4] & 0x7F80) == 0x7F80 and (out[0, 4] & 0x7F) != 0       # NaN
    assert out[0, 6] == 0x4760                                              # 57344
    assert out[0, 7] == 0x3780                                              # 2^-16
