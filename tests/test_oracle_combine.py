"""Pins of the oracle's MoE combine: out[t] = sum_j gates[t][j] * y[rows[t][j]]
(the gate-weighted sum of a token's routed rows after the grouped GEMM of a
block-scale fused MoE; ROCm 7.0 article, section 2; 8 active experts per
token in the DeepSeek-V3 guide's configuration table)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


def test_hand_worked_case():
    # y rows (exact in bf16), two tokens with two slots each
    y = _bf16_bits([[1, 2], [3, -4], [8, 0.5], [-2, 6]])
    rows = np.array([[2, 0], [1, 3]], np.int32)
    gates = np.array([[0.5, 0.25], [0.75, 0.125]], np.float32)
    out, bnd = O.moe_combine(y, rows, gates)
    # token 0: 0.5*[8, 0.5] + 0.25*[1, 2] = [4.25, 0.75]
    # token 1: 0.75*[3, -4] + 0.125*[-2, 6] = [2.0, -2.25]
    np.testing.assert_array_equal(out, [[4.25, 0.75], [2.0, -2.25]])
    np.testing.assert_array_equal(bnd, [[4.25, 0.75], [2.5, 3.75]])


def test_single_slot_unit_gate_is_a_gather():
    rng = np.random.default_rng(1)
    y = _bf16_bits(rng.standard_normal((50, 24)))
    rows = rng.integers(0, 50, size=(30, 1)).astype(np.int32)
    out, _ = O.moe_combine(y, rows, np.ones((30, 1), np.float32))
    yv = torch.from_numpy(y.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(out, yv[rows[:, 0]])


def test_linear_in_gates_and_symmetric_in_slots():
    rng = np.random.default_rng(2)
    y = _bf16_bits(rng.integers(-40, 40, size=(64, 16)))      # small integers: exact sums
    rows = rng.integers(0, 64, size=(20, 8)).astype(np.int32)
    gates = (rng.integers(1, 64, size=(20, 8)) / 64.0).astype(np.float32)
    out, _ = O.moe_combine(y, rows, gates)
    out2, _ = O.moe_combine(y, rows, gates * 2)
    np.testing.assert_array_equal(out2, 2 * out)
    perm = rng.permutation(8)
    out3, _ = O.moe_combine(y, rows[:, perm], gates[:, perm])
    np.testing.assert_array_equal(out3, out)


def test_routing_map_covers_every_row_once():
    r = W.routing_full(64, 16, 4, 1.0, W.gen(5))
    tr = r["token_rows"].numpy()
    assert sorted(tr.reshape(-1).tolist()) == list(range(64 * 4))
    ri = r["row_index"].numpy()
    assert (ri[tr] == np.arange(64)[:, None]).all()
    np.testing.assert_allclose(r["gates"].sum(1).numpy(), 1.0, rtol=1e-6)


def test_rejects_rows_out_of_range():
    y = _bf16_bits(np.zeros((4, 8)))
    with pytest.raises(ValueError):
        O.moe_combine(y, np.array([[4]], np.int32), np.ones((1, 1), np.float32))
