"""fp8_delayed_quant_noalloc (the step-in-flight scratch in the library's
static per-GPU array instead of the state) against fp8_delayed_quant,
called through the C ABI on states that start equal.  Codes, the scale
used and the whole state after each call must be equal bit for bit; the
second call of each pair runs on a smaller input (fewer workgroups than
amax slots), so it relies on the first leaving the scratch cleared."""
import ctypes

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


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _new_state(F, L):
    nbytes = (F.DELAYED_HEADER_BYTES + 4 * L + 15) // 16 * 16
    st = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=DEV)
    assert F.lib().fp8_delayed_state_init(_ptr(st), L, _stream()) == 0
    return st


def _step(fn, x, st, L, algo):
    q = torch.full(x.shape, 0x5A, dtype=torch.uint8, device=DEV)
    su = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    rc = fn(_ptr(x), x.numel(), _ptr(st), L, algo, ctypes.c_float(400.0), _ptr(q), _ptr(su), _stream())
    assert rc == 0, rc
    return q, su


def _inputs(sizes, seed):
    g = W.gen(seed, DEV)
    out = []
    for i, n in enumerate(sizes):
        mag = 2.0 ** (4 - 3 * i)
        out.append((torch.randn(n, generator=g, device=DEV) * mag).to(torch.bfloat16))
    return out


@pytest.mark.parametrize("L,algo", [(4, 0), (128, 1)])
def test_noalloc_matches_delayed_quant_two_calls(F, L, algo):
    lib = F.lib()
    # 38 workgroups (more than the 16 amax slots, ragged last one), then 4
    sizes = [8192 * 37 + 320, 8192 * 3 + 8]
    xs = _inputs(sizes, 7 + L)
    ref, nal = _new_state(F, L), _new_state(F, L)
    torch.cuda.synchronize()
    assert torch.equal(ref, nal)
    for i, x in enumerate(xs):
        q_ref, s_ref = _step(lib.fp8_delayed_quant, x, ref, L, algo)
        q_nal, s_nal = _step(lib.fp8_delayed_quant_noalloc, x, nal, L, algo)
        torch.cuda.synchronize()
        bad = torch.nonzero(q_ref != q_nal)
        assert bad.numel() == 0, f"call {i} (n {x.numel()}): {bad.shape[0]} code mismatches, first {bad[0].item()}"
        assert s_ref.view(torch.int32).item() == s_nal.view(torch.int32).item(), i
        # the whole state: scale, history position and count, history; the
        # reference's slot lines are back at zero, and the variant never
        # touched the state's
        assert torch.equal(ref, nal), f"call {i}: states differ"
    assert s_ref.item() != 1.0                                 # the second call used a learned scale


def test_noalloc_interleaved_states_and_sizes(F):
    """Two states advanced in turn through the variant alone, against two
    advanced through fp8_delayed_quant: the shared scratch carries nothing
    from one call to the next."""
    lib = F.lib()
    L = 3
    sizes = [8192 * 20, 8192 * 2, 8, 8192 * 17 + 8, 8192]
    xs = _inputs(sizes, 99)
    ref = [_new_state(F, L), _new_state(F, L)]
    nal = [_new_state(F, L), _new_state(F, L)]
    for i, x in enumerate(xs):
        k = i % 2
        q_ref, s_ref = _step(lib.fp8_delayed_quant, x, ref[k], L, 0)
        q_nal, s_nal = _step(lib.fp8_delayed_quant_noalloc, x, nal[k], L, 0)
        torch.cuda.synchronize()
        assert torch.equal(q_ref, q_nal), i
        assert s_ref.view(torch.int32).item() == s_nal.view(torch.int32).item(), i
        assert torch.equal(ref[k], nal[k]), i


def test_noalloc_rejects_what_delayed_quant_rejects(F):
    lib = F.lib()
    x = torch.zeros(64, dtype=torch.bfloat16, device=DEV)
    st = _new_state(F, 4)
    q = torch.empty(64, dtype=torch.uint8, device=DEV)
    su = torch.empty(1, dtype=torch.float32, device=DEV)
    f = lib.fp8_delayed_quant_noalloc
    assert f(_ptr(x), 60, _ptr(st), 4, 0, ctypes.c_float(400.0), _ptr(q), _ptr(su), _stream()) == -1
    assert f(_ptr(x), (1 << 31) * 8192, _ptr(st), 4, 0, ctypes.c_float(400.0), _ptr(q), _ptr(su), _stream()) == -1
    assert f(_ptr(x), 64, _ptr(st), 4, 2, ctypes.c_float(400.0), _ptr(q), _ptr(su), _stream()) == -3
    torch.cuda.synchronize()


def test_noalloc_step_replays_from_a_graph(F, orc):
    """The use the entry point is for: a step captured in a HIP graph (no
    allocation inside the capture) and replayed on new inputs, with eager
    work and synchronisations between the replays, follows the oracle's
    scale sequence; the state is advanced only by the replays."""
    L, S, n = 4, 5, 8192 * 9 + 64
    g = W.gen(2024, DEV)
    mag = torch.exp2(torch.tensor([3.0, -2.0, 5.0, 0.0, -6.0], device=DEV)).reshape(S, 1)
    x = (torch.randn(S, n, generator=g, device=DEV) * mag).to(torch.bfloat16)
    ds = F.DelayedScaler(L, "max", 400.0)
    buf = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    q = torch.empty(n, dtype=torch.uint8, device=DEV)
    su = torch.empty(1, dtype=torch.float32, device=DEV)
    buf.copy_(x[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # an eager step first (the library's set-up on this GPU)
        ds.quantize_noalloc(buf, q, su)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ds.reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ds.quantize_noalloc(buf, q, su)
    ds.reset()                          # capture does not run the step
    q2, s2 = orc.delayed_scaling(W.bits(x.cpu()), L, 0, 400.0)
    for s in range(S):
        buf.copy_(x[s])
        graph.replay()
        torch.cuda.synchronize()
        assert su.item() == s2[s], s
        assert (q.cpu().numpy() == q2[s]).all(), s
        _ = (x[s].float() * 2).sum().item()   # eager work between replays
