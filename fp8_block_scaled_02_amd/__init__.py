"""Python binding of libfp8blk, the MI355X (gfx950) W8A8 block-scaled FP8
linear-layer library.

Argument marshalling only: every step of the hot path runs in the HIP
kernels behind the C ABI declared in include/fp8blk.h.  torch provides the
device memory and the stream (the current torch stream of the tensors'
device).  The functions carry the C names (fp8_act_quant, fp8_weight_quant,
fp8_block_gemm, mxfp8_gemm, fp8_grouped_gemm, fp8_cast_f32) and take torch
tensors; outputs are allocated with torch when not supplied.

There is no fallback: if libfp8blk.so is missing this module raises on
first use.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8blk.so")

# enums of include/fp8blk.h
FP8B_OK = 0
SCALE_FP32, SCALE_UE8M0, SCALE_E8M0_BYTE = 0, 1, 2
OUT_F32, OUT_BF16 = 0, 1
FMT_E4M3, FMT_E5M2 = 0, 1
MFMA_BF16_16X16X32, MFMA_FP8_16X16X128 = 0, 1
PROBE_COPY, PROBE_EMPTY = 0, 1
GEMM_PROBE_TILE0 = 0
MFMA_LOOP_FLOPS = {MFMA_BF16_16X16X32: 16384, MFMA_FP8_16X16X128: 65536}   # per MFMA instruction
DELAYED_HEADER_BYTES = 128 + 128 * 16    # FP8B_DELAYED_HEADER_BYTES of include/fp8blk.h

_SCALE_FMT = {"fp32": SCALE_FP32, "ue8m0": SCALE_UE8M0, "e8m0": SCALE_E8M0_BYTE}

_lib = None


class Fp8Error(RuntimeError):
    """A negative status from libfp8blk."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


def lib():
    """The loaded libfp8blk.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m fp8_block_scaled_02_amd.build` (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.fp8b_abi_version.restype = ci
        L.fp8b_abi_version.argtypes = []
        L.fp8b_status_string.restype = ctypes.c_char_p
        L.fp8b_status_string.argtypes = [ci]
        L.fp8_act_quant.restype = ci
        L.fp8_act_quant.argtypes = [vp, i64, i64, i64, ci, ci, vp, i64, vp, vp]
        L.fp8_weight_quant.restype = ci
        L.fp8_weight_quant.argtypes = [vp, i64, i64, i64, ci, vp, i64, vp, vp]
        L.fp8_block_gemm.restype = ci
        L.fp8_block_gemm.argtypes = [vp, i64, vp, vp, i64, vp, i64, i64, i64, vp, i64, ci, vp]
        L.mxfp8_gemm.restype = ci
        L.mxfp8_gemm.argtypes = [vp, i64, vp, vp, i64, vp, i64, i64, i64, vp, i64, vp]
        L.fp8_grouped_gemm.restype = ci
        L.fp8_grouped_gemm.argtypes = [vp, vp, i64, vp, vp, i64, i64, vp, vp, i64, i64, vp, ci, vp]
        L.fp8_weight_pack.restype = ci
        L.fp8_weight_pack.argtypes = [vp, i64, i64, i64, i64, vp, vp]
        L.fp8_block_gemm_packed.restype = ci
        L.fp8_block_gemm_packed.argtypes = [vp, i64, vp, vp, vp, i64, i64, i64, vp, i64, ci, vp]
        L.fp8_grouped_gemm_packed.restype = ci
        L.fp8_grouped_gemm_packed.argtypes = [vp, vp, i64, vp, vp, i64, i64, vp, vp, i64, i64, vp, ci, vp]
        L.fp8_weight_dequant.restype = ci
        L.fp8_weight_dequant.argtypes = [vp, i64, i64, i64, vp, vp, i64, vp]
        L.fp8_moe_combine.restype = ci
        L.fp8_moe_combine.argtypes = [vp, i64, i64, vp, vp, i64, i64, vp, ci, vp]
        L.fp8_kv_quant.restype = ci
        L.fp8_kv_quant.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp]
        L.fp8_kv_dequant.restype = ci
        L.fp8_kv_dequant.argtypes = [vp, i64, i64, i64, vp, vp, i64, vp]
        L.fp8_delayed_state_init.restype = ci
        L.fp8_delayed_state_init.argtypes = [vp, i64, vp]
        L.fp8_delayed_quant.restype = ci
        L.fp8_delayed_quant.argtypes = [vp, i64, vp, i64, ci, ctypes.c_float, vp, vp, vp]
        L.fp8_delayed_quant_noalloc.restype = ci
        L.fp8_delayed_quant_noalloc.argtypes = [vp, i64, vp, i64, ci, ctypes.c_float, vp, vp, vp]
        L.fp8_cast_f32.restype = ci
        L.fp8_cast_f32.argtypes = [vp, i64, ci, vp, vp]
        L.fp8b_stream_probe.restype = ci
        L.fp8b_stream_probe.argtypes = [ci, vp, i64, i64, vp, vp, vp]
        L.fp8b_gemm_probe.restype = ci
        L.fp8b_gemm_probe.argtypes = [ci, vp, vp, vp, vp, i64, i64, i64, vp, vp]
        L.fp8b_mfma_loop.restype = ci
        L.fp8b_mfma_loop.argtypes = [ci, vp, i64, i64, vp, vp]
        _lib = L
    return _lib


def abi_version() -> int:
    return int(lib().fp8b_abi_version())


def status_string(status: int) -> str:
    return lib().fp8b_status_string(int(status)).decode()


def _check(fn, rc):
    if rc != FP8B_OK:
        raise Fp8Error(fn, rc)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _fmt(scale_fmt):
    return _SCALE_FMT[scale_fmt] if isinstance(scale_fmt, str) else int(scale_fmt)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _on_gpu(*ts):
    """Every tensor is on the same GPU as the first: the kernels dereference
    data_ptr() as device memory, so a host tensor (or one on another GPU)
    must never reach them."""
    dev = ts[0].device
    for t in ts:
        _need(t.is_cuda, f"every tensor must be on a GPU (found one on {t.device})")
        _need(t.device == dev, f"every tensor must be on {dev} (found one on {t.device})")


def _shape(t, shape, name):
    _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")


def fp8_act_quant(x: torch.Tensor, block_k: int = 128, scale_fmt="fp32", q=None, scales=None):
    """Dynamic per-token, per-block activation quantisation.

    x: bf16 [M, K] on a GPU (row stride x.stride(0)).  Returns
    (q uint8 [M, K], scales [M, K/block_k]) -- float32 scales, or uint8 E8M0
    bytes for scale_fmt "e8m0"."""
    _need(x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1, "x must be 2-D bf16, rows contiguous")
    M, K = x.shape
    f = _fmt(scale_fmt)
    if q is None:
        q = torch.empty(M, K, dtype=torch.uint8, device=x.device)
    if scales is None:
        sdt = torch.uint8 if f == SCALE_E8M0_BYTE else torch.float32
        scales = torch.empty(M, max(K // block_k, 0), dtype=sdt, device=x.device)
    _need(q.dtype == torch.uint8 and q.dim() == 2 and q.stride(1) == 1, "q must be 2-D uint8, rows contiguous")
    _shape(q, (M, K), "q")
    _need(scales.dtype == (torch.uint8 if f == SCALE_E8M0_BYTE else torch.float32),
          "scales must be uint8 for e8m0, float32 otherwise")
    _need(scales.is_contiguous(), "scales must be contiguous")
    _shape(scales, (M, K // block_k if block_k > 0 else 0), "scales")
    _on_gpu(x, q, scales)
    rc = lib().fp8_act_quant(_p(x), M, K, x.stride(0) if M else K, block_k, f, _p(q),
                             q.stride(0) if M else K, _p(scales), _stream(x))
    _check("fp8_act_quant", rc)
    return q, scales


def fp8_weight_quant(w: torch.Tensor, scale_fmt="fp32", q=None, scales=None):
    """128x128-block weight quantisation: w bf16 [N, K] -> (q uint8 [N, K],
    float32 scales [N/128, K/128])."""
    _need(w.dtype == torch.bfloat16 and w.dim() == 2 and w.stride(1) == 1, "w must be 2-D bf16, rows contiguous")
    N, K = w.shape
    if q is None:
        q = torch.empty(N, K, dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(N // 128, K // 128, dtype=torch.float32, device=w.device)
    _need(q.dtype == torch.uint8 and q.dim() == 2 and q.stride(1) == 1, "q must be 2-D uint8, rows contiguous")
    _shape(q, (N, K), "q")
    _need(scales.dtype == torch.float32 and scales.is_contiguous(), "scales must be contiguous float32")
    _shape(scales, (N // 128, K // 128), "scales")
    _on_gpu(w, q, scales)
    rc = lib().fp8_weight_quant(_p(w), N, K, w.stride(0), _fmt(scale_fmt), _p(q), q.stride(0),
                                _p(scales), _stream(w))
    _check("fp8_weight_quant", rc)
    return q, scales


def fp8_weight_dequant(q: torch.Tensor, scales: torch.Tensor, w=None):
    """FP8 weights with 128x128 block scales back to bf16:
    w[n, k] = bf16(fp32(value(q[n, k]) * scales[n/128, k/128]))."""
    _need(q.dtype == torch.uint8 and q.dim() == 2 and q.stride(1) == 1, "q must be 2-D uint8, rows contiguous")
    _need(scales.dtype == torch.float32 and scales.is_contiguous(), "scales must be contiguous float32")
    N, K = q.shape
    if w is None:
        w = torch.empty(N, K, dtype=torch.bfloat16, device=q.device)
    _need(w.dtype == torch.bfloat16 and w.dim() == 2 and w.stride(1) == 1, "w must be 2-D bf16, rows contiguous")
    _shape(scales, (N // 128, K // 128), "scales")
    _shape(w, (N, K), "w")
    _on_gpu(q, scales, w)
    rc = lib().fp8_weight_dequant(_p(q), N, K, q.stride(0), _p(scales), _p(w), w.stride(0), _stream(q))
    _check("fp8_weight_dequant", rc)
    return w


def fp8_moe_combine(y: torch.Tensor, token_rows: torch.Tensor, gates: torch.Tensor, out_dtype=torch.bfloat16,
                    out=None):
    """out[t] = sum_j gates[t, j] * y[token_rows[t, j]] (fp32 accumulation):
    y bf16 [R, N] routed rows, token_rows int32 [T, k], gates fp32 [T, k]."""
    _need(y.dtype == torch.bfloat16 and y.dim() == 2 and y.is_contiguous(), "y must be contiguous 2-D bf16")
    _need(token_rows.dtype == torch.int32 and token_rows.is_contiguous(), "token_rows must be contiguous int32")
    _need(gates.dtype == torch.float32 and gates.is_contiguous(), "gates must be contiguous float32")
    _need(token_rows.shape == gates.shape and token_rows.dim() == 2, "token_rows and gates must be [T, k]")
    R, N = y.shape
    T, k = token_rows.shape
    _need(out_dtype in (torch.bfloat16, torch.float32), "out_dtype must be bfloat16 or float32")
    od = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    if out is None:
        out = torch.empty(T, N, dtype=out_dtype, device=y.device)
    _need(out.is_contiguous() and out.dtype == out_dtype, "out must be contiguous of out_dtype")
    _shape(out, (T, N), "out")
    _on_gpu(y, token_rows, gates, out)
    rc = lib().fp8_moe_combine(_p(y), R, N, _p(token_rows), _p(gates), T, k, _p(out), od, _stream(y))
    _check("fp8_moe_combine", rc)
    return out


def moe_forward(x: torch.Tensor, row_index, expert_offsets, token_rows, gates, w_q, w_scales,
                out_dtype=torch.bfloat16, packed=False):
    """One block-scale MoE expert projection as a kernel sequence: act_quant
    of the tokens (once per token, per 128 channels, fp32 scales), the
    grouped GEMM over the routed rows (gather inside), then the gate-weighted
    combine back to tokens.  packed: w_q is fp8_weight_pack of the expert
    weights.  Returns (out [T, N], y routed rows [R, N])."""
    a, sa = fp8_act_quant(x, 128, "fp32")
    gemm = fp8_grouped_gemm_packed if packed else fp8_grouped_gemm
    y = gemm(a, sa, row_index, expert_offsets, w_q, w_scales, torch.bfloat16)
    return fp8_moe_combine(y, token_rows, gates, out_dtype), y


def fp8_kv_quant(x: torch.Tensor, q=None, scales=None):
    """KV-cache rows x bf16 [T, D] -> (E5M2 codes uint8 [T, D], fp32 scales [T]),
    one scale per row (d = amax / 57344)."""
    _need(x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1, "x must be 2-D bf16, rows contiguous")
    T, D = x.shape
    if q is None:
        q = torch.empty(T, D, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(T, dtype=torch.float32, device=x.device)
    _need(q.dtype == torch.uint8 and q.dim() == 2 and q.stride(1) == 1, "q must be 2-D uint8, rows contiguous")
    _shape(q, (T, D), "q")
    _need(scales.dtype == torch.float32 and scales.is_contiguous(), "scales must be contiguous float32")
    _shape(scales, (T,), "scales")
    _on_gpu(x, q, scales)
    rc = lib().fp8_kv_quant(_p(x), T, D, x.stride(0), _p(q), q.stride(0), _p(scales), _stream(x))
    _check("fp8_kv_quant", rc)
    return q, scales


def fp8_kv_dequant(q: torch.Tensor, scales: torch.Tensor, out=None):
    """E5M2 codes [T, D] + fp32 row scales [T] -> bf16 [T, D]."""
    _need(q.dtype == torch.uint8 and q.dim() == 2 and q.stride(1) == 1, "q must be 2-D uint8, rows contiguous")
    _need(scales.dtype == torch.float32 and scales.is_contiguous(), "scales must be contiguous float32")
    T, D = q.shape
    if out is None:
        out = torch.empty(T, D, dtype=torch.bfloat16, device=q.device)
    _shape(scales, (T,), "scales")
    _need(out.dtype == torch.bfloat16 and out.dim() == 2 and out.stride(1) == 1, "out must be 2-D bf16, rows contiguous")
    _shape(out, (T, D), "out")
    _on_gpu(q, scales, out)
    rc = lib().fp8_kv_dequant(_p(q), T, D, q.stride(0), _p(scales), _p(out), out.stride(0), _stream(q))
    _check("fp8_kv_dequant", rc)
    return out


class DelayedScaler:
    """Per-tensor delayed scaling with an amax history (state in device
    memory): quantize(x) uses the scale from earlier steps and returns
    (codes uint8, scale_used float32 [1]); the state then holds the next
    scale.  algo "max" (window maximum) or "latest"; divisor 400 by default."""

    def __init__(self, history_len=16, algo="max", divisor=400.0, device="cuda"):
        _need(algo in ("max", "latest"), "algo must be 'max' or 'latest'")
        self.history_len = int(history_len)
        self.algo = 0 if algo == "max" else 1
        self.divisor = float(divisor)
        nbytes = DELAYED_HEADER_BYTES + 4 * self.history_len
        self.state = torch.empty((nbytes + 15) // 16 * 16, dtype=torch.uint8, device=device)
        self.reset()

    def reset(self):
        _on_gpu(self.state)
        rc = lib().fp8_delayed_state_init(_p(self.state), self.history_len, _stream(self.state))
        _check("fp8_delayed_state_init", rc)

    def quantize(self, x: torch.Tensor, q=None, scale_used=None):
        _need(x.dtype == torch.bfloat16 and x.is_contiguous(), "x must be contiguous bf16")
        if q is None:
            q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        if scale_used is None:
            scale_used = torch.empty(1, dtype=torch.float32, device=x.device)
        _need(q.dtype == torch.uint8 and q.is_contiguous() and q.numel() == x.numel(),
              "q must be contiguous uint8 with one code per element of x")
        _need(scale_used.dtype == torch.float32 and scale_used.numel() >= 1, "scale_used must be float32 [1]")
        _on_gpu(x, self.state, q, scale_used)
        rc = lib().fp8_delayed_quant(_p(x), x.numel(), _p(self.state), self.history_len, self.algo,
                                     self.divisor, _p(q), _p(scale_used), _stream(x))
        _check("fp8_delayed_quant", rc)
        return q, scale_used

    def quantize_noalloc(self, x: torch.Tensor, q: torch.Tensor, scale_used: torch.Tensor):
        """The same step through fp8_delayed_quant_noalloc: the caller
        passes the outputs, and the library's static per-GPU scratch holds
        the step in flight (steps on one GPU must not overlap)."""
        _need(x.dtype == torch.bfloat16 and x.is_contiguous(), "x must be contiguous bf16")
        _need(q.dtype == torch.uint8 and q.is_contiguous() and q.numel() == x.numel(),
              "q must be contiguous uint8 with one code per element of x")
        _need(scale_used.dtype == torch.float32 and scale_used.numel() >= 1, "scale_used must be float32 [1]")
        _on_gpu(x, self.state, q, scale_used)
        rc = lib().fp8_delayed_quant_noalloc(_p(x), x.numel(), _p(self.state), self.history_len, self.algo,
                                             self.divisor, _p(q), _p(scale_used), _stream(x))
        _check("fp8_delayed_quant_noalloc", rc)
        return q, scale_used


def _codes(t, name):
    _need(t.dtype == torch.uint8 and t.dim() == 2 and t.stride(1) == 1, f"{name} must be 2-D uint8 codes, rows contiguous")


def _gemm_operands(a, a_scales, w, w_scales):
    """Codes a [M, K] and w [N, K]; fp32 scales [M, K/128] and
    [N/128, K/128], contiguous (the layouts the kernels index)."""
    _codes(a, "a")
    _codes(w, "w")
    M, K = a.shape
    N = w.shape[0]
    _need(w.shape[1] == K, f"w must be [N, K] with K = {K}")
    _need(a_scales.dtype == torch.float32 and w_scales.dtype == torch.float32, "scales must be float32")
    _need(a_scales.is_contiguous() and w_scales.is_contiguous(), "scales must be contiguous")
    _shape(a_scales, (M, K // 128), "a_scales")
    _shape(w_scales, (N // 128, K // 128), "w_scales")


def _gemm_output(y, rows, N, out_dtype):
    _need(out_dtype in (torch.bfloat16, torch.float32), "out_dtype must be bfloat16 or float32")
    _need(y.dtype == out_dtype and y.dim() == 2 and y.stride(1) == 1, f"y must be 2-D {out_dtype}, rows contiguous")
    _shape(y, (rows, N), "y")


def _grouped_operands(a, a_scales, row_index, expert_offsets, w, w_scales, out_dtype):
    """Token codes a [T, K] and scales [T, K/128], routing int32 row_index [R]
    and expert_offsets [E+1], expert weights [E, N, K] with scales
    [E, N/128, K/128], all contiguous."""
    _need(a.dtype == torch.uint8 and a.dim() == 2 and a.is_contiguous(), "a must be contiguous 2-D uint8 codes")
    _need(w.dtype == torch.uint8 and w.dim() == 3 and w.is_contiguous(), "w must be contiguous uint8 [E, N, K]")
    T, K = a.shape
    E, N, Kw = w.shape
    _need(Kw == K, f"w must be [E, N, K] with K = {K}")
    _need(row_index.dtype == torch.int32 and expert_offsets.dtype == torch.int32, "routing must be int32")
    _need(row_index.dim() == 1 and row_index.is_contiguous(), "row_index must be a contiguous 1-D tensor")
    _need(expert_offsets.dim() == 1 and expert_offsets.is_contiguous(), "expert_offsets must be a contiguous 1-D tensor")
    _need(expert_offsets.numel() == E + 1, f"expert_offsets must hold E + 1 = {E + 1} entries")
    _need(a_scales.dtype == torch.float32 and a_scales.is_contiguous(), "a_scales must be contiguous float32")
    _shape(a_scales, (T, K // 128), "a_scales")
    _need(w_scales.dtype == torch.float32 and w_scales.is_contiguous(), "w_scales must be contiguous float32")
    _shape(w_scales, (E, N // 128, K // 128), "w_scales")
    _need(out_dtype in (torch.bfloat16, torch.float32), "out_dtype must be bfloat16 or float32")
    od = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    return T, row_index.shape[0], E, N, K, od


def fp8_block_gemm(a, a_scales, w, w_scales, out_dtype=torch.bfloat16, y=None):
    """y[M, N] = block-scaled FP8 GEMM of codes a [M, K] and w [N, K] with
    fp32 scales a_scales [M, K/128] and w_scales [N/128, K/128]."""
    _gemm_operands(a, a_scales, w, w_scales)
    M, K = a.shape
    N = w.shape[0]
    od = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    if y is None:
        y = torch.empty(M, N, dtype=out_dtype, device=a.device)
    _gemm_output(y, M, N, out_dtype)
    _on_gpu(a, a_scales, w, w_scales, y)
    rc = lib().fp8_block_gemm(_p(a), a.stride(0) if M else K, _p(a_scales), _p(w), w.stride(0),
                              _p(w_scales), M, N, K, _p(y), y.stride(0) if M else N, od, _stream(a))
    _check("fp8_block_gemm", rc)
    return y


def fp8_weight_pack(w: torch.Tensor, out=None):
    """Weight codes uint8 [N, K] or [G, N, K] (row-major) -> the packed
    layout read by fp8_block_gemm_packed / fp8_grouped_gemm_packed, returned
    as a contiguous uint8 tensor of the same shape whose bytes are in packed
    order (1 KB chunks of 16 rows x 64 codes, K outermost)."""
    _need(w.dtype == torch.uint8 and w.dim() in (2, 3), "w must be uint8 [N, K] or [G, N, K]")
    _need(w.stride(-1) == 1, "w rows must be contiguous")
    G = 1 if w.dim() == 2 else w.shape[0]
    N, K = w.shape[-2], w.shape[-1]
    ld = w.stride(-2)
    _need(w.dim() == 2 or G == 1 or w.stride(0) == N * ld, "matrices of w must be [N][ld] one after another")
    if out is None:
        out = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    _need(out.dtype == torch.uint8 and out.is_contiguous() and out.numel() == G * N * K,
          "out must be contiguous uint8 with G*N*K bytes")
    _on_gpu(w, out)
    rc = lib().fp8_weight_pack(_p(w), G, N, K, ld, _p(out), _stream(w))
    _check("fp8_weight_pack", rc)
    return out


def fp8_block_gemm_packed(a, a_scales, w_packed, w_scales, out_dtype=torch.bfloat16, y=None):
    """fp8_block_gemm with the weight codes from fp8_weight_pack (shape [N, K])."""
    _need(w_packed.dim() == 2 and w_packed.is_contiguous(), "w_packed must be a contiguous [N, K] tensor")
    _gemm_operands(a, a_scales, w_packed, w_scales)
    M, K = a.shape
    N = w_packed.shape[0]
    od = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    if y is None:
        y = torch.empty(M, N, dtype=out_dtype, device=a.device)
    _gemm_output(y, M, N, out_dtype)
    _on_gpu(a, a_scales, w_packed, w_scales, y)
    rc = lib().fp8_block_gemm_packed(_p(a), a.stride(0) if M else K, _p(a_scales), _p(w_packed), _p(w_scales),
                                     M, N, K, _p(y), y.stride(0) if M else N, od, _stream(a))
    _check("fp8_block_gemm_packed", rc)
    return y


def fp8b_gemm_probe(kind: int, a, a_scales, w_packed, w_scales, y=None):
    """The prefill block GEMM kernel with every tile reading tile (0, 0)'s
    operands (a measurement aid, not a step of the method): the same work as
    fp8_block_gemm_packed with bf16 output, no operand traffic beyond L2.
    a [M, K] contiguous, w_packed [N, K]; M, N, K multiples of 128."""
    _need(w_packed.dim() == 2 and w_packed.is_contiguous(), "w_packed must be a contiguous [N, K] tensor")
    _gemm_operands(a, a_scales, w_packed, w_scales)
    _need(a.is_contiguous(), "a must be contiguous")
    M, K = a.shape
    N = w_packed.shape[0]
    if y is None:
        y = torch.empty(M, N, dtype=torch.bfloat16, device=a.device)
    _gemm_output(y, M, N, torch.bfloat16)
    _need(y.is_contiguous(), "y must be contiguous")
    _on_gpu(a, a_scales, w_packed, w_scales, y)
    rc = lib().fp8b_gemm_probe(int(kind), _p(a), _p(a_scales), _p(w_packed), _p(w_scales), M, N, K, _p(y),
                               _stream(a))
    _check("fp8b_gemm_probe", rc)
    return y


def mxfp8_gemm(a, a_e8m0, b, b_e8m0, y=None):
    """y[M, N] (fp32) = MXFP8 GEMM of codes a [M, K], b [N, K] with E8M0
    bytes a_e8m0 [M, K/32], b_e8m0 [N, K/32]."""
    _codes(a, "a")
    _codes(b, "b")
    M, K = a.shape
    N = b.shape[0]
    _need(b.shape[1] == K, f"b must be [N, K] with K = {K}")
    for t, rows, name in ((a_e8m0, M, "a_e8m0"), (b_e8m0, N, "b_e8m0")):
        _need(t.dtype == torch.uint8 and t.is_contiguous(), f"{name} must be contiguous uint8 E8M0 bytes")
        _shape(t, (rows, K // 32), name)
    if y is None:
        y = torch.empty(M, N, dtype=torch.float32, device=a.device)
    _gemm_output(y, M, N, torch.float32)
    _on_gpu(a, a_e8m0, b, b_e8m0, y)
    rc = lib().mxfp8_gemm(_p(a), a.stride(0) if M else K, _p(a_e8m0), _p(b), b.stride(0), _p(b_e8m0),
                          M, N, K, _p(y), y.stride(0) if M else N, _stream(a))
    _check("mxfp8_gemm", rc)
    return y


def fp8_grouped_gemm(a, a_scales, row_index, expert_offsets, w, w_scales, out_dtype=torch.bfloat16, y=None):
    """Grouped MoE GEMM: a [T, K] token codes, a_scales [T, K/128],
    row_index int32 [R], expert_offsets int32 [E+1] (device), w [E, N, K],
    w_scales [E, N/128, K/128] -> y [R, N] in routed order."""
    T, R, E, N, K, od = _grouped_operands(a, a_scales, row_index, expert_offsets, w, w_scales, out_dtype)
    if y is None:
        y = torch.empty(R, N, dtype=out_dtype, device=a.device)
    _need(y.is_contiguous(), "y must be contiguous")
    _gemm_output(y, R, N, out_dtype)
    _on_gpu(a, a_scales, row_index, expert_offsets, w, w_scales, y)
    rc = lib().fp8_grouped_gemm(_p(a), _p(a_scales), T, _p(row_index), _p(expert_offsets), R, E,
                                _p(w), _p(w_scales), N, K, _p(y), od, _stream(a))
    _check("fp8_grouped_gemm", rc)
    return y


def fp8_grouped_gemm_packed(a, a_scales, row_index, expert_offsets, w_packed, w_scales, out_dtype=torch.bfloat16,
                            y=None):
    """fp8_grouped_gemm with the expert weights from fp8_weight_pack (shape [E, N, K])."""
    T, R, E, N, K, od = _grouped_operands(a, a_scales, row_index, expert_offsets, w_packed, w_scales, out_dtype)
    if y is None:
        y = torch.empty(R, N, dtype=out_dtype, device=a.device)
    _need(y.is_contiguous(), "y must be contiguous")
    _gemm_output(y, R, N, out_dtype)
    _on_gpu(a, a_scales, row_index, expert_offsets, w_packed, w_scales, y)
    rc = lib().fp8_grouped_gemm_packed(_p(a), _p(a_scales), T, _p(row_index), _p(expert_offsets), R, E,
                                       _p(w_packed), _p(w_scales), N, K, _p(y), od, _stream(a))
    _check("fp8_grouped_gemm_packed", rc)
    return y


def fp8_cast_f32(x: torch.Tensor, fmt=FMT_E4M3, q=None):
    """FP8Cast with unit scale: clamp to +-Fmax, round to nearest even."""
    _need(x.dtype == torch.float32 and x.is_contiguous(), "x must be contiguous float32")
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _need(q.dtype == torch.uint8 and q.is_contiguous() and q.numel() == x.numel(),
          "q must be contiguous uint8 with one code per element of x")
    _on_gpu(x, q)
    rc = lib().fp8_cast_f32(_p(x), x.numel(), int(fmt), _p(q), _stream(x))
    _check("fp8_cast_f32", rc)
    return q


def linear(x: torch.Tensor, w_q, w_scales, scale_fmt="fp32", out_dtype=torch.bfloat16, packed=False):
    """W8A8 linear layer: act_quant(x) then the block-scaled GEMM (packed:
    w_q is fp8_weight_pack of the weight codes)."""
    a, sa = fp8_act_quant(x, 128, scale_fmt)
    if sa.dtype != torch.float32:
        raise ValueError("the block GEMM takes fp32 or ue8m0 (fp32-stored) scales")
    gemm = fp8_block_gemm_packed if packed else fp8_block_gemm
    return gemm(a, sa, w_q, w_scales, out_dtype)


def fp8b_mfma_loop(kind: int, ops: torch.Tensor, iters: int, workgroups: int, out=None):
    """The MFMA-only measurement loop (a measurement aid, not a step of the
    method): ops is int32/uint32-sized [64, 64] operand words on the device;
    returns out, float32 [workgroups, 256].  FLOPs of one call:
    workgroups * 4 * iters * 2 * MFMA_LOOP_FLOPS[kind]."""
    _need(ops.is_cuda and ops.element_size() == 4 and ops.numel() == 64 * 64 and ops.is_contiguous(),
          "ops must be 64 x 64 contiguous 4-byte words on the GPU")
    if out is None:
        out = torch.empty(workgroups, 256, dtype=torch.float32, device=ops.device)
    _need(out.dtype == torch.float32 and out.numel() >= workgroups * 256 and out.is_contiguous(),
          "out must hold workgroups * 256 contiguous float32")
    _on_gpu(ops, out)
    rc = lib().fp8b_mfma_loop(int(kind), _p(ops), int(iters), int(workgroups), _p(out), _stream(ops))
    _check("fp8b_mfma_loop", rc)
    return out


def fp8b_stream_probe(kind: int, x: torch.Tensor, q: torch.Tensor, scales: torch.Tensor):
    """The act_quant launch with its arithmetic removed (a measurement aid,
    not a step of the method): PROBE_COPY moves the same bytes (q = low byte
    of each bf16, scales = 0), PROBE_EMPTY launches the same grid and does
    nothing.  x bf16 [M, K], q uint8 [M, K], scales float32 [M, K/128], all
    contiguous on one GPU."""
    _need(x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_contiguous(), "x must be contiguous 2-D bf16")
    M, K = x.shape
    _need(q.dtype == torch.uint8 and q.is_contiguous(), "q must be contiguous uint8")
    _shape(q, (M, K), "q")
    _need(scales.dtype == torch.float32 and scales.is_contiguous(), "scales must be contiguous float32")
    _shape(scales, (M, K // 128), "scales")
    _on_gpu(x, q, scales)
    rc = lib().fp8b_stream_probe(int(kind), _p(x), M, K, _p(q), _p(scales), _stream(x))
    _check("fp8b_stream_probe", rc)
    return q
