"""CPU oracle for the W8A8 block-scaled FP8 linear layer.

TEST INFRASTRUCTURE ONLY: a plain, slow, obviously correct implementation of
what the GPU path computes, written from the pages (see ``fp8_oracle.h`` for
the sources and readings).  Only the tests, ``__graft_entry__.smoke()`` and
the benchmark's CPU-baseline leg may import this package.  It shares no code
with the HIP library and never imports it.

The arithmetic lives in ``fp8_oracle.c``; this module only marshals numpy
arrays through ctypes.  Every function takes and returns numpy arrays:
bf16 tensors travel as their uint16 bit patterns.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

SCALE_FP32 = 0
SCALE_UE8M0 = 1
SCALE_E8M0_BYTE = 2

_c_u8p = ctypes.POINTER(ctypes.c_uint8)
_c_u16p = ctypes.POINTER(ctypes.c_uint16)
_c_f32p = ctypes.POINTER(ctypes.c_float)
_c_f64p = ctypes.POINTER(ctypes.c_double)
_c_i32p = ctypes.POINTER(ctypes.c_int32)
_c_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def lib():
    """Load (building first if absent) the oracle shared library, or the one
    FP8_ORACLE_LIB names (the sanitizer build of the same source)."""
    global _LIB
    if _LIB is None:
        path = os.environ.get("FP8_ORACLE_LIB") or _build.LIB
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e5m2_value.restype = ctypes.c_double
        L.orc_e5m2_value.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_value.restype = ctypes.c_double
        L.orc_e8m0_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e5m2_encode.restype = ctypes.c_uint8
        L.orc_e5m2_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode_array.argtypes = [_c_f32p, _i64, _c_u8p]
        L.orc_e5m2_encode_array.argtypes = [_c_f32p, _i64, _c_u8p]
        L.orc_scale_fp32.restype = ctypes.c_float
        L.orc_scale_fp32.argtypes = [ctypes.c_float]
        L.orc_scale_pow2_exp.restype = ctypes.c_int
        L.orc_scale_pow2_exp.argtypes = [ctypes.c_float]
        L.orc_act_quant.argtypes = [_c_u16p, _i64, _i64, _i64, ctypes.c_int,
                                    ctypes.c_int, _c_u8p, _i64, ctypes.c_void_p]
        L.orc_dequant_one.restype = ctypes.c_uint16
        L.orc_dequant_one.argtypes = [ctypes.c_uint8, ctypes.c_float]
        L.orc_weight_dequant.argtypes = [_c_u8p, _i64, _i64, _i64, _c_f32p, _c_u16p, _i64]
        L.orc_weight_pack.argtypes = [_c_u8p, _i64, _i64, _i64, _i64, _c_u8p]
        L.orc_kv_quant.argtypes = [_c_u16p, _i64, _i64, _i64, _c_u8p, _i64, _c_f32p]
        L.orc_kv_dequant.argtypes = [_c_u8p, _i64, _i64, _i64, _c_f32p, _c_u16p, _i64]
        L.orc_moe_combine.argtypes = [_c_u16p, _i64, _i64, _c_i32p, _c_f32p, _i64, _i64, _c_f64p, _c_f64p]
        L.orc_delayed_scaling.argtypes = [_c_u16p, _i64, _i64, _i64, ctypes.c_int, ctypes.c_float, _c_u8p, _c_f32p]
        L.orc_weight_quant.argtypes = [_c_u16p, _i64, _i64, _i64, ctypes.c_int,
                                       _c_u8p, _i64, _c_f32p]
        L.orc_block_gemm.argtypes = [_c_u8p, _i64, _c_f32p, _c_u8p, _i64, _c_f32p,
                                     _i64, _i64, _i64, _c_f64p, _c_f64p]
        L.orc_mx_gemm.argtypes = [_c_u8p, _i64, _c_u8p, _c_u8p, _i64, _c_u8p,
                                  _i64, _i64, _i64, _c_f64p, _c_f64p]
        L.orc_grouped_gemm.argtypes = [
            _c_u8p, _c_f32p, _i64, _c_i32p, _c_i32p, _i64, _i64,
            ctypes.POINTER(_c_u8p), ctypes.POINTER(_c_f32p), _i64, _i64,
            _c_i64p, _i64, _c_f64p, _c_f64p]
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_set_num_threads.argtypes = [ctypes.c_int]
        _LIB = L
    return _LIB


def _p(arr, ctype):
    return arr.ctypes.data_as(ctype)


def _c(arr, dtype):
    return np.ascontiguousarray(arr, dtype=dtype)


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the oracle's parallel loops use from now on (n >= 1)."""
    lib().orc_set_num_threads(int(n))


# ---- codecs --------------------------------------------------------------
def e4m3_table() -> np.ndarray:
    """Value of each of the 256 E4M3 codes (fp64; NaN for 0x7F/0xFF)."""
    return np.array([lib().orc_e4m3_value(c) for c in range(256)])


def e5m2_table() -> np.ndarray:
    return np.array([lib().orc_e5m2_value(c) for c in range(256)])


def e8m0_table() -> np.ndarray:
    return np.array([lib().orc_e8m0_value(c) for c in range(256)])


def e4m3_encode(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e4m3_encode_array(_p(v, _c_f32p), v.size, _p(out, _c_u8p))
    return out


def e5m2_encode(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e5m2_encode_array(_p(v, _c_f32p), v.size, _p(out, _c_u8p))
    return out


def scale_fp32(amax: float) -> float:
    return float(lib().orc_scale_fp32(float(amax)))


def scale_pow2_exp(amax: float) -> int:
    return int(lib().orc_scale_pow2_exp(float(amax)))


# ---- quantisers ----------------------------------------------------------
def act_quant(x_bits, block: int, scale_fmt: int):
    """x_bits: uint16 [M, K] bf16 patterns -> (codes uint8 [M, K], scales).

    scales are fp32 [M, K/block] (SCALE_FP32 / SCALE_UE8M0) or uint8
    [M, K/block] (SCALE_E8M0_BYTE)."""
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    q = np.empty((M, K), np.uint8)
    sdt = np.uint8 if scale_fmt == SCALE_E8M0_BYTE else np.float32
    s = np.empty((M, K // block), sdt)
    rc = lib().orc_act_quant(_p(x, _c_u16p), M, K, K, block, scale_fmt,
                             _p(q, _c_u8p), K, s.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError("orc_act_quant rejected its arguments")
    return q, s


def weight_quant(w_bits, scale_fmt: int):
    """w_bits: uint16 [N, K] -> (codes [N, K], fp32 scales [N/128, K/128])."""
    w = _c(w_bits, np.uint16)
    N, K = w.shape
    q = np.empty((N, K), np.uint8)
    s = np.empty((N // 128, K // 128), np.float32)
    rc = lib().orc_weight_quant(_p(w, _c_u16p), N, K, K, scale_fmt,
                                _p(q, _c_u8p), K, _p(s, _c_f32p))
    if rc != 0:
        raise ValueError("orc_weight_quant rejected its arguments")
    return q, s


def weight_dequant(q, scales):
    """codes uint8 [N, K] + fp32 scales [N/128, K/128] -> bf16 bits uint16 [N, K]."""
    q = _c(q, np.uint8)
    s = _c(scales, np.float32)
    N, K = q.shape
    w = np.empty((N, K), np.uint16)
    rc = lib().orc_weight_dequant(_p(q, _c_u8p), N, K, K, _p(s, _c_f32p), _p(w, _c_u16p), K)
    if rc != 0:
        raise ValueError("orc_weight_dequant rejected its arguments")
    return w


def weight_pack(w):
    """Codes uint8 [N, K] or [G, N, K] -> the packed byte order (same shape):
    1 KB chunks (kc, p) of 16 rows x 64 codes at (kc*N/16 + p)*1024, byte
    256g + 16r + b = code [16p + r][64kc + 16g + b] (a storage layout of the
    GPU library; the oracle states it element by element)."""
    w = _c(w, np.uint8)
    shape = w.shape
    if w.ndim == 2:
        w = w[None]
    G, N, K = w.shape
    out = np.empty((G, N, K), np.uint8)
    rc = lib().orc_weight_pack(_p(w, _c_u8p), G, N, K, K, _p(out, _c_u8p))
    if rc != 0:
        raise ValueError("orc_weight_pack rejected its arguments")
    return out.reshape(shape)


def dequant_one(code: int, d: float) -> int:
    return int(lib().orc_dequant_one(int(code), float(d)))


def kv_quant(x_bits):
    """x_bits: uint16 (bf16) [T, D] -> (E5M2 codes uint8 [T, D], fp32 scales [T])."""
    x = _c(x_bits, np.uint16)
    T, D = x.shape
    q = np.empty((T, D), np.uint8)
    s = np.empty(T, np.float32)
    if lib().orc_kv_quant(_p(x, _c_u16p), T, D, D, _p(q, _c_u8p), D, _p(s, _c_f32p)) != 0:
        raise ValueError("orc_kv_quant rejected its arguments")
    return q, s


def kv_dequant(q, scales):
    """E5M2 codes [T, D] + fp32 scales [T] -> bf16 bits uint16 [T, D]."""
    q = _c(q, np.uint8)
    s = _c(scales, np.float32)
    T, D = q.shape
    out = np.empty((T, D), np.uint16)
    if lib().orc_kv_dequant(_p(q, _c_u8p), T, D, D, _p(s, _c_f32p), _p(out, _c_u16p), D) != 0:
        raise ValueError("orc_kv_dequant rejected its arguments")
    return out


def moe_combine(y_bits, token_rows, gates):
    """y bf16 bits [R, N], token_rows int32 [T, k], gates fp32 [T, k] ->
    (out fp64 [T, N], bound fp64 [T, N])."""
    y = _c(y_bits, np.uint16)
    tr = _c(token_rows, np.int32)
    g = _c(gates, np.float32)
    R, N = y.shape
    T, k = tr.shape
    out = np.empty((T, N), np.float64)
    b = np.empty((T, N), np.float64)
    if lib().orc_moe_combine(_p(y, _c_u16p), R, N, _p(tr, _c_i32p), _p(g, _c_f32p), T, k,
                             _p(out, _c_f64p), _p(b, _c_f64p)) != 0:
        raise ValueError("orc_moe_combine rejected its arguments")
    return out, b


def delayed_scaling(x_bits, history_len: int, algo: int, divisor: float = 400.0):
    """x_bits uint16 [S, n] (one bf16 tensor per step) -> (codes [S, n],
    scales used per step fp32 [S])."""
    x = _c(x_bits, np.uint16)
    S, n = x.shape
    q = np.empty((S, n), np.uint8)
    sc = np.empty(S, np.float32)
    if lib().orc_delayed_scaling(_p(x, _c_u16p), S, n, history_len, algo, divisor, _p(q, _c_u8p),
                                 _p(sc, _c_f32p)) != 0:
        raise ValueError("orc_delayed_scaling rejected its arguments")
    return q, sc


# ---- GEMM references -----------------------------------------------------
def block_gemm(a, sa, w, sw):
    """Block-scaled GEMM reference -> (y fp64 [M, N], bound fp64 [M, N])."""
    a = _c(a, np.uint8)
    w = _c(w, np.uint8)
    sa = _c(sa, np.float32)
    sw = _c(sw, np.float32)
    M, K = a.shape
    N = w.shape[0]
    y = np.empty((M, N), np.float64)
    b = np.empty((M, N), np.float64)
    rc = lib().orc_block_gemm(_p(a, _c_u8p), K, _p(sa, _c_f32p), _p(w, _c_u8p), K,
                              _p(sw, _c_f32p), M, N, K, _p(y, _c_f64p), _p(b, _c_f64p))
    if rc != 0:
        raise ValueError("orc_block_gemm rejected its arguments")
    return y, b


def mx_gemm(a, ea, b, eb):
    """MXFP8 GEMM reference -> (y fp64 [M, N], bound fp64 [M, N])."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    ea = _c(ea, np.uint8)
    eb = _c(eb, np.uint8)
    M, K = a.shape
    N = b.shape[0]
    y = np.empty((M, N), np.float64)
    bd = np.empty((M, N), np.float64)
    rc = lib().orc_mx_gemm(_p(a, _c_u8p), K, _p(ea, _c_u8p), _p(b, _c_u8p), K,
                           _p(eb, _c_u8p), M, N, K, _p(y, _c_f64p), _p(bd, _c_f64p))
    if rc != 0:
        raise ValueError("orc_mx_gemm rejected its arguments")
    return y, bd


def grouped_gemm(a, sa, row_index, offs, w_list, sw_list, rows=None):
    """Grouped (MoE) GEMM reference.

    a uint8 [T, K], sa fp32 [T, K/128], row_index int32 [R], offs int32
    [E+1]; w_list / sw_list: length-E lists of per-expert arrays ([N, K]
    codes, [N/128, K/128] scales) or None for experts whose rows are not
    wanted.  rows: optional int64 list of output rows.  Returns (y, bound)
    with one row per requested output row."""
    a = _c(a, np.uint8)
    sa = _c(sa, np.float32)
    ri = _c(row_index, np.int32)
    of = _c(offs, np.int32)
    T, K = a.shape
    E = len(of) - 1
    R = len(ri)
    keep = []
    wp = (_c_u8p * E)()
    sp = (_c_f32p * E)()
    N = None
    for e in range(E):
        if w_list[e] is None:
            wp[e] = _c_u8p()
            sp[e] = _c_f32p()
            continue
        we = _c(w_list[e], np.uint8)
        se = _c(sw_list[e], np.float32)
        keep += [we, se]
        N = we.shape[0]
        wp[e] = _p(we, _c_u8p)
        sp[e] = _p(se, _c_f32p)
    if N is None:
        raise ValueError("no expert weights given")
    if rows is None:
        rr = None
        cnt = R
    else:
        rr = _c(rows, np.int64)
        cnt = len(rr)
    y = np.full((cnt, N), np.nan)
    b = np.full((cnt, N), np.nan)
    rc = lib().orc_grouped_gemm(
        _p(a, _c_u8p), _p(sa, _c_f32p), T, _p(ri, _c_i32p), _p(of, _c_i32p), E, R,
        wp, sp, N, K, None if rr is None else _p(rr, _c_i64p), cnt,
        _p(y, _c_f64p), _p(b, _c_f64p))
    if rc != 0:
        raise ValueError("orc_grouped_gemm rejected its arguments")
    return y, b
