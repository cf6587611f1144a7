"""Parity criteria shared by the GPU tests.

fp32 output:  |y - y_ref| <= 1e-5 * B, with B = sum_k |deq a_k * deq w_k|.
bf16 output:  |y - RN_bf16(y_ref)| <= 1 ulp_bf16(RN_bf16(y_ref)), or, for
              cancellation-dominated elements,
              |y - y_ref| <= 1e-5 * B + ulp_bf16(y_ref) / 2.
y_ref and B come from the CPU oracle (exact block sums, fp64 combination).
"""
import numpy as np

REL = 1e-5


def rn_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), in fp64."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                  # x = m * 2^e, |m| in [0.5, 1)
    e = np.maximum(e, -125)             # bf16 subnormal spacing 2^-133
    return np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    return np.ldexp(1.0, e - 8)


def check_f32(y, y_ref, bnd, rel=REL):
    """Returns (ok mask, worst err / allowed)."""
    y = np.asarray(y, np.float64)
    err = np.abs(y - y_ref)
    allowed = rel * bnd
    ok = (err <= allowed) | ((bnd == 0) & (y == 0))
    ratio = np.where(allowed > 0, err / np.where(allowed > 0, allowed, 1), np.where(err > 0, np.inf, 0))
    return ok, float(np.max(ratio)) if ratio.size else 0.0


def check_bf16(y, y_ref, bnd, rel=REL):
    y = np.asarray(y, np.float64)
    r = rn_bf16(y_ref)
    ok1 = (r != 0) & (np.abs(y - r) <= ulp_bf16(r))
    ok2 = np.abs(y - y_ref) <= rel * bnd + 0.5 * ulp_bf16(y_ref)
    ok = ok1 | ok2 | ((bnd == 0) & (y == 0))
    allowed = np.maximum(np.where(r != 0, ulp_bf16(r), 0), rel * bnd + 0.5 * ulp_bf16(y_ref))
    ratio = np.abs(y - r) / np.where(allowed > 0, allowed, 1)
    return ok, float(np.max(ratio)) if ratio.size else 0.0


def assert_parity(y, y_ref, bnd, bf16: bool, what="", rel=REL):
    ok, worst = (check_bf16 if bf16 else check_f32)(y, y_ref, bnd, rel)
    if not ok.all():
        idx = np.argwhere(~ok)
        i = tuple(idx[0])
        raise AssertionError(
            f"{what}: {len(idx)} of {ok.size} outputs out of tolerance; first at {i}: "
            f"y={float(np.asarray(y)[i])!r} ref={float(y_ref[i])!r} bound={float(bnd[i])!r}")
    return worst
