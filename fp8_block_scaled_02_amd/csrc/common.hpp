// common.hpp -- device helpers shared by the gfx950 kernels of libfp8blk.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Maxima of non-negative floats (block amax values) on their bit patterns,
// which order like unsigned integers: one v_max_u32 with a DPP operand per
// step and no float canonicalisation.  row16: quad swaps, then half-row and
// row mirrors (every lane of a 16-lane row ends with the row maximum); quad:
// each aligned quad of lanes.
template <int CTRL>
__device__ __forceinline__ uint32_t umax_dpp(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
  return o > v ? o : v;
}
__device__ __forceinline__ float row16_max_nonneg(float v) {
  uint32_t u = __float_as_uint(v);
  u = umax_dpp<0xB1>(u);
  u = umax_dpp<0x4E>(u);
  u = umax_dpp<0x141>(u);
  u = umax_dpp<0x140>(u);
  return __uint_as_float(u);
}
__device__ __forceinline__ float quad_max_nonneg(float v) {
  uint32_t u = __float_as_uint(v);
  u = umax_dpp<0xB1>(u);
  u = umax_dpp<0x4E>(u);
  return __uint_as_float(u);
}

// max over the 16 lanes of a DPP row (quad swaps, then half-row and row
// mirrors); every lane of the row ends with the row maximum.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

// max over each aligned quad of lanes.
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  return v;
}

// Exponent e of the power-of-two scale: smallest integer with
// amax <= 448 * 2^e, clamped to [-127, 127]; 0 for amax == 0.
// With amax = sig * 2^E (sig in [1, 2)), amax / 448 = (sig / 1.75) * 2^(E-8),
// so e = E - 8 + (sig > 1.75).  Subnormal amax lies far below 448 * 2^-127.
__device__ __forceinline__ int pow2_scale_exp(float amax) {
  uint32_t u = __float_as_uint(amax) & 0x7fffffffu;
  if (u == 0) return 0;
  int ef = (int)(u >> 23);
  if (ef == 0) return -127;
  int e = ef - 127 - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^e as fp32 for e in [-127, 127] (2^-127 is a subnormal).
__device__ __forceinline__ float exp2i(int e) {
  return e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
}

// Pack four fp32 values (already clamped to +-448) into four E4M3 bytes,
// round to nearest even.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

__device__ __forceinline__ uint32_t pack4_e5m2(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, r, true);
  return (uint32_t)r;
}

__device__ __forceinline__ float clamp448(float v) {
  return fminf(fmaxf(v, -448.0f), 448.0f);
}

// Division by a block scale d = fp32(amax / Fmax) (Fmax 448 for E4M3 codes,
// 57344 for E5M2), correctly rounded like the IEEE quotient x / d, at a
// fraction of its cost.  Per block: y ~ 1 / d (a reciprocal estimate and one
// Newton step).  Per element: q = x * y, one residual r = x - q * d (exact
// with FMA) and one correction q + r * y (Markstein's method), then the sign
// of x restored (the correction turns (-0) into +0).  Blocks with
// amax < 2^-62 would put the residual below fp32's normal range and use the
// IEEE division instead.  (With amax >= 2^-62 the residual of every quotient
// that can round to a nonzero code, E4M3 or E5M2, is a normal fp32.)  The
// GPU sweep tests run every positive finite bf16 amax with every bf16 x with
// |x| <= amax through act_quant (E4M3) and the KV quantiser (E5M2) and
// require the oracle's codes -- which, since inputs are bf16, covers every
// (amax, x) pair these kernels can see.
struct BlockDivisor {
  float d, y;
  bool fast;
};

__device__ __forceinline__ BlockDivisor make_divisor(float amax, float d) {
  BlockDivisor b;
  b.d = d;
  b.fast = amax >= 0x1.0p-62f;
  // reciprocal estimate refined by one Newton step (d is normal on the fast
  // path); the per-element correction then rounds the quotient correctly,
  // which the exhaustive sweep (every bf16 amax with every |x| <= amax)
  // checks against the IEEE division on gfx950
  const float y0 = __builtin_amdgcn_rcpf(d);
  b.y = __builtin_fmaf(__builtin_fmaf(-d, y0, 1.0f), y0, y0);
  return b;
}

// d = fp32(amax / fmax) for a positive finite amax, without an IEEE
// division: d0 = RN(amax * c) with c = RN(1 / fmax), the exact residual
// r = amax - d0 * fmax (FMA), then d = RN(d0 + r * c) -- one correction
// step (Markstein's method).  Verified in exact rational arithmetic for
// every positive finite bf16 amax with fmax = 448 and 57344 (the only
// values amax takes here, the maximum of bf16 inputs); amax = 0 gives 1.
__device__ __forceinline__ float block_scale(float amax, float fmax, float c) {
  const float d0 = amax * c;
  const float r = __builtin_fmaf(-d0, fmax, amax);
  const float d = __builtin_fmaf(r, c, d0);
  return amax == 0.0f ? 1.0f : d;
}

__device__ __forceinline__ float divide(float x, const BlockDivisor& b) {
  if (!b.fast) return x / b.d;
  const float q = x * b.y;
  const float r = __builtin_fmaf(-q, b.d, x);
  return copysignf(__builtin_fmaf(r, b.y, q), x);
}

// The same quotient for N values of one block, with the fast / IEEE choice
// taken once for the block (a branch per element cost more than the
// quotient itself).
template <int N>
__device__ __forceinline__ void divide_block(const float (&x)[N], float (&q)[N], const BlockDivisor& b) {
  if (b.fast) {
    // with the residual negated, r' = t * d - x and q = t - r' * y, the
    // zero cases keep the sign of x (x = -0: r' = +0 and q = -0 + -0 = -0)
    // with no copysign; the negations are free source modifiers
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float t = x[i] * b.y;
      const float rn = __builtin_fmaf(t, b.d, -x[i]);
      q[i] = __builtin_fmaf(-rn, b.y, t);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) q[i] = x[i] / b.d;
  }
}

}  // namespace fp8blk
