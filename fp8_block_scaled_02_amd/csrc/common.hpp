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
// fraction of its cost.  Per block: y = 1 / d
// (one IEEE division).  Per element: q = x * y, one residual r = x - q * d
// (exact with FMA) and one correction q + r * y (Markstein's method for a
// correctly rounded reciprocal), then the sign of x restored (the
// correction turns (-0) into +0).  Blocks with amax < 2^-62 would put the
// residual below fp32's normal range and use the IEEE division instead.
// (With amax >= 2^-62 the residual of every quotient that can round to a
// nonzero code, E4M3 or E5M2, is a normal fp32.)  Verified exhaustively on
// gfx950 for E4M3: for every positive finite bf16 amax and every bf16 x with
// |x| <= amax, the code of the clamped quotient is identical to the one from
// the IEEE division; the parity tests run one block per bf16 amax for both
// formats.
struct BlockDivisor {
  float d, y;
  bool fast;
};

__device__ __forceinline__ BlockDivisor make_divisor(float amax, float d) {
  BlockDivisor b;
  b.d = d;
  b.fast = amax >= 0x1.0p-62f;
  b.y = 1.0f / d;
  return b;
}

__device__ __forceinline__ float divide(float x, const BlockDivisor& b) {
  if (!b.fast) return x / b.d;
  const float q = x * b.y;
  const float r = __builtin_fmaf(-q, b.d, x);
  return copysignf(__builtin_fmaf(r, b.y, q), x);
}

}  // namespace fp8blk
