// api.hip -- the C ABI of libfp8blk (declared in include/fp8blk.h): host-side
// argument validation, then one launch on the caller's stream.  No
// allocation, no synchronisation, no exceptions across the boundary.
#include <stdint.h>
#include <limits.h>

#include "launch.hpp"

namespace {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }
constexpr int64_t kMaxDim = (int64_t)1 << 30;  // keeps every 32-bit tile index in range
constexpr int64_t kMaxLd = (int64_t)1 << 24;   // GEMM leading dimensions: 32-bit offsets inside a tile
constexpr int64_t kMaxPackedN = (int64_t)1 << 25;  // packed weights: 64 * N bytes per K chunk row, 32-bit

// Arguments shared by the grouped GEMM entry points.
int grouped_check(const uint8_t* a, const float* a_scales, int64_t T, const int32_t* row_index,
                  const int32_t* expert_offsets, int64_t R, int64_t E, const uint8_t* w, const float* w_scales,
                  int64_t N, int64_t K, void* y, int out_dtype) {
  if (out_dtype != FP8B_OUT_F32 && out_dtype != FP8B_OUT_BF16) return FP8B_EUNSUPPORTED;
  if (T < 1 || R < 0 || E < 1 || E > 1024 || N <= 0 || K <= 0) return FP8B_EINVAL;
  if (T > kMaxDim || R > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8B_EINVAL;
  if (N % 128 != 0 || K % 128 != 0) return FP8B_EINVAL;
  if (R == 0) return FP8B_OK;  // no routed rows: nothing is read or written
  if (!a || !a_scales || !row_index || !expert_offsets || !w || !w_scales || !y) return FP8B_EINVAL;
  // the in-kernel work map counts tile items (128 x 128) and stream items
  // (64 weight rows) in 32-bit integers
  if ((R / 128 + E) * (N / 128) + E * (N / 64) >= INT32_MAX) return FP8B_EINVAL;
  // token rows are gathered with 32-bit offsets from the start of a: the
  // token matrix must stay below 4 GiB
  if (T * K >= ((int64_t)1 << 32) || K >= kMaxLd) return FP8B_EINVAL;
  if (!aligned(a, 16) || !aligned(w, 16) || !aligned(y, 16)) return FP8B_EALIGN;
  if (!aligned(a_scales, 4) || !aligned(w_scales, 4) || !aligned(row_index, 4) || !aligned(expert_offsets, 4))
    return FP8B_EALIGN;
  return FP8B_OK;
}

// Arguments shared by the delayed-scaling steps.
int delayed_check(const void* x, int64_t n, const void* state, int64_t history_len, int algo, float amax_divisor,
                  const uint8_t* q, const float* scale_used) {
  if (algo != FP8B_AMAX_MAX && algo != FP8B_AMAX_LATEST) return FP8B_EUNSUPPORTED;
  if (!x || !state || !q || !scale_used) return FP8B_EINVAL;
  if (n <= 0 || n % 8 != 0 || n / 8 / 1024 >= INT32_MAX) return FP8B_EINVAL;
  if (history_len < 1 || history_len > FP8B_DELAYED_MAX_HISTORY) return FP8B_EINVAL;
  if (!(amax_divisor > 0.0f) || amax_divisor > 3.0e38f) return FP8B_EINVAL;
  if (!aligned(x, 16) || !aligned(q, 8) || !aligned(state, 16) || !aligned(scale_used, 4)) return FP8B_EALIGN;
  return FP8B_OK;
}

}  // namespace

#define FP8B_EXPORT __attribute__((visibility("default")))

extern "C" {

FP8B_EXPORT int fp8b_abi_version(void) { return FP8B_ABI_VERSION; }

FP8B_EXPORT const char* fp8b_status_string(int status) {
  switch (status) {
    case FP8B_OK: return "ok";
    case FP8B_EINVAL: return "invalid argument (null pointer, size or multiple)";
    case FP8B_EALIGN: return "misaligned pointer or leading dimension";
    case FP8B_EUNSUPPORTED: return "unsupported format/enum value for this call";
    case FP8B_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

FP8B_EXPORT int fp8_act_quant(const void* x, int64_t M, int64_t K, int64_t ld_x, int block_k, int scale_fmt, uint8_t* q,
                  int64_t ld_q, void* scales, void* stream) {
  if (block_k != 128 && block_k != 32) return FP8B_EUNSUPPORTED;
  if (scale_fmt < FP8B_SCALE_FP32 || scale_fmt > FP8B_SCALE_E8M0_BYTE) return FP8B_EUNSUPPORTED;
  if (scale_fmt == FP8B_SCALE_E8M0_BYTE && block_k != 32) return FP8B_EUNSUPPORTED;
  if (M < 0 || K <= 0 || M > kMaxDim || K > kMaxDim || K % block_k != 0) return FP8B_EINVAL;
  if (ld_x < K || ld_q < K) return FP8B_EINVAL;
  if (M == 0) return FP8B_OK;  // nothing is read or written; empty arrays may be NULL
  if (!x || !q || !scales) return FP8B_EINVAL;
  if (!aligned(x, 16) || ld_x % 8 != 0 || !aligned(q, 8) || ld_q % 8 != 0) return FP8B_EALIGN;
  if (scale_fmt != FP8B_SCALE_E8M0_BYTE && !aligned(scales, 4)) return FP8B_EALIGN;
  if (M * (K / 8) / 512 >= INT32_MAX) return FP8B_EINVAL;
  return fp8blk::launch_act_quant(x, M, K, ld_x, block_k, scale_fmt, q, ld_q, scales, as_stream(stream));
}

FP8B_EXPORT int fp8_weight_quant(const void* w, int64_t N, int64_t K, int64_t ld_w, int scale_fmt, uint8_t* q, int64_t ld_q,
                     float* scales, void* stream) {
  if (scale_fmt != FP8B_SCALE_FP32 && scale_fmt != FP8B_SCALE_UE8M0) return FP8B_EUNSUPPORTED;
  if (!w || !q || !scales) return FP8B_EINVAL;
  if (N <= 0 || K <= 0 || N > kMaxDim || K > kMaxDim || N % 128 != 0 || K % 128 != 0) return FP8B_EINVAL;
  if (ld_w < K || ld_q < K) return FP8B_EINVAL;
  if (!aligned(w, 16) || ld_w % 8 != 0 || !aligned(q, 8) || ld_q % 8 != 0 || !aligned(scales, 4))
    return FP8B_EALIGN;
  return fp8blk::launch_weight_quant(w, N, K, ld_w, scale_fmt, q, ld_q, scales, as_stream(stream));
}

FP8B_EXPORT int fp8_block_gemm(const uint8_t* a, int64_t ld_a, const float* a_scales, const uint8_t* w, int64_t ld_w,
                   const float* w_scales, int64_t M, int64_t N, int64_t K, void* y, int64_t ld_y, int out_dtype,
                   void* stream) {
  if (out_dtype != FP8B_OUT_F32 && out_dtype != FP8B_OUT_BF16) return FP8B_EUNSUPPORTED;
  if (M < 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8B_EINVAL;
  if (N % 128 != 0 || K % 128 != 0 || ld_a < K || ld_w < K || ld_y < N) return FP8B_EINVAL;
  if (ld_a >= kMaxLd || ld_w >= kMaxLd) return FP8B_EINVAL;
  if (M == 0) return FP8B_OK;  // nothing is read or written; empty arrays may be NULL
  if (!a || !a_scales || !w || !w_scales || !y) return FP8B_EINVAL;
  if (!aligned(a, 16) || !aligned(w, 16) || ld_a % 16 != 0 || ld_w % 16 != 0) return FP8B_EALIGN;
  if (!aligned(a_scales, 4) || !aligned(w_scales, 4) || !aligned(y, 16) || ld_y % 8 != 0) return FP8B_EALIGN;
  if (((M + 127) / 128) * (N / 128) >= INT32_MAX) return FP8B_EINVAL;
  return fp8blk::launch_block_gemm(a, ld_a, a_scales, w, ld_w, w_scales, M, N, K, y, ld_y,
                                   out_dtype == FP8B_OUT_BF16, false, as_stream(stream));
}

FP8B_EXPORT int fp8_weight_pack(const uint8_t* w, int64_t G, int64_t N, int64_t K, int64_t ld_w, uint8_t* w_packed,
                                void* stream) {
  if (!w || !w_packed) return FP8B_EINVAL;
  if (G < 1 || N <= 0 || K <= 0 || G > kMaxDim || N > kMaxPackedN || K > kMaxDim) return FP8B_EINVAL;
  if (N % 128 != 0 || K % 128 != 0 || ld_w < K) return FP8B_EINVAL;
  if (!aligned(w, 16) || ld_w % 16 != 0 || !aligned(w_packed, 16)) return FP8B_EALIGN;
  // one thread per 16-byte piece, G * N * K / 16 of them, in one grid
  // dimension (the quotient form cannot overflow)
  if (G > (int64_t)INT32_MAX * 256 / (N * (K / 16))) return FP8B_EINVAL;
  return fp8blk::launch_weight_pack(w, G, N, K, ld_w, w_packed, as_stream(stream));
}

FP8B_EXPORT int fp8_block_gemm_packed(const uint8_t* a, int64_t ld_a, const float* a_scales, const uint8_t* w_packed,
                                      const float* w_scales, int64_t M, int64_t N, int64_t K, void* y, int64_t ld_y,
                                      int out_dtype, void* stream) {
  if (out_dtype != FP8B_OUT_F32 && out_dtype != FP8B_OUT_BF16) return FP8B_EUNSUPPORTED;
  if (M < 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxPackedN || K > kMaxDim) return FP8B_EINVAL;
  if (N % 128 != 0 || K % 128 != 0 || ld_a < K || ld_y < N || ld_a >= kMaxLd) return FP8B_EINVAL;
  if (M == 0) return FP8B_OK;  // nothing is read or written; empty arrays may be NULL
  if (!a || !a_scales || !w_packed || !w_scales || !y) return FP8B_EINVAL;
  if (!aligned(a, 16) || !aligned(w_packed, 16) || ld_a % 16 != 0) return FP8B_EALIGN;
  if (!aligned(a_scales, 4) || !aligned(w_scales, 4) || !aligned(y, 16) || ld_y % 8 != 0) return FP8B_EALIGN;
  if (((M + 127) / 128) * (N / 128) >= INT32_MAX) return FP8B_EINVAL;
  return fp8blk::launch_block_gemm(a, ld_a, a_scales, w_packed, 0, w_scales, M, N, K, y, ld_y,
                                   out_dtype == FP8B_OUT_BF16, true, as_stream(stream));
}

FP8B_EXPORT int mxfp8_gemm(const uint8_t* a, int64_t ld_a, const uint8_t* a_e8m0, const uint8_t* b, int64_t ld_b,
               const uint8_t* b_e8m0, int64_t M, int64_t N, int64_t K, float* y, int64_t ld_y, void* stream) {
  if (M < 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8B_EINVAL;
  if (N % 128 != 0 || K % 128 != 0 || ld_a < K || ld_b < K || ld_y < N) return FP8B_EINVAL;
  if (ld_a >= kMaxLd || ld_b >= kMaxLd) return FP8B_EINVAL;
  if (M == 0) return FP8B_OK;  // nothing is read or written; empty arrays may be NULL
  if (!a || !a_e8m0 || !b || !b_e8m0 || !y) return FP8B_EINVAL;
  if (!aligned(a, 16) || !aligned(b, 16) || ld_a % 16 != 0 || ld_b % 16 != 0) return FP8B_EALIGN;
  if (!aligned(a_e8m0, 4) || !aligned(b_e8m0, 4) || !aligned(y, 16) || ld_y % 4 != 0) return FP8B_EALIGN;
  if (((M + 127) / 128) * (N / 128) >= INT32_MAX) return FP8B_EINVAL;
  return fp8blk::launch_mx_gemm(a, ld_a, a_e8m0, b, ld_b, b_e8m0, M, N, K, y, ld_y, as_stream(stream));
}

FP8B_EXPORT int fp8_grouped_gemm(const uint8_t* a, const float* a_scales, int64_t T, const int32_t* row_index,
                     const int32_t* expert_offsets, int64_t R, int64_t E, const uint8_t* w, const float* w_scales,
                     int64_t N, int64_t K, void* y, int out_dtype, void* stream) {
  const int rc = grouped_check(a, a_scales, T, row_index, expert_offsets, R, E, w, w_scales, N, K, y, out_dtype);
  if (rc != FP8B_OK || R == 0) return rc;
  return fp8blk::launch_grouped_gemm(a, a_scales, T, row_index, expert_offsets, R, E, w, w_scales, N, K, y,
                                     out_dtype == FP8B_OUT_BF16, false, as_stream(stream));
}

FP8B_EXPORT int fp8_grouped_gemm_packed(const uint8_t* a, const float* a_scales, int64_t T, const int32_t* row_index,
                                        const int32_t* expert_offsets, int64_t R, int64_t E, const uint8_t* w_packed,
                                        const float* w_scales, int64_t N, int64_t K, void* y, int out_dtype,
                                        void* stream) {
  const int rc =
      grouped_check(a, a_scales, T, row_index, expert_offsets, R, E, w_packed, w_scales, N, K, y, out_dtype);
  if (rc != FP8B_OK) return rc;
  if (N > kMaxPackedN) return FP8B_EINVAL;
  if (R == 0) return FP8B_OK;
  return fp8blk::launch_grouped_gemm(a, a_scales, T, row_index, expert_offsets, R, E, w_packed, w_scales, N, K, y,
                                     out_dtype == FP8B_OUT_BF16, true, as_stream(stream));
}

FP8B_EXPORT int fp8_weight_dequant(const uint8_t* q, int64_t N, int64_t K, int64_t ld_q, const float* scales, void* w,
                                   int64_t ld_w, void* stream) {
  if (!q || !scales || !w) return FP8B_EINVAL;
  if (N <= 0 || K <= 0 || N > kMaxDim || K > kMaxDim || N % 128 != 0 || K % 128 != 0) return FP8B_EINVAL;
  if (ld_q < K || ld_w < K) return FP8B_EINVAL;
  if (!aligned(q, 16) || ld_q % 16 != 0 || !aligned(w, 16) || ld_w % 8 != 0 || !aligned(scales, 4))
    return FP8B_EALIGN;
  if (N * (K / 16) / 256 >= INT32_MAX) return FP8B_EINVAL;
  return fp8blk::launch_weight_dequant(q, N, K, ld_q, scales, w, ld_w, as_stream(stream));
}

FP8B_EXPORT int fp8_moe_combine(const void* y, int64_t R, int64_t N, const int32_t* token_rows, const float* gates,
                                int64_t T, int64_t topk, void* out, int out_dtype, void* stream) {
  if (out_dtype != FP8B_OUT_F32 && out_dtype != FP8B_OUT_BF16) return FP8B_EUNSUPPORTED;
  if (R < 0 || R > kMaxDim || N <= 0 || N > kMaxDim || N % 8 != 0 || T < 0 || T > kMaxDim) return FP8B_EINVAL;
  if (topk < 1 || topk > 64) return FP8B_EINVAL;
  if (T == 0) return FP8B_OK;  // nothing is read or written; empty arrays may be NULL
  if (R < 1 || !y || !token_rows || !gates || !out) return FP8B_EINVAL;
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(token_rows, 4) || !aligned(gates, 4)) return FP8B_EALIGN;
  if (T * (N / 8) / 256 >= INT32_MAX) return FP8B_EINVAL;
  return fp8blk::launch_moe_combine(y, R, N, token_rows, gates, T, topk, out, out_dtype == FP8B_OUT_BF16,
                                    as_stream(stream));
}

FP8B_EXPORT int fp8_kv_quant(const void* x, int64_t T, int64_t D, int64_t ld_x, uint8_t* q, int64_t ld_q, float* scales,
                             void* stream) {
  if (T < 0 || T > kMaxDim || D <= 0 || D > 16384 || D % 16 != 0 || ld_x < D || ld_q < D) return FP8B_EINVAL;
  if (T == 0) return FP8B_OK;  // nothing is read or written; empty arrays may be NULL
  if (!x || !q || !scales) return FP8B_EINVAL;
  if (!aligned(x, 16) || ld_x % 8 != 0 || !aligned(q, 8) || ld_q % 8 != 0 || !aligned(scales, 4))
    return FP8B_EALIGN;
  return fp8blk::launch_kv_quant(x, T, D, ld_x, q, ld_q, scales, as_stream(stream));
}

FP8B_EXPORT int fp8_kv_dequant(const uint8_t* q, int64_t T, int64_t D, int64_t ld_q, const float* scales, void* out,
                               int64_t ld_out, void* stream) {
  if (T < 0 || T > kMaxDim || D <= 0 || D > 16384 || D % 16 != 0 || ld_q < D || ld_out < D) return FP8B_EINVAL;
  if (T == 0) return FP8B_OK;  // nothing is read or written; empty arrays may be NULL
  if (!q || !scales || !out) return FP8B_EINVAL;
  if (!aligned(q, 16) || ld_q % 16 != 0 || !aligned(out, 16) || ld_out % 8 != 0 || !aligned(scales, 4))
    return FP8B_EALIGN;
  return fp8blk::launch_kv_dequant(q, T, D, ld_q, scales, out, ld_out, as_stream(stream));
}

FP8B_EXPORT int fp8_delayed_state_init(void* state, int64_t history_len, void* stream) {
  if (!state) return FP8B_EINVAL;
  if (history_len < 1 || history_len > FP8B_DELAYED_MAX_HISTORY) return FP8B_EINVAL;
  if (!aligned(state, 16)) return FP8B_EALIGN;
  return fp8blk::launch_delayed_init(state, history_len, as_stream(stream));
}

FP8B_EXPORT int fp8_delayed_quant(const void* x, int64_t n, void* state, int64_t history_len, int algo,
                                  float amax_divisor, uint8_t* q, float* scale_used, void* stream) {
  const int rc = delayed_check(x, n, state, history_len, algo, amax_divisor, q, scale_used);
  if (rc != FP8B_OK) return rc;
  return fp8blk::launch_delayed_quant(x, n, state, history_len, algo, amax_divisor, q, scale_used,
                                      as_stream(stream));
}

FP8B_EXPORT int fp8_delayed_quant_noalloc(const void* x, int64_t n, void* state, int64_t history_len, int algo,
                                          float amax_divisor, uint8_t* q, float* scale_used, void* stream) {
  const int rc = delayed_check(x, n, state, history_len, algo, amax_divisor, q, scale_used);
  if (rc != FP8B_OK) return rc;
  return fp8blk::launch_delayed_quant_noalloc(x, n, state, history_len, algo, amax_divisor, q, scale_used,
                                              as_stream(stream));
}

FP8B_EXPORT int fp8_cast_f32(const float* x, int64_t n, int fmt, uint8_t* q, void* stream) {
  if (fmt != FP8B_FMT_E4M3 && fmt != FP8B_FMT_E5M2) return FP8B_EUNSUPPORTED;
  if (n < 0 || n / 1024 >= INT32_MAX) return FP8B_EINVAL;
  if (n == 0) return FP8B_OK;  // nothing is read or written; empty arrays may be NULL
  if (!x || !q) return FP8B_EINVAL;
  if (!aligned(x, 4)) return FP8B_EALIGN;
  return fp8blk::launch_cast(x, n, fmt, q, as_stream(stream));
}

FP8B_EXPORT int fp8b_stream_probe(int kind, const void* x, int64_t M, int64_t K, uint8_t* q, float* scales,
                                  void* stream) {
  if (kind != FP8B_PROBE_COPY && kind != FP8B_PROBE_EMPTY) return FP8B_EUNSUPPORTED;
  if (!x || !q || !scales) return FP8B_EINVAL;
  if (M < 1 || K <= 0 || M > kMaxDim || K > kMaxDim || K % 128 != 0) return FP8B_EINVAL;
  if (!aligned(x, 16) || !aligned(q, 8) || !aligned(scales, 4)) return FP8B_EALIGN;
  if (M * (K / 8) / 512 >= INT32_MAX) return FP8B_EINVAL;
  return fp8blk::launch_stream_probe(kind, x, M, K, q, scales, as_stream(stream));
}

FP8B_EXPORT int fp8b_gemm_probe(int kind, const uint8_t* a, const float* a_scales, const uint8_t* w_packed,
                                const float* w_scales, int64_t M, int64_t N, int64_t K, void* y, void* stream) {
  if (kind != FP8B_GEMM_PROBE_TILE0) return FP8B_EUNSUPPORTED;
  if (!a || !a_scales || !w_packed || !w_scales || !y) return FP8B_EINVAL;
  if (M < 128 || N < 128 || K < 128 || M % 128 != 0 || N % 128 != 0 || K % 128 != 0) return FP8B_EINVAL;
  if (M > kMaxDim || N > kMaxPackedN || K >= kMaxLd || N >= kMaxLd) return FP8B_EINVAL;
  if ((M / 128) * (N / 128) >= INT32_MAX) return FP8B_EINVAL;
  if (!aligned(a, 16) || !aligned(w_packed, 16) || !aligned(y, 16) || !aligned(a_scales, 4) ||
      !aligned(w_scales, 4))
    return FP8B_EALIGN;
  return fp8blk::launch_gemm_probe(a, a_scales, w_packed, w_scales, M, N, K, y, as_stream(stream));
}

FP8B_EXPORT int fp8b_mfma_loop(int kind, const uint32_t* ops, int64_t iters, int64_t workgroups, float* out,
                               void* stream) {
  if (kind != FP8B_MFMA_BF16_16X16X32 && kind != FP8B_MFMA_FP8_16X16X128) return FP8B_EUNSUPPORTED;
  if (!ops || !out) return FP8B_EINVAL;
  if (iters < 1 || iters > ((int64_t)1 << 30) || workgroups < 1 || workgroups > ((int64_t)1 << 20))
    return FP8B_EINVAL;
  if (!aligned(ops, 16) || !aligned(out, 4)) return FP8B_EALIGN;
  return fp8blk::launch_mfma_loop(kind, ops, iters, workgroups, out, as_stream(stream));
}

}  // extern "C"
