// launch.hpp -- host-side launch plumbing shared by the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp8blk.h"

namespace fp8blk {

inline int check_launch() {
  return hipGetLastError() == hipSuccess ? FP8B_OK : FP8B_ELAUNCH;
}

int launch_act_quant(const void* x, int64_t M, int64_t K, int64_t ldx, int block, int fmt,
                     uint8_t* q, int64_t ldq, void* scales, hipStream_t s);
int launch_stream_probe(int kind, const void* x, int64_t M, int64_t K, uint8_t* q, float* scales,
                        hipStream_t s);
int launch_weight_quant(const void* w, int64_t N, int64_t K, int64_t ldw, int fmt, uint8_t* q,
                        int64_t ldq, float* scales, hipStream_t s);
int launch_cast(const float* x, int64_t n, int fmt, uint8_t* q, hipStream_t s);
int launch_kv_quant(const void* x, int64_t T, int64_t D, int64_t ldx, uint8_t* q, int64_t ldq, float* scales,
                    hipStream_t s);
int launch_kv_dequant(const uint8_t* q, int64_t T, int64_t D, int64_t ldq, const float* scales, void* out,
                      int64_t ldo, hipStream_t s);
int launch_moe_combine(const void* y, int64_t R, int64_t N, const int32_t* token_rows, const float* gates,
                       int64_t T, int64_t topk, void* out, int out_bf16, hipStream_t s);
int launch_delayed_init(void* state, int64_t L, hipStream_t s);
int launch_delayed_quant(const void* x, int64_t n, void* state, int64_t L, int algo, float divisor, uint8_t* q,
                         float* scale_used, hipStream_t s);
int launch_delayed_quant_noalloc(const void* x, int64_t n, void* state, int64_t L, int algo, float divisor,
                                 uint8_t* q, float* scale_used, hipStream_t s);
int launch_weight_dequant(const uint8_t* q, int64_t N, int64_t K, int64_t ldq, const float* scales,
                          void* w, int64_t ldw, hipStream_t s);
int launch_weight_pack(const uint8_t* w, int64_t G, int64_t N, int64_t K, int64_t ldw, uint8_t* out,
                       hipStream_t s);
// packed: w is in the packed layout of launch_weight_pack (ldw unused)
int launch_block_gemm(const uint8_t* a, int64_t lda, const float* sa, const uint8_t* w,
                      int64_t ldw, const float* sw, int64_t M, int64_t N, int64_t K, void* y,
                      int64_t ldy, int out_bf16, bool packed, hipStream_t s);
int launch_gemm_probe(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, int64_t M, int64_t N,
                      int64_t K, void* y, hipStream_t s);
int launch_mx_gemm(const uint8_t* a, int64_t lda, const uint8_t* ea, const uint8_t* b,
                   int64_t ldb, const uint8_t* eb, int64_t M, int64_t N, int64_t K, float* y,
                   int64_t ldy, hipStream_t s);
int launch_mfma_loop(int kind, const uint32_t* ops, int64_t iters, int64_t workgroups, float* out,
                     hipStream_t s);
int launch_grouped_gemm(const uint8_t* a, const float* sa, int64_t T, const int32_t* row_index,
                        const int32_t* offs, int64_t R, int64_t E, const uint8_t* w,
                        const float* sw, int64_t N, int64_t K, void* y, int out_bf16,
                        bool packed, hipStream_t s);

}  // namespace fp8blk
