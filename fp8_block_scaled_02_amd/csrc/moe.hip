// moe.hip -- the gate-weighted combine that closes a block-scale MoE layer
// (ROCm 7.0 FP8 article, section 2: the block-scale fused MoE operator; the
// DeepSeek-V3 guide's configuration: 8 active experts per token).
//
// After the grouped GEMM has produced one output row per routed (token,
// slot) pair, each token's output is the gate-weighted sum of its rows:
//   out[t][n] = sum_j gates[t][j] * y[token_rows[t][j]][n],
// accumulated in fp32 in slot order (one FMA per slot), then written as
// fp32 or bf16 (nearest even).  HBM-bound: every routed row is read once
// (2 bytes per element) and every token row written once; each thread
// covers 8 consecutive columns (one 16-byte load per slot).
#include "common.hpp"
#include "launch.hpp"

namespace fp8blk {

template <bool BF16>
__global__ __launch_bounds__(256) void moe_combine_kernel(
    const uint16_t* __restrict__ y, int64_t R, int64_t N, const int32_t* __restrict__ token_rows,
    const float* __restrict__ gates, int64_t T, int topk, void* __restrict__ out) {
  const int64_t cpr = N / 8;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= T * cpr) return;
  const int64_t t = c / cpr, n = (c - t * cpr) * 8;
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  // slots in batches of 8: all loads of a batch are issued before its FMAs,
  // which then run in slot order
  for (int j0 = 0; j0 < topk; j0 += 8) {
    uint4 v[8];
    float g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = make_uint4(0, 0, 0, 0);
      g[j] = 0.0f;
      if (j0 + j < topk) {
        // rows outside [0, R) are a contract violation: clamp so nothing faults
        const int64_t r = min(max((int64_t)token_rows[t * topk + j0 + j], (int64_t)0), R - 1);
        g[j] = gates[t * topk + j0 + j];
        v[j] = *reinterpret_cast<const uint4*>(y + r * N + n);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j0 + j < topk) {
        const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = __builtin_fmaf(g[j], bf16_bits_to_f32(w[i] & 0xffffu), acc[2 * i]);
          acc[2 * i + 1] = __builtin_fmaf(g[j], __uint_as_float(w[i] & 0xffff0000u), acc[2 * i + 1]);
        }
      }
    }
  }
  if (BF16) {
    uint4 o;
    o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
    o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
    o.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
    o.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
    __builtin_nontemporal_store(u32x4{o.x, o.y, o.z, o.w},
                                reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + t * N + n));
  } else {
    float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + t * N + n);
    o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

int launch_moe_combine(const void* y, int64_t R, int64_t N, const int32_t* token_rows, const float* gates,
                       int64_t T, int64_t topk, void* out, int out_bf16, hipStream_t s) {
  const dim3 grid((unsigned)((T * (N / 8) + 255) / 256));
  const uint16_t* yp = static_cast<const uint16_t*>(y);
  if (out_bf16)
    hipLaunchKernelGGL(moe_combine_kernel<true>, grid, dim3(256), 0, s, yp, R, N, token_rows, gates, T, (int)topk,
                       out);
  else
    hipLaunchKernelGGL(moe_combine_kernel<false>, grid, dim3(256), 0, s, yp, R, N, token_rows, gates, T, (int)topk,
                       out);
  return check_launch();
}

}  // namespace fp8blk
