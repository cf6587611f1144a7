// probe.hip -- measurement aids, not steps of the method:
//  * the MFMA-only loop behind fp8b_mfma_loop: dense matrix-core work on
//    operands held in registers, with no memory traffic, conversion or
//    rescale.  Its rate is the ceiling this part sustains for one MFMA
//    instruction, clock and power limits included, measured beside the GEMMs;
//  * the streaming copy and the empty launch behind fp8b_stream_probe: the
//    grid, workgroup shape, loads and stores of act_quant (128-blocks, fp32
//    scales) without its arithmetic, and the same grid returning at once,
//    which time act_quant's streaming rate and its launch and drain.
#include "common.hpp"
#include "launch.hpp"

namespace fp8blk {
namespace {

// Independent accumulators per wave.  Two chains compile to a loop of bare
// MFMAs; with four or more the compiler rotated the accumulators through
// AGPRs with a dozen register moves per round.  Latency is hidden by
// several waves per SIMD instead.
constexpr int kChains = 2;
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Lane l of every wave reads its 64 operand words ops[l][0..63] once, then
// runs iters rounds of kChains MFMAs, chain c on its own operands; each
// lane writes the sum of its accumulators (which keeps the work live).
// Words past those the chains use are not read.
template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop_kernel(const uint32_t* __restrict__ ops, int iters,
                                                        float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const u32x4* my = reinterpret_cast<const u32x4*>(ops + 64 * lane);
  v4f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (KIND == FP8B_MFMA_BF16_16X16X32) {
    bf16x8 a[kChains], b[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      a[c] = __builtin_bit_cast(bf16x8, my[2 * c]);
      b[c] = __builtin_bit_cast(bf16x8, my[2 * c + 1]);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c], b[c], acc[c], 0, 0, 0);
    }
  } else {
    i32x8 a[kChains], b[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      const u32x4 a0 = my[4 * c], a1 = my[4 * c + 1], b0 = my[4 * c + 2], b1 = my[4 * c + 3];
      a[c] = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
      b[c] = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    }
    // E4M3 operands (format 0 for both), unit E8M0 scales (127)
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[c], b[c], acc[c], 0, 0, 0, 127, 0, 127);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) s += acc[c][r];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Grid: x = row, y = segment of 256 * UNROLL 16-byte chunks of the row;
// each thread non-temporally loads UNROLL chunks 256 apart (all before any
// store, as act_quant does) and writes the low byte of each bf16 element as
// its code (8-byte non-temporal stores) and 0 as the scale of each
// 128-element block it leads.
constexpr int kCopyUnroll = 4;  // act_quant's chunks per lane

__global__ __launch_bounds__(256) void stream_copy_kernel(const uint16_t* __restrict__ x, int64_t K,
                                                          uint8_t* __restrict__ q, float* __restrict__ scales) {
  const int cpr = (int)(K / 8), nblk = (int)(K / 128);
  const int64_t row = blockIdx.x;
  const int base = (int)blockIdx.y * 256 * kCopyUnroll + (int)threadIdx.x;
  const uint16_t* xr = x + row * K;
  uint8_t* qr = q + row * K;
  u32x4 raw[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int c = base + u * 256;
    raw[u] = c < cpr ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + 8 * c)) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int c = base + u * 256;
    if (c < cpr) {
      u32x2 out;
      out[0] = __builtin_amdgcn_perm(raw[u][1], raw[u][0], 0x06040200u);
      out[1] = __builtin_amdgcn_perm(raw[u][3], raw[u][2], 0x06040200u);
      __builtin_nontemporal_store(out, reinterpret_cast<u32x2*>(qr + 8 * c));
      if ((c % 16) == 0) scales[row * nblk + c / 16] = 0.0f;
    }
  }
}

__global__ __launch_bounds__(256) void empty_kernel() {}

}  // namespace

int launch_stream_probe(int kind, const void* x, int64_t M, int64_t K, uint8_t* q, float* scales,
                        hipStream_t s) {
  const int64_t cpr = K / 8;
  const int64_t segs = (cpr + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll);
  if (segs > 65535 || M > 0x7fffffff) return FP8B_EINVAL;
  const dim3 grid((unsigned)M, (unsigned)segs);
  if (kind == FP8B_PROBE_COPY)
    hipLaunchKernelGGL(stream_copy_kernel, grid, dim3(256), 0, s, static_cast<const uint16_t*>(x), K, q, scales);
  else
    hipLaunchKernelGGL(empty_kernel, grid, dim3(256), 0, s);
  return check_launch();
}

int launch_mfma_loop(int kind, const uint32_t* ops, int64_t iters, int64_t workgroups, float* out,
                     hipStream_t s) {
  const dim3 grid((unsigned)workgroups), block(256);
  if (kind == FP8B_MFMA_BF16_16X16X32)
    hipLaunchKernelGGL((mfma_loop_kernel<FP8B_MFMA_BF16_16X16X32>), grid, block, 0, s, ops, (int)iters, out);
  else
    hipLaunchKernelGGL((mfma_loop_kernel<FP8B_MFMA_FP8_16X16X128>), grid, block, 0, s, ops, (int)iters, out);
  return check_launch();
}

}  // namespace fp8blk
