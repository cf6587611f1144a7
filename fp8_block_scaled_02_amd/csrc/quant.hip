// quant.hip -- quantisation kernels for gfx950.
//
// act_quant: per token, per block of 128 (or 32) channels, amax -> scale ->
// E4M3 codes (DeepSeek-V3 guide, runtime-dispatch snippet; quantizer of
// "FP8 engineering 2026" section 2; Dynamic Scaling of the "FP8 推理"
// notes: scale = amax / 448, fp8 = x / scale).
//
// The work is HBM-bound (2 bytes in, 1 byte + a scale out per element), so
// the kernel is built for streaming: every lane owns 8 consecutive bf16
// (one 16-byte load), the lanes of one quantisation block are adjacent in a
// wavefront, the block maximum is reduced with DPP inside the wave (no LDS,
// no barrier), and each lane writes its 8 codes with one 8-byte
// non-temporal store.
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace fp8blk {

// FMT: 0 fp32 scales, 1 power-of-two scales stored as fp32, 2 E8M0 bytes.
// Grid: x = token row, y = segment of 256 * UNROLL 16-byte chunks of the
// row (so no index needs a division); each thread owns UNROLL chunks 256
// apart, all loaded before any is processed (bytes in flight per lane =
// 16 * UNROLL).
template <int BLOCK, int FMT, int UNROLL>
__global__ __launch_bounds__(256) void act_quant_kernel(
    const uint16_t* __restrict__ x, int64_t K, int64_t ldx,
    uint8_t* __restrict__ q, int64_t ldq, void* __restrict__ scales) {
  constexpr int LPB = BLOCK / 8;  // lanes per quantisation block
  const int cpr = (int)(K / 8);   // 16-byte chunks per row
  const int nblk = (int)(K / BLOCK);
  const int64_t row = blockIdx.x;
  const int base = (int)blockIdx.y * 256 * UNROLL + (int)threadIdx.x;
  const uint16_t* xr = x + row * ldx;
  uint8_t* qr = q + row * ldq;

  uint4 raw[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int c = base + u * 256;
    u32x4 v = {0, 0, 0, 0};
    if (c < cpr) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + 8 * c));
    raw[u] = make_uint4(v[0], v[1], v[2], v[3]);
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int c = base + u * 256;
    float f[8];
    const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = (LPB == 16) ? row16_max_nonneg(amax) : quad_max_nonneg(amax);

    float qv[8];
    const bool ok = c < cpr;
    const bool lead = ok && (c % LPB) == 0;
    const int64_t sidx = row * nblk + c / LPB;
    if (FMT == 0) {
      const float d = block_scale(amax, 448.0f, 1.0f / 448.0f);
      const BlockDivisor bd = make_divisor(amax, d);
      divide_block(f, qv, bd);
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[i] = clamp448(qv[i]);
      if (lead) reinterpret_cast<float*>(scales)[sidx] = d;
    } else {
      const int e = pow2_scale_exp(amax);
      // x / 2^e == x * 2^-e exactly (both are the correctly rounded quotient)
      const float rinv = exp2i(-e);
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[i] = clamp448(f[i] * rinv);
      if (lead) {
        if (FMT == 1)
          reinterpret_cast<float*>(scales)[sidx] = exp2i(e);
        else
          reinterpret_cast<uint8_t*>(scales)[sidx] = (uint8_t)(127 + e);
      }
    }
    if (ok) {
      u32x2 out;
      out[0] = pack4_e4m3(qv[0], qv[1], qv[2], qv[3]);
      out[1] = pack4_e4m3(qv[4], qv[5], qv[6], qv[7]);
      // codes are written once and read by a later kernel: non-temporal
      // (measured 13-18% faster than a plain store)
      __builtin_nontemporal_store(out, reinterpret_cast<u32x2*>(qr + 8 * c));
    }
  }
}

// Weight quantisation: one workgroup per 128x128 tile.  256 threads, each
// owns 8 chunks of 8 bf16; amax is reduced in-wave with DPP, across waves
// through LDS.
template <int FMT>
__global__ __launch_bounds__(256) void weight_quant_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, int64_t ldw,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ scales) {
  __shared__ float red[4];
  const int64_t kt = K / 128;
  const int64_t ti = blockIdx.x / kt, tj = blockIdx.x % kt;
  const int tid = threadIdx.x;
  uint4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 4, ch = c & 15;
    raw[i] = *reinterpret_cast<const uint4*>(w + (ti * 128 + r) * ldw + tj * 128 + ch * 8);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t v[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[j] & 0xffffu)));
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[j] >> 16)));
    }
  }
  amax = row16_max(amax);
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  float d, rinv = 1.0f;
  BlockDivisor bd{};
  if (FMT == 0) {
    d = block_scale(amax, 448.0f, 1.0f / 448.0f);
    bd = make_divisor(amax, d);
  } else {
    const int e = pow2_scale_exp(amax);
    d = exp2i(e);
    rinv = exp2i(-e);
  }
  if (tid == 0) scales[ti * kt + tj] = d;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 4, ch = c & 15;
    const uint32_t v[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
    float f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = bf16_bits_to_f32(v[j] & 0xffffu);
      f[2 * j + 1] = bf16_bits_to_f32(v[j] >> 16);
    }
    if (FMT == 0) {
      divide_block(f, f, bd);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] *= rinv;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = clamp448(f[j]);
    uint2 out;
    out.x = pack4_e4m3(f[0], f[1], f[2], f[3]);
    out.y = pack4_e4m3(f[4], f[5], f[6], f[7]);
    *reinterpret_cast<uint2*>(q + (ti * 128 + r) * ldq + tj * 128 + ch * 8) = out;
  }
}

// FP8Cast with s = 1: clamp to +-Fmax, round to nearest even.  4 values per
// thread.
template <int FMT>
__global__ __launch_bounds__(256) void cast_kernel(const float* __restrict__ x, int64_t n,
                                                   uint8_t* __restrict__ q) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float t = (i + j < n) ? x[i + j] : 0.0f;
    v[j] = FMT == 0 ? clamp448(t) : fminf(fmaxf(t, -57344.0f), 57344.0f);
  }
  const uint32_t p = FMT == 0 ? pack4_e4m3(v[0], v[1], v[2], v[3]) : pack4_e5m2(v[0], v[1], v[2], v[3]);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (i + j < n) q[i + j] = (uint8_t)(p >> (8 * j));
}

// Weight packing: G row-major code matrices [N][ld] -> the packed layout the
// GEMMs can stream (chunk (kc, p) of 1 KB at (kc * N/16 + p) * 1024 holds
// rows 16p .. 16p+15, K bytes 64kc .. 64kc+63, byte 256g + 16r + b = code
// [16p + r][64kc + 16g + b]; matrix i at i * N * K).  A pure permutation,
// done once per weight: each thread writes one 16-byte piece of the output
// in order and reads its 16 codes from one row.
__global__ __launch_bounds__(256) void weight_pack_kernel(
    const uint8_t* __restrict__ w, int64_t G, int64_t N, int64_t K, int64_t ldw, uint8_t* __restrict__ out) {
  const int64_t piece = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 16-byte output piece
  const int64_t per_mat = N * K / 16;
  if (piece >= G * per_mat) return;
  const int64_t mat = piece / per_mat, in_mat = piece - mat * per_mat;
  const int64_t chunk = in_mat >> 6, np = N / 16;
  const int lane = (int)(in_mat & 63), r = lane & 15, g = lane >> 4;
  const int64_t kc = chunk / np, p = chunk - kc * np;
  const u32x4 v = *reinterpret_cast<const u32x4*>(w + (mat * N + 16 * p + r) * ldw + 64 * kc + 16 * g);
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + piece * 16));
}

// KV-cache quantisation ("LLM 推理的 FP8 混合精度工程 2026", section 4: the
// KV cache stored in E5M2 for its range, one scale per token from the
// token's real-time amax).  One cache row (a token's K or V, D values) per
// wave: each lane owns U 16-byte chunks (chunk lane + 64u), the row maximum
// is reduced in-wave (DPP, then two cross-row shuffles), d = amax / 57344,
// codes = E5M2(clamp(x / d)).  Rows past T exit; chunks past D are zeros.
template <int U>
__global__ __launch_bounds__(256) void kv_quant_kernel(
    const uint16_t* __restrict__ x, int64_t T, int64_t D, int64_t ldx,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t nch = D / 8;
  uint4 raw[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = lane + 64 * u;
    u32x4 v = {0, 0, 0, 0};
    if (c < nch) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + t * ldx + 8 * c));
    raw[u] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[i] & 0xffffu)));
      amax = fmaxf(amax, fabsf(__uint_as_float(w[i] & 0xffff0000u)));
    }
  }
  amax = row16_max(amax);
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  const float d = block_scale(amax, 57344.0f, 1.0f / 57344.0f);
  const BlockDivisor bd = make_divisor(amax, d);
  if (lane == 0) scales[t] = d;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = lane + 64 * u;
    if (c >= nch) continue;
    const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
    float f[8], v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    divide_block(f, v, bd);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = fminf(fmaxf(v[i], -57344.0f), 57344.0f);
    u32x2 out;
    out[0] = pack4_e5m2(v[0], v[1], v[2], v[3]);
    out[1] = pack4_e5m2(v[4], v[5], v[6], v[7]);
    __builtin_nontemporal_store(out, reinterpret_cast<u32x2*>(q + t * ldq + 8 * c));
  }
}

// Delayed scaling (ROCm 7.0 FP8/MXFP8/MXFP4 article, training part,
// "Delayed Scaling": a step is quantised with the scale derived from
// earlier steps, and the next scale is taken from the current amax with a
// margin, amax / 400; its pitfall section adds an amax history window with
// the "max" algorithm).  One scale per tensor.  The state lives in device
// memory, laid out as fp8b_delayed_state (scale, running amax bits, next
// history slot, filled count, then the history), so a step is two kernels
// in stream order and never needs the host.
// Mirrors fp8b_delayed_state (include/fp8blk.h).
struct DelayedHeader {
  float scale;
  uint32_t done;
  int32_t pos;
  int32_t filled;
  uint32_t reserved[28];
  uint32_t amax[FP8B_DELAYED_AMAX_SLOTS][32];
};
static_assert(sizeof(DelayedHeader) == FP8B_DELAYED_HEADER_BYTES, "state header layout");
static_assert(sizeof(DelayedHeader) == sizeof(fp8b_delayed_state), "state header layout");

__global__ __launch_bounds__(256) void delayed_init_kernel(uint8_t* __restrict__ st, int L) {
  DelayedHeader* h = reinterpret_cast<DelayedHeader*>(st);
  float* hist = reinterpret_cast<float*>(st + sizeof(DelayedHeader));
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < L) hist[i] = 0.0f;
  if (i < FP8B_DELAYED_AMAX_SLOTS * 32) (&h->amax[0][0])[i] = 0u;
  if (i < 28) h->reserved[i] = 0u;
  if (i == 0) {
    h->scale = 1.0f;
    h->done = 0u;
    h->pos = 0;
    h->filled = 0;
  }
}

// One step: codes = E4M3(clamp(x / d, +-448)) with the stored scale d
// (IEEE division: d comes from another tensor, so the quotient can take any
// magnitude), one chunk of 8192 values per workgroup.  Each workgroup folds
// its amax into one of 16 amax slots (workgroup b into slot b mod 16; the
// 128-byte line at slots + 32 b holds the slot's maximum in word 0 and its
// ticket in word 1: the state's slots, or the library's static scratch for
// fp8_delayed_quant_noalloc) with an atomic max (non-negative floats order
// like their bit patterns), then takes a ticket of its slot; the workgroup
// completing a slot takes a ticket of the step (*done), and the one
// completing the step has
// every workgroup's maximum in the slots (each one's atomic max completed
// before its tickets).  Spreading the atomics over 16 lines keeps them from
// queueing on one word.  That workgroup closes the step: it merges and
// clears the slots, pushes the amax into
// the history, sets the next scale = h / divisor (1 if h = 0), h = the
// window maximum (algo 0) or this step's amax (algo 1), and resets the
// ticket.  Every workgroup has read the old scale before taking its ticket.
constexpr int kDelayedUnroll = 4;

__global__ __launch_bounds__(256) void delayed_step_kernel(
    const uint16_t* __restrict__ x, int64_t n, uint8_t* __restrict__ st, uint32_t* slots, uint32_t* done, int L,
    int algo, float divisor, uint8_t* __restrict__ q, float* __restrict__ scale_used) {
  DelayedHeader* hd = reinterpret_cast<DelayedHeader*>(st);
  float* hist = reinterpret_cast<float*>(st + sizeof(DelayedHeader));
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const float d = hd->scale;
  const int64_t nch = n / 8;
  const int64_t base = (int64_t)blockIdx.x * 256 * kDelayedUnroll + tid;
  float amax = 0.0f;
  uint4 raw[kDelayedUnroll];
#pragma unroll
  for (int u = 0; u < kDelayedUnroll; ++u) {
    const int64_t c = base + (int64_t)u * 256;
    u32x4 v = {0, 0, 0, 0};
    if (c < nch) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + 8 * c));
    raw[u] = make_uint4(v[0], v[1], v[2], v[3]);
  }
#pragma unroll
  for (int u = 0; u < kDelayedUnroll; ++u) {
    const int64_t c = base + (int64_t)u * 256;
    const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    if (c < nch) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = clamp448(f[i] / d);
      u32x2 out;
      out[0] = pack4_e4m3(v[0], v[1], v[2], v[3]);
      out[1] = pack4_e4m3(v[4], v[5], v[6], v[7]);
      __builtin_nontemporal_store(out, reinterpret_cast<u32x2*>(q + 8 * c));
    }
  }
  amax = row16_max(amax);
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  if (tid >= 64) return;  // one wave carries on
  int closer = 0;
  if (tid == 0) {
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (blockIdx.x == 0) *scale_used = d;
    // Slot sl's line holds its running maximum ([0]) and how many of its
    // workgroups have finished ([1]).  Each atomic returns its old value,
    // which proves it done; the empty asm statements (taking that value,
    // clobbering memory) keep the next atomic behind it.  All are
    // device-scope atomics, performed where every XCD sees them, so no
    // fence is needed: the closing workgroup reads nothing else.
    const int sl = (int)(blockIdx.x % FP8B_DELAYED_AMAX_SLOTS);
    uint32_t* line = slots + 32 * sl;
    const uint32_t prev = __hip_atomic_fetch_max(line, __float_as_uint(amax), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::"v"(prev) : "memory");
    const uint32_t in_slot = (gridDim.x - sl + FP8B_DELAYED_AMAX_SLOTS - 1) / FP8B_DELAYED_AMAX_SLOTS;
    const uint32_t t = __hip_atomic_fetch_add(line + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t == in_slot - 1) {  // this slot is complete
      asm volatile("" ::"v"(t) : "memory");
      const uint32_t nslots = min(gridDim.x, (unsigned)FP8B_DELAYED_AMAX_SLOTS);
      closer = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nslots - 1;
    }
  }
  if (!__shfl(closer, 0)) return;

  // the last workgroup, one wave: close the step
  const int lane = tid;
  uint32_t ab = 0u;
  if (lane < FP8B_DELAYED_AMAX_SLOTS) {
    ab = __hip_atomic_load(slots + 32 * lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(slots + 32 * lane, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(slots + 32 * lane + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  float a = __uint_as_float(ab);
  a = row16_max(a);
  a = fmaxf(a, __shfl_xor(a, 16));
  a = fmaxf(a, __shfl_xor(a, 32));
  const int pos = hd->pos;
  const int filled = min(hd->filled + 1, L);
  float h = a;
  if (algo == 0) {
    for (int i = lane; i < filled; i += 64) h = fmaxf(h, i == pos ? a : hist[i]);
    h = row16_max(h);
    h = fmaxf(h, __shfl_xor(h, 16));
    h = fmaxf(h, __shfl_xor(h, 32));
  }
  if (lane == 0) {
    hist[pos] = a;
    hd->pos = (pos + 1) % L;
    hd->filled = filled;
    hd->scale = (h == 0.0f) ? 1.0f : h / divisor;
    __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Dequantisation to bf16, out = bf16_RNE(fp32(value(code) * d)) (x_hat =
// s * x_fp8 of "量化: FP8 与混合精度推理", section "FP8 也需要 scale"), for
// the weights (the bf16 branch of the DeepSeek-V3 guide's dispatch snippet,
// weight_dequant(weight, weight.scale): E4M3 codes, 128 x 128 block scales;
// KIND 0) and the KV cache (E5M2 codes, one scale per row; KIND 1).  The
// code -> fp32 conversion is exact, the product is one fp32 rounding and
// v_cvt_pk_bf16_f32 the second (round to nearest even).  Each lane turns 8 codes per step
// into 8 bf16 (an 8-byte load, a 16-byte store), so a wave instruction reads
// 512 and writes 1024 contiguous bytes (16 codes per lane, stored as two
// 16-byte halves 32 bytes apart, wrote ~10% more bytes than the output and
// took 72.2 / 21.0 us against 67.1 / 19.7 us for 18432 x 7168 weights and a
// 32768 x 1024 cache).  Grid: x = a block of rows, y = a
// segment of 256 * UNROLL 8-code groups of a row; rows shorter than 256
// groups (a power-of-two count) share a workgroup, UNROLL * 256 / groups
// of them, each lane taking one group in each of UNROLL rows.
template <int KIND, int UNROLL>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ q, int64_t rows, int64_t cols,
                                                      int64_t ldq, const float* __restrict__ scales,
                                                      uint16_t* __restrict__ out, int64_t ldo, int row_shift) {
  const int gpr = (int)(cols / 8);  // 8-code groups per row
  const int tid = threadIdx.x;
  // the lane's UNROLL groups: (row, group) pairs, all loaded before any is
  // converted (bytes in flight per lane = 8 * UNROLL)
  int64_t row[UNROLL];
  int grp[UNROLL];
  if (row_shift > 0) {  // UNROLL * 2^row_shift rows per workgroup, gpr = 256 >> row_shift
    const int64_t r0 = ((int64_t)blockIdx.x * UNROLL << row_shift) + (tid >> (8 - row_shift));
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      row[u] = r0 + ((int64_t)u << row_shift);
      grp[u] = tid & (gpr - 1);
    }
  } else {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      row[u] = blockIdx.x;
      grp[u] = (int)blockIdx.y * 256 * UNROLL + tid + 256 * u;
    }
  }
  u32x2 raw[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    raw[u] = u32x2{0u, 0u};
    if (row[u] < rows && grp[u] < gpr)
      raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(q + row[u] * ldq + 8 * grp[u]));
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t r = row[u];
    const int g = grp[u];
    if (r >= rows || g >= gpr) break;  // later pairs lie further out in the same order
    const float d = KIND == 0 ? scales[(r >> 7) * (cols >> 7) + (g >> 4)] : scales[r];
    typedef float f2 __attribute__((ext_vector_type(2)));
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      f2 lo, hi;
      if (KIND == 0) {
        lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)raw[u][i], 1.0f, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)raw[u][i], 1.0f, true);
      } else {
        lo = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8((int)raw[u][i], 1.0f, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8((int)raw[u][i], 1.0f, true);
      }
      // fp32 products, then one RNE rounding to bf16 per value (v_cvt_pk_bf16_f32)
      const bf16x2 b0 = {(__bf16)(lo[0] * d), (__bf16)(lo[1] * d)};
      const bf16x2 b1 = {(__bf16)(hi[0] * d), (__bf16)(hi[1] * d)};
      o[2 * i] = __builtin_bit_cast(uint32_t, b0);
      o[2 * i + 1] = __builtin_bit_cast(uint32_t, b1);
    }
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + r * ldo + 8 * g));
  }
}

// 8-code groups per row up to 256 * kDqUnroll take one segment (7168 and
// 8192 columns: 896 and 1024 groups).
constexpr int kDqUnroll = 4;

template <int KIND>
static int launch_dequant(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const float* scales,
                          uint16_t* out, int64_t ldo, hipStream_t s) {
  const int64_t gpr = cols / 8;
  int shift = 0;
  while (shift < 7 && (gpr << (shift + 1)) <= 256 && (256 % (gpr << (shift + 1))) == 0) ++shift;
  if (shift > 0 && (gpr << shift) != 256) shift = 0;  // only exact divisors of 256 share workgroups
  // Rows that share a workgroup take kDqUnroll of them per lane while that
  // leaves at least 512 workgroups (measured on MI355X: 32768 x 1024 KV
  // rows 19.0 -> 17.9 us, 4096 x 1024 weights 4.07 -> 3.79 us; a 1001 x 512
  // cache, 63 workgroups, 2.36 -> 2.97 us, so small launches keep one).
  if (shift > 0 && (rows >> shift) < 4 * 512) {
    const int64_t bx = (rows + (1 << shift) - 1) >> shift;
    if (bx > 0x7fffffff) return FP8B_EINVAL;  // grid limit
    hipLaunchKernelGGL((dequant_kernel<KIND, 1>), dim3((unsigned)bx), dim3(256), 0, s, q, rows, cols, ldq, scales,
                       out, ldo, shift);
    return check_launch();
  }
  const int64_t per_wg = (int64_t)kDqUnroll << shift;  // rows per workgroup when rows share one
  const int64_t bx = shift > 0 ? (rows + per_wg - 1) / per_wg : rows;
  const int64_t segs = shift > 0 ? 1 : (gpr + 256 * kDqUnroll - 1) / (256 * kDqUnroll);
  if (bx > 0x7fffffff || segs > 65535) return FP8B_EINVAL;  // grid limits
  hipLaunchKernelGGL((dequant_kernel<KIND, kDqUnroll>), dim3((unsigned)bx, (unsigned)segs), dim3(256), 0, s, q, rows,
                     cols, ldq, scales, out, ldo, shift);
  return check_launch();
}

// ---- host launchers --------------------------------------------------------
// 4 chunks per lane: a 7168- or 8192-wide row is one segment of 1024
// chunks (2 and 8 measured slower on 4096 x 7168).
constexpr int kActUnroll = 4;

int launch_act_quant(const void* x, int64_t M, int64_t K, int64_t ldx, int block, int fmt,
                     uint8_t* q, int64_t ldq, void* scales, hipStream_t s) {
  const int64_t cpr = K / 8;
  const int64_t segs = (cpr + 256 * kActUnroll - 1) / (256 * kActUnroll);
  if (segs > 65535 || M > 0x7fffffff) return FP8B_EINVAL;  // grid limits
  const dim3 grid((unsigned)M, (unsigned)segs);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
#define FP8B_AQ(B, F) \
  hipLaunchKernelGGL((act_quant_kernel<B, F, kActUnroll>), grid, dim3(256), 0, s, xp, K, ldx, q, ldq, scales)
  if (block == 128) {
    if (fmt == 0) FP8B_AQ(128, 0);
    else if (fmt == 1) FP8B_AQ(128, 1);
    else FP8B_AQ(128, 2);
  } else {
    if (fmt == 0) FP8B_AQ(32, 0);
    else if (fmt == 1) FP8B_AQ(32, 1);
    else FP8B_AQ(32, 2);
  }
#undef FP8B_AQ
  return check_launch();
}

int launch_weight_quant(const void* w, int64_t N, int64_t K, int64_t ldw, int fmt, uint8_t* q,
                        int64_t ldq, float* scales, hipStream_t s) {
  const dim3 grid((unsigned)((N / 128) * (K / 128)));
  const uint16_t* wp = static_cast<const uint16_t*>(w);
  if (fmt == 0)
    hipLaunchKernelGGL(weight_quant_kernel<0>, grid, dim3(256), 0, s, wp, N, K, ldw, q, ldq, scales);
  else
    hipLaunchKernelGGL(weight_quant_kernel<1>, grid, dim3(256), 0, s, wp, N, K, ldw, q, ldq, scales);
  return check_launch();
}

int launch_weight_dequant(const uint8_t* q, int64_t N, int64_t K, int64_t ldq, const float* scales,
                          void* w, int64_t ldw, hipStream_t s) {
  return launch_dequant<0>(q, N, K, ldq, scales, static_cast<uint16_t*>(w), ldw, s);
}

int launch_weight_pack(const uint8_t* w, int64_t G, int64_t N, int64_t K, int64_t ldw, uint8_t* out,
                       hipStream_t s) {
  const dim3 grid((unsigned)((G * N * (K / 16) + 255) / 256));
  hipLaunchKernelGGL(weight_pack_kernel, grid, dim3(256), 0, s, w, G, N, K, ldw, out);
  return check_launch();
}

int launch_kv_quant(const void* x, int64_t T, int64_t D, int64_t ldx, uint8_t* q, int64_t ldq, float* scales,
                    hipStream_t s) {
  const dim3 grid((unsigned)((T + 3) / 4));
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const int64_t per_lane = (D / 8 + 63) / 64;  // 16-byte chunks per lane
#define FP8B_KV(U) hipLaunchKernelGGL(kv_quant_kernel<U>, grid, dim3(256), 0, s, xp, T, D, ldx, q, ldq, scales)
  if (per_lane <= 1) FP8B_KV(1);
  else if (per_lane <= 2) FP8B_KV(2);
  else if (per_lane <= 4) FP8B_KV(4);
  else if (per_lane <= 8) FP8B_KV(8);
  else if (per_lane <= 16) FP8B_KV(16);
  else FP8B_KV(32);
#undef FP8B_KV
  return check_launch();
}

int launch_kv_dequant(const uint8_t* q, int64_t T, int64_t D, int64_t ldq, const float* scales, void* out,
                      int64_t ldo, hipStream_t s) {
  return launch_dequant<1>(q, T, D, ldq, scales, static_cast<uint16_t*>(out), ldo, s);
}

int launch_delayed_init(void* state, int64_t L, hipStream_t s) {
  const int64_t words = std::max<int64_t>(L, FP8B_DELAYED_AMAX_SLOTS * 32);
  hipLaunchKernelGGL(delayed_init_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s,
                     static_cast<uint8_t*>(state), (int)L);
  return check_launch();
}

static int delayed_step(const void* x, int64_t n, void* state, uint32_t* slots, uint32_t* done, int64_t L,
                        int algo, float divisor, uint8_t* q, float* scale_used, hipStream_t s) {
  const int64_t per_wg = 256 * kDelayedUnroll;
  const dim3 grid((unsigned)((n / 8 + per_wg - 1) / per_wg));
  hipLaunchKernelGGL(delayed_step_kernel, grid, dim3(256), 0, s, static_cast<const uint16_t*>(x), n,
                     static_cast<uint8_t*>(state), slots, done, (int)L, algo, divisor, q, scale_used);
  return check_launch();
}

int launch_delayed_quant(const void* x, int64_t n, void* state, int64_t L, int algo, float divisor, uint8_t* q,
                         float* scale_used, hipStream_t s) {
  DelayedHeader* h = static_cast<DelayedHeader*>(state);
  return delayed_step(x, n, state, &h->amax[0][0], &h->done, L, algo, divisor, q, scale_used, s);
}

// ---- delayed scaling without a caller-provided scratch -------------------------
// fp8_delayed_quant_noalloc keeps the step-in-flight scratch (the 16 amax
// slot lines and the step ticket, one 128-byte line each) in this array
// instead of the state.  Every GPU holds its own copy at its own address
// until the process ends.  In host code `scratch` is only a stand-in for
// the symbol: its device address is looked up once per device and kept in
// scratch_dev, and only that address is passed to kernels.
constexpr int kDelayedScratchWords = (FP8B_DELAYED_AMAX_SLOTS + 1) * 32;
static_assert(kDelayedScratchWords * 4 == FP8B_DELAYED_NOALLOC_SCRATCH_BYTES, "scratch size in the header");
static __device__ __align__(256) uint32_t scratch[kDelayedScratchWords];

__global__ __launch_bounds__(256) void scratch_clear_kernel(uint32_t* __restrict__ p, int words) {
  for (int i = threadIdx.x; i < words; i += 256) p[i] = 0u;
}

constexpr int kMaxScratchDevices = 64;
static uint32_t* scratch_dev[kMaxScratchDevices];  // device address of `scratch`, per device
static std::mutex scratch_mu;

// Device address of this stream's device's scratch.  The first call on a
// device looks the address up with that device current and clears the
// array with a kernel on the caller's stream (ordered before the step that
// follows; later steps leave it cleared: the closing workgroup zeroes the
// slots and the ticket).
static int delayed_scratch(hipStream_t s, uint32_t** out) {
  hipDevice_t dev = 0;
  if (s == nullptr || hipStreamGetDevice(s, &dev) != hipSuccess) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return FP8B_ELAUNCH;
    dev = cur;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return FP8B_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_dev[dev] == nullptr) {
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) return FP8B_ELAUNCH;
    if (prev != dev && hipSetDevice(dev) != hipSuccess) return FP8B_ELAUNCH;
    void* p = nullptr;
    int rc = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p != nullptr ? FP8B_OK : FP8B_ELAUNCH;
    if (rc == FP8B_OK) {  // cleared on the caller's stream, with its device still current
      hipLaunchKernelGGL(scratch_clear_kernel, dim3(1), dim3(256), 0, s, static_cast<uint32_t*>(p),
                         kDelayedScratchWords);
      rc = check_launch();
    }
    if (prev != dev) (void)hipSetDevice(prev);
    if (rc != FP8B_OK) return FP8B_ELAUNCH;
    scratch_dev[dev] = static_cast<uint32_t*>(p);
  }
  *out = scratch_dev[dev];
  return FP8B_OK;
}

int launch_delayed_quant_noalloc(const void* x, int64_t n, void* state, int64_t L, int algo, float divisor,
                                 uint8_t* q, float* scale_used, hipStream_t s) {
  uint32_t* p = nullptr;
  const int rc = delayed_scratch(s, &p);
  if (rc != FP8B_OK) return rc;
  return delayed_step(x, n, state, p, p + FP8B_DELAYED_AMAX_SLOTS * 32, L, algo, divisor, q, scale_used, s);
}

int launch_cast(const float* x, int64_t n, int fmt, uint8_t* q, hipStream_t s) {
  const dim3 grid((unsigned)((n + 1023) / 1024));
  if (fmt == 0)
    hipLaunchKernelGGL(cast_kernel<0>, grid, dim3(256), 0, s, x, n, q);
  else
    hipLaunchKernelGGL(cast_kernel<1>, grid, dim3(256), 0, s, x, n, q);
  return check_launch();
}

}  // namespace fp8blk
