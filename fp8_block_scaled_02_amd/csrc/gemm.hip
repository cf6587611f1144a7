// gemm.hip -- block-scaled FP8 GEMM, MXFP8 GEMM and grouped (MoE) GEMM for
// gfx950.
//
// Method (sources by page title and section):
//  * DeepSeek-V3 on MI250 guide, configuration table and dispatch snippet:
//    E4M3 weights with one scale per 128x128 block, activations with one
//    scale per token per 128 channels, fp8_gemm(x, scale, weight, weight.scale).
//  * "FP8 engineering 2026", section 3: FP8 products accumulated in FP32,
//    blockwise scales applied per 128x128 block.
//  * ROCm 7.0 FP8 article, sections 1.1-1.2: MXFP8 blocks of 32 elements
//    sharing one E8M0 exponent.
//
// Design for CDNA4 (the pages' Hopper TMA/WGMMA pipeline is prior art only):
//  * Arithmetic.  gfx950's FP8 MFMA (v_mfma_*_f8f6f4) sums its products in
//    groups of 8 aligned to the group's largest exponent with 13 fraction
//    bits, truncating the rest; with the activation outliers these layers see,
//    that misses an fp32-accumulation error budget.  E4M3 -> bf16 is exact,
//    and the bf16 MFMA accumulates products at fp32 precision, so the codes
//    stay FP8 in HBM and LDS (the bytes the method saves) and are widened in
//    registers (v_cvt_scalef32_pk_bf16_fp8) right before
//    v_mfma_f32_16x16x32_bf16.
//  * One K step is one 128-wide scale block: four chained bf16 MFMAs give
//    the block's partial product P in fp32, then the VALU folds it in with
//    one FMA per output: acc += P * (sa * sw).  MX scales are powers of two
//    and are folded into the conversion instead, so the MX loop accumulates
//    straight in the MFMAs.
//  * The MFMA operands are swapped (A-operand = weight rows, B-operand =
//    activation rows) so that each lane's four results share one token row:
//    the combined scale is one value per lane, and the four outputs are
//    four consecutive columns of y (one packed store).
//  * Operand tiles go HBM/L2 -> LDS with direct-to-LDS loads
//    (global_load_lds_dwordx4), no register staging: each wave instruction
//    fills 1 KB = 8 tile rows; the XOR chunk swizzle that keeps ds_read_b128
//    conflict-free is applied on the global-address side.  The per-step
//    scales ride along with dword direct loads into the same LDS buffer.
//  * Two LDS buffers declared as separate arrays (so the compiler can see
//    that the prefetch target never aliases the buffer being read), one
//    barrier per K step.
//  * Tile order is remapped so that each XCD (8 per chip, each with its own
//    L2) works on a contiguous, grouped patch of output tiles.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace fp8blk {

constexpr int kBK = 128;
constexpr int kGroupM = 8;  // m-tiles per tile-order group

template <int BM_, int BN_, int WM_, int WN_, bool MX_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr bool MX = MX_;
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int MI = TM / 16, NJ = TN / 16;  // 16x16 subtiles per wave
  static constexpr int GROUPS = (BM + BN) / 8;      // 1 KB row groups per K step
  static constexpr int NI = GROUPS / NW;            // code DMA instructions per wave
  // scale DMA instructions per K step (64 lanes x 4 bytes each)
  static constexpr int NS_A = BM / 64;
  static constexpr int NS_B = MX ? BN / 64 : 1;
  static constexpr int NS = NS_A + NS_B;
  // LDS layout of one buffer
  static constexpr int OFF_W = BM * 128;
  static constexpr int OFF_SA = (BM + BN) * 128;
  static constexpr int OFF_SB = OFF_SA + BM * 4;
  static constexpr int BUF = OFF_SB + (MX ? BN * 4 : 256);
  static_assert(GROUPS % NW == 0, "row groups must split evenly over waves");
  static_assert(NS <= NW, "at most one scale load per wave");
  static_assert(TM % 16 == 0 && TN % 16 == 0 && BM % 64 == 0 && BN % 128 == 0, "tile shape");
};

// LDS byte offset of logical 16-byte chunk `ch` (0..7) of tile row `r`.
__device__ __forceinline__ int lds_off(int r, int ch) { return r * 128 + ((ch ^ (r & 7)) << 4); }

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void* src, uint8_t* dst_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst_wave_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, uint8_t* dst_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst_wave_base, 4, 0, 0);
}

// vmcnt(0) with the other counters left alone (gfx9 s_waitcnt encoding).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Map a linear workgroup id to an output tile (tm, tn): first give each XCD
// a contiguous range of ids (workgroups are dealt to the 8 XCDs round
// robin), then walk tiles in groups of kGroupM m-tiles so that concurrently
// running workgroups share A rows and W rows in that XCD's L2.
__device__ __forceinline__ void tile_of(int pid, int nwg, int tiles_m, int tiles_n, int& tm, int& tn) {
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  const int per_group = kGroupM * tiles_n;
  const int group = pid / per_group;
  const int first_m = group * kGroupM;
  const int gsz = min(tiles_m - first_m, kGroupM);
  const int in = pid - group * per_group;
  tm = first_m + in % gsz;
  tn = in / gsz;
}

// Per-lane sources of one output tile's direct-to-LDS loads.
template <class C>
struct Src {
  const uint8_t* code[C::NI];  // row pointer + swizzled chunk offset, K step 0
  const uint8_t* scale;        // this wave's scale load (K step 0), if any
  int scale_dst;               // its LDS offset in the buffer, or -1
};

// Row-group bookkeeping: wave w, instruction i fills row group q = w + NW*i,
// i.e. tile rows 8q .. 8q+7 (A rows first, then W rows); lane l covers row
// 8q + (l >> 3) and LDS position (l & 7), which holds logical chunk
// (l & 7) ^ (row & 7) = (l & 7) ^ (l >> 3).
template <class C, class ARow, class WRow>
__device__ __forceinline__ void make_code_src(Src<C>& s, ARow arow, WRow wrow) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunk = (lane & 7) ^ (lane >> 3);
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    const int q = wave + C::NW * i;
    const int r = 8 * q + (lane >> 3);
    s.code[i] = (r < C::BM ? arow(r) : wrow(r - C::BM)) + chunk * 16;
  }
}

template <class C>
__device__ __forceinline__ void issue(uint8_t* buf, const Src<C>& s, int kb) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < C::NI; ++i) dma16(s.code[i] + (int64_t)kb * kBK, buf + (wave + C::NW * i) * 1024);
  if (s.scale_dst >= 0) dma4(s.scale + (int64_t)kb * 4, buf + s.scale_dst);
}

// FP8 -> bf16 (exact for every finite E4M3 code; `scale` is a power of two
// folded into the conversion) for the 8 codes of a dword pair.
__device__ __forceinline__ bf16x8 cvt8(uint32_t lo, uint32_t hi, float scale) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, scale, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, scale, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, scale, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, scale, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The 32 FP8 codes of a lane's fragment (16x128 operand, lane group g holds
// chunks g and g+4 of its row) as four bf16x8 MFMA operands, one per 32-wide
// K sub-step.  Both operands of an MFMA use the same byte -> K assignment, so
// every K of the block is multiplied exactly once.  s_lo / s_hi scale the
// first / second 16 codes (chunk g / chunk g+4).
struct Frag16 {
  bf16x8 k[4];
};

__device__ __forceinline__ Frag16 load_frag(const uint8_t* t, int r, int g, float s_lo, float s_hi) {
  const uint4 lo = *reinterpret_cast<const uint4*>(t + lds_off(r, g));
  const uint4 hi = *reinterpret_cast<const uint4*>(t + lds_off(r, g + 4));
  Frag16 f;
  f.k[0] = cvt8(lo.x, lo.y, s_lo);
  f.k[1] = cvt8(lo.z, lo.w, s_lo);
  f.k[2] = cvt8(hi.x, hi.y, s_hi);
  f.k[3] = cvt8(hi.z, hi.w, s_hi);
  return f;
}

__device__ __forceinline__ v4f mfma_bf16(bf16x8 a, bf16x8 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16 tile product over one 128-wide K block: four chained bf16 MFMAs
// (fp32 accumulation inside the block).
__device__ __forceinline__ v4f block_product(const Frag16& w, const Frag16& x, v4f c) {
  c = mfma_bf16(w.k[0], x.k[0], c);
  c = mfma_bf16(w.k[1], x.k[1], c);
  c = mfma_bf16(w.k[2], x.k[2], c);
  return mfma_bf16(w.k[3], x.k[3], c);
}

// One K step of the block-scaled GEMM on the wave's MI x NJ subtiles:
// P = block product (fp32), then acc += P * (sa * sw).
template <class C>
__device__ __forceinline__ void compute_block(const uint8_t* buf, v4f (&acc)[C::MI][C::NJ]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % C::WM, wn = wave / C::WM, l16 = lane & 15, g = lane >> 4;
  const float* sa = reinterpret_cast<const float*>(buf + C::OFF_SA);
  const float* sw = reinterpret_cast<const float*>(buf + C::OFF_SB);
  Frag16 xf[C::MI];
  float s[C::MI];
  const float sw0 = sw[(wn * C::TN) / 128];
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    const int r = wm * C::TM + 16 * i + l16;
    xf[i] = load_frag(buf, r, g, 1.0f, 1.0f);
    s[i] = sa[r] * sw0;
  }
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) {
    const int rn = wn * C::TN + 16 * j;
    const Frag16 wf = load_frag(buf + C::OFF_W, rn + l16, g, 1.0f, 1.0f);
    float swj = sw0;
    if (C::TN > 128) swj = sw[rn / 128];
#pragma unroll
    for (int i = 0; i < C::MI; ++i) {
      const v4f p = block_product(wf, xf[i], zero);
      const float si = (C::TN > 128) ? sa[wm * C::TM + 16 * i + l16] * swj : s[i];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], si, acc[i][j][r]);
    }
  }
}

// 2^(e - 127) for an E8M0 byte e in [1, 254] (fp32 normal); e = 0 gives
// 2^-127 (fp32 subnormal).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
}

// One K step of the MXFP8 GEMM.  Each 32-block's E8M0 scale is folded into
// the FP8 -> bf16 conversion of its codes (exact while the scaled values stay
// in bf16's normal range), so the MFMAs accumulate straight into acc.  The
// lane's first 16 codes (K 16g..) lie in 32-block g/2 and its last 16
// (K 64+16g..) in 32-block 2 + g/2; scale bytes are one dword per row.
template <class C>
__device__ __forceinline__ void compute_mx(const uint8_t* buf, v4f (&acc)[C::MI][C::NJ]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % C::WM, wn = wave / C::WM, l16 = lane & 15, g = lane >> 4;
  const uint32_t* ea = reinterpret_cast<const uint32_t*>(buf + C::OFF_SA);
  const uint32_t* eb = reinterpret_cast<const uint32_t*>(buf + C::OFF_SB);
  const int b0 = 8 * (g >> 1), b1 = 8 * (2 + (g >> 1));
  Frag16 xf[C::MI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    const int r = wm * C::TM + 16 * i + l16;
    const uint32_t e = ea[r];
    xf[i] = load_frag(buf, r, g, e8m0_to_f32((e >> b0) & 0xffu), e8m0_to_f32((e >> b1) & 0xffu));
  }
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) {
    const int r = wn * C::TN + 16 * j + l16;
    const uint32_t e = eb[r];
    const Frag16 wf = load_frag(buf + C::OFF_W, r, g, e8m0_to_f32((e >> b0) & 0xffu),
                                e8m0_to_f32((e >> b1) & 0xffu));
#pragma unroll
    for (int i = 0; i < C::MI; ++i) acc[i][j] = block_product(wf, xf[i], acc[i][j]);
  }
}

// Full K loop of one output tile.  Buffer b is filled by the loads issued
// one step earlier; every step waits for its own loads, then one barrier
// makes everyone's loads visible and guarantees the other buffer is no
// longer being read, then the next step's loads go out and the math runs.
template <class C>
__device__ __forceinline__ void k_loop(uint8_t* lds0, uint8_t* lds1, const Src<C>& src, int nkb,
                                       v4f (&acc)[C::MI][C::NJ]) {
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  issue<C>(lds0, src, 0);
  for (int kb = 0; kb < nkb; kb += 2) {
    wait_vmem();
    __syncthreads();
    if (kb + 1 < nkb) issue<C>(lds1, src, kb + 1);
    if (C::MX) compute_mx<C>(lds0, acc); else compute_block<C>(lds0, acc);
    if (kb + 1 < nkb) {
      wait_vmem();
      __syncthreads();
      if (kb + 2 < nkb) issue<C>(lds0, src, kb + 2);
      if (C::MX) compute_mx<C>(lds1, acc); else compute_block<C>(lds1, acc);
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void store4(void* __restrict__ y, int64_t off, const v4f v) {
  if (BF16) {
    uint2 p;
    p.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
    p.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + off) = p;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + off) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Lane's outputs: m-subtile i is tile row wm*TM + 16i + l16, n-subtile j
// covers columns n0 + wn*TN + 16j + 4g .. +3.  row_off(r) gives the element
// offset of tile row r in y, or -1 for rows that are not stored.
template <class C, bool BF16, class RowOff>
__device__ __forceinline__ void epilogue(void* __restrict__ y, const v4f (&acc)[C::MI][C::NJ], int n0,
                                         RowOff row_off) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % C::WM, wn = wave / C::WM, l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    const int64_t base = row_off(wm * C::TM + 16 * i + l16);
    if (base >= 0) {
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) store4<BF16>(y, base + n0 + wn * C::TN + 16 * j + 4 * g, acc[i][j]);
    }
  }
}

// ---- block-scaled GEMM ------------------------------------------------------
template <class C, bool BF16>
__global__ __launch_bounds__(C::NT, 2) void block_gemm_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ SA,
    const uint8_t* __restrict__ W, int64_t ldw, const float* __restrict__ SW, int M, int N, int K,
    void* __restrict__ Y, int64_t ldy) {
  __shared__ __attribute__((aligned(16))) uint8_t lds0[C::BUF];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[C::BUF];
  const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = N / C::BN;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN, nkb = K / kBK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  Src<C> src;
  // rows past M re-read the last row; their results are never stored
  make_code_src<C>(src, [&](int r) { return A + (int64_t)min(m0 + r, M - 1) * lda; },
                   [&](int r) { return W + (int64_t)(n0 + r) * ldw; });
  src.scale_dst = -1;
  src.scale = A;
  if (wave < C::NS_A) {
    src.scale = reinterpret_cast<const uint8_t*>(SA + (int64_t)min(m0 + 64 * wave + lane, M - 1) * nkb);
    src.scale_dst = C::OFF_SA + 256 * wave;
  } else if (wave == C::NS_A) {
    const int nb = n0 / 128 + min(lane, C::BN / 128 - 1);
    src.scale = reinterpret_cast<const uint8_t*>(SW + (int64_t)nb * nkb);
    src.scale_dst = C::OFF_SB;
  }

  v4f acc[C::MI][C::NJ];
  k_loop<C>(lds0, lds1, src, nkb, acc);
  epilogue<C, BF16>(Y, acc, n0, [&](int r) -> int64_t { return m0 + r < M ? (int64_t)(m0 + r) * ldy : -1; });
}

// ---- MXFP8 GEMM ---------------------------------------------------------------
template <class C>
__global__ __launch_bounds__(C::NT, 2) void mx_gemm_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ EA,
    const uint8_t* __restrict__ B, int64_t ldb, const uint8_t* __restrict__ EB, int M, int N, int K,
    float* __restrict__ Y, int64_t ldy) {
  __shared__ __attribute__((aligned(16))) uint8_t lds0[C::BUF];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[C::BUF];
  const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = N / C::BN;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN, nkb = K / kBK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t srow = K / 32;  // E8M0 bytes per row

  Src<C> src;
  make_code_src<C>(src, [&](int r) { return A + (int64_t)min(m0 + r, M - 1) * lda; },
                   [&](int r) { return B + (int64_t)(n0 + r) * ldb; });
  src.scale_dst = -1;
  src.scale = A;
  if (wave < C::NS_A) {
    src.scale = EA + (int64_t)min(m0 + 64 * wave + lane, M - 1) * srow;
    src.scale_dst = C::OFF_SA + 256 * wave;
  } else if (wave < C::NS) {
    const int t = wave - C::NS_A;
    src.scale = EB + (int64_t)(n0 + 64 * t + lane) * srow;
    src.scale_dst = C::OFF_SB + 256 * t;
  }

  v4f acc[C::MI][C::NJ];
  k_loop<C>(lds0, lds1, src, nkb, acc);
  epilogue<C, false>(Y, acc, n0, [&](int r) -> int64_t { return m0 + r < M ? (int64_t)(m0 + r) * ldy : -1; });
}

// ---- grouped (MoE) GEMM -----------------------------------------------------
// Persistent workgroups; the tile map is rebuilt in LDS by every workgroup
// from expert_offsets (a prefix sum of per-expert tile counts), so the host
// never reads the routing.  Work ids are ordered (expert, n-tile, m-tile)
// with m fastest, so concurrently running m-tiles of a heavy expert share
// that expert's weight tile in L2.
constexpr int kMaxExperts = 1024;

template <class C, bool BF16>
__global__ __launch_bounds__(C::NT, 2) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ SA, int T,
    const int32_t* __restrict__ RI, const int32_t* __restrict__ OFFS, int R, int E,
    const uint8_t* __restrict__ W, const float* __restrict__ SW, int N, int K, void* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) uint8_t lds0[C::BUF];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[C::BUF];
  __shared__ int tstart[kMaxExperts + 1];
  __shared__ int part[C::NT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles_n = N / C::BN, nkb = K / kBK;

  auto off_at = [&](int e) { return min(max(OFFS[e], 0), R); };
  auto ntiles = [&](int e) { return ((max(off_at(e + 1) - off_at(e), 0) + C::BM - 1) / C::BM) * tiles_n; };

  // tile map: tstart[e] = first work id of expert e
  const int per = (E + C::NT - 1) / C::NT;
  const int e0 = min(tid * per, E), e1 = min(e0 + per, E);
  int local = 0;
  for (int e = e0; e < e1; ++e) local += ntiles(e);
  part[tid] = local;
  __syncthreads();
  for (int o = 1; o < C::NT; o <<= 1) {
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = tid ? part[tid - 1] : 0;
  for (int e = e0; e < e1; ++e) {
    tstart[e] = run;
    run += ntiles(e);
  }
  if (tid == C::NT - 1) tstart[E] = part[C::NT - 1];
  __syncthreads();
  const int total = tstart[E];

  for (int wk = blockIdx.x; wk < total; wk += gridDim.x) {
    int lo = 0, hi = E;  // largest e with tstart[e] <= wk
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tstart[mid] <= wk) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int rb = off_at(e), re = off_at(e + 1);
    const int mt = (re - rb + C::BM - 1) / C::BM;
    const int loc = wk - tstart[e];
    const int tn = loc / mt, tm = loc - tn * mt;
    const int r0 = rb + tm * C::BM, n0 = tn * C::BN;
    const uint8_t* We = W + (int64_t)e * N * K;
    auto token = [&](int r) { return min(max(RI[min(r0 + r, re - 1)], 0), T - 1); };

    Src<C> src;
    make_code_src<C>(src, [&](int r) { return A + (int64_t)token(r) * K; },
                     [&](int r) { return We + (int64_t)(n0 + r) * K; });
    src.scale_dst = -1;
    src.scale = A;
    if (wave < C::NS_A) {
      src.scale = reinterpret_cast<const uint8_t*>(SA + (int64_t)token(64 * wave + lane) * nkb);
      src.scale_dst = C::OFF_SA + 256 * wave;
    } else if (wave == C::NS_A) {
      const int nb = n0 / 128 + min(lane, C::BN / 128 - 1);
      src.scale = reinterpret_cast<const uint8_t*>(SW + ((int64_t)e * (N / 128) + nb) * nkb);
      src.scale_dst = C::OFF_SB;
    }

    __syncthreads();  // the previous tile's last step may still read lds0/lds1
    v4f acc[C::MI][C::NJ];
    k_loop<C>(lds0, lds1, src, nkb, acc);
    epilogue<C, BF16>(Y, acc, n0,
                      [&](int r) -> int64_t { return r0 + r < re ? (int64_t)(r0 + r) * N : -1; });
  }
}

// ---- host launchers ---------------------------------------------------------
using BlockCfg = Cfg<128, 128, 2, 2, false>;
using MxCfg = Cfg<128, 128, 2, 2, true>;

static int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

int launch_block_gemm(const uint8_t* a, int64_t lda, const float* sa, const uint8_t* w, int64_t ldw,
                      const float* sw, int64_t M, int64_t N, int64_t K, void* y, int64_t ldy, int out_bf16,
                      hipStream_t s) {
  using C = BlockCfg;
  const int64_t tiles = ((M + C::BM - 1) / C::BM) * (N / C::BN);
  const dim3 grid((unsigned)tiles), block(C::NT);
  if (out_bf16)
    hipLaunchKernelGGL((block_gemm_kernel<C, true>), grid, block, 0, s, a, lda, sa, w, ldw, sw, (int)M, (int)N,
                       (int)K, y, ldy);
  else
    hipLaunchKernelGGL((block_gemm_kernel<C, false>), grid, block, 0, s, a, lda, sa, w, ldw, sw, (int)M, (int)N,
                       (int)K, y, ldy);
  return check_launch();
}

int launch_mx_gemm(const uint8_t* a, int64_t lda, const uint8_t* ea, const uint8_t* b, int64_t ldb,
                   const uint8_t* eb, int64_t M, int64_t N, int64_t K, float* y, int64_t ldy, hipStream_t s) {
  using C = MxCfg;
  const int64_t tiles = ((M + C::BM - 1) / C::BM) * (N / C::BN);
  hipLaunchKernelGGL(mx_gemm_kernel<C>, dim3((unsigned)tiles), dim3(C::NT), 0, s, a, lda, ea, b, ldb, eb, (int)M,
                     (int)N, (int)K, y, ldy);
  return check_launch();
}

int launch_grouped_gemm(const uint8_t* a, const float* sa, int64_t T, const int32_t* ri, const int32_t* offs,
                        int64_t R, int64_t E, const uint8_t* w, const float* sw, int64_t N, int64_t K, void* y,
                        int out_bf16, hipStream_t s) {
  using C = BlockCfg;
  // enough persistent workgroups to fill every CU twice, never more than
  // the largest possible number of tiles
  const int64_t max_tiles = ((R + C::BM - 1) / C::BM + E) * (N / C::BN);
  const int64_t nwg = std::max<int64_t>(1, std::min<int64_t>(2 * (int64_t)cu_count(), max_tiles));
  const dim3 grid((unsigned)nwg), block(C::NT);
  if (out_bf16)
    hipLaunchKernelGGL((grouped_gemm_kernel<C, true>), grid, block, 0, s, a, sa, (int)T, ri, offs, (int)R, (int)E,
                       w, sw, (int)N, (int)K, y);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<C, false>), grid, block, 0, s, a, sa, (int)T, ri, offs, (int)R, (int)E,
                       w, sw, (int)N, (int)K, y);
  return check_launch();
}

}  // namespace fp8blk
