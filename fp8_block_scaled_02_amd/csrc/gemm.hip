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
//    (buffer_load_dwordx4 ... lds through a buffer descriptor whose base
//    moves one K step at a time in SGPRs), no register staging: each wave
//    instruction
//    fills 1 KB = 8 tile rows; the XOR chunk swizzle that keeps ds_read_b128
//    conflict-free is applied on the global-address side.  The per-step
//    scales ride along with dword direct loads into the same LDS buffer.
//  * Two LDS buffers declared as separate arrays (so the compiler can see
//    that the prefetch target never aliases the buffer being read), one
//    barrier per K step.
//  * Tile order is remapped so that each XCD (8 per chip, each with its own
//    L2) works on a contiguous, grouped patch of output tiles.
//  * Weights may also come in a packed layout (1 KB chunks of 16 rows x 64
//    codes, K outermost; see packed_woff): each wave load is one contiguous
//    chunk, and weight-streaming launches read one advancing front of HBM.
//  * Up to 64 tokens (decode, the short tails of MoE experts) the weights
//    are streamed once through registers instead of being tiled through LDS
//    (stream_rows), the K range split over the workgroup's four waves.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace fp8blk {


constexpr int kBK = 128;
constexpr int kGroupM = 8;  // m-tiles per tile-order group

// Tile configuration: BM x BN output tile, WM x WN waves (each TM x TN),
// S LDS stages (prefetch distance S-1 K steps).
template <int BM_, int BN_, int WM_, int WN_, bool MX_, int S_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, S = S_;
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
  // LDS layout of one stage
  static constexpr int OFF_W = BM * 128;
  static constexpr int OFF_SA = (BM + BN) * 128;
  static constexpr int OFF_SB = OFF_SA + BM * 4;
  static constexpr int BUF = OFF_SB + (MX ? BN * 4 : 256);
  static_assert(GROUPS % NW == 0, "row groups must split evenly over waves");
  static_assert(NS <= NW, "at most one scale load per wave");
  static_assert(TM % 16 == 0 && TN % 16 == 0 && BM % 64 == 0 && BN % 128 == 0, "tile shape");
  static_assert(TN <= 128, "a wave's columns lie in one weight-scale block");
  static_assert(S == 2 || S == 3, "two or three LDS stages");
  static_assert(S * BUF <= 160 * 1024, "LDS capacity");
};

// LDS byte offset of logical 16-byte chunk `ch` (0..7) of tile row `r`.
__device__ __forceinline__ int lds_off(int r, int ch) { return r * 128 + ((ch ^ (r & 7)) << 4); }

typedef __attribute__((address_space(3))) void lds_void;

// A raw buffer (stride 0) over the 4 GiB from base; the third descriptor
// word is the gfx9 default (32-bit data format), which raw loads ignore.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)0xFFFFFFFFu, 0x00020000);
}
// Direct-to-LDS loads through a buffer descriptor: the base lives in SGPRs
// and the lane's 32-bit offset needs no 64-bit address arithmetic (the
// global form took a 64-bit VALU add per load: 5 VALU instructions per K
// step of the 128 x 128 tile, about 1% of the block and MX GEMMs' time).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint8_t* dst_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst_wave_base, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint8_t* dst_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst_wave_base, 4, voff, 0, 0, 0);
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt bits
// [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The wave index as a scalar (it is uniform; saying so keeps LDS bases and
// M0 setup in SALU).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

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

// Per-lane sources of one output tile's direct-to-LDS loads: a uniform base
// (activation or weight matrix) plus a 32-bit per-lane byte offset, so the
// loads use scalar-base addressing and each K step only moves the base.
template <class C>
struct Src {
  const uint8_t* abase;        // uniform
  const uint8_t* wbase;        // uniform
  size_t wstep;                // bytes the weight base moves per K step
  uint32_t code[C::NI];        // row offset + swizzled chunk offset, K step 0
  const uint8_t* sbase;        // uniform base of this wave's scale load
  uint32_t soff;               // per-lane offset of that load
  int scale_dst;               // its LDS offset in the stage (uniform), or -1
};

// Row-group bookkeeping: wave w, instruction i fills 1 KB group q = w + NW*i
// of the stage (A groups first, then W groups).  An A group (and a W group
// of row-major weights) is tile rows 8q .. 8q+7: lane l covers row
// 8q + (l >> 3) and LDS position (l & 7), which holds logical chunk
// (l & 7) ^ (row & 7) = (l & 7) ^ (l >> 3).  arow_off(r) is the byte offset
// of activation row r from abase; woff(qw, lane) that of lane's 16 bytes of
// W group qw from wbase (row_major_woff or packed_woff).
template <class C, class ARow, class WOff>
__device__ __forceinline__ void make_code_src(Src<C>& s, ARow arow_off, WOff woff) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const uint32_t chunk = (uint32_t)((lane & 7) ^ (lane >> 3));
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    const int q = wave + C::NW * i;
    s.code[i] = q < C::BM / 8 ? arow_off(8 * q + (lane >> 3)) + chunk * 16u : woff(q - C::BM / 8, lane);
  }
}

// Row-major weights [rows][ld]: W group qw is tile rows 8qw .. 8qw+7, in the
// swizzled row layout of the A groups.
__device__ __forceinline__ uint32_t row_major_woff(int qw, int lane, int64_t ld) {
  const int r = 8 * qw + (lane >> 3);
  return (uint32_t)(r * ld) + (uint32_t)(((lane & 7) ^ (lane >> 3)) * 16);
}

// ---- packed weight layout ---------------------------------------------------
// A weight matrix [N][K] of codes is stored as N*K/1024 chunks of 1 KB: chunk
// (kc, p), for K bytes 64kc .. 64kc+63 of rows 16p .. 16p+15, sits at byte
// (kc * N/16 + p) * 1024, and inside it byte 256g + 16r + b is code
// [16p + r][64kc + 16g + b].  Lane l = 16g + r of a wave reading chunk
// (kc, p) at 16l therefore holds exactly the 16 codes its MFMA fragment
// takes from that K half, and the whole wave reads 1 KB contiguously.  With
// K outermost, all workgroups of a weight-streaming GEMM read one contiguous
// front of HBM at a time (measured on MI355X for 28672 x 8192 codes: 6.3
// TB/s pure-read against 5.2 TB/s for 16-row panels of the row-major matrix).
// A tile's K step is 2 x BN/16 whole chunks: W group qw = h * BN/16 + pp is
// chunk (2kb + h, p0 + pp), copied verbatim (lane l moves bytes 16l ..
// 16l+15, one 1 KB line-contiguous load per wave), so the stage holds the
// chunks in that order and a lane reads its fragment's two 16-byte halves
// at 16 * lane of chunks (0, pp) and (1, pp) (read_w).
//
// Offset of lane's 16 bytes of W group qw from the tile's packed base (its
// first panel at kc = 0); np = N / 16, nb = BN / 16 panels per tile.
__device__ __forceinline__ uint32_t packed_woff(int qw, int lane, int np, int nb) {
  const int h = qw / nb, pp = qw - h * nb;
  return ((uint32_t)(h * np + pp) << 10) + (uint32_t)(16 * lane);
}

template <class C>
__device__ __forceinline__ void issue(uint8_t* buf, const Src<C>& s, int kb) {
  const int wave = wave_id();
  const __amdgpu_buffer_rsrc_t ra = rsrc_at(s.abase + (size_t)kb * kBK);
  const __amdgpu_buffer_rsrc_t rw = rsrc_at(s.wbase + (size_t)kb * s.wstep);
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    const int q = wave + C::NW * i;
    dma16(q < C::BM / 8 ? ra : rw, s.code[i], buf + q * 1024);
  }
  if (s.scale_dst >= 0) dma4(rsrc_at(s.sbase + (size_t)kb * 4), s.soff, buf + s.scale_dst);
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

struct Raw16 {
  uint4 lo, hi;
};

__device__ __forceinline__ Raw16 read_raw(const uint8_t* t, int r, int g) {
  Raw16 v;
  v.lo = *reinterpret_cast<const uint4*>(t + lds_off(r, g));
  v.hi = *reinterpret_cast<const uint4*>(t + lds_off(r, g + 4));
  return v;
}

// A lane's weight fragment for tile rows row0 .. row0+15 (row0 a multiple
// of 16) from the stage's W region: swizzled rows, or packed chunks (see
// packed_woff).
template <class C, bool PK>
__device__ __forceinline__ Raw16 read_w(const uint8_t* wt, int row0, int lane) {
  if (PK) {
    const uint8_t* p = wt + (row0 >> 4) * 1024 + 16 * lane;
    Raw16 v;
    v.lo = *reinterpret_cast<const uint4*>(p);
    v.hi = *reinterpret_cast<const uint4*>(p + (C::BN / 16) * 1024);
    return v;
  }
  return read_raw(wt, row0 + (lane & 15), lane >> 4);
}

__device__ __forceinline__ Frag16 widen(const Raw16& v, float s_lo, float s_hi) {
  Frag16 f;
  f.k[0] = cvt8(v.lo.x, v.lo.y, s_lo);
  f.k[1] = cvt8(v.lo.z, v.lo.w, s_lo);
  f.k[2] = cvt8(v.hi.x, v.hi.y, s_hi);
  f.k[3] = cvt8(v.hi.z, v.hi.w, s_hi);
  return f;
}

// One K step of the block-scaled GEMM on the wave's MI x NJ subtiles.
// For each weight fragment j the MI block products run as MI chains of four
// bf16 MFMAs in k-outer / i-inner order, so consecutive MFMAs are
// independent: a dependent MFMA issued right behind its producer stalls on
// gfx950.  Inside window k (register ties keep the windows apart) the VALU
// widens a quarter of fragment j+1 and folds fragment j-1's product for
// subtile row k into acc (acc += P * sa * sw); those have long been
// complete, so no VALU op waits on an MFMA in flight.
template <class C, bool PK, class Hook>
__device__ __forceinline__ void compute_block(const uint8_t* buf, v4f (&acc)[C::MI][C::NJ], Hook hook) {
  static_assert(C::MI == 4, "one rescale row per K sub-step window");
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave % C::WM, wn = wave / C::WM, l16 = lane & 15, g = lane >> 4;
  const float* sa = reinterpret_cast<const float*>(buf + C::OFF_SA);
  const float* sw = reinterpret_cast<const float*>(buf + C::OFF_SB);
  const uint8_t* wt = buf + C::OFF_W;
  // LDS reads: the scales, the four A fragments and the first two weight
  // fragments go out together (15 reads, the most the LDS wait counter can
  // track), later weight fragments two subtiles ahead of their use inside
  // the MFMA loop.
  Raw16 wraw[C::NJ];
  Frag16 xf[C::MI];
  float s[C::MI];
  float sar[C::MI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i) sar[i] = sa[wm * C::TM + 16 * i + l16];
  const float sw0 = sw[(wn * C::TN) / 128];
  Raw16 araw[C::MI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i) araw[i] = read_raw(buf, wm * C::TM + 16 * i + l16, g);
#pragma unroll
  for (int j = 0; j < 2 && j < C::NJ; ++j) wraw[j] = read_w<C, PK>(wt, wn * C::TN + 16 * j, lane);
  // Only the first 32-wide K window of the activation fragments is widened
  // up front; windows 1..3 are widened between the MFMAs of the first weight
  // fragment, so the step does not open with a VALU-only burst that leaves
  // the matrix unit idle.
  auto widen_a = [&](int i, int k) {
    const uint4& h = k < 2 ? araw[i].lo : araw[i].hi;
    xf[i].k[k] = (k & 1) ? cvt8(h.z, h.w, 1.0f) : cvt8(h.x, h.y, 1.0f);
  };
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    widen_a(i, 0);
    s[i] = sar[i] * sw0;
  }
  Frag16 wcur = widen(wraw[0], 1.0f, 1.0f), wnext;
  // the next stage's direct-to-LDS loads (see k_step); the compiler places
  // them right behind the first reads, which measured best for this loop
  hook();
  v4f p[C::MI], prev[C::MI];
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) {
    if (j + 2 < C::NJ) wraw[j + 2] = read_w<C, PK>(wt, wn * C::TN + 16 * (j + 2), lane);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
        p[i] = mfma_bf16(wcur.k[k], xf[i].k[k], k == 0 ? v4f{0.0f, 0.0f, 0.0f, 0.0f} : p[i]);
      if (j == 0 && k < 3) {
#pragma unroll
        for (int i = 0; i < C::MI; ++i) widen_a(i, k + 1);
      }
      if (j + 1 < C::NJ) {
        const uint4& h = k < 2 ? wraw[j + 1].lo : wraw[j + 1].hi;
        wnext.k[k] = (k & 1) ? cvt8(h.z, h.w, 1.0f) : cvt8(h.x, h.y, 1.0f);
      }
      if (j > 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[k][j - 1][r] = __builtin_fmaf(prev[k][r], s[k], acc[k][j - 1][r]);
      }
      // order: this window's VALU results exist before the next window's
      // MFMAs read their operands (empty asm statements tie the registers;
      // measured ahead of sched_barrier windows and iglp_opt)
      if (k < 3) {
        if (j > 0) asm volatile("" : "+v"(wcur.k[k + 1]), "+v"(acc[k][j - 1]));
        if (j + 1 < C::NJ) asm volatile("" : "+v"(wcur.k[k + 1]), "+v"(wnext.k[k]));
        asm volatile("" : "+v"(wcur.k[k + 1]), "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]));
        if (j == 0)
          asm volatile("" : "+v"(wcur.k[k + 1]), "+v"(xf[0].k[k + 1]), "+v"(xf[1].k[k + 1]), "+v"(xf[2].k[k + 1]),
                       "+v"(xf[3].k[k + 1]));
      }
    }
#pragma unroll
    for (int i = 0; i < C::MI; ++i) prev[i] = p[i];
    if (j + 1 < C::NJ) wcur = wnext;
  }
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      acc[i][C::NJ - 1][r] = __builtin_fmaf(prev[i][r], s[i], acc[i][C::NJ - 1][r]);
}

// 2^(e - 127) for an E8M0 byte e in [1, 254] (fp32 normal); e = 0 gives
// 2^-127 (fp32 subnormal).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  // 2^-127 (the fp32 subnormal 0x00400000) times 2^e: exact for every
  // byte 0..254, one v_ldexp_f32
  return __builtin_amdgcn_ldexpf(__uint_as_float(0x00400000u), (int)e);
}

// One K step of the MXFP8 GEMM.  Each 32-block's E8M0 scale is folded into
// the FP8 -> bf16 conversion of its codes (exact while the scaled values stay
// in bf16's normal range), so the MFMAs accumulate straight into acc.  The
// lane's first 16 codes (K 16g..) lie in 32-block g/2 and its last 16
// (K 64+16g..) in 32-block 2 + g/2; scale bytes are one dword per row.
template <class C, class Hook>
__device__ __forceinline__ void compute_mx(const uint8_t* buf, v4f (&acc)[C::MI][C::NJ], Hook hook) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave % C::WM, wn = wave / C::WM, l16 = lane & 15, g = lane >> 4;
  const uint32_t* ea = reinterpret_cast<const uint32_t*>(buf + C::OFF_SA);
  const uint32_t* eb = reinterpret_cast<const uint32_t*>(buf + C::OFF_SB);
  const int b0 = 8 * (g >> 1), b1 = 8 * (2 + (g >> 1));
  // reads first (A fragments, their scales, the first weight fragment),
  // then the conversions; later weight fragments one subtile ahead
  Raw16 araw[C::MI], wraw[2];
  uint32_t eav[C::MI], ebv[2];
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    const int r = wm * C::TM + 16 * i + l16;
    eav[i] = ea[r];
    araw[i] = read_raw(buf, r, g);
  }
  ebv[0] = eb[wn * C::TN + l16];
  wraw[0] = read_raw(buf + C::OFF_W, wn * C::TN + l16, g);
  Frag16 xf[C::MI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
    xf[i] = widen(araw[i], e8m0_to_f32((eav[i] >> b0) & 0xffu), e8m0_to_f32((eav[i] >> b1) & 0xffu));
  // the conversions above are pinned before the next stage's direct-to-LDS
  // loads (see k_step), so their LDS waits stay exact (9% faster at 8192^3
  // than letting the compiler hoist the loads)
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
    asm volatile("" : "+v"(xf[i].k[0]), "+v"(xf[i].k[1]), "+v"(xf[i].k[2]), "+v"(xf[i].k[3])::"memory");
  hook();
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) {
    if (j + 1 < C::NJ) {
      const int rn = wn * C::TN + 16 * (j + 1) + l16;
      ebv[(j + 1) & 1] = eb[rn];
      wraw[(j + 1) & 1] = read_raw(buf + C::OFF_W, rn, g);
    }
    const uint32_t e = ebv[j & 1];
    const Frag16 wf = widen(wraw[j & 1], e8m0_to_f32((e >> b0) & 0xffu), e8m0_to_f32((e >> b1) & 0xffu));
    // k-outer order: consecutive MFMAs go to different accumulators
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int i = 0; i < C::MI; ++i) acc[i][j] = mfma_bf16(wf.k[k], xf[i].k[k], acc[i][j]);
  }
}

// Full K loop of one output tile over an S-stage LDS ring (separate arrays,
// so the compiler sees that the stage being filled never aliases the one
// being read).  Step kb: wait for this wave's loads of step kb (the loads of
// the S-2 later steps may stay in flight), one barrier (everyone's loads of
// step kb are visible and everyone is done reading the stage about to be
// refilled), compute step kb, and issue step kb+S-1 from inside it, once
// the step's first LDS reads have been consumed.  (While a direct-to-LDS
// load is in flight the compiler can only wait for all outstanding LDS
// reads at once, so issuing the loads first would expose the full LDS
// latency before every fragment; issued after the first batch of reads,
// the later full waits only cover reads that have long landed.)
template <class C, bool PK>
__device__ __forceinline__ void k_step(uint8_t* cur, uint8_t* refill, const Src<C>& src, int kb, int nkb,
                                       v4f (&acc)[C::MI][C::NJ]) {
  if (C::S == 3 && kb + 1 < nkb) wait_vmem<C::NI>(); else wait_vmem<0>();
  __syncthreads();
  auto hook = [&]() {
    if (kb + C::S - 1 < nkb) issue<C>(refill, src, kb + C::S - 1);
  };
  if constexpr (C::MX)
    compute_mx<C>(cur, acc, hook);
  else
    compute_block<C, PK>(cur, acc, hook);
}

// PK: the weight stages hold packed chunks (see packed_woff).
template <class C, bool PK = false>
__device__ __forceinline__ void k_loop(uint8_t* l0, uint8_t* l1, uint8_t* l2, const Src<C>& src, int nkb,
                                       v4f (&acc)[C::MI][C::NJ]) {
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  issue<C>(l0, src, 0);
  if (C::S == 2) {
    for (int kb = 0; kb < nkb; kb += 2) {
      k_step<C, PK>(l0, l1, src, kb, nkb, acc);
      if (kb + 1 < nkb) k_step<C, PK>(l1, l0, src, kb + 1, nkb, acc);
    }
  } else {
    if (nkb > 1) issue<C>(l1, src, 1);
    for (int kb = 0; kb < nkb; kb += 3) {
      k_step<C, PK>(l0, l2, src, kb, nkb, acc);
      if (kb + 1 < nkb) k_step<C, PK>(l1, l0, src, kb + 1, nkb, acc);
      if (kb + 2 < nkb) k_step<C, PK>(l2, l1, src, kb + 2, nkb, acc);
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
  const int lane = threadIdx.x & 63, wave = wave_id();
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

// Stage arrays: a kernel declares all three (unused ones cost nothing; the
// compiler drops them) so one body serves S = 2 and S = 3.
#define FP8B_STAGES(C)                                                          \
  __shared__ __attribute__((aligned(16))) uint8_t lds0[C::BUF];                 \
  __shared__ __attribute__((aligned(16))) uint8_t lds1[C::BUF];                 \
  __shared__ __attribute__((aligned(16))) uint8_t lds2[C::S == 3 ? C::BUF : 16]

// ---- block-scaled GEMM ------------------------------------------------------
// Occupancy: 512-thread tiles run one workgroup per CU (2 waves per SIMD);
// 256-thread tiles two.
template <class C, bool BF16, bool PK>
__global__ __launch_bounds__(C::NT, 512 / C::NT) void block_gemm_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ SA,
    const uint8_t* __restrict__ W, int64_t ldw, const float* __restrict__ SW, int M, int N, int K,
    void* __restrict__ Y, int64_t ldy) {
  FP8B_STAGES(C);
  const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = N / C::BN;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN, nkb = K / kBK;
  const int lane = threadIdx.x & 63, wave = wave_id();

  Src<C> src;
  // 64-bit tile bases, 32-bit per-lane offsets inside the tile (the entry
  // point keeps every leading dimension below 2^24); rows past M re-read
  // the last row and their results are never stored
  const int mlast = M - 1 - m0;
  src.abase = A + (int64_t)m0 * lda;
  if (PK) {
    src.wbase = W + (int64_t)(n0 / 16) * 1024;
    src.wstep = (size_t)N * kBK;
    make_code_src<C>(src, [&](int r) { return (uint32_t)(min(r, mlast) * lda); },
                     [&](int qw, int l) { return packed_woff(qw, l, N / 16, C::BN / 16); });
  } else {
    src.wbase = W + (int64_t)n0 * ldw;
    src.wstep = kBK;
    make_code_src<C>(src, [&](int r) { return (uint32_t)(min(r, mlast) * lda); },
                     [&](int qw, int l) { return row_major_woff(qw, l, ldw); });
  }
  src.scale_dst = -1;
  src.sbase = reinterpret_cast<const uint8_t*>(SA + (int64_t)m0 * nkb);
  src.soff = 0;
  if (wave < C::NS_A) {
    src.soff = (uint32_t)(min(64 * wave + lane, mlast) * nkb * 4);
    src.scale_dst = C::OFF_SA + 256 * wave;
  } else if (wave == C::NS_A) {
    src.sbase = reinterpret_cast<const uint8_t*>(SW + (int64_t)(n0 / 128) * nkb);
    src.soff = (uint32_t)(min(lane, C::BN / 128 - 1) * nkb * 4);
    src.scale_dst = C::OFF_SB;
  }

  v4f acc[C::MI][C::NJ];
  k_loop<C, PK>(lds0, lds1, lds2, src, nkb, acc);
  epilogue<C, BF16>(Y, acc, n0, [&](int r) -> int64_t { return m0 + r < M ? (int64_t)(m0 + r) * ldy : -1; });
}

// ---- MXFP8 GEMM ---------------------------------------------------------------
template <class C>
__global__ __launch_bounds__(C::NT, 512 / C::NT) void mx_gemm_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ EA,
    const uint8_t* __restrict__ B, int64_t ldb, const uint8_t* __restrict__ EB, int M, int N, int K,
    float* __restrict__ Y, int64_t ldy) {
  FP8B_STAGES(C);
  const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = N / C::BN;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN, nkb = K / kBK;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int srow = K / 32;  // E8M0 bytes per row

  Src<C> src;
  // 64-bit tile bases, 32-bit per-lane offsets inside the tile
  const int mlast = M - 1 - m0;
  src.abase = A + (int64_t)m0 * lda;
  src.wbase = B + (int64_t)n0 * ldb;
  src.wstep = kBK;
  make_code_src<C>(src, [&](int r) { return (uint32_t)(min(r, mlast) * lda); },
                   [&](int qw, int l) { return row_major_woff(qw, l, ldb); });
  src.scale_dst = -1;
  src.sbase = EA + (int64_t)m0 * srow;
  src.soff = 0;
  if (wave < C::NS_A) {
    src.soff = (uint32_t)(min(64 * wave + lane, mlast) * srow);
    src.scale_dst = C::OFF_SA + 256 * wave;
  } else if (wave < C::NS) {
    const int t = wave - C::NS_A;
    src.sbase = EB + (int64_t)n0 * srow;
    src.soff = (uint32_t)((64 * t + lane) * srow);
    src.scale_dst = C::OFF_SB + 256 * t;
  }

  v4f acc[C::MI][C::NJ];
  k_loop<C>(lds0, lds1, lds2, src, nkb, acc);
  epilogue<C, false>(Y, acc, n0, [&](int r) -> int64_t { return m0 + r < M ? (int64_t)(m0 + r) * ldy : -1; });
}

// ---- streaming few-row block GEMM -------------------------------------------
// With few activation rows (decode, small MoE experts) a layer streams W once
// from HBM and the math is small, so this path is built for bandwidth.  A
// workgroup owns 64 weight rows (4 subtiles of 16 per wave) and up to 16*MI
// activation rows; its 4 waves take every 4th K block, so together they read
// contiguous 512-byte runs of each weight row (one contiguous front in the
// packed layout).  Each wave loads its weight fragments straight from
// global memory into a register ring kStreamDepth K blocks ahead (no
// barrier in the loop).  The activation rows (L2 resident, read by every
// workgroup) are loaded as whole 128-byte lines, eight lanes to a line, and
// turned into MFMA fragments through a wave-private LDS tile: fragment-order
// loads would split every line over two instructions and made M = 32 about
// 20% slower than M = 16.  Each activation fragment is loaded once per K
// block and shared by the 4 weight subtiles.  The 4 partial sums are added
// in a fixed order through LDS at the end.  Measured on MI355X (8192 ->
// 28672): 64 rows per workgroup beat 16 and 32 by 10-45%, and a deeper ring
// or a 2-way K split was slower.
constexpr int kStreamDepth = 2;
constexpr int kStreamNJ = 4;
constexpr int kStreamRows = 16 * kStreamNJ;  // weight rows per workgroup

struct Raw16g {
  uint4 lo, hi;
};

// A lane's 32 codes of one 16-row x 128-K fragment, read from global memory
// (row_k = this lane's row at the K block).
__device__ __forceinline__ Raw16g load_frag_global(const uint8_t* row_k) {
  const int g = (threadIdx.x & 63) >> 4;
  Raw16g v;
  v.lo = *reinterpret_cast<const uint4*>(row_k + 16 * g);
  v.hi = *reinterpret_cast<const uint4*>(row_k + 16 * (g + 4));
  return v;
}

// The same fragment from the packed layout: the wave's subtile j of K block
// kb is chunk (2kb, p0 + j) for the first 16 codes and (2kb + 1, p0 + j) for
// the last 16.  lane_base = the panel p0's chunk at kc = 0 plus 16 * lane;
// cstride = N/16 * 1024, the distance between consecutive K chunks.  The
// codes are read once per layer, so the loads are non-temporal (measured
// 7% faster than plain loads in this layout).
__device__ __forceinline__ Raw16g load_frag_packed(const uint8_t* lane_base, int64_t cstride, int j, int kb) {
  const uint8_t* p = lane_base + 1024 * j + 2 * (int64_t)kb * cstride;
  const u32x4 lo = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  const u32x4 hi = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + cstride));
  Raw16g v;
  v.lo = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  v.hi = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  return v;
}

// Two whole 128-byte activation lines of a lane (rows r and r + 8 of a
// fragment, bytes 16 * (lane & 7) ..), kept as native vectors.
struct Lines2 {
  u32x4 lo, hi;
};

__device__ __forceinline__ Lines2 load_lines(const uint8_t* p0, const uint8_t* p1) {
  Lines2 v;
  v.lo = *reinterpret_cast<const u32x4*>(p0);
  v.hi = *reinterpret_cast<const u32x4*>(p1);
  return v;
}

// LDS needed by stream_rows<MI>: partial sums of waves 1..3.
template <int MI, int NJ = kStreamNJ>
constexpr int stream_part_bytes() {
  return 3 * MI * NJ * 64 * (int)sizeof(v4f);
}

// acc[i][j] = y rows 16i + l16 of the chunk, weight rows 16j + 4g .. +3 of
// the workgroup's 16*NJ, over all nkb K blocks.  aline[i][q]: row
// 16i + 8q + (lane >> 3) of the activation codes at byte 16 * (lane & 7)
// (eight lanes read each 128-byte line of a K block whole; the wave turns
// the lines into its MFMA fragment through a private LDS tile in lds_a,
// 4 * MI * 2048 bytes per workgroup); sarow[i]: the per-block scales of
// this lane's row 16i + l16; wload(j, kb): this lane's fragment of weight
// subtile j at K block kb; swrow: the weight-scale row of these rows.
// Every wave of the workgroup must call it; the sums are complete in wave 0
// only (the return value says which), and `part` may be reused by the
// caller only after a barrier.
template <int MI, int NJ = kStreamNJ, int D = kStreamDepth, class WLoad>
__device__ __forceinline__ bool stream_rows(const uint8_t* const (&aline)[MI][2], const float* const (&sarow)[MI],
                                            WLoad wload, const float* swrow, int nkb, uint8_t* lds_a,
                                            v4f* part, v4f (&acc)[MI][NJ]) {
  const int lane = threadIdx.x & 63, ks = wave_id();
  const int nmine = ks < nkb ? (nkb - ks + 3) / 4 : 0;  // K blocks this wave adds
  // the t-th K block of this wave; t past the end repeats its last block
  auto kblock = [&](int t) { return ks + 4 * min(t, max(nmine - 1, 0)); };

  Raw16g wr[D][NJ];
  Lines2 ar[D][MI];
  float sar[D][MI], swr[D];
  auto fetch = [&](int sl, int kb) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) wr[sl][j] = wload(j, kb);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      ar[sl][i] = load_lines(aline[i][0] + (int64_t)kb * kBK, aline[i][1] + (int64_t)kb * kBK);
      sar[sl][i] = sarow[i][kb];
    }
    swr[sl] = swrow[kb];
  };
  // the ring slots are compile-time indices (the ring stays in registers)
  auto each_slot = [&](auto f) {
    f(std::integral_constant<int, 0>{});
    if constexpr (D > 1) f(std::integral_constant<int, 1>{});
    if constexpr (D > 2) f(std::integral_constant<int, 2>{});
    static_assert(D <= 3, "ring depth");
  };
  if (nmine > 0) each_slot([&](auto slc) { fetch(decltype(slc)::value, kblock(decltype(slc)::value)); });
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};

  for (int t0 = 0; t0 < nmine; t0 += D) {
    each_slot([&](auto slc) {
      constexpr int sl = decltype(slc)::value;
      if (t0 + sl < nmine) {
        Frag16 xf[MI];
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          // lines -> fragment through the wave's swizzled 16 x 128-byte tile
          uint8_t* la = lds_a + (ks * MI + i) * 2048;
          *reinterpret_cast<u32x4*>(la + lds_off(lane >> 3, lane & 7)) = ar[sl][i].lo;
          *reinterpret_cast<u32x4*>(la + lds_off(8 + (lane >> 3), lane & 7)) = ar[sl][i].hi;
          xf[i] = widen(read_raw(la, lane & 15, lane >> 4), 1.0f, 1.0f);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const Frag16 wf = widen(Raw16{wr[sl][j].lo, wr[sl][j].hi}, 1.0f, 1.0f);
#pragma unroll
          for (int i = 0; i < MI; ++i) {
            const v4f pr = block_product(wf, xf[i], zero);
            const float sc = sar[sl][i] * swr[sl];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(pr[r], sc, acc[i][j][r]);
          }
        }
        fetch(sl, kblock(t0 + sl + D));  // refill this slot with the block D steps ahead
      }
    });
  }

  if (ks > 0) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) part[(((ks - 1) * MI + i) * NJ + j) * 64 + lane] = acc[i][j];
  }
  __syncthreads();
  if (ks > 0) return false;
#pragma unroll
  for (int q = 0; q < 3; ++q)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const v4f o = part[((q * MI + i) * NJ + j) * 64 + lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] += o[r];
      }
  return true;
}

// Lane's outputs of stream_rows: chunk row 16i + l16 at element offset
// row_off(16i + l16) of y (skipped when negative), columns n0 + 16j + 4g .. +3.
template <int MI, bool BF16, int NJ = kStreamNJ, class RowOff>
__device__ __forceinline__ void stream_store(void* __restrict__ y, const v4f (&acc)[MI][NJ], int n0,
                                             RowOff row_off) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int64_t base = row_off(16 * i + l16);
    if (base >= 0) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) store4<BF16>(y, base + n0 + 16 * j + 4 * g, acc[i][j]);
    }
  }
}

// Block GEMM for M <= 16*MI: one workgroup per 16*NJ weight rows, a
// D-deep register ring; W row-major (PK false) or packed.
template <int MI, bool BF16, bool PK, int NJ, int D>
__global__ __launch_bounds__(256) void decode_gemm_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ SA,
    const uint8_t* __restrict__ W, int64_t ldw, const float* __restrict__ SW, int M, int N, int K,
    void* __restrict__ Y, int64_t ldy) {
  __shared__ v4f part[stream_part_bytes<MI, NJ>() / sizeof(v4f)];
  __shared__ __align__(16) uint8_t lds_a[4 * MI * 2048];
  const int lane = threadIdx.x & 63, l16 = lane & 15;
  const int n0 = blockIdx.x * 16 * NJ, nkb = K / kBK;
  const uint8_t* aline[MI][2];
  const float* sarow[MI];
  // rows past M repeat the last; never stored
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    sarow[i] = SA + (int64_t)min(16 * i + l16, M - 1) * nkb;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      aline[i][q] = A + (int64_t)min(16 * i + 8 * q + (lane >> 3), M - 1) * lda + 16 * (lane & 7);
  }
  const float* swrow = SW + (int64_t)(n0 / 128) * nkb;
  v4f acc[MI][NJ];
  bool mine;
  if (PK) {
    const int64_t cs = (int64_t)(N / 16) * 1024;
    const uint8_t* wl = W + (int64_t)(n0 / 16) * 1024 + 16 * (threadIdx.x & 63);
    mine = stream_rows<MI, NJ, D>(aline, sarow, [&](int j, int kb) { return load_frag_packed(wl, cs, j, kb); },
                                  swrow, nkb, lds_a, part, acc);
  } else {
    const uint8_t* wrow = W + (int64_t)(n0 + l16) * ldw;
    mine = stream_rows<MI, NJ, D>(
        aline, sarow, [&](int j, int kb) { return load_frag_global(wrow + (int64_t)16 * j * ldw + (int64_t)kb * kBK); },
        swrow, nkb, lds_a, part, acc);
  }
  if (!mine) return;
  stream_store<MI, BF16, NJ>(Y, acc, n0, [&](int r) -> int64_t { return r < M ? (int64_t)r * ldy : -1; });
}

// ---- grouped (MoE) GEMM -----------------------------------------------------
// Persistent workgroups over two kinds of work item, both mapped in LDS by
// every workgroup from expert_offsets (prefix sums of per-expert counts), so
// the host never reads the routing:
//  * tile items: 128 x 128 output tiles of an expert's rows, ordered
//    (expert, n-tile, m-tile) with m fastest, so concurrently running m-tiles
//    of a heavy expert share its weight tile in L2;
//  * stream items: an expert's last (rows mod 128) rows when there are at
//    most kStreamTail of them (most experts of a skewed routing have only a
//    few rows): 64 weight rows each, on the streaming path, so a 5-row
//    expert costs one pass over its weights instead of 128-row tiles of MFMA
//    work.
// Tile items come first and the fine-grained stream items fill the end of the
// run (measured on MI355X with a Zipf-skewed 256-expert routing: 3-6% faster
// than interleaving the two kinds evenly or putting stream items first).
// Each XCD gets a contiguous run of work ids per round (workgroups are dealt
// to the 8 XCDs round robin), so consecutive m-tiles of one weight tile meet
// in one L2 (7-15% faster than the plain order).
constexpr int kMaxExperts = 1024;
constexpr int kStreamTail = 32;

template <class C, bool BF16, bool PK>
__global__ __launch_bounds__(C::NT, 512 / C::NT) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ SA, int T,
    const int32_t* __restrict__ RI, const int32_t* __restrict__ OFFS, int R, int E,
    const uint8_t* __restrict__ W, const float* __restrict__ SW, int N, int K, void* __restrict__ Y) {
  static_assert(C::NT == 256, "stream items use 4 waves");
  static_assert(stream_part_bytes<2>() <= C::BUF, "stream partials fit in one stage");
  static_assert(4 * 2 * 2048 <= C::BUF, "stream activation tiles fit in one stage");
  FP8B_STAGES(C);
  __shared__ int tstart[kMaxExperts + 1];  // first tile item of expert e
  __shared__ int sstart[kMaxExperts + 1];  // first stream item of expert e
  __shared__ int scan[2][C::NT];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int tiles_n = N / C::BN, nkb = K / kBK, sblocks = N / kStreamRows;

  auto off_at = [&](int e) { return min(max(OFFS[e], 0), R); };
  auto rows_of = [&](int e) { return max(off_at(e + 1) - off_at(e), 0); };
  auto tail_of = [&](int e) {  // rows handled by stream items
    const int t = rows_of(e) % C::BM;
    return t <= kStreamTail ? t : 0;
  };
  auto ntiles = [&](int e) { return ((rows_of(e) - tail_of(e) + C::BM - 1) / C::BM) * tiles_n; };
  auto nstream = [&](int e) { return tail_of(e) > 0 ? sblocks : 0; };

  // the two maps: block-wide inclusive scans of per-thread expert ranges
  const int per = (E + C::NT - 1) / C::NT;
  const int e0 = min(tid * per, E), e1 = min(e0 + per, E);
  int lt = 0, ls = 0;
  for (int e = e0; e < e1; ++e) {
    lt += ntiles(e);
    ls += nstream(e);
  }
  scan[0][tid] = lt;
  scan[1][tid] = ls;
  __syncthreads();
  for (int o = 1; o < C::NT; o <<= 1) {
    const int vt = tid >= o ? scan[0][tid - o] : 0;
    const int vs = tid >= o ? scan[1][tid - o] : 0;
    __syncthreads();
    scan[0][tid] += vt;
    scan[1][tid] += vs;
    __syncthreads();
  }
  int rt = tid ? scan[0][tid - 1] : 0, rs = tid ? scan[1][tid - 1] : 0;
  for (int e = e0; e < e1; ++e) {
    tstart[e] = rt;
    sstart[e] = rs;
    rt += ntiles(e);
    rs += nstream(e);
  }
  if (tid == C::NT - 1) {
    tstart[E] = scan[0][C::NT - 1];
    sstart[E] = scan[1][C::NT - 1];
  }
  __syncthreads();
  const int n_tile = tstart[E], n_stream = sstart[E];
  const int total = n_tile + n_stream;
  // largest e with start[e] <= w
  auto expert_of = [&](const int* start, int w) {
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (start[mid] <= w) lo = mid; else hi = mid;
    }
    return lo;
  };

  const int G = gridDim.x;
  const int slot = (G & 7) == 0 ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  for (int base = 0; base < total; base += G) {
    const int wk = base + slot;
    if (wk >= total) break;
    __syncthreads();  // the previous item may still read the stages / partials

    if (wk < n_tile) {
      const int e = expert_of(tstart, wk);
      const int rb = off_at(e), re = rb + rows_of(e) - tail_of(e);
      const int mt = (re - rb + C::BM - 1) / C::BM;
      const int loc = wk - tstart[e];
      const int tn = loc / mt, tm = loc - tn * mt;
      const int r0 = rb + tm * C::BM, n0 = tn * C::BN;
      auto token = [&](int r) { return min(max(RI[min(r0 + r, re - 1)], 0), T - 1); };

      Src<C> src;
      src.abase = A;
      if (PK) {
        src.wbase = W + (int64_t)e * N * K + (int64_t)(n0 / 16) * 1024;
        src.wstep = (size_t)N * kBK;
        make_code_src<C>(src, [&](int r) { return (uint32_t)token(r) * (uint32_t)K; },
                         [&](int qw, int l) { return packed_woff(qw, l, N / 16, C::BN / 16); });
      } else {
        src.wbase = W + ((int64_t)e * N + n0) * K;
        src.wstep = kBK;
        make_code_src<C>(src, [&](int r) { return (uint32_t)token(r) * (uint32_t)K; },
                         [&](int qw, int l) { return row_major_woff(qw, l, K); });
      }
      src.scale_dst = -1;
      src.sbase = reinterpret_cast<const uint8_t*>(SA);
      src.soff = 0;
      if (wave < C::NS_A) {
        src.soff = (uint32_t)token(64 * wave + lane) * (uint32_t)(nkb * 4);
        src.scale_dst = C::OFF_SA + 256 * wave;
      } else if (wave == C::NS_A) {
        src.sbase = reinterpret_cast<const uint8_t*>(SW + ((int64_t)e * (N / 128) + n0 / 128) * nkb);
        src.soff = (uint32_t)(min(lane, C::BN / 128 - 1) * nkb * 4);
        src.scale_dst = C::OFF_SB;
      }
      v4f acc[C::MI][C::NJ];
      k_loop<C, PK>(lds0, lds1, lds2, src, nkb, acc);
      epilogue<C, BF16>(Y, acc, n0,
                        [&](int r) -> int64_t { return r0 + r < re ? (int64_t)(r0 + r) * N : -1; });
    } else {
      const int sb = wk - n_tile;  // stream item index
      const int e = expert_of(sstart, sb);
      const int t = tail_of(e), r0 = off_at(e) + rows_of(e) - t;
      const int n0 = (sb - sstart[e]) * kStreamRows;
      const int l16 = lane & 15;
      const uint8_t* wrow = PK ? W + (int64_t)e * N * K + (int64_t)(n0 / 16) * 1024 + 16 * lane
                               : W + ((int64_t)e * N + n0 + l16) * K;
      const int64_t cs = (int64_t)(N / 16) * 1024;
      const float* swrow = SW + ((int64_t)e * (N / 128) + n0 / 128) * nkb;
      v4f* part = reinterpret_cast<v4f*>(lds0);
      auto row_off = [&](int r) -> int64_t { return r < t ? (int64_t)(r0 + r) * N : -1; };
      auto run = [&](auto mi) {
        constexpr int MI = decltype(mi)::value;
        auto token = [&](int r) { return min(max(RI[r0 + min(r, t - 1)], 0), T - 1); };
        const uint8_t* aline[MI][2];
        const float* sarow[MI];
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          sarow[i] = SA + (int64_t)token(16 * i + l16) * nkb;
#pragma unroll
          for (int q = 0; q < 2; ++q)
            aline[i][q] = A + (int64_t)token(16 * i + 8 * q + (lane >> 3)) * K + 16 * (lane & 7);
        }
        v4f acc[MI][kStreamNJ];
        bool mine;
        if (PK)
          mine = stream_rows<MI>(aline, sarow, [&](int j, int kb) { return load_frag_packed(wrow, cs, j, kb); },
                                 swrow, nkb, lds1, part, acc);
        else
          mine = stream_rows<MI>(aline, sarow, [&](int j, int kb) {
            return load_frag_global(wrow + (int64_t)16 * j * K + (int64_t)kb * kBK);
          }, swrow, nkb, lds1, part, acc);
        if (mine) stream_store<MI, BF16>(Y, acc, n0, row_off);
      };
      if (t <= 16)
        run(std::integral_constant<int, 1>{});
      else
        run(std::integral_constant<int, 2>{});
    }
  }
}

// ---- host launchers ---------------------------------------------------------
// Tile configurations (BM, BN, WM, WN) and LDS stages, chosen by measurement
// on MI355X (4096 x 18432 x 7168 and 8192^3); overridable at build time.
// Block GEMM: 128 x 128 tiles, 64 x 64 per wave, two stages, two workgroups
// per CU (larger tiles or deeper rings measured no faster: the wave's
// MFMA + widening + rescale issue is the limit, not L2 or latency).
// MX GEMM (no VALU rescale): 256 x 256 tiles, 64 x 128 per wave.
#ifndef FP8B_BLOCK_CFG
#define FP8B_BLOCK_CFG 128, 128, 2, 2
#endif
#ifndef FP8B_BLOCK_STAGES
#define FP8B_BLOCK_STAGES 2
#endif
#ifndef FP8B_MX_CFG
#define FP8B_MX_CFG 256, 256, 4, 2
#endif
#ifndef FP8B_MX_STAGES
#define FP8B_MX_STAGES 2
#endif
using BlockCfg = Cfg<FP8B_BLOCK_CFG, false, FP8B_BLOCK_STAGES>;
// M up to 128 past the streaming kernel: 64 x 128 tiles (4 waves of
// 64 x 32), twice the tiles of 128 x 128 so a decode-sized layer fills the
// chip (measured at 8192 -> 28672: M 64 93 -> 72 us, M 128 95 -> 89 us;
// three stages were slower).
#ifndef FP8B_SMALL_CFG
#define FP8B_SMALL_CFG 64, 128, 1, 4, false, 2
#endif
using SmallMCfg = Cfg<FP8B_SMALL_CFG>;
using MxCfg = Cfg<FP8B_MX_CFG, true, FP8B_MX_STAGES>;
using MxSmallCfg = Cfg<128, 128, 2, 2, true, 2>;
using GroupedCfg = Cfg<128, 128, 2, 2, false, 2>;

static int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

#ifndef FP8B_DEC1
#define FP8B_DEC1 4, 2
#endif
#ifndef FP8B_DEC2
#define FP8B_DEC2 4, 1
#endif
// Streaming-kernel shapes per 16-token subtile count MI on packed weights:
// (weight subtiles per wave NJ, register ring depth D).  Row-major weights
// keep (4, 2) and M <= 32 (their fragment loads split every 128-byte line
// over two instructions and need the deeper ring: M 32 on a 1-deep ring
// took 82 us against 60-67).  Measured on MI355X at 8192 -> 28672: one
// subtile keeps a 2-deep ring (M 1: 39.9 us against 41.4 with 1); from two
// subtiles on a 1-deep ring wins, its registers leaving room for more waves
// (M 32: 47.4 -> 42.9 us), and the streaming kernel beats the 64 x 128
// tiles up to M = 64 (M 33 / 48 / 49: 47.3 / 51.4 / 57.6 us against 62.3 /
// 62.5 / 62.8).  A sweep of NJ in {2, 4, 8} and D in {1, 2, 3} for one and
// two subtiles found nothing faster than these.
#ifndef FP8B_STREAM_MAX_M
#define FP8B_STREAM_MAX_M 64  // 32 or 64
#endif
#ifndef FP8B_DEC3
#define FP8B_DEC3 4, 1
#endif
#ifndef FP8B_DEC4
#define FP8B_DEC4 4, 1
#endif
template <int MI, bool PK, int NJ, int D>
static void launch_decode_nj(const uint8_t* a, int64_t lda, const float* sa, const uint8_t* w, int64_t ldw,
                             const float* sw, int64_t M, int64_t N, int64_t K, void* y, int64_t ldy, int out_bf16,
                             hipStream_t s) {
  const dim3 grid((unsigned)(N / (16 * NJ))), block(256);
  if (out_bf16)
    hipLaunchKernelGGL((decode_gemm_kernel<MI, true, PK, NJ, D>), grid, block, 0, s, a, lda, sa, w, ldw, sw,
                       (int)M, (int)N, (int)K, y, ldy);
  else
    hipLaunchKernelGGL((decode_gemm_kernel<MI, false, PK, NJ, D>), grid, block, 0, s, a, lda, sa, w, ldw, sw,
                       (int)M, (int)N, (int)K, y, ldy);
}

template <int MI, bool PK>
static void launch_decode(const uint8_t* a, int64_t lda, const float* sa, const uint8_t* w, int64_t ldw,
                          const float* sw, int64_t M, int64_t N, int64_t K, void* y, int64_t ldy, int out_bf16,
                          hipStream_t s) {
  if constexpr (!PK)  // row-major weights: two loads per 128-byte line, a 2-deep ring
    launch_decode_nj<MI, PK, 4, 2>(a, lda, sa, w, ldw, sw, M, N, K, y, ldy, out_bf16, s);
  else if constexpr (MI == 1)
    launch_decode_nj<1, PK, FP8B_DEC1>(a, lda, sa, w, ldw, sw, M, N, K, y, ldy, out_bf16, s);
  else if constexpr (MI == 2)
    launch_decode_nj<2, PK, FP8B_DEC2>(a, lda, sa, w, ldw, sw, M, N, K, y, ldy, out_bf16, s);
  else if constexpr (MI == 3)
    launch_decode_nj<3, PK, FP8B_DEC3>(a, lda, sa, w, ldw, sw, M, N, K, y, ldy, out_bf16, s);
  else
    launch_decode_nj<4, PK, FP8B_DEC4>(a, lda, sa, w, ldw, sw, M, N, K, y, ldy, out_bf16, s);
}

template <class C, bool PK>
static void launch_block(const uint8_t* a, int64_t lda, const float* sa, const uint8_t* w, int64_t ldw,
                         const float* sw, int64_t M, int64_t N, int64_t K, void* y, int64_t ldy, int out_bf16,
                         hipStream_t s) {
  const int64_t tiles = ((M + C::BM - 1) / C::BM) * (N / C::BN);
  const dim3 grid((unsigned)tiles), block(C::NT);
  if (out_bf16)
    hipLaunchKernelGGL((block_gemm_kernel<C, true, PK>), grid, block, 0, s, a, lda, sa, w, ldw, sw, (int)M,
                       (int)N, (int)K, y, ldy);
  else
    hipLaunchKernelGGL((block_gemm_kernel<C, false, PK>), grid, block, 0, s, a, lda, sa, w, ldw, sw, (int)M,
                       (int)N, (int)K, y, ldy);
}

template <bool PK>
static void launch_block_any(const uint8_t* a, int64_t lda, const float* sa, const uint8_t* w, int64_t ldw,
                             const float* sw, int64_t M, int64_t N, int64_t K, void* y, int64_t ldy, int out_bf16,
                             hipStream_t s) {
  // the streaming kernel for M <= 64 on packed weights (one to four 16-token
  // subtiles), M <= 32 on row-major ones
  if (M <= 16)
    launch_decode<1, PK>(a, lda, sa, w, ldw, sw, M, N, K, y, ldy, out_bf16, s);
  else if (M <= 32)
    launch_decode<2, PK>(a, lda, sa, w, ldw, sw, M, N, K, y, ldy, out_bf16, s);
  else if (PK && FP8B_STREAM_MAX_M >= 64 && M <= 64) {
    if constexpr (PK) {
      if (M <= 48)
        launch_decode<3, PK>(a, lda, sa, w, ldw, sw, M, N, K, y, ldy, out_bf16, s);
      else
        launch_decode<4, PK>(a, lda, sa, w, ldw, sw, M, N, K, y, ldy, out_bf16, s);
    }
  } else if (M <= 128)
    launch_block<SmallMCfg, PK>(a, lda, sa, w, ldw, sw, M, N, K, y, ldy, out_bf16, s);
  else
    launch_block<BlockCfg, PK>(a, lda, sa, w, ldw, sw, M, N, K, y, ldy, out_bf16, s);
}

int launch_block_gemm(const uint8_t* a, int64_t lda, const float* sa, const uint8_t* w, int64_t ldw,
                      const float* sw, int64_t M, int64_t N, int64_t K, void* y, int64_t ldy, int out_bf16,
                      bool packed, hipStream_t s) {
  if (packed)
    launch_block_any<true>(a, lda, sa, w, 0, sw, M, N, K, y, ldy, out_bf16, s);
  else
    launch_block_any<false>(a, lda, sa, w, ldw, sw, M, N, K, y, ldy, out_bf16, s);
  return check_launch();
}

template <class C>
static void launch_mx(const uint8_t* a, int64_t lda, const uint8_t* ea, const uint8_t* b, int64_t ldb,
                      const uint8_t* eb, int64_t M, int64_t N, int64_t K, float* y, int64_t ldy, hipStream_t s) {
  const int64_t tiles = ((M + C::BM - 1) / C::BM) * (N / C::BN);
  hipLaunchKernelGGL(mx_gemm_kernel<C>, dim3((unsigned)tiles), dim3(C::NT), 0, s, a, lda, ea, b, ldb, eb, (int)M,
                     (int)N, (int)K, y, ldy);
}

int launch_mx_gemm(const uint8_t* a, int64_t lda, const uint8_t* ea, const uint8_t* b, int64_t ldb,
                   const uint8_t* eb, int64_t M, int64_t N, int64_t K, float* y, int64_t ldy, hipStream_t s) {
  // the big tile once there are enough tiles to fill the chip
  if (N % MxCfg::BN == 0 && M >= 8 * MxCfg::BM)
    launch_mx<MxCfg>(a, lda, ea, b, ldb, eb, M, N, K, y, ldy, s);
  else
    launch_mx<MxSmallCfg>(a, lda, ea, b, ldb, eb, M, N, K, y, ldy, s);
  return check_launch();
}

int launch_grouped_gemm(const uint8_t* a, const float* sa, int64_t T, const int32_t* ri, const int32_t* offs,
                        int64_t R, int64_t E, const uint8_t* w, const float* sw, int64_t N, int64_t K, void* y,
                        int out_bf16, bool packed, hipStream_t s) {
  using C = GroupedCfg;
  // enough persistent workgroups to fill every CU (at its occupancy), never
  // more than the largest possible number of tiles
  const int64_t max_tiles = ((R + C::BM - 1) / C::BM + E) * (N / C::BN) + E * (N / kStreamRows);
  const int64_t nwg = std::max<int64_t>(1, std::min<int64_t>((512 / C::NT) * (int64_t)cu_count(), max_tiles));
  const dim3 grid((unsigned)nwg), block(C::NT);
#define FP8B_GROUPED(BF, PK)                                                                                  \
  hipLaunchKernelGGL((grouped_gemm_kernel<C, BF, PK>), grid, block, 0, s, a, sa, (int)T, ri, offs, (int)R, \
                     (int)E, w, sw, (int)N, (int)K, y)
  if (out_bf16) {
    if (packed) FP8B_GROUPED(true, true); else FP8B_GROUPED(true, false);
  } else {
    if (packed) FP8B_GROUPED(false, true); else FP8B_GROUPED(false, false);
  }
#undef FP8B_GROUPED
  return check_launch();
}

}  // namespace fp8blk
