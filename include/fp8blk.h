/*
 * fp8blk.h -- C ABI of the MI355X (gfx950) W8A8 block-scaled FP8 linear
 * layer library (libfp8blk.so).
 *
 * What it computes (sources named by page title and section):
 *  - "FP8 推理提速 83.6%: DeepSeek-V3 在 AMD MI250 上的完整落地指南",
 *    runtime-dispatch snippet: a linear layer in fp8 mode runs
 *    act_quant(x, block_size, scale_fmt) -> (x_fp8, scale) and then
 *    fp8_gemm(x, scale, weight, weight.scale); its configuration table fixes
 *    E4M3 weights with one scale per 128x128 block, scale_fmt ue8m0, 256
 *    routed experts and 8 active experts per token.
 *  - "LLM 推理的 FP8 混合精度工程 2026", section 2: the quantizer
 *    Q(x) = clamp(round(x*s), -Fmax, Fmax) * s^-1 with Fmax = 448 (E4M3),
 *    57344 (E5M2); section 3: FP32 accumulation and blockwise scales.
 *  - "FP8 推理" study notes, Dynamic Scaling: scale = max|x| / 448 and
 *    fp8 value = x / scale.
 *  - "量化: FP8 与混合精度推理", section "FP8 也需要 scale":
 *    x_fp8 = FP8Cast(x / s), x_hat = s * x_fp8.
 *  - ROCm 7.0 FP8/MXFP8 article, sections 1.1-1.2: MXFP8 = 32-element
 *    blocks sharing one 8-bit exponent (E8M0).
 *
 * Conventions for every entry point:
 *  - All data pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or keeps them after the call returns.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default
 *    stream.  Work is enqueued asynchronously; FP8B_OK means the launch was
 *    accepted, not that the kernel finished.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    negative status means nothing was launched (except FP8B_ELAUNCH).
 *  - Where a call allows an empty dimension (M, T, R or n = 0), it reads
 *    and writes nothing and returns FP8B_OK once its sizes and enum values
 *    are valid; the pointers of the empty arrays may then be NULL.
 *  - Matrices are row-major with a leading dimension `ld_*` in elements.
 *    "Codes" are E4M3 (OCP, no Inf, largest finite 448) bytes.
 *  - Scale d is the dequantisation multiplier: x ~= d * value(code).
 *    Codes are computed from the fp32 quotient x / d, clamped to +-448 and
 *    rounded to nearest, ties to even.  A negative value that rounds to
 *    zero gives code 0x80.
 *  - Non-finite inputs give unspecified codes/outputs but never fault.
 *  - Thread-safe.  Global state: the compute-unit count of each device,
 *    queried once and cached, and the static device scratch of
 *    fp8_delayed_quant_noalloc (see there).
 */
#ifndef FP8BLK_H
#define FP8BLK_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8B_ABI_VERSION 1

typedef enum {
  FP8B_OK = 0,
  FP8B_EINVAL = -1,       /* NULL pointer, bad size, size not a multiple  */
  FP8B_EALIGN = -2,       /* pointer or leading dimension misaligned      */
  FP8B_EUNSUPPORTED = -3, /* enum value not valid for this call          */
  FP8B_ELAUNCH = -4       /* the HIP launch failed (hipGetLastError)     */
} fp8b_status;

typedef enum {
  FP8B_SCALE_FP32 = 0,      /* fp32 d = fp32(amax / 448); d = 1 if amax=0 */
  FP8B_SCALE_UE8M0 = 1,     /* fp32 storage of d = 2^e, e the smallest
                               integer with amax <= 448 * 2^e, clamped to
                               [-127, 127]; e = 0 if amax = 0            */
  FP8B_SCALE_E8M0_BYTE = 2  /* the same e stored as one byte 127 + e      */
} fp8b_scale_fmt;

typedef enum { FP8B_OUT_F32 = 0, FP8B_OUT_BF16 = 1 } fp8b_out_dtype;

typedef enum { FP8B_FMT_E4M3 = 0, FP8B_FMT_E5M2 = 1 } fp8b_elem_fmt;

/* Version of this ABI (FP8B_ABI_VERSION). */
int fp8b_abi_version(void);

/* Static description of a status code; never NULL. */
const char *fp8b_status_string(int status);

/*
 * fp8_act_quant -- dynamic activation quantisation (act_quant of the
 * DeepSeek-V3 guide's dispatch snippet; Dynamic Scaling of the "FP8 推理"
 * notes; quantizer of "FP8 engineering 2026" section 2).
 *
 *   For every row m and block j of `block_k` consecutive columns:
 *     amax = max |x[m][j*block_k ...]|, d from `scale_fmt`,
 *     q[m][k] = E4M3(clamp(fp32(x[m][k] / d), -448, 448)).
 *
 *   x       bf16 [M][ld_x], 16-byte aligned, ld_x % 8 == 0, ld_x >= K.
 *   M       rows (tokens), >= 0 (0 is a no-op).
 *   K       columns, > 0, K % block_k == 0.
 *   block_k 128 (per token per 128 channels) or 32 (MX blocks).
 *   scale_fmt FP8B_SCALE_FP32 | FP8B_SCALE_UE8M0 (fp32 scales) or
 *           FP8B_SCALE_E8M0_BYTE (one byte per block; block_k must be 32).
 *   q       uint8 codes [M][ld_q], 8-byte aligned, ld_q % 8 == 0, >= K.
 *   scales  [M][K/block_k], contiguous: float (4-byte aligned) or uint8.
 */
int fp8_act_quant(const void *x, int64_t M, int64_t K, int64_t ld_x,
                  int block_k, int scale_fmt, uint8_t *q, int64_t ld_q,
                  void *scales, void *stream);

/*
 * fp8_weight_quant -- offline weight quantisation with one scale per
 * 128x128 block (the "FP8 weights carry 128x128 block scales
 * (weight_scale_inv)" statement of the DeepSeek-V3 guide, scale_fmt ue8m0
 * in its configuration table).  Same rule as fp8_act_quant with amax taken
 * over each 128x128 tile.
 *
 *   w       bf16 [N][ld_w], 16-byte aligned, ld_w % 8 == 0, ld_w >= K.
 *   N, K    > 0, multiples of 128.
 *   scale_fmt FP8B_SCALE_FP32 or FP8B_SCALE_UE8M0.
 *   q       uint8 [N][ld_q], 8-byte aligned, ld_q % 8 == 0, ld_q >= K.
 *   scales  float [N/128][K/128], contiguous.
 */
int fp8_weight_quant(const void *w, int64_t N, int64_t K, int64_t ld_w,
                     int scale_fmt, uint8_t *q, int64_t ld_q, float *scales,
                     void *stream);

/*
 * fp8_block_gemm -- block-scaled FP8 GEMM (fp8_gemm(x, scale, weight,
 * weight.scale) of the DeepSeek-V3 guide; blockwise per-block-scale GEMM
 * with FP32 accumulation of "FP8 engineering 2026" section 3).
 *
 *   y[m][n] = sum_kb a_scales[m][kb] * w_scales[n/128][kb] *
 *             sum_{k in block kb} value(a[m][k]) * value(w[n][k])
 *   with fp32 accumulation and a per-128-K-block rescale; y is written as
 *   fp32 or bf16 (round to nearest even).  The rescale multiplies each
 *   block's fp32 partial sum by the fp32 product a_scales * w_scales: y
 *   meets the stated tolerance while that product is a normal fp32 number
 *   (at least 2^-126) and y is finite; a smaller product carries fp32's
 *   subnormal rounding (with fp8_act_quant scales, only for blocks whose
 *   activation and weight amax are both tiny).  The same holds for the
 *   packed and grouped variants below.
 *
 *   a         codes [M][ld_a], 16-byte aligned, ld_a % 16 == 0, >= K.
 *   a_scales  float [M][K/128], contiguous (fp8_act_quant with block 128).
 *   w         codes [N][ld_w], 16-byte aligned, ld_w % 16 == 0, >= K.
 *   w_scales  float [N/128][K/128], contiguous.
 *   M >= 0 (0 is a no-op); N, K > 0 and multiples of 128;
 *   ld_a, ld_w < 2^24.
 *   y         [M][ld_y] fp32 or bf16, 16-byte aligned, ld_y >= N,
 *             ld_y % 8 == 0.
 *   out_dtype FP8B_OUT_F32 or FP8B_OUT_BF16.
 */
int fp8_block_gemm(const uint8_t *a, int64_t ld_a, const float *a_scales,
                   const uint8_t *w, int64_t ld_w, const float *w_scales,
                   int64_t M, int64_t N, int64_t K, void *y, int64_t ld_y,
                   int out_dtype, void *stream);

/*
 * fp8_weight_pack -- rearrange quantised weight codes into the packed
 * layout that fp8_block_gemm_packed and fp8_grouped_gemm_packed read.  A
 * storage layout of this library, not part of the method: the codes and
 * their values are unchanged, only their order in memory.
 *
 * Layout of one [N][K] matrix (N*K bytes): 1024-byte chunks (kc, p) for
 * kc < K/64, p < N/16, chunk (kc, p) at byte (kc * N/16 + p) * 1024; byte
 * 256*g + 16*r + b of a chunk (g < 4, r < 16, b < 16) is the code of row
 * 16p + r at column 64kc + 16g + b.  K is outermost, so a GEMM that
 * streams the weights once reads them front to back, and each 64-lane
 * 16-byte load is one contiguous chunk.  G matrices are packed one after
 * the other (matrix i at i*N*K), e.g. the experts of a MoE layer.
 *
 *   w         codes [G][N][ld_w] (row-major, from fp8_weight_quant),
 *             16-byte aligned, ld_w % 16 == 0, ld_w >= K.
 *   G >= 1; N, K > 0 and multiples of 128; N <= 2^25.
 *   w_packed  G*N*K bytes, 16-byte aligned, not overlapping w.
 */
int fp8_weight_pack(const uint8_t *w, int64_t G, int64_t N, int64_t K,
                    int64_t ld_w, uint8_t *w_packed, void *stream);

/*
 * fp8_block_gemm_packed -- fp8_block_gemm (same operation, same passages,
 * same tolerance) with the weight codes in the packed layout of
 * fp8_weight_pack.  The output is bit-identical to fp8_block_gemm's for
 * M <= 32 and M > 64; for 33 <= M <= 64 the packed path streams the
 * weights while the row-major one runs tiles, so the fp32 sums are taken in
 * another (fixed) order.  Arguments as for fp8_block_gemm, except:
 *
 *   w_packed  N*K bytes from fp8_weight_pack (G = 1), 16-byte aligned.
 *   N <= 2^25.
 */
int fp8_block_gemm_packed(const uint8_t *a, int64_t ld_a,
                          const float *a_scales, const uint8_t *w_packed,
                          const float *w_scales, int64_t M, int64_t N,
                          int64_t K, void *y, int64_t ld_y, int out_dtype,
                          void *stream);

/*
 * mxfp8_gemm -- MXFP8 GEMM (ROCm 7.0 FP8 article, sections 1.1-1.2: blocks
 * of 32 elements along K share one E8M0 exponent).
 *
 *   y[m][n] = sum_kb 2^(a_e8m0[m][kb] - 127) * 2^(b_e8m0[n][kb] - 127) *
 *             sum_{k in 32-block kb} value(a[m][k]) * value(b[n][k])
 *   accumulated in fp32, written as fp32.
 *
 *   a       codes [M][ld_a]; b codes [N][ld_b]; both 16-byte aligned,
 *           ld % 16 == 0, ld >= K.
 *   a_e8m0  uint8 [M][K/32]; b_e8m0 uint8 [N][K/32]; contiguous, 4-byte
 *           aligned (fp8_act_quant with block 32, FP8B_SCALE_E8M0_BYTE).
 *   M >= 0; N, K > 0 and multiples of 128; ld_a, ld_b < 2^24.
 *   y       float [M][ld_y], 16-byte aligned, ld_y % 4 == 0, ld_y >= N.
 *
 * y meets the fp32 tolerance of the other GEMMs for every scale byte
 * 0 .. 254 while each scaled product 2^(ea + eb - 254) * value(a) *
 * value(b) and the sums lie in fp32's normal range (outside it, fp32's
 * subnormal rounding or overflow applies).  Output tiles whose scale bytes
 * all lie in 10 .. 246 fold each scale into the exact FP8 -> bf16 widening
 * of its block's codes; a tile with any byte outside that range (from
 * fp8_act_quant only for blocks with amax <= 448 * 2^-118 or above
 * 448 * 2^119) takes each 32-block's partial sum in fp32 and scales it by
 * an exact power of two instead (slower, same result contract).  Scale
 * byte 0xFF (NaN) gives unspecified outputs.
 */
int mxfp8_gemm(const uint8_t *a, int64_t ld_a, const uint8_t *a_e8m0,
               const uint8_t *b, int64_t ld_b, const uint8_t *b_e8m0,
               int64_t M, int64_t N, int64_t K, float *y, int64_t ld_y,
               void *stream);

/*
 * fp8_grouped_gemm -- grouped block-scaled GEMM for mixture-of-experts
 * layers (the DeepSeek-V3 guide's 256 routed / 8 active experts; the
 * block-scale fused MoE operator of the ROCm 7.0 article, section 2).
 *
 *   Output row r (0 <= r < R) belongs to the expert e with
 *   expert_offsets[e] <= r < expert_offsets[e+1] and reads token
 *   t = row_index[r]:
 *     y[r][n] = sum_kb a_scales[t][kb] * w_scales[e][n/128][kb] *
 *               sum_{k in kb} value(a[t][k]) * value(w[e][n][k])
 *   (the gather happens inside the kernel; rows are written in routed
 *   order).  The per-expert tile map is derived on the device from
 *   expert_offsets: no host synchronisation and no workspace.
 *
 *   a               token codes [T][K] (contiguous, 16-byte aligned).
 *   a_scales        float [T][K/128].
 *   row_index       int32 [R] (device) token of each routed row.
 *   expert_offsets  int32 [E+1] (device), non-decreasing, [0] = 0,
 *                   [E] = R.  Entries outside that contract, or token ids
 *                   outside [0, T), give unspecified rows but never fault.
 *   T >= 1, R >= 0 (0 is a no-op), 1 <= E <= 1024; T * K < 2^32 (the
 *   token matrix is gathered with 32-bit offsets).
 *   w               codes [E][N][K] (contiguous, 16-byte aligned).
 *   w_scales        float [E][N/128][K/128].
 *   N, K            > 0, multiples of 128.
 *   y               [R][N] fp32 or bf16, 16-byte aligned.
 *   out_dtype       FP8B_OUT_F32 or FP8B_OUT_BF16.
 */
int fp8_grouped_gemm(const uint8_t *a, const float *a_scales, int64_t T,
                     const int32_t *row_index, const int32_t *expert_offsets,
                     int64_t R, int64_t E, const uint8_t *w,
                     const float *w_scales, int64_t N, int64_t K, void *y,
                     int out_dtype, void *stream);

/*
 * fp8_grouped_gemm_packed -- fp8_grouped_gemm (same operation, same
 * passages, bit-identical output) with the expert weights in the packed
 * layout: w_packed is fp8_weight_pack of the [E][N][K] codes with G = E
 * (16-byte aligned).  Other arguments as for fp8_grouped_gemm; N <= 2^25.
 */
int fp8_grouped_gemm_packed(const uint8_t *a, const float *a_scales,
                            int64_t T, const int32_t *row_index,
                            const int32_t *expert_offsets, int64_t R,
                            int64_t E, const uint8_t *w_packed,
                            const float *w_scales, int64_t N, int64_t K,
                            void *y, int out_dtype, void *stream);

/*
 * fp8_moe_combine -- the gate-weighted combine after fp8_grouped_gemm,
 * closing a block-scale MoE layer (ROCm 7.0 FP8 article, section 2: the
 * block-scale fused MoE operator; the DeepSeek-V3 guide: 8 active experts
 * per token):
 *
 *   out[t][n] = sum_{j < topk} gates[t][j] * y[token_rows[t][j]][n]
 *   accumulated in fp32 in slot order (one fused multiply-add per slot),
 *   written as fp32 or bf16 (nearest even).
 *
 *   y           bf16 [R][N] (the grouped GEMM's rows in routed order),
 *               contiguous, 16-byte aligned; R >= 1.
 *   N           > 0, N % 8 == 0.
 *   token_rows  int32 [T][topk]: routed row of (token, slot); rows outside
 *               [0, R) give unspecified outputs but never fault.
 *   gates       float [T][topk] gate weights (the model's gating function
 *               is the caller's).
 *   T >= 0 (0 is a no-op); 1 <= topk <= 64.
 *   out         [T][N] fp32 or bf16, contiguous, 16-byte aligned.
 *   out_dtype   FP8B_OUT_F32 or FP8B_OUT_BF16.
 */
int fp8_moe_combine(const void *y, int64_t R, int64_t N,
                    const int32_t *token_rows, const float *gates, int64_t T,
                    int64_t topk, void *out, int out_dtype, void *stream);

/*
 * fp8_weight_dequant -- weight dequantisation, the bf16 branch of the
 * DeepSeek-V3 guide's dispatch snippet (weight_dequant(weight,
 * weight.scale), used to turn the FP8 checkpoint into bf16) and
 * x_hat = s * x_fp8 of "量化: FP8 与混合精度推理", section "FP8 也需要 scale":
 *
 *   w[n][k] = bf16_RNE(fp32(value(q[n][k]) * scales[n/128][k/128]))
 *   (the product is rounded once to fp32, then to bf16, nearest even).
 *
 *   q       codes [N][ld_q], 16-byte aligned, ld_q % 16 == 0, ld_q >= K.
 *   N, K    > 0, multiples of 128.
 *   scales  float [N/128][K/128], contiguous (fp8_weight_quant's layout).
 *   w       bf16 [N][ld_w], 16-byte aligned, ld_w % 8 == 0, ld_w >= K.
 *   NaN codes (0x7F, 0xFF) give NaN; products beyond bf16's range give
 *   +-Inf.
 */
int fp8_weight_dequant(const uint8_t *q, int64_t N, int64_t K, int64_t ld_q,
                       const float *scales, void *w, int64_t ld_w,
                       void *stream);

/*
 * fp8_kv_quant / fp8_kv_dequant -- KV-cache quantisation of "LLM 推理的 FP8
 * 混合精度工程 2026", section 4 (E5M2 rather than E4M3 for the KV cache, for
 * its range; one scale per token from the token's real-time amax, as in the
 * section's precision table):
 *
 *   per row t of x [T][D] (one token's K or V):
 *     amax = max_k |x[t][k]|,  d = fp32(amax / 57344)  (d = 1 if amax = 0),
 *     q[t][k] = E5M2(clamp(fp32(x[t][k] / d), -57344, 57344)),  scales[t] = d;
 *   dequantisation: out[t][k] = bf16_RNE(fp32(value(q[t][k]) * scales[t])).
 *
 *   T >= 0 (0 is a no-op); D in (0, 16384], D % 16 == 0.  Per-head scales:
 *   pass the cache as T*heads rows of D = head_dim.
 *   x       bf16 [T][ld_x], 16-byte aligned, ld_x % 8 == 0, ld_x >= D.
 *   q       E5M2 bytes [T][ld_q], ld_q >= D; quant: 8-byte aligned,
 *           ld_q % 8 == 0; dequant: 16-byte aligned, ld_q % 16 == 0.
 *   scales  float [T], contiguous.
 *   out     bf16 [T][ld_out], 16-byte aligned, ld_out % 8 == 0, >= D.
 *   Inf codes give +-Inf, NaN codes NaN.
 */
int fp8_kv_quant(const void *x, int64_t T, int64_t D, int64_t ld_x,
                 uint8_t *q, int64_t ld_q, float *scales, void *stream);
int fp8_kv_dequant(const uint8_t *q, int64_t T, int64_t D, int64_t ld_q,
                   const float *scales, void *out, int64_t ld_out,
                   void *stream);

/*
 * Delayed scaling (ROCm 7.0 FP8/MXFP8/MXFP4 article, training part,
 * "Delayed Scaling": quantise a step with the scale derived from earlier
 * steps, then take the next scale from the current amax with a safety
 * margin, amax / 400, starting from scale 1; its pitfall section: an amax
 * history window (amax_history_len) and the "max" compute algorithm).
 * One scale per tensor.  The state is device memory owned by the caller:
 *
 *   fp8b_delayed_state header (FP8B_DELAYED_HEADER_BYTES) followed by
 *   float history[len].
 *
 * fp8_delayed_state_init writes the initial state (scale 1, empty history)
 * with a kernel (no memset, so it may be captured in a graph).
 *
 * fp8_delayed_quant runs one step on the stream:
 *   d = state.scale;  q[i] = E4M3(clamp(fp32(x[i] / d), -448, 448));
 *   *scale_used = d (the dequantisation scale of these codes);
 *   amax = max_i |x[i]| pushed into the history (the oldest entry leaves
 *   once `history_len` are held);
 *   state.scale = fp32(h / amax_divisor), or 1 if h = 0, where h is the
 *   history maximum (FP8B_AMAX_MAX) or this step's amax (FP8B_AMAX_LATEST).
 *   One kernel does the whole step: the workgroup that finishes last
 *   (counted through the amax slots and state.done) updates the history
 *   and the scale, so the scale the next call reads is in place when this
 *   call's work is done.
 *   Calls that share a state must be ordered (one stream); the same
 *   history_len must be passed to every call on a state.
 *
 *   x            bf16 [n], 16-byte aligned; n > 0, n % 8 == 0.
 *   state        FP8B_DELAYED_STATE_BYTES(history_len) bytes, 16-byte
 *                aligned; 1 <= history_len <= FP8B_DELAYED_MAX_HISTORY.
 *   amax_divisor > 0 (the article uses 400: 448 with about 10% margin).
 *   q            uint8 codes [n], 8-byte aligned.
 *   scale_used   float [1].
 */
#define FP8B_DELAYED_MAX_HISTORY 65536
#define FP8B_DELAYED_AMAX_SLOTS 16
#define FP8B_DELAYED_HEADER_BYTES (128 + 128 * FP8B_DELAYED_AMAX_SLOTS)
#define FP8B_DELAYED_STATE_BYTES(len) (FP8B_DELAYED_HEADER_BYTES + 4 * (int64_t)(len))
typedef struct {
  float scale;        /* the scale the next step uses                   */
  uint32_t done;      /* amax slots of a step in flight that completed  */
  int32_t pos;        /* next history slot                              */
  int32_t filled;     /* history entries written so far (<= len)       */
  uint32_t reserved[28];
  /* running amax of a step in flight, spread over slots so that the
   * workgroups' atomics do not all meet on one word: slot s holds the
   * float bits of its maximum in step_amax[s][0] and the number of its
   * workgroups that finished in step_amax[s][1], one 128-byte line per
   * slot; zero between steps */
  uint32_t step_amax[FP8B_DELAYED_AMAX_SLOTS][32];
  /* float history[len] follows */
} fp8b_delayed_state;
typedef enum { FP8B_AMAX_MAX = 0, FP8B_AMAX_LATEST = 1 } fp8b_amax_algo;

int fp8_delayed_state_init(void *state, int64_t history_len, void *stream);
int fp8_delayed_quant(const void *x, int64_t n, void *state,
                      int64_t history_len, int algo, float amax_divisor,
                      uint8_t *q, float *scale_used, void *stream);

/*
 * fp8_delayed_quant_noalloc -- for callers that cannot allocate device
 * memory or bring a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): fp8_delayed_quant with the
 * step-in-flight scratch (the amax slots and the step ticket) kept in a
 * file-scope static device array of the library instead of the state.
 * Same arguments, checks, results and state layout as fp8_delayed_quant;
 * the state's step_amax lines and `done` word are left untouched, and a
 * state may be advanced by either entry point.
 *
 *   The scratch is FP8B_DELAYED_NOALLOC_SCRATCH_BYTES (2176) bytes per GPU,
 *   whatever n is, held from the first call on that GPU until the process
 *   ends.  n is bounded as for fp8_delayed_quant (n % 8 == 0,
 *   n / 8192 < 2^31): larger sizes return FP8B_EINVAL.
 *   The first call on a GPU looks up the array's device address (with that
 *   GPU current) and clears it with a kernel on `stream`; each step leaves
 *   it cleared for the next.  No hipMalloc/hipFree or other allocation.
 *   Every call on one GPU shares that GPU's scratch: calls that overlap on
 *   one GPU (on different streams, or in one graph without an order
 *   between them) race and give wrong scales.  Order them.
 *   Returns FP8B_ELAUNCH if the symbol lookup or a launch fails, and
 *   FP8B_EUNSUPPORTED on a device index of 64 or more.
 */
#define FP8B_DELAYED_NOALLOC_SCRATCH_BYTES (128 * (FP8B_DELAYED_AMAX_SLOTS + 1))
int fp8_delayed_quant_noalloc(const void *x, int64_t n, void *state,
                              int64_t history_len, int algo,
                              float amax_divisor, uint8_t *q,
                              float *scale_used, void *stream);

/*
 * fp8_cast_f32 -- FP8Cast of "量化: FP8 与混合精度推理" (x_fp8 =
 * FP8Cast(x / s)) with s = 1: clamp each fp32 value to +-Fmax (448 for
 * E4M3, 57344 for E5M2) and round to nearest, ties to even.
 *
 *   x    float [n] (4-byte aligned); n >= 0.
 *   fmt  FP8B_FMT_E4M3 or FP8B_FMT_E5M2.
 *   q    uint8 [n].
 */
int fp8_cast_f32(const float *x, int64_t n, int fmt, uint8_t *q, void *stream);

/*
 * fp8b_mfma_loop -- a measurement aid, not a step of the method: a dense
 * loop of one MFMA instruction on operands held in registers, with no
 * memory traffic, conversion or rescale.  Its rate is the matrix-core
 * ceiling the part sustains for that instruction, clock and power limits
 * included; benchmarks set the GEMMs' rates beside it.
 *
 *   kind        FP8B_MFMA_BF16_16X16X32: v_mfma_f32_16x16x32_bf16, the
 *               instruction every GEMM of this library runs its products
 *               on; FP8B_MFMA_FP8_16X16X128: v_mfma_scale_f32_16x16x128_f8f6f4
 *               on E4M3 operands with unit scales.
 *   ops         uint32 [64][64], device, 16-byte aligned: row l is lane l's
 *               operand words (bf16 pairs for kind 0, E4M3 bytes for kind
 *               1), the same for every wave.  Chain c (0 or 1) takes A from
 *               words 8c..8c+3 and B from 8c+4..8c+7 (kind 0), or A from
 *               16c..16c+7 and B from 16c+8..16c+15 (kind 1); the other
 *               words are not read.
 *   iters       rounds per wave, 1 .. 2^30; a round is one MFMA on each of
 *               the 2 chains, each accumulating into its own registers.
 *   workgroups  1 .. 2^20 workgroups of 4 waves (256 threads).
 *   out         float [workgroups][256], device, 4-byte aligned: each lane's
 *               sum of its 8 accumulator values.
 *
 * FLOPs per call: workgroups * 4 * iters * 2 * 16384 (kind 0) or * 65536
 * (kind 1).  Returns FP8B_EUNSUPPORTED for another kind.
 */
typedef enum { FP8B_MFMA_BF16_16X16X32 = 0, FP8B_MFMA_FP8_16X16X128 = 1 } fp8b_mfma_kind;

int fp8b_mfma_loop(int kind, const uint32_t *ops, int64_t iters, int64_t workgroups,
                   float *out, void *stream);

/*
 * fp8b_stream_probe -- a measurement aid, not a step of the method: two
 * kernels of their own with the grid and workgroup shape of fp8_act_quant
 * (block 128, fp32 scales) on x bf16 [M][K] (contiguous rows):
 *   FP8B_PROBE_COPY:  act_quant's loads and stores without its arithmetic --
 *                     q[m][k] = low byte of x[m][k] and scales[m][k/128] = 0
 *                     (the same bytes moved);
 *   FP8B_PROBE_EMPTY: every workgroup returns at once (launch and drain).
 * Timed beside fp8_act_quant it separates the memory system's rate for this
 * access pattern, and the launch's fixed cost, from the quantiser's own work.
 *
 *   x        bf16 [M][K], 16-byte aligned; M >= 1; K > 0, K % 128 == 0.
 *   q        uint8 [M][K], 8-byte aligned.
 *   scales   float [M][K/128], 4-byte aligned.
 *   Returns FP8B_EUNSUPPORTED for another kind.
 */
typedef enum { FP8B_PROBE_COPY = 0, FP8B_PROBE_EMPTY = 1 } fp8b_probe_kind;

int fp8b_stream_probe(int kind, const void *x, int64_t M, int64_t K,
                      uint8_t *q, float *scales, void *stream);

/*
 * fp8b_gemm_probe -- a measurement aid, not a step of the method: the
 * 128 x 128 tile kernel fp8_block_gemm_packed runs for these sizes (with
 * its K split when the grid has at most one tile per CU and the number of
 * K blocks is even, as at 65 .. 128 tokens), bf16 output, with every
 * workgroup reading the codes and scales of output tile (0, 0) and writing
 * its results to its own output tile, so the operands stay resident in L2.
 * It does the same work per tile as the GEMM; timed beside it, it shows
 * what the operand traffic beyond L2 costs.  Tile (0, 0) of y is the
 * GEMM's own result; the others hold copies of it.
 *
 *   kind      FP8B_GEMM_PROBE_TILE0.
 *   a, a_scales, w_packed, w_scales: as for fp8_block_gemm_packed with
 *             ld_a = K.
 *   M, N, K   multiples of 128, each >= 128 (M <= 2^30, N < 2^24, K < 2^24,
 *             (M/128) x (N/128) < 2^31 tiles).
 *   y         bf16 [M][N], 16-byte aligned (ld_y = N).
 *   Returns FP8B_EUNSUPPORTED for another kind.
 */
typedef enum { FP8B_GEMM_PROBE_TILE0 = 0 } fp8b_gemm_probe_kind;
int fp8b_gemm_probe(int kind, const uint8_t *a, const float *a_scales,
                    const uint8_t *w_packed, const float *w_scales, int64_t M,
                    int64_t N, int64_t K, void *y, void *stream);

#ifdef __cplusplus
}
#endif
#endif
