/*
 * fp8_oracle.h -- plain CPU oracle for the W8A8 block-scaled FP8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, obviously-correct
 * statement of what the GPU path must compute.  Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the product path
 * never calls it, and it shares no code, header or table with the HIP
 * library.
 *
 * Sources (the pages this oracle is written from):
 *  [P1] "ROCm 7.0 FP8/MXFP8/MXFP4" article (devpress.csdn.net, AMD channel),
 *       section 1.1 (format table: E4M3 max 448, E5M2 max 57344, MXFP8 =
 *       8 bit + shared exponent), section 1.2 (MXFP8: 32-element blocks, one
 *       scale each), section 2 (block-scale fused MoE operator), and the
 *       "Delayed Scaling" listing of the training part (order of operations:
 *       divide by the scale, clamp to +-448, cast).
 *  [P2] "LLM 推理的 FP8 混合精度工程 2026" (blog.lonae.com), section 2
 *       (quantizer Q(x) = clamp(round(x*s), -Fmax, Fmax) * s^-1, Fmax 448 /
 *       57344), section 3 (FP32 accumulation, 128x128 blockwise scales) and
 *       section 4 (KV cache in E5M2 with per-token scales).
 *  [P3] "FP8 推理" study notes (luoboask.github.io), the format tables and
 *       the "Dynamic Scaling" section (scale = max|tensor| / 448,
 *       FP8 value = FP32 value / scale).
 *  [P4] "FP8 推理提速 83.6%: DeepSeek-V3 在 AMD MI250 上的完整落地指南"
 *       (xdnf.cn), the configuration-parameter table (dtype fp8, scale_fmt
 *       ue8m0 for the 128x128 block scales, 256 routed experts, 8 active)
 *       and the runtime-dispatch snippet (act_quant per token per 128
 *       channels, then fp8_gemm(x, scale, weight, weight.scale)).
 *  [P5] "量化: FP8 与混合精度推理" (charles2530.github.io), section
 *       "FP8 也需要 scale": x_fp8 = FP8Cast(x / s), x_hat = s * x_fp8.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - The stored scale d is the dequantisation multiplier (page 2's s^-1);
 *    codes are computed from the fp32 quotient x / d (one IEEE division).
 *  - Rounding is round-to-nearest, ties to even, on the fp32 quotient, after
 *    clamping it to +-Fmax.
 *  - ue8m0 / E8M0 scales: d = 2^e with e the smallest integer such that
 *    amax <= 448 * 2^e, clamped to [-127, 127].
 *  - amax == 0: d = 1 (e = 0).
 *  - A negative value that rounds to zero keeps its sign (code 0x80).
 *  - Weight dequantisation forms value(code) * scale in fp32 and rounds that
 *    to bf16 (nearest even): two roundings, as the scales are fp32.
 *  - KV cache: one E5M2 scale per cache row (a token's K or V), from the
 *    row's amax; percentile clipping is a calibration policy, not modelled.
 *
 * All functions are reentrant; buffers are owned by the caller.
 */
#ifndef FP8_ORACLE_H
#define FP8_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* scale formats (mirror the meaning, not the code, of the product ABI) */
#define ORC_SCALE_FP32 0       /* fp32 d = fp32(amax / 448)               */
#define ORC_SCALE_UE8M0 1      /* fp32 storage of d = 2^e                 */
#define ORC_SCALE_E8M0_BYTE 2  /* one byte 127 + e per block              */

/* ---- codecs: value of each 8-bit code ([P1] 1.1, [P3] format tables) ---- */
double orc_e4m3_value(uint8_t code);  /* NaN for 0x7F / 0xFF, no Inf        */
double orc_e5m2_value(uint8_t code);  /* +-Inf for 0x7C / 0xFC, NaN e=31,m>0 */
double orc_e8m0_value(uint8_t code);  /* 2^(code-127); NaN for 0xFF         */

/* ---- encoders: clamp to +-Fmax, then nearest grid value, ties to even ---- */
uint8_t orc_e4m3_encode(float v);
uint8_t orc_e5m2_encode(float v);
void orc_e4m3_encode_array(const float *v, int64_t n, uint8_t *out);
void orc_e5m2_encode_array(const float *v, int64_t n, uint8_t *out);

/* ---- scale rules ([P3] Dynamic Scaling; [P4] scale_fmt ue8m0) ---- */
float orc_scale_fp32(float amax);    /* fp32(amax / 448); 1 when amax == 0 */
int orc_scale_pow2_exp(float amax);  /* smallest e: amax <= 448*2^e, clamped */

/* ---- act_quant: per row, per block of B consecutive elements along K ----
 * x: bf16 bit patterns, [M][ldx] (first K used).  q: [M][ldq] codes.
 * scales: fp32 [M][K/B] for ORC_SCALE_FP32 / ORC_SCALE_UE8M0, or
 *         uint8 [M][K/B] for ORC_SCALE_E8M0_BYTE.
 * Returns 0, or -1 on a bad argument. */
int orc_act_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                  int block, int scale_fmt, uint8_t *q, int64_t ldq,
                  void *scales);

/* ---- weight quant: one scale per 128x128 tile of W[N][K] ----
 * scales fp32 [N/128][K/128]. scale_fmt is ORC_SCALE_FP32 or _UE8M0. */
int orc_weight_quant(const uint16_t *w, int64_t N, int64_t K, int64_t ldw,
                     int scale_fmt, uint8_t *q, int64_t ldq, float *scales);

/* ---- weight dequantisation ([P4] weight_dequant; [P5] x_hat = s * x_fp8) --
 * w[n][k] = bf16_RNE(fp32(value(q[n][k]) * scales[n/128][k/128])): the
 * product is rounded once to fp32, then to bf16.  NaN codes give 0x7FC0.
 * N, K multiples of 128.  Returns 0, or -1 on bad arguments. */
uint16_t orc_dequant_one(uint8_t code, float d);
int orc_weight_dequant(const uint8_t *q, int64_t N, int64_t K, int64_t ldq,
                       const float *scales, uint16_t *w, int64_t ldw);

/* ---- packed weight layout (a storage order of the GPU library, not part of
 * the method: the GEMMs on packed weights compute the same y) --------------
 * For each of G matrices [N][ldw] of codes: out[i*N*K + (kc*(N/16) + p)*1024
 * + 256*g + 16*r + b] = w[i][16p + r][64kc + 16g + b] for kc < K/64,
 * p < N/16, g < 4, r < 16, b < 16.  N a multiple of 16, K of 64, ldw >= K.
 * Returns 0, or -1 on bad arguments. */
int orc_weight_pack(const uint8_t *w, int64_t G, int64_t N, int64_t K,
                    int64_t ldw, uint8_t *out);

/* ---- KV cache ([P2] section 4: E5M2, one scale per token) ----------------
 * Per row t of x [T][D]: amax over the row, d = fp32(amax / 57344) (1 if
 * amax = 0), q = E5M2(clamp(fp32(x / d), +-57344)), scales[t] = d.
 * Dequantisation: out = bf16_RNE(fp32(value(q) * d)); NaN codes give
 * 0x7FC0, Inf codes give +-Inf.  Return 0, or -1 on bad arguments. */
int orc_kv_quant(const uint16_t *x, int64_t T, int64_t D, int64_t ldx, uint8_t *q,
                 int64_t ldq, float *scales);
int orc_kv_dequant(const uint8_t *q, int64_t T, int64_t D, int64_t ldq, const float *scales,
                   uint16_t *out, int64_t ldo);

/* ---- MoE combine ([P1] section 2, fused MoE; 8 active experts per token) --
 * out[t][n] = sum_j gates[t][j] * y[token_rows[t][j]][n] (fp64, exact
 * products), bnd[t][n] = sum_j |gates[t][j] * y[...][n]|.  y is bf16 bits
 * [R][N]; gates fp32 [T][topk]; token_rows int32 [T][topk] in [0, R).
 * Returns 0, or -1 on bad arguments (including a row outside [0, R)). */
int orc_moe_combine(const uint16_t *y, int64_t R, int64_t N, const int32_t *token_rows,
                    const float *gates, int64_t T, int64_t topk, double *out, double *bnd);

/* ---- delayed scaling ([P1] "Delayed Scaling"; amax history, algo "max") ---
 * Runs S steps over x [S][n] (bf16 bits) from the initial state (scale 1,
 * empty history of length L): step s writes q[s] = E4M3(clamp(fp32(x[s] /
 * scale), +-448)) and scales_used[s] = scale, then pushes amax(x[s]) into
 * the history and sets scale = fp32(h / divisor) (1 if h = 0), h the
 * history maximum (algo 0) or the latest amax (algo 1). */
int orc_delayed_scaling(const uint16_t *x, int64_t S, int64_t n, int64_t L, int algo,
                        float divisor, uint8_t *q, float *scales_used);

/* ---- block-scaled GEMM reference: y[m][n] = sum_kb sa[m][kb] *
 * sw[n/128][kb] * sum_{k in kb} val(a[m][k]) * val(w[n][k]).
 * Inner sums are exact integers (val * 2^9 is an integer for every finite
 * E4M3 code); the combination is in fp64.  bnd[m][n] = sum_k
 * |deq a * deq w|.  Either output may be NULL.  Returns 0 / -1. */
int orc_block_gemm(const uint8_t *a, int64_t lda, const float *sa,
                   const uint8_t *w, int64_t ldw, const float *sw,
                   int64_t M, int64_t N, int64_t K, double *y, double *bnd);

/* ---- MXFP8 GEMM reference: 32-element K blocks, E8M0 byte scales for
 * both operands.  ea [M][K/32], eb [N][K/32]. */
int orc_mx_gemm(const uint8_t *a, int64_t lda, const uint8_t *ea,
                const uint8_t *b, int64_t ldb, const uint8_t *eb,
                int64_t M, int64_t N, int64_t K, double *y, double *bnd);

/* ---- grouped (MoE) GEMM reference.
 * a: [T][K] token codes, sa: [T][K/128].  Row r of the output belongs to the
 * expert e with offs[e] <= r < offs[e+1] and reads token row_index[r].
 * w_e[e] / sw_e[e]: that expert's [N][K] codes and [N/128][K/128] scales; a
 * NULL entry marks an expert whose rows are not wanted (they are skipped).
 * rows: optional list of nrows output rows to compute (NULL = all R).
 * y / bnd: [nrows or R][N]. */
int orc_grouped_gemm(const uint8_t *a, const float *sa, int64_t T,
                     const int32_t *row_index, const int32_t *offs,
                     int64_t E, int64_t R,
                     const uint8_t *const *w_e, const float *const *sw_e,
                     int64_t N, int64_t K, const int64_t *rows,
                     int64_t nrows, double *y, double *bnd);

/* number of OpenMP threads the oracle uses */
int orc_num_threads(void);
/* Threads the parallel loops use from now on (n >= 1; other values are ignored). */
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
