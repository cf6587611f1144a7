/*
 * fp8_oracle.c -- plain CPU oracle (TEST INFRASTRUCTURE ONLY; see the header
 * for the sources and the readings it follows).
 *
 * Deliberately simple: scalar loops, exact integer inner sums, fp64 outer
 * combination, OpenMP only over independent output rows.  No blocking, no
 * reordering beyond what the definitions state.  Build with -O2 and without
 * fast-math or floating-point contraction.
 */
#include "fp8_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* Codecs.  [P1] 1.1 and [P3] format tables: E4M3 = 1 sign, 4 exponent,     */
/* 3 mantissa bits (bias 7, largest finite 448, NaN only); E5M2 = 1 sign,   */
/* 5 exponent, 2 mantissa (bias 15, largest finite 57344, Inf and NaN).     */
/* E8M0 is the shared 8-bit exponent of the MX blocks ([P1] 1.1).           */
/* ------------------------------------------------------------------------ */
double orc_e4m3_value(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);            /* 2^(1-7) * m/8 */
  else
    mag = ldexp((double)(8 + m), e - 10);  /* 2^(e-7) * (1 + m/8) */
  return sign ? -mag : mag;
}

double orc_e5m2_value(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 2) & 0x1F;
  int m = code & 0x3;
  double mag;
  if (e == 0x1F) {
    if (m != 0) return NAN;
    return sign ? -INFINITY : INFINITY;
  }
  if (e == 0)
    mag = ldexp((double)m, -16);           /* 2^(1-15) * m/4 */
  else
    mag = ldexp((double)(4 + m), e - 17);  /* 2^(e-15) * (1 + m/4) */
  return sign ? -mag : mag;
}

double orc_e8m0_value(uint8_t code) {
  if (code == 0xFF) return NAN;
  return ldexp(1.0, (int)code - 127);
}

/* Generic "clamp, then round to the nearest point of the binary grid with
 * mbits mantissa bits and minimum normal exponent emin, ties to even".
 * Works in fp64 where every step is exact: a is an fp32 value, the grid
 * spacing is a power of two, and nearbyint() rounds half to even in the
 * default rounding mode.  Returns the rounded magnitude. */
static double round_to_grid(double a, int mbits, int emin, double fmax) {
  int exp2;
  double spacing, n;
  if (a > fmax) a = fmax;
  if (a < ldexp(1.0, emin)) {
    spacing = ldexp(1.0, emin - mbits);    /* subnormal spacing */
  } else {
    (void)frexp(a, &exp2);                 /* a = f * 2^exp2, f in [0.5,1) */
    spacing = ldexp(1.0, (exp2 - 1) - mbits);
  }
  n = nearbyint(a / spacing);              /* a / spacing is exact */
  return n * spacing;
}

/* code of a finite, non-negative magnitude that lies on the grid */
static uint8_t grid_code(double mag, int mbits, int bias) {
  int emin = 1 - bias, exp2, e;
  double frac;
  if (mag == 0.0) return 0;
  if (mag < ldexp(1.0, emin))
    return (uint8_t)(int)(mag / ldexp(1.0, emin - mbits));  /* e field 0 */
  frac = frexp(mag, &exp2);                /* mag = frac * 2^exp2 */
  e = exp2 - 1;                            /* mag in [2^e, 2^(e+1)) */
  /* mantissa field = (mag / 2^e - 1) * 2^mbits, exact */
  return (uint8_t)(((e + bias) << mbits) |
                   (int)((frac * 2.0 - 1.0) * ldexp(1.0, mbits)));
}

uint8_t orc_e4m3_encode(float v) {
  double a;
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  if (isnan(v)) return (uint8_t)(sign | 0x7F);
  a = fabs((double)v);
  return (uint8_t)(sign | grid_code(round_to_grid(a, 3, -6, 448.0), 3, 7));
}

uint8_t orc_e5m2_encode(float v) {
  double a;
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  if (isnan(v)) return (uint8_t)(sign | 0x7F);
  a = fabs((double)v);
  return (uint8_t)(sign | grid_code(round_to_grid(a, 2, -14, 57344.0), 2, 15));
}

void orc_e4m3_encode_array(const float *v, int64_t n, uint8_t *out) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]);
}

void orc_e5m2_encode_array(const float *v, int64_t n, uint8_t *out) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i) out[i] = orc_e5m2_encode(v[i]);
}

/* ------------------------------------------------------------------------ */
/* Scale rules.  [P3] Dynamic Scaling: scale = max|tensor| / 448 and        */
/* fp8 = x / scale.  [P4]: scale_fmt ue8m0, i.e. a power-of-two scale; we   */
/* take the smallest power of two that keeps amax / scale <= 448.           */
/* ------------------------------------------------------------------------ */
float orc_scale_fp32(float amax) {
  volatile float q;
  if (amax == 0.0f) return 1.0f;
  q = amax / 448.0f;  /* one IEEE binary32 division, round to nearest even */
  return q;
}

int orc_scale_pow2_exp(float amax) {
  int e = -127;
  if (amax == 0.0f) return 0;
  while (e < 127 && (double)amax > ldexp(448.0, e)) ++e;
  return e;
}

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* one block: amax -> scale -> codes.  Returns the scale (as d) and writes
 * the exponent for the power-of-two formats. */
static float block_scale(float amax, int scale_fmt, int *exp_out) {
  int e;
  if (scale_fmt == ORC_SCALE_FP32) {
    *exp_out = 0;
    return orc_scale_fp32(amax);
  }
  e = orc_scale_pow2_exp(amax);
  *exp_out = e;
  return ldexpf(1.0f, e);
}

/* [P2] section 2 quantizer and [P5] FP8Cast(x / s): divide in fp32, clamp
 * to +-448 (the order of [P1]'s delayed-scaling listing), round. */
static uint8_t quantize_one(float x, float d) {
  volatile float t = x / d;
  float c = t;
  if (c > 448.0f) c = 448.0f;
  if (c < -448.0f) c = -448.0f;
  return orc_e4m3_encode(c);
}

int orc_act_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                  int block, int scale_fmt, uint8_t *q, int64_t ldq,
                  void *scales) {
  int64_t m, nblk;
  if (!x || !q || !scales || M < 0 || K < 0) return -1;
  if (block != 128 && block != 32) return -1;
  if (K % block != 0 || ldx < K || ldq < K) return -1;
  if (scale_fmt < 0 || scale_fmt > 2) return -1;
  nblk = K / block;
#pragma omp parallel for schedule(static)
  for (m = 0; m < M; ++m) {
    int64_t j, k;
    for (j = 0; j < nblk; ++j) {
      float amax = 0.0f, d;
      int e;
      for (k = j * block; k < (j + 1) * block; ++k) {
        float a = fabsf(bf16_to_f32(x[m * ldx + k]));
        if (a > amax) amax = a;
      }
      d = block_scale(amax, scale_fmt, &e);
      for (k = j * block; k < (j + 1) * block; ++k)
        q[m * ldq + k] = quantize_one(bf16_to_f32(x[m * ldx + k]), d);
      if (scale_fmt == ORC_SCALE_E8M0_BYTE)
        ((uint8_t *)scales)[m * nblk + j] = (uint8_t)(127 + e);
      else
        ((float *)scales)[m * nblk + j] = d;
    }
  }
  return 0;
}

/* [P4]: FP8 weights carry one scale per 128x128 block. */
int orc_weight_quant(const uint16_t *w, int64_t N, int64_t K, int64_t ldw,
                     int scale_fmt, uint8_t *q, int64_t ldq, float *scales) {
  int64_t tile, nt, kt;
  if (!w || !q || !scales || N < 0 || K < 0) return -1;
  if (N % 128 != 0 || K % 128 != 0 || ldw < K || ldq < K) return -1;
  if (scale_fmt != ORC_SCALE_FP32 && scale_fmt != ORC_SCALE_UE8M0) return -1;
  nt = N / 128;
  kt = K / 128;
#pragma omp parallel for schedule(static)
  for (tile = 0; tile < nt * kt; ++tile) {
    int64_t i = tile / kt, j = tile % kt, n, k;
    float amax = 0.0f, d;
    int e;
    for (n = i * 128; n < (i + 1) * 128; ++n)
      for (k = j * 128; k < (j + 1) * 128; ++k) {
        float a = fabsf(bf16_to_f32(w[n * ldw + k]));
        if (a > amax) amax = a;
      }
    d = block_scale(amax, scale_fmt, &e);
    for (n = i * 128; n < (i + 1) * 128; ++n)
      for (k = j * 128; k < (j + 1) * 128; ++k)
        q[n * ldq + k] = quantize_one(bf16_to_f32(w[n * ldw + k]), d);
    scales[i * kt + j] = d;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Weight dequantisation.  [P4] dispatch snippet, bf16 branch:              */
/* weight_dequant(weight, weight.scale) turns the FP8 weights with their    */
/* 128x128 block scales back into bf16 (the fp8_cast_bf16 conversion);     */
/* [P5] "FP8 也需要 scale": x_hat = s * x_fp8.  Reading: the product of a   */
/* code's value and its block scale is formed in fp32 (the scales' type),   */
/* i.e. rounded once to fp32, and that fp32 value is rounded to bf16,       */
/* nearest even.                                                            */
/* ------------------------------------------------------------------------ */

/* Round a finite double that is exactly an fp32 value to bf16 (8
   significant bits, fp32's exponent range, subnormals down to 2^-133),
   nearest, ties to even; overflow gives +-Inf.  Returns the bf16 bits. */
static uint16_t round_f32_to_bf16(float f) {
  union { float f; uint32_t u; } cv;
  double v = (double)f, q, r;
  int e;
  if (isnan(f)) {
    cv.f = f;
    return (uint16_t)((cv.u >> 16) | 0x40u);
  }
  if (v == 0.0 || isinf(v)) {
    cv.f = f;
    return (uint16_t)(cv.u >> 16);
  }
  frexp(fabs(v), &e);                     /* |v| in [2^(e-1), 2^e)          */
  if (e - 1 < -126) e = -125;             /* subnormal range: fixed quantum */
  q = ldexp(1.0, e - 1 - 7);              /* bf16 spacing at this binade    */
  r = nearbyint(v / q) * q;               /* exact: v/q and r*q are exact   */
  if (fabs(r) >= ldexp(1.0, 128)) r = copysign(INFINITY, v);
  cv.f = (float)r;                        /* r is a bf16 value: exact       */
  if (r == 0.0) cv.f = (float)copysign(0.0, v);
  return (uint16_t)(cv.u >> 16);
}

uint16_t orc_dequant_one(uint8_t code, float d) {
  double v = orc_e4m3_value(code);
  float p;
  if (isnan(v)) return 0x7FC0u;
  p = (float)(v * (double)d);  /* exact product (<= 28 bits), one rounding */
  return round_f32_to_bf16(p);
}

/* The packed order, element by element: chunk (kc, p) holds the 16 x 64
 * codes of rows 16p.., columns 64kc..; inside it, byte 256g + 16r + b. */
int orc_weight_pack(const uint8_t *w, int64_t G, int64_t N, int64_t K,
                    int64_t ldw, uint8_t *out) {
  int64_t i;
  if (!w || !out || G < 0 || N < 0 || K < 0) return -1;
  if (N % 16 != 0 || K % 64 != 0 || ldw < K) return -1;
  for (i = 0; i < G; ++i) {
    int64_t kc, p, g, r, b;
    for (kc = 0; kc < K / 64; ++kc)
      for (p = 0; p < N / 16; ++p)
        for (g = 0; g < 4; ++g)
          for (r = 0; r < 16; ++r)
            for (b = 0; b < 16; ++b) {
              const int64_t row = i * N + 16 * p + r, col = 64 * kc + 16 * g + b;
              out[i * N * K + (kc * (N / 16) + p) * 1024 + 256 * g + 16 * r + b] = w[row * ldw + col];
            }
  }
  return 0;
}

int orc_weight_dequant(const uint8_t *q, int64_t N, int64_t K, int64_t ldq,
                       const float *scales, uint16_t *w, int64_t ldw) {
  int64_t n;
  if (!q || !scales || !w || N < 0 || K < 0) return -1;
  if (N % 128 != 0 || K % 128 != 0 || ldq < K || ldw < K) return -1;
#pragma omp parallel for schedule(static)
  for (n = 0; n < N; ++n) {
    int64_t k;
    for (k = 0; k < K; ++k)
      w[n * ldw + k] = orc_dequant_one(q[n * ldq + k], scales[(n / 128) * (K / 128) + k / 128]);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* KV-cache quantisation.  [P2] section 4 (KV cache): E5M2 rather than     */
/* E4M3 for its range (largest finite 57344), with one scale per token     */
/* taken from the token's real-time amax ([P2]'s precision table row "KV   */
/* cache | E5M2 | per-token").  Reading: one row of the cache (a token's   */
/* K or V) is one block: d = fp32(amax / 57344) (d = 1 for amax = 0),      */
/* q = E5M2(clamp(fp32(x / d), +-57344)); dequantisation is                */
/* bf16_RNE(fp32(value(q) * d)).                                            */
/* ------------------------------------------------------------------------ */
int orc_kv_quant(const uint16_t *x, int64_t T, int64_t D, int64_t ldx, uint8_t *q,
                 int64_t ldq, float *scales) {
  int64_t t;
  if (!x || !q || !scales || T < 0 || D <= 0 || ldx < D || ldq < D) return -1;
#pragma omp parallel for schedule(static)
  for (t = 0; t < T; ++t) {
    int64_t k;
    float amax = 0.0f, d;
    for (k = 0; k < D; ++k) {
      float a = fabsf(bf16_to_f32(x[t * ldx + k]));
      if (a > amax) amax = a;
    }
    d = (amax == 0.0f) ? 1.0f : amax / 57344.0f;  /* one IEEE division */
    for (k = 0; k < D; ++k) {
      float v = bf16_to_f32(x[t * ldx + k]) / d;  /* fp32 quotient      */
      if (v > 57344.0f) v = 57344.0f;
      if (v < -57344.0f) v = -57344.0f;
      q[t * ldq + k] = orc_e5m2_encode(v);
    }
    scales[t] = d;
  }
  return 0;
}

int orc_kv_dequant(const uint8_t *q, int64_t T, int64_t D, int64_t ldq, const float *scales,
                   uint16_t *out, int64_t ldo) {
  int64_t t;
  if (!q || !scales || !out || T < 0 || D <= 0 || ldq < D || ldo < D) return -1;
#pragma omp parallel for schedule(static)
  for (t = 0; t < T; ++t) {
    int64_t k;
    for (k = 0; k < D; ++k) {
      double v = orc_e5m2_value(q[t * ldq + k]);
      out[t * ldo + k] = isnan(v) ? (uint16_t)0x7FC0u
                                  : round_f32_to_bf16((float)(v * (double)scales[t]));
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* MoE combine.  [P1] section 2 (block-scale fused MoE) and the DeepSeek-V3 */
/* guide's 8 active experts per token: after the grouped GEMM, each token's */
/* output is the gate-weighted sum of its routed rows.  The gate weights    */
/* and the (token, slot) -> routed-row map are inputs (the model's gating   */
/* function is not part of the method).  Reference: the exact sum in fp64  */
/* (each product of a bf16 and an fp32 is exact in fp64; k <= 16 terms are */
/* summed in fp64), plus the bound sum |gate * y| for tolerance checks.     */
/* ------------------------------------------------------------------------ */
int orc_moe_combine(const uint16_t *y, int64_t R, int64_t N, const int32_t *token_rows,
                    const float *gates, int64_t T, int64_t topk, double *out, double *bnd) {
  int64_t t;
  if (!y || !token_rows || !gates || !out || !bnd || R < 0 || N <= 0 || T < 0 || topk < 1)
    return -1;
  for (t = 0; t < T * topk; ++t)
    if (token_rows[t] < 0 || token_rows[t] >= R) return -1;
#pragma omp parallel for schedule(static)
  for (t = 0; t < T; ++t) {
    int64_t n, j;
    for (n = 0; n < N; ++n) {
      double acc = 0.0, b = 0.0;
      for (j = 0; j < topk; ++j) {
        const int64_t r = token_rows[t * topk + j];
        const double p = (double)gates[t * topk + j] * (double)bf16_to_f32(y[r * N + n]);
        acc += p;
        b += fabs(p);
      }
      out[t * N + n] = acc;
      bnd[t * N + n] = b;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Delayed scaling.  [P1] "Delayed Scaling" (training part): the current     */
/* step is quantised with the scale derived from earlier steps (code =       */
/* E4M3(clamp(x / scale, +-448))), then the scale for the next step is set   */
/* from the current tensor's amax with a safety margin (amax / 400); the     */
/* initial scale is 1.  [P1] pitfall section: an amax history window         */
/* (amax_history_len) and a compute algorithm "max" (the window maximum      */
/* rather than the latest value).  Readings: one scale per tensor; the       */
/* history holds the last L amaxes (fewer at the start); algo 0 = window     */
/* maximum, algo 1 = latest; next scale = fp32(h / divisor) with one IEEE    */
/* division, or 1 when h = 0.                                                */
/* ------------------------------------------------------------------------ */
int orc_delayed_scaling(const uint16_t *x, int64_t S, int64_t n, int64_t L, int algo,
                        float divisor, uint8_t *q, float *scales_used) {
  int64_t s, i;
  float scale = 1.0f;
  float *hist;
  int64_t filled = 0, pos = 0;
  if (!x || !q || !scales_used || S < 0 || n <= 0 || L < 1 || (algo != 0 && algo != 1) ||
      !(divisor > 0.0f))
    return -1;
  hist = (float *)calloc((size_t)L, sizeof(float));
  if (!hist) return -1;
  for (s = 0; s < S; ++s) {
    const uint16_t *xs = x + s * n;
    float amax = 0.0f, h = 0.0f;
    scales_used[s] = scale;
    for (i = 0; i < n; ++i) {
      float v = bf16_to_f32(xs[i]);
      float t = v / scale;               /* fp32 quotient */
      if (t > 448.0f) t = 448.0f;
      if (t < -448.0f) t = -448.0f;
      q[s * n + i] = orc_e4m3_encode(t);
      if (fabsf(v) > amax) amax = fabsf(v);
    }
    hist[pos] = amax;
    pos = (pos + 1) % L;
    if (filled < L) ++filled;
    if (algo == 1) {
      h = amax;
    } else {
      for (i = 0; i < filled; ++i)
        if (hist[i] > h) h = hist[i];
    }
    scale = (h == 0.0f) ? 1.0f : h / divisor;
  }
  free(hist);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* GEMM references.  [P2] section 3: FP8 x FP8 products accumulated in FP32 */
/* with per-block scales; [P4]: fp8_gemm(x, scale, weight, weight.scale).   */
/* Here the inner products are exact: 512 * val(code) is an integer for    */
/* every finite E4M3 code (smallest step 2^-9), so a block partial sum is   */
/* an exact int64 in units of 2^-18.                                        */
/* ------------------------------------------------------------------------ */
static void e4m3_int_table(int32_t tab[256]) {
  int c;
  for (c = 0; c < 256; ++c) {
    double v = orc_e4m3_value((uint8_t)c);
    tab[c] = isnan(v) ? 0 : (int32_t)(v * 512.0);
  }
}

int orc_block_gemm(const uint8_t *a, int64_t lda, const float *sa,
                   const uint8_t *w, int64_t ldw, const float *sw,
                   int64_t M, int64_t N, int64_t K, double *y, double *bnd) {
  int32_t tab[256];
  int64_t m, nkb;
  if (!a || !sa || !w || !sw || M < 0 || N < 0 || K < 0) return -1;
  if (N % 128 != 0 || K % 128 != 0 || lda < K || ldw < K) return -1;
  e4m3_int_table(tab);
  nkb = K / 128;
#pragma omp parallel for schedule(dynamic, 1)
  for (m = 0; m < M; ++m) {
    int64_t n, kb, k;
    for (n = 0; n < N; ++n) {
      double acc = 0.0, babs = 0.0;
      for (kb = 0; kb < nkb; ++kb) {
        int64_t p = 0, pabs = 0;
        double s = (double)sa[m * nkb + kb] * (double)sw[(n / 128) * nkb + kb];
        for (k = kb * 128; k < (kb + 1) * 128; ++k) {
          int64_t t = (int64_t)tab[a[m * lda + k]] * (int64_t)tab[w[n * ldw + k]];
          p += t;
          pabs += t < 0 ? -t : t;
        }
        acc += s * ldexp((double)p, -18);
        babs += fabs(s) * ldexp((double)pabs, -18);
      }
      if (y) y[m * N + n] = acc;
      if (bnd) bnd[m * N + n] = babs;
    }
  }
  return 0;
}

int orc_mx_gemm(const uint8_t *a, int64_t lda, const uint8_t *ea,
                const uint8_t *b, int64_t ldb, const uint8_t *eb,
                int64_t M, int64_t N, int64_t K, double *y, double *bnd) {
  int32_t tab[256];
  int64_t m, nkb;
  if (!a || !ea || !b || !eb || M < 0 || N < 0 || K < 0) return -1;
  if (K % 32 != 0 || lda < K || ldb < K) return -1;
  e4m3_int_table(tab);
  nkb = K / 32;
#pragma omp parallel for schedule(dynamic, 1)
  for (m = 0; m < M; ++m) {
    int64_t n, kb, k;
    for (n = 0; n < N; ++n) {
      double acc = 0.0, babs = 0.0;
      for (kb = 0; kb < nkb; ++kb) {
        int64_t p = 0, pabs = 0;
        /* 2^(ea-127) * 2^(eb-127) applied exactly with ldexp */
        int sh = (int)ea[m * nkb + kb] + (int)eb[n * nkb + kb] - 254 - 18;
        for (k = kb * 32; k < (kb + 1) * 32; ++k) {
          int64_t t = (int64_t)tab[a[m * lda + k]] * (int64_t)tab[b[n * ldb + k]];
          p += t;
          pabs += t < 0 ? -t : t;
        }
        acc += ldexp((double)p, sh);
        babs += ldexp((double)pabs, sh);
      }
      if (y) y[m * N + n] = acc;
      if (bnd) bnd[m * N + n] = babs;
    }
  }
  return 0;
}

int orc_grouped_gemm(const uint8_t *a, const float *sa, int64_t T,
                     const int32_t *row_index, const int32_t *offs,
                     int64_t E, int64_t R,
                     const uint8_t *const *w_e, const float *const *sw_e,
                     int64_t N, int64_t K, const int64_t *rows,
                     int64_t nrows, double *y, double *bnd) {
  int32_t tab[256];
  int64_t i, nkb, count;
  if (!a || !sa || !row_index || !offs || !w_e || !sw_e) return -1;
  if (N % 128 != 0 || K % 128 != 0 || E < 1 || R < 0 || T < 0) return -1;
  if (offs[0] != 0 || offs[E] != R) return -1;
  e4m3_int_table(tab);
  nkb = K / 128;
  count = rows ? nrows : R;
#pragma omp parallel for schedule(dynamic, 1)
  for (i = 0; i < count; ++i) {
    int64_t r = rows ? rows[i] : i, e = 0, n, kb, k, t;
    const uint8_t *we;
    const float *swe;
    if (r < 0 || r >= R) continue;
    while (e < E && !(offs[e] <= r && r < offs[e + 1])) ++e;  /* owning expert */
    if (e == E || !w_e[e] || !sw_e[e]) continue;
    we = w_e[e];
    swe = sw_e[e];
    t = row_index[r];
    if (t < 0 || t >= T) continue;
    for (n = 0; n < N; ++n) {
      double acc = 0.0, babs = 0.0;
      for (kb = 0; kb < nkb; ++kb) {
        int64_t p = 0, pabs = 0;
        double s = (double)sa[t * nkb + kb] * (double)swe[(n / 128) * nkb + kb];
        for (k = kb * 128; k < (kb + 1) * 128; ++k) {
          int64_t v = (int64_t)tab[a[t * K + k]] * (int64_t)tab[we[n * K + k]];
          p += v;
          pabs += v < 0 ? -v : v;
        }
        acc += s * ldexp((double)p, -18);
        babs += fabs(s) * ldexp((double)pabs, -18);
      }
      if (y) y[i * N + n] = acc;
      if (bnd) bnd[i * N + n] = babs;
    }
  }
  return 0;
}
