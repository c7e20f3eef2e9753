/*
 * CPU oracle for the W8A8 INT8 linear layer -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The GPU library shares no code, header, table or
 * helper with it; each side implements the definitions on its own.
 *
 * What it computes is the layer described in "Realizing Native INT8 Compute
 * for Diffusion Transformers on Consumer GPUs: A Fused INT8 GEMM Kernel for
 * Ideogram 4.0" (Asaria, Salomone, Gandhi; arXiv 2606.14598), Abstract: the
 * activations are quantized per token and the weights per output channel to
 * int8, the int8 x int8 product is accumulated in int32, and the epilogue
 * applies the per-token x per-channel dequantization and adds the bias; the
 * Spanish news write-up of the same paper (aiexpert.news, "Núcleo Tritón Fuso
 * Reduce el Tiempo de Generación de Imágenes en 9,5% en Ampere de Consumo",
 * second paragraph) adds that the result is emitted as bf16.
 *
 * Where the pages leave a step open, this file takes these readings:
 *   - symmetric quantization, no zero point; scale = absmax / 127 in fp32
 *     (one IEEE division); code = round-half-to-even(fp32 quotient x / scale),
 *     clamped to [-127, 127]; a row whose scale is zero gets all-zero codes;
 *   - accumulation: exact, here in int64, checked to fit int32;
 *   - epilogue: fp32, each operation rounded to nearest, no fused multiply-add:
 *       y = bf16_rne( (s_x[m] * s_w[n]) * float(acc) + float(bias[n]) );
 *   - GELU (not on the pages; used between the MLP layers of the workloads):
 *       gelu(v) = v * Phi(v) = 0.5 * v * erfc(-v / sqrt(2)), evaluated in fp64
 *     and rounded once, directly, to bf16.
 *
 * FP8 variant (the pages' FP8 comparison point; same per-token x per-channel
 * scheme with OCP e4m3 codes in place of int8), readings:
 *   - scale = absmax / 448 in fp32 (448 is the largest finite e4m3 value);
 *     code = e4m3_rne( clamp(fp32 quotient x / scale, -448, 448) ), the
 *     e4m3 rounding being round-half-to-even on the e4m3 grid (subnormal
 *     quantum 2^-9); a row whose scale is zero gets all-zero codes;
 *   - accumulation: the exact sum of the decoded products, computed in fp64
 *     (a product of two e4m3 values is a multiple of 2^-18 below 2^17.6, so
 *     for K <= 2^17 every partial sum is an integer multiple of 2^-18 below
 *     2^53: fp64 holds it exactly), rounded once to fp32 for the epilogue;
 *   - epilogue: the int8 one, on that fp32 value.  (Matrix cores accumulate
 *     fp8 products with rounding of their own, so a GPU result is compared
 *     with this one within a derived error bound, not bit for bit.)
 *
 * Build: plain C99, -ffp-contract=off, no fast-math, so every float operation
 * below is exactly one IEEE operation.  OpenMP only splits independent rows.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_INT32 1 /* an accumulator does not fit in int32 */

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------- bf16 -- */

/* bf16 -> fp32: the 16 bits are the top half of the fp32 pattern (exact). */
static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Any double -> nearest bf16, ties to even, in one rounding.
 * bf16 keeps 8 significant bits; below 2^-126 its spacing is fixed at 2^-133.
 * a / quantum and r are exact in double (power-of-two scaling), nearbyint
 * rounds half to even in the default rounding mode, and the rounded value has
 * at most 8 significant bits, so the final conversion to float is exact. */
static uint16_t f64_to_bf16(double d) {
  if (isnan(d)) return (uint16_t)(signbit(d) ? 0xFFC0u : 0x7FC0u);
  uint16_t sign = signbit(d) ? 0x8000u : 0u;
  double a = fabs(d);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
  int e = ilogb(a); /* a in [2^e, 2^(e+1)) */
  double quantum = (e < -126) ? ldexp(1.0, -133) : ldexp(1.0, e - 7);
  double r = nearbyint(a / quantum) * quantum;
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u); /* overflow */
  float f = (float)r;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (uint16_t)(u >> 16));
}

/* fp32 -> bf16 RNE: widening to double is exact, then one rounding. */
static uint16_t f32_to_bf16(float f) { return f64_to_bf16((double)f); }

void oracle_bf16_to_f32(const uint16_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_f32(in[i]);
}
void oracle_f32_to_bf16(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
}
void oracle_f64_to_bf16(const double* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f64_to_bf16(in[i]);
}

/* ------------------------------------------------- quantization (H1,H2) -- */

/* One row of fp32 values -> int8 codes and one fp32 scale. */
static void quantize_row(const float* x, int64_t K, int8_t* q, float* scale) {
  float amax = 0.0f;
  for (int64_t k = 0; k < K; ++k) {
    float a = fabsf(x[k]);
    if (a > amax) amax = a;
  }
  float s = amax / 127.0f;
  *scale = s;
  for (int64_t k = 0; k < K; ++k) {
    if (s == 0.0f) {
      q[k] = 0;
      continue;
    }
    float t = x[k] / s;  /* one IEEE fp32 division */
    float r = rintf(t);  /* half to even (default rounding mode) */
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    q[k] = (int8_t)r;
  }
}

/* Rows of fp32 values (weights, per output channel). */
void oracle_quantize_rows_f32(const float* x, int64_t rows, int64_t K, int64_t ldx,
                              int8_t* q, int64_t ldq, float* scale) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) quantize_row(x + r * ldx, K, q + r * ldq, scale + r);
}

/* Rows of bf16 values (activations, per token): widen exactly, then as above. */
void oracle_quantize_rows_bf16(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx,
                               int8_t* q, int64_t ldq, float* scale, float* tmp_rows) {
  /* tmp_rows: caller-provided rows*K floats of scratch */
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    float* t = tmp_rows + r * K;
    for (int64_t k = 0; k < K; ++k) t[k] = bf16_to_f32(x[r * ldx + k]);
    quantize_row(t, K, q + r * ldq, scale + r);
  }
}

/* ------------------------------------------------------ FP8 (e4m3) -- */

/* OCP e4m3 code -> value: sign, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent field 0 holds the subnormals m * 2^-9; 0x7F / 0xFF are NaN. */
static double e4m3_decode(uint8_t c) {
  int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = e ? ldexp(8.0 + m, e - 10) : ldexp((double)m, -9);
  return sgn ? -v : v;
}

/* fp32 value -> OCP e4m3 code, round half to even.  Magnitudes that round
 * beyond 448 give NaN (no saturation; callers clamp first). */
static uint8_t e4m3_encode(float f) {
  if (isnan(f)) return 0x7F;
  uint8_t sgn = signbit(f) ? 0x80 : 0x00;
  double a = fabs((double)f);
  if (a == 0.0) return sgn;
  int E;
  frexp(a, &E);            /* a = frac * 2^E, frac in [0.5, 1): a in [2^(E-1), 2^E) */
  int e = E - 1;           /* unbiased exponent of a */
  if (e < -6) e = -6;      /* subnormal range shares the quantum of 2^-6 .. 2^-5 */
  double quantum = ldexp(1.0, e - 3);
  double r = nearbyint(a / quantum) * quantum;   /* exact division by a power of two */
  if (r == 0.0) return sgn;
  if (r > 448.0) return (uint8_t)(sgn | 0x7F);
  if (r < ldexp(1.0, -6)) return (uint8_t)(sgn | (uint8_t)(r / ldexp(1.0, -9)));  /* subnormal */
  frexp(r, &E);
  int er = E - 1;
  int m = (int)(r / ldexp(1.0, er - 3)) - 8;
  return (uint8_t)(sgn | ((er + 7) << 3) | m);
}

void oracle_e4m3_decode(const uint8_t* c, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_decode(c[i]);
}
void oracle_e4m3_encode(const float* f, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(f[i]);
}

/* One row of fp32 values -> e4m3 codes and one fp32 scale. */
static void quantize_row_fp8(const float* x, int64_t K, uint8_t* q, float* scale) {
  float amax = 0.0f;
  for (int64_t k = 0; k < K; ++k) {
    float a = fabsf(x[k]);
    if (a > amax) amax = a;
  }
  float s = amax / 448.0f;
  *scale = s;
  for (int64_t k = 0; k < K; ++k) {
    if (s == 0.0f) {
      q[k] = 0;
      continue;
    }
    float t = x[k] / s;  /* one IEEE fp32 division */
    if (t > 448.0f) t = 448.0f;
    if (t < -448.0f) t = -448.0f;
    q[k] = e4m3_encode(t);
  }
}

void oracle_quantize_rows_f32_fp8(const float* x, int64_t rows, int64_t K, int64_t ldx,
                                  uint8_t* q, int64_t ldq, float* scale) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) quantize_row_fp8(x + r * ldx, K, q + r * ldq, scale + r);
}

void oracle_quantize_rows_bf16_fp8(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx,
                                   uint8_t* q, int64_t ldq, float* scale, float* tmp_rows) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    float* t = tmp_rows + r * K;
    for (int64_t k = 0; k < K; ++k) t[k] = bf16_to_f32(x[r * ldx + k]);
    quantize_row_fp8(t, K, q + r * ldq, scale + r);
  }
}

/* acc[m][n] = sum_k decode(a[m][k]) * decode(b[n][k]), exact in fp64 (see header).
 * Each output is summed over k = 0, 1, ... from 0.0, as written; the codes go
 * through a 256-entry table of e4m3_decode's values (the decode depends on the
 * byte alone), and eight outputs of a row advance together, which only
 * interleaves independent sums. */
void oracle_gemm_fp8(const uint8_t* a, int64_t lda, const uint8_t* b, int64_t ldb, int64_t M,
                     int64_t N, int64_t K, double* acc) {
  double val[256];
  for (int c = 0; c < 256; ++c) val[c] = e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    const uint8_t* ar = a + m * lda;
    int64_t n = 0;
    for (; n + 8 <= N; n += 8) {
      double sum[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
      for (int64_t k = 0; k < K; ++k) {
        const double x = val[ar[k]];
        for (int j = 0; j < 8; ++j) sum[j] += x * val[b[(n + j) * ldb + k]];
      }
      for (int j = 0; j < 8; ++j) acc[m * N + n + j] = sum[j];
    }
    for (; n < N; ++n) {
      double sum = 0.0;
      for (int64_t k = 0; k < K; ++k) sum += val[ar[k]] * val[b[n * ldb + k]];
      acc[m * N + n] = sum;
    }
  }
}

/* y = bf16( (s_x[m] * s_w[n]) * fp32(acc) + float(bias[n]) ); bias may be NULL. */
void oracle_epilogue_f64acc(const double* acc, int64_t M, int64_t N, const float* s_x,
                            const float* s_w, const uint16_t* bias, uint16_t* y) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      float f = s_x[m] * s_w[n];
      float v = f * (float)acc[m * N + n];
      float o = bias ? v + bf16_to_f32(bias[n]) : v;
      y[m * N + n] = f32_to_bf16(o);
    }
  }
}

/* ------------------------------------------------------ int GEMM (H4) -- */

/* acc[m][n] = sum_k a[m][k] * b[n][k]  (both operands K-contiguous). */
void oracle_gemm_i64(const int8_t* a, int64_t lda, const int8_t* b, int64_t ldb,
                     int64_t M, int64_t N, int64_t K, int64_t* acc) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      int64_t sum = 0;
      for (int64_t k = 0; k < K; ++k) sum += (int64_t)a[m * lda + k] * (int64_t)b[n * ldb + k];
      acc[m * N + n] = sum;
    }
  }
}

/* ------------------------------------------------- epilogue (H5, H6) -- */

/* y = bf16( (s_x[m] * s_w[n]) * float(acc) + float(bias[n]) ); bias may be NULL.
 * Returns ORACLE_ERR_INT32 (and writes nothing further) if an accumulator does
 * not fit in int32, which the int32 accumulation of the method rules out. */
int oracle_epilogue(const int64_t* acc, int64_t M, int64_t N, const float* s_x,
                    const float* s_w, const uint16_t* bias, uint16_t* y) {
  for (int64_t i = 0; i < M * N; ++i)
    if (acc[i] > INT32_MAX || acc[i] < INT32_MIN) return ORACLE_ERR_INT32;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      float f = s_x[m] * s_w[n];
      float v = f * (float)(int32_t)acc[m * N + n];
      float o = bias ? v + bf16_to_f32(bias[n]) : v;
      y[m * N + n] = f32_to_bf16(o);
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------ GELU (H8) -- */

static double gelu64(double v) { return 0.5 * v * erfc(-v / sqrt(2.0)); }

void oracle_gelu_f64(const double* v, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = gelu64(v[i]);
}

/* bf16 in -> GELU in fp64 -> bf16 (one rounding). */
void oracle_gelu_bf16(const uint16_t* y, int64_t n, uint16_t* h) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) h[i] = f64_to_bf16(gelu64((double)bf16_to_f32(y[i])));
}
