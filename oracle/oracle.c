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
