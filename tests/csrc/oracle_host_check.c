/* Sanitizer build of the CPU oracle (oracle/oracle.c): each exported function
 * runs on small odd-sized inputs held in exactly sized heap buffers, with
 * leading dimensions larger than the row length, empty inputs and the edge
 * values the oracle special-cases (zero rows, subnormal scales, int32
 * overflow, e4m3 ties and NaN codes).  Built with -fsanitize=address,undefined
 * by tests/test_host_sanitizers.py; a few closed-form values are checked on
 * the way.  Exits 0 after printing "oracle ok". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_num_threads(void);
void oracle_bf16_to_f32(const uint16_t* in, float* out, int64_t n);
void oracle_f32_to_bf16(const float* in, uint16_t* out, int64_t n);
void oracle_f64_to_bf16(const double* in, uint16_t* out, int64_t n);
void oracle_quantize_rows_f32(const float* x, int64_t rows, int64_t K, int64_t ldx, int8_t* q,
                              int64_t ldq, float* scale);
void oracle_quantize_rows_bf16(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, int8_t* q,
                               int64_t ldq, float* scale, float* tmp_rows);
void oracle_gemm_i64(const int8_t* a, int64_t lda, const int8_t* b, int64_t ldb, int64_t M,
                     int64_t N, int64_t K, int64_t* acc);
int oracle_epilogue(const int64_t* acc, int64_t M, int64_t N, const float* s_x, const float* s_w,
                    const uint16_t* bias, uint16_t* y);
void oracle_gelu_f64(const double* v, double* out, int64_t n);
void oracle_gelu_bf16(const uint16_t* y, int64_t n, uint16_t* h);
void oracle_e4m3_decode(const uint8_t* c, double* out, int64_t n);
void oracle_e4m3_encode(const float* f, uint8_t* out, int64_t n);
void oracle_quantize_rows_f32_fp8(const float* x, int64_t rows, int64_t K, int64_t ldx, uint8_t* q,
                                  int64_t ldq, float* scale);
void oracle_quantize_rows_bf16_fp8(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx,
                                   uint8_t* q, int64_t ldq, float* scale, float* tmp_rows);
void oracle_gemm_fp8(const uint8_t* a, int64_t lda, const uint8_t* b, int64_t ldb, int64_t M,
                     int64_t N, int64_t K, double* acc);
void oracle_epilogue_f64acc(const double* acc, int64_t M, int64_t N, const float* s_x,
                            const float* s_w, const uint16_t* bias, uint16_t* y);

static int failures = 0;
#define CHECK(c)                                                         \
  do {                                                                   \
    if (!(c)) {                                                          \
      fprintf(stderr, "check failed, line %d: %s\n", __LINE__, #c);      \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) abort();
  return p;
}

int main(void) {
  CHECK(oracle_num_threads() >= 1);
  enum { R = 3, K = 40, LD = 56, N = 9 };
  /* bf16 conversions, including every pattern once */
  {
    uint16_t* pat = xmalloc(65536 * sizeof *pat);
    float* f = xmalloc(65536 * sizeof *f);
    uint16_t* back = xmalloc(65536 * sizeof *back);
    double* d = xmalloc(65536 * sizeof *d);
    for (int i = 0; i < 65536; ++i) pat[i] = (uint16_t)i;
    oracle_bf16_to_f32(pat, f, 65536);
    oracle_f32_to_bf16(f, back, 65536);
    for (int i = 0; i < 65536; ++i) {
      d[i] = (double)f[i];
      if (!isnan(f[i])) CHECK(back[i] == pat[i]);
    }
    oracle_f64_to_bf16(d, back, 65536);
    for (int i = 0; i < 65536; ++i)
      if (!isnan(f[i])) CHECK(back[i] == pat[i]);
    free(pat); free(f); free(back); free(d);
  }
  /* int8 quantization: strided rows, a zero row, a subnormal row */
  {
    float* x = xmalloc(R * LD * sizeof *x);
    int8_t* q = xmalloc(R * LD);
    float* s = xmalloc(R * sizeof *s);
    for (int r = 0; r < R; ++r)
      for (int k = 0; k < LD; ++k) x[r * LD + k] = (float)((k * 7 + r) % 23) - 11.0f;
    memset(x + LD, 0, K * sizeof *x);                          /* row 1: all zero */
    for (int k = 0; k < K; ++k) x[2 * LD + k] = ldexpf((float)(k % 5) - 2.0f, -140);
    oracle_quantize_rows_f32(x, R, K, LD, q, LD, s);
    CHECK(s[1] == 0.0f);
    for (int k = 0; k < K; ++k) CHECK(q[LD + k] == 0);
    int m0 = 0;
    for (int k = 0; k < K; ++k) m0 = abs(q[k]) > m0 ? abs(q[k]) : m0;
    CHECK(m0 == 127);
    oracle_quantize_rows_f32(x, 0, K, LD, q, LD, s);            /* no rows */
    uint16_t* xb = xmalloc(R * LD * sizeof *xb);
    oracle_f32_to_bf16(x, xb, R * LD);
    float* tmp = xmalloc(R * K * sizeof *tmp);
    oracle_quantize_rows_bf16(xb, R, K, LD, q, LD, s, tmp);
    CHECK(s[1] == 0.0f);
    free(x); free(q); free(s); free(xb); free(tmp);
  }
  /* int GEMM + epilogue: all-ones closed form, overflow rejected, K = 0 */
  {
    int8_t* a = xmalloc(R * LD);
    int8_t* b = xmalloc(N * LD);
    int64_t* acc = xmalloc(R * N * sizeof *acc);
    memset(a, 1, R * LD);
    memset(b, 1, N * LD);
    oracle_gemm_i64(a, LD, b, LD, R, N, K, acc);
    for (int i = 0; i < R * N; ++i) CHECK(acc[i] == K);
    float* sx = xmalloc(R * sizeof *sx);
    float* sw = xmalloc(N * sizeof *sw);
    uint16_t* bias = xmalloc(N * sizeof *bias);
    uint16_t* y = xmalloc(R * N * sizeof *y);
    for (int i = 0; i < R; ++i) sx[i] = 0.5f;
    for (int i = 0; i < N; ++i) { sw[i] = 2.0f; bias[i] = 0x3F80; } /* bias 1.0 */
    CHECK(oracle_epilogue(acc, R, N, sx, sw, bias, y) == 0);
    for (int i = 0; i < R * N; ++i) CHECK(y[i] == 0x4224);          /* 40 + 1 = 41 */
    CHECK(oracle_epilogue(acc, R, N, sx, sw, NULL, y) == 0);
    acc[4] = (int64_t)1 << 31;
    CHECK(oracle_epilogue(acc, R, N, sx, sw, bias, y) != 0);
    oracle_gemm_i64(a, LD, b, LD, R, N, 0, acc);
    for (int i = 0; i < R * N; ++i) CHECK(acc[i] == 0);
    free(a); free(b); free(acc); free(sx); free(sw); free(bias); free(y);
  }
  /* GELU */
  {
    double v[5] = {0.0, 1.0, -1.0, 8.0, -40.0}, g[5];
    oracle_gelu_f64(v, g, 5);
    CHECK(g[0] == 0.0 && fabs(g[3] - 8.0) < 1e-12 && g[1] - g[2] > 0.999999999 && g[1] - g[2] < 1.000000001);
    uint16_t* in = xmalloc(65536 * sizeof *in);
    uint16_t* h = xmalloc(65536 * sizeof *h);
    for (int i = 0; i < 65536; ++i) in[i] = (uint16_t)i;
    oracle_gelu_bf16(in, 65536, h);
    CHECK(h[0] == 0 && h[0x3F80] != 0);
    free(in); free(h);
  }
  /* FP8: every code decoded, ties encoded, quantize, GEMM, epilogue */
  {
    uint8_t* c = xmalloc(256);
    double* dv = xmalloc(256 * sizeof *dv);
    for (int i = 0; i < 256; ++i) c[i] = (uint8_t)i;
    oracle_e4m3_decode(c, dv, 256);
    CHECK(dv[0x7E] == 448.0 && dv[0xFE] == -448.0 && isnan(dv[0x7F]) && dv[1] == ldexp(1.0, -9));
    float t[4] = {1.0625f, 1.1875f, -0.0f, 1000.0f};
    uint8_t e[4];
    oracle_e4m3_encode(t, e, 4);
    CHECK(e[0] == 0x38 && e[1] == 0x3A && e[2] == 0x80 && e[3] == 0x7F);
    float* x = xmalloc(R * LD * sizeof *x);
    for (int i = 0; i < R * LD; ++i) x[i] = (float)(i % 17) - 8.0f;
    uint8_t* q = xmalloc(R * LD);
    uint8_t* w = xmalloc(N * LD);
    float* s = xmalloc(R * sizeof *s);
    float* sw = xmalloc(N * sizeof *sw);
    oracle_quantize_rows_f32_fp8(x, R, K, LD, q, LD, s);
    uint16_t* xb = xmalloc(R * LD * sizeof *xb);
    float* tmp = xmalloc(R * K * sizeof *tmp);
    oracle_f32_to_bf16(x, xb, R * LD);
    oracle_quantize_rows_bf16_fp8(xb, R, K, LD, q, LD, s, tmp);
    memset(w, 0x38, N * LD);                                       /* every weight 1.0 */
    for (int i = 0; i < N; ++i) sw[i] = 1.0f;
    double* acc = xmalloc(R * N * sizeof *acc);
    oracle_gemm_fp8(q, LD, w, LD, R, N, K, acc);
    double* row = xmalloc(K * sizeof *row);
    for (int r = 0; r < R; ++r) {
      oracle_e4m3_decode(q + r * LD, row, K);
      double sum = 0.0;
      for (int k = 0; k < K; ++k) sum += row[k];
      for (int n = 0; n < N; ++n) CHECK(acc[r * N + n] == sum);
    }
    uint16_t* y = xmalloc(R * N * sizeof *y);
    oracle_epilogue_f64acc(acc, R, N, s, sw, NULL, y);
    free(c); free(dv); free(x); free(q); free(w); free(s); free(sw); free(xb); free(tmp);
    free(acc); free(row); free(y);
  }
  if (failures) return 1;
  printf("oracle ok\n");
  return 0;
}
