/*
 * w8a8.h -- C ABI of libw8a8.so, a W8A8 INT8 linear layer for AMD MI355X
 * (gfx950, CDNA4).
 *
 * The operation is the fused INT8 linear of "Realizing Native INT8 Compute for
 * Diffusion Transformers on Consumer GPUs: A Fused INT8 GEMM Kernel for
 * Ideogram 4.0" (Asaria, Salomone, Gandhi; arXiv 2606.14598), Abstract:
 * activations are quantized to int8 per token and weights per output channel
 * (post-training), the int8 x int8 products are accumulated in int32 on the
 * integer matrix units, and the per-token x per-channel dequantization and the
 * bias are applied in the GEMM epilogue.  The Spanish write-up of the same
 * paper (aiexpert.news, "Núcleo Tritón Fuso Reduce el Tiempo de Generación de
 * Imágenes en 9,5% en Ampere de Consumo", second paragraph) adds that the
 * epilogue emits bf16 directly, without an extra round trip through memory.
 *
 * Numerical contract (the pages leave these open; this library fixes them):
 *   scale  = fl32(absmax_of_row / 127)                       (IEEE division)
 *   code   = clamp(round_half_even(fl32(x / scale)), -127, 127); scale 0 -> 0
 *   acc    = sum_k code_x[m,k] * code_w[n,k]                  (exact, int32)
 *   y      = bf16_rne( fl32( fl32( fl32(s_x[m]*s_w[n]) * fl32(acc) ) + bias[n] ) )
 *            -- every step one IEEE fp32 operation, no fused multiply-add.
 *
 * Conventions for every entry point below:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing; its only mutable state is a per-device cache of
 *     kernel occupancy figures, filled on first use (calls are thread-safe).
 *   - Matrices are row-major with the reduction dimension K contiguous.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Work is enqueued asynchronously on it; the return value covers argument
 *     validation and launch errors only.
 *   - Sizes: M, N >= 0 and 0 <= K <= W8A8_MAX_K with K % 16 == 0.  A call with
 *     nothing to compute returns W8A8_OK and enqueues nothing.  Pointers to
 *     tensors with zero elements may be NULL.
 *   - Alignment: int8 / bf16 / int32 matrix pointers 16-byte aligned; leading
 *     dimensions (in elements) such that every row starts 16-byte aligned;
 *     fp32 scale vectors 4-byte aligned, bf16 bias 2-byte aligned.
 *   - On any status other than W8A8_OK nothing has been enqueued (for
 *     W8A8_ERR_HIP: the launch itself failed).
 *   - Non-finite inputs are outside the contract: outputs are then
 *     unspecified, but every access stays in bounds.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest K for which |acc| <= 127*127*K cannot overflow int32, rounded down
 * to a multiple of 16:  16129 * 133136 = 2147350544 <= 2^31 - 1. */
#define W8A8_MAX_K 133136

enum w8a8_status {
  W8A8_OK = 0,
  W8A8_ERR_NULL = 1,       /* a required pointer is NULL */
  W8A8_ERR_SHAPE = 2,      /* negative size, K % 16 != 0, or ld < K */
  W8A8_ERR_ALIGN = 3,      /* pointer or row stride not aligned as above */
  W8A8_ERR_K_OVERFLOW = 4, /* K > W8A8_MAX_K: int32 accumulation could overflow */
  W8A8_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than required */
  W8A8_ERR_HIP = 6,        /* the HIP runtime rejected a launch */
  W8A8_ERR_CONFIG = 7,     /* unknown GEMM kernel configuration id */
  W8A8_ERR_SCRATCH = 8     /* w8a8_linear_noalloc: problem exceeds its static scratch */
};

/* Human-readable name of a status code (static storage; never NULL). */
const char* w8a8_status_string(int status);

/*
 * Per-token activation quantization.
 *   x      bf16 [M, K], row stride ldx elements (ldx >= K, ldx % 8 == 0)
 *   q      int8 [M, K] out, row stride ldq (ldq >= K, ldq % 16 == 0)
 *   scale  fp32 [M] out: scale[m] = absmax(x[m, :]) / 127 (IEEE fp32)
 *   q[m,k] = clamp(round_half_even(fp32(x[m,k] / scale[m])), -127, 127),
 *   all zero where scale[m] == 0.  Inputs must be finite; rows holding NaN
 *   or Inf get unspecified codes.
 * Source: the Abstract's per-token activation quantization.
 */
int w8a8_quantize_act(const void* x_bf16, int64_t M, int64_t K, int64_t ldx,
                      int8_t* q, int64_t ldq, float* scale, void* stream);

/*
 * Per-output-channel weight quantization (run once, offline), same rule on
 * fp32 rows.
 *   w      fp32 [N, K], row stride ldw (ldw >= K, ldw % 4 == 0)
 *   q      int8 [N, K] out, row stride ldq (ldq >= K, ldq % 16 == 0)
 *   scale  fp32 [N] out
 * Source: the Abstract's per-channel weight quantization; the news write-up
 * (second-to-last paragraph of its body) says it is done after training.
 */
int w8a8_quantize_weight(const float* w, int64_t N, int64_t K, int64_t ldw,
                         int8_t* q, int64_t ldq, float* scale, void* stream);

/*
 * Debug entry: the int32 accumulators alone, written to memory.
 *   q_x  int8 [M, K] (row stride K), w_q int8 [N, K] (row stride K)
 *   acc  int32 [M, N] out (row stride N): acc[m,n] = sum_k q_x[m,k] * w_q[n,k]
 * Source: the Abstract's int8 x int8 -> int32 accumulation, which the paper
 * checks bit for bit against a reference integer matmul.
 */
int w8a8_gemm_i32(const int8_t* q_x, const int8_t* w_q, int64_t M, int64_t N, int64_t K,
                  int32_t* acc, void* stream);

/*
 * int8 GEMM with the fused dequantization + bias epilogue, on activations
 * that are already quantized (e.g. by w8a8_gelu_quantize_act).
 *   q_x  int8 [M, K], s_x fp32 [M], w_q int8 [N, K], s_w fp32 [N]
 *   bias bf16 [N] or NULL (no bias)
 *   y    bf16 [M, N] out (row stride N)
 * The int32 accumulators never leave registers.
 * Source: the Abstract's epilogue folding of dequantization and bias.
 */
int w8a8_gemm_dequant(const int8_t* q_x, const float* s_x, const int8_t* w_q,
                      const float* s_w, const void* bias_bf16, int64_t M, int64_t N,
                      int64_t K, void* y_bf16, void* stream);

/* Bytes of device workspace w8a8_linear needs: the int8 codes [M, K] and the
 * fp32 scales [M] of the activations, each padded to 256 bytes.  0 when
 * M <= 0 or K < 0; SIZE_MAX when the size does not fit in size_t. */
size_t w8a8_linear_workspace_bytes(int64_t M, int64_t K);

/*
 * The fused W8A8 linear: per-token quantization of x into the workspace, then
 * the int8 GEMM with the dequantization + bias epilogue.
 *   x     bf16 [M, K] (row stride K)
 *   w_q   int8 [N, K], s_w fp32 [N]   (from w8a8_quantize_weight)
 *   bias  bf16 [N] or NULL
 *   y     bf16 [M, N] out
 *   workspace  device memory of at least w8a8_linear_workspace_bytes(M, K),
 *              16-byte aligned; its contents on return are the codes and
 *              scales of x.  Calls sharing one workspace must be ordered.
 * For a few token rows (M <= 16 with N <= 4096, M <= 12 above; K <= 3072)
 * the quantization, the GEMM and the epilogue run in one kernel launch.
 * Source: the Abstract's fused INT8 GEMM that replaces the
 * dequantize-to-bf16 linear forward.
 */
int w8a8_linear(const void* x_bf16, const int8_t* w_q, const float* s_w,
                const void* bias_bf16, int64_t M, int64_t N, int64_t K, void* y_bf16,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * The fused linear for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation and result as w8a8_linear, with the activation codes
 * and scales kept in a static device scratch array of the library instead of
 * a caller workspace.  Nothing is allocated by the call (no hipMalloc or
 * allocating library routine); each GPU holds its own copy of the array,
 * w8a8_linear_noalloc_max_bytes() = 64 MiB, from its first use until the
 * process ends.  Problems whose codes and scales exceed it
 * (w8a8_linear_workspace_bytes(M, K) > w8a8_linear_noalloc_max_bytes()) fail
 * with W8A8_ERR_SCRATCH.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (concurrent streams, or threads without
 * ordering) race on it and must be ordered by the caller.  On return the
 * array holds this call's codes and scales; nothing in it needs clearing.
 */
int w8a8_linear_noalloc(const void* x_bf16, const int8_t* w_q, const float* s_w,
                        const void* bias_bf16, int64_t M, int64_t N, int64_t K, void* y_bf16,
                        void* stream);
size_t w8a8_linear_noalloc_max_bytes(void);

/*
 * GELU followed by per-token quantization, for the activation between the
 * two linears of a DiT MLP (not on the pages; part of the DiT MLP workload):
 *   h[m,k] = bf16_rne(gelu(y[m,k])),  gelu(v) = 0.5 * v * erfc(-v / sqrt(2))
 *   correctly rounded (one rounding of the exact value; the kernel looks it
 *   up in a 65536-entry table of bf16 results built in double precision),
 *   then q, scale from h exactly as w8a8_quantize_act.
 *   Inputs must be finite; rows holding NaN or Inf get unspecified codes.
 *   y      bf16 [M, K], row stride ldy (ldy >= K, ldy % 8 == 0)
 *   q      int8 [M, K] out (row stride ldq), scale fp32 [M] out
 *   h_out  bf16 [M, K] out (row stride K) or NULL: the GELU values that were
 *          quantized, for inspection.
 */
int w8a8_gelu_quantize_act(const void* y_bf16, int64_t M, int64_t K, int64_t ldy,
                           int8_t* q, int64_t ldq, float* scale, void* h_out_bf16,
                           void* stream);

/*
 * Inter-layer fusion variant for the DiT MLP (GELU is not on the pages; the
 * fusion follows the Abstract's principle of folding the work around the
 * matmul into its epilogue).  w8a8_gemm_dequant_gelu_amax is
 * w8a8_gemm_dequant whose epilogue also applies GELU, writing
 *   h[m,n] = bf16_rne(gelu(y[m,n]))   (y the bf16 output of w8a8_gemm_dequant,
 *                                      the same table as w8a8_gelu_quantize_act)
 * and the row maxima amax[m] = max_n |h[m,n]| as fp32 bit patterns (uint32
 * [M]; the call overwrites them).  w8a8_quantize_act_amax then quantizes h
 * per token from those maxima without reducing the rows again: its codes and
 * scales equal w8a8_quantize_act(h) bit for bit.  Together they replace
 * w8a8_gemm_dequant + w8a8_gelu_quantize_act between the MLP's linears.
 *   Shapes: M and N multiples of 256, K a multiple of 64 and >= 256
 *   (W8A8_ERR_SHAPE otherwise); s_x, s_w and bias 16-byte aligned
 *   (W8A8_ERR_ALIGN otherwise).  w8a8_quantize_act_amax: K <= 12288.
 * Both variants move the same HBM bytes (a bf16 [M, N] tensor written and
 * read back, then the codes); on the 4096 x 3072 -> 12288 up-projection the
 * table gathers in the epilogue make this pair slower than the one it
 * replaces (218 us against 185.5 us for quantize + up-proj + inter-layer),
 * so the library's own MLP step keeps w8a8_gelu_quantize_act.
 */
int w8a8_gemm_dequant_gelu_amax(const int8_t* q_x, const float* s_x, const int8_t* w_q,
                                const float* s_w, const void* bias_bf16, int64_t M, int64_t N,
                                int64_t K, void* h_bf16, uint32_t* amax, void* stream);
int w8a8_quantize_act_amax(const void* h_bf16, int64_t M, int64_t K, int64_t ldh,
                           const uint32_t* amax, int8_t* q, int64_t ldq, float* scale,
                           void* stream);

/*
 * GEMM kernel configurations (tile shapes), chosen per GEMM shape -- the
 * Abstract's per-shape autotuning, here a fixed table built from measurement.
 */
int w8a8_gemm_num_configs(void);
/* Name of configuration `config` (static storage), or NULL if out of range. */
const char* w8a8_gemm_config_name(int config);
/* The configuration the library uses for an (M, N, K) GEMM. */
int w8a8_gemm_select_config(int64_t M, int64_t N, int64_t K);

/*
 * w8a8_gemm_i32 / w8a8_gemm_dequant with an explicit configuration
 * (config = -1: the library's choice).  out_int32 != 0 writes int32
 * accumulators to `out` (s_x, s_w, bias ignored); otherwise bf16 as
 * w8a8_gemm_dequant.  Every configuration computes the same bits.
 */
int w8a8_gemm_ex(const int8_t* q_x, const float* s_x, const int8_t* w_q, const float* s_w,
                 const void* bias_bf16, int64_t M, int64_t N, int64_t K, void* out,
                 int out_int32, int config, void* stream);

/*
 * FP8 variant: the same per-token x per-channel scheme with OCP e4m3 codes
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest finite
 * value 448; bytes 0x7F and 0xFF are NaN) in place of int8 -- the FP8 path
 * the pages compare the INT8 one with (Abstract; news write-up, third
 * paragraph).  Same sizes, alignment, leading-dimension, workspace and error
 * rules as the int8 entry points above.
 *
 * Quantization (per token for bf16 activations, per output channel for fp32
 * weights):  scale = fl32(absmax / 448);  code = e4m3_rne(clamp(fl32(x /
 * scale), -448, 448)), round half to even on the e4m3 grid (subnormal step
 * 2^-9); a row whose scale is 0 gets all-zero codes.  Codes are uint8 bytes.
 */
int w8a8_quantize_act_fp8(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                          int64_t ldq, float* scale, void* stream);
int w8a8_quantize_weight_fp8(const float* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                             int64_t ldq, float* scale, void* stream);

/* GELU then per-token e4m3 quantization: h as in w8a8_gelu_quantize_act, then
 * codes and scales from h as in w8a8_quantize_act_fp8. */
int w8a8_gelu_quantize_act_fp8(const void* y_bf16, int64_t M, int64_t K, int64_t ldy, uint8_t* q,
                               int64_t ldq, float* scale, void* h_out_bf16, void* stream);

/*
 * y[m,n] = bf16_rne((s_x[m] * s_w[n]) * acc[m,n] + bias[n]) with acc the sum
 * over k of e4m3(q_x[m,k]) * e4m3(w_q[n,k]) accumulated in fp32 on the FP8
 * matrix cores (their accumulation rounds, so acc matches the exact sum
 * within a small relative error, not bit for bit).  Codes must be finite (no
 * NaN bytes); the quantizers above never produce them.  Fastest when K is a
 * multiple of 128.  config: -1 for the library's choice, else 0 ..
 * w8a8_gemm_fp8_num_configs() - 1.
 */
int w8a8_gemm_dequant_fp8(const uint8_t* q_x, const float* s_x, const uint8_t* w_q,
                          const float* s_w, const void* bias_bf16, int64_t M, int64_t N, int64_t K,
                          void* y_bf16, void* stream);
int w8a8_gemm_fp8_ex(const uint8_t* q_x, const float* s_x, const uint8_t* w_q, const float* s_w,
                     const void* bias_bf16, int64_t M, int64_t N, int64_t K, void* y_bf16,
                     int config, void* stream);
int w8a8_gemm_fp8_num_configs(void);
const char* w8a8_gemm_fp8_config_name(int config);

/*
 * The fused FP8 linear: w8a8_quantize_act_fp8 of x into the workspace (same
 * size as w8a8_linear's: w8a8_linear_workspace_bytes(M, K)), then
 * w8a8_gemm_dequant_fp8.  w_q, s_w from w8a8_quantize_weight_fp8.  Up to 8
 * token rows (K <= 3072) run in one launch, with the same output bits.
 */
int w8a8_linear_fp8(const void* x_bf16, const uint8_t* w_q, const float* s_w,
                    const void* bias_bf16, int64_t M, int64_t N, int64_t K, void* y_bf16,
                    void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
