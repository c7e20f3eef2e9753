// Internal declarations shared by the HIP translation units of libw8a8.so.
// Not part of the public ABI (that is include/w8a8.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w8a8 {

// ---------------------------------------------------------- quantization --
// Row-wise symmetric int8 quantization of bf16 (per token) or fp32 (per
// channel) rows, optionally with GELU applied to bf16 rows first; the *Fp8
// sources write OCP e4m3 codes (scale absmax / 448) instead.  All sizes
// already validated by the API layer; M >= 1.
enum class QuantSrc { kBf16, kF32, kBf16Gelu, kBf16Fp8, kF32Fp8, kBf16GeluFp8 };

hipError_t launch_quantize_rows(QuantSrc src, const void* x, int64_t M, int64_t K, int64_t ldx,
                                int8_t* q, int64_t ldq, float* scale, uint16_t* h_out,
                                hipStream_t stream);

// ------------------------------------------------------------------ GEMM --
struct GemmArgs {
  const int8_t* qx;   // [M, K] activations (codes), row stride K
  const int8_t* qw;   // [N, K] weights (codes), row stride K
  const float* sx;    // [M] per-token scales (bf16 output only)
  const float* sw;    // [N] per-channel scales (bf16 output only)
  const uint16_t* bias;  // [N] bf16 or nullptr
  void* out;          // [M, N] bf16 or int32
  int64_t M, N, K;
  // GELU epilogue variant only (launch_gemm_gelu_amax): the [M] row maxima
  // of |h| (fp32 bit patterns)
  uint32_t* amax = nullptr;
};

// The fused linear for a handful of token rows in one launch (quantize +
// GEMM + epilogue); the codes and scales of x also go to qx_out / sx_out.
struct RowsArgs {
  const uint16_t* x;     // [M, K] bf16 activations, row stride K
  const int8_t* qw;      // [N, K] weight codes
  const float* sw;       // [N]
  const uint16_t* bias;  // [N] bf16 or nullptr
  uint16_t* y;           // [M, N] bf16
  int8_t* qx_out;        // [M, K] codes of x, or nullptr
  float* sx_out;         // [M] scales of x, or nullptr
  int64_t M, N, K;
};
// (fp8: e4m3 codes of x and weights, the FP8 GEMM's few-row kernel's bits)
bool linear_few_rows_supported(int64_t M, int64_t N, int64_t K, bool fp8);
hipError_t launch_linear_few_rows(const RowsArgs& a, bool fp8, hipStream_t stream);

// The GEMM whose epilogue also applies GELU and raises the row maxima of |h|
// (the inter-layer fusion variant): out = h = bf16(gelu(y)) [M, N] bf16,
// amax[m] = max |h[m, :]| (fp32 bits; zeroed first).  Interior shapes only.
bool gemm_gelu_amax_supported(const GemmArgs& a);
hipError_t launch_gemm_gelu_amax(const GemmArgs& a, hipStream_t stream);
// Per-token quantization of bf16 rows whose absmax is already known
// (amax[m]: fp32 bits): the same codes and scales as launch_quantize_rows.
hipError_t launch_quantize_with_amax(const void* x, int64_t M, int64_t K, int64_t ldx,
                                     const uint32_t* amax, int8_t* q, int64_t ldq, float* scale,
                                     hipStream_t stream);

int gemm_num_configs();
const char* gemm_config_name(int cfg);
int gemm_select_config(int64_t M, int64_t N, int64_t K);
// out_int32: write raw accumulators instead of the dequantized bf16.
hipError_t launch_gemm(const GemmArgs& a, bool out_int32, int cfg, hipStream_t stream);

// The same GEMM on OCP e4m3 codes (qx, qw hold fp8 bytes), fp32 accumulation,
// bf16 output with the same epilogue; its own table of tile configurations.
int gemm_fp8_num_configs();
const char* gemm_fp8_config_name(int cfg);
int gemm_fp8_select_config(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_fp8(const GemmArgs& a, int cfg, hipStream_t stream);

// ------------------------------------------------------ no-alloc scratch --
// Bytes of the static device scratch behind w8a8_linear_noalloc (codes and
// scales of the activations, laid out as w8a8_linear's workspace).
constexpr size_t kNoAllocScratchBytes = size_t{64} << 20;
// This device's address of that scratch (looked up once per device).
hipError_t noalloc_scratch(void** ptr);

}  // namespace w8a8
