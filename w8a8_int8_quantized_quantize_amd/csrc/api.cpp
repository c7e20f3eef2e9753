// C ABI of libw8a8.so (declared in include/w8a8.h): argument validation,
// per-shape kernel selection and launches on the caller's stream.
//
// Validation happens entirely on the host before any HIP call, so every error
// path is reachable (and tested) on a machine without a GPU.
#include "w8a8.h"

#include "internal.h"

namespace {

using w8a8::GemmArgs;
using w8a8::QuantSrc;

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

inline int hip_status(hipError_t e) { return e == hipSuccess ? W8A8_OK : W8A8_ERR_HIP; }

constexpr size_t kPad = 256;
inline size_t pad(size_t b) { return (b + kPad - 1) / kPad * kPad; }

// Shared checks for K: 0 <= K <= W8A8_MAX_K, K % 16 == 0.
inline int check_k(int64_t K) {
  if (K < 0 || (K % 16) != 0) return W8A8_ERR_SHAPE;
  if (K > W8A8_MAX_K) return W8A8_ERR_K_OVERFLOW;
  return W8A8_OK;
}

// Row quantization: x [rows, K] (elem_bytes per element, stride ldx),
// q [rows, K] (stride ldq), scale [rows].
int check_rows(const void* x, int64_t rows, int64_t K, int64_t ldx, size_t elem_bytes,
               const int8_t* q, int64_t ldq, const float* scale) {
  if (rows < 0) return W8A8_ERR_SHAPE;
  if (int rc = check_k(K)) return rc;
  if (ldx < K || ldq < K) return W8A8_ERR_SHAPE;
  if (rows == 0) return W8A8_OK;
  if (scale == nullptr) return W8A8_ERR_NULL;
  if (K > 0 && (x == nullptr || q == nullptr)) return W8A8_ERR_NULL;
  if (!aligned(scale, 4)) return W8A8_ERR_ALIGN;
  if (K > 0) {
    if (!aligned(x, 16) || !aligned(q, 16)) return W8A8_ERR_ALIGN;
    if ((static_cast<size_t>(ldx) * elem_bytes) % 16 != 0 || ldq % 16 != 0) return W8A8_ERR_ALIGN;
  }
  return W8A8_OK;
}

int check_gemm(const int8_t* qx, const int8_t* qw, int64_t M, int64_t N, int64_t K,
               const void* out) {
  if (M < 0 || N < 0) return W8A8_ERR_SHAPE;
  if (int rc = check_k(K)) return rc;
  if (M == 0 || N == 0) return W8A8_OK;
  if (out == nullptr) return W8A8_ERR_NULL;
  if (K > 0 && (qx == nullptr || qw == nullptr)) return W8A8_ERR_NULL;
  if (!aligned(out, 16)) return W8A8_ERR_ALIGN;
  if (K > 0 && (!aligned(qx, 16) || !aligned(qw, 16))) return W8A8_ERR_ALIGN;
  return W8A8_OK;
}

int check_dequant(const float* sx, const float* sw, const void* bias, int64_t M, int64_t N) {
  if (M == 0 || N == 0) return W8A8_OK;
  if (sx == nullptr || sw == nullptr) return W8A8_ERR_NULL;
  if (!aligned(sx, 4) || !aligned(sw, 4)) return W8A8_ERR_ALIGN;
  if (bias != nullptr && !aligned(bias, 2)) return W8A8_ERR_ALIGN;
  return W8A8_OK;
}

int gemm_any(const int8_t* q_x, const float* s_x, const int8_t* w_q, const float* s_w,
             const void* bias, int64_t M, int64_t N, int64_t K, void* out, bool out_i32,
             int config, void* stream) {
  if (int rc = check_gemm(q_x, w_q, M, N, K, out)) return rc;
  if (!out_i32) {
    if (int rc = check_dequant(s_x, s_w, bias, M, N)) return rc;
  }
  if (config < -1 || config >= w8a8::gemm_num_configs()) return W8A8_ERR_CONFIG;
  if (M == 0 || N == 0) return W8A8_OK;
  const int cfg = config >= 0 ? config : w8a8::gemm_select_config(M, N, K);
  GemmArgs a;
  a.qx = q_x;
  a.qw = w_q;
  a.sx = s_x;
  a.sw = s_w;
  a.bias = static_cast<const uint16_t*>(bias);
  a.out = out;
  a.M = M;
  a.N = N;
  a.K = K;
  return hip_status(w8a8::launch_gemm(a, out_i32, cfg, as_stream(stream)));
}

int gemm_fp8_any(const uint8_t* q_x, const float* s_x, const uint8_t* w_q, const float* s_w,
                 const void* bias, int64_t M, int64_t N, int64_t K, void* y, int config,
                 void* stream) {
  const int8_t* qx = reinterpret_cast<const int8_t*>(q_x);
  const int8_t* qw = reinterpret_cast<const int8_t*>(w_q);
  if (int rc = check_gemm(qx, qw, M, N, K, y)) return rc;
  if (int rc = check_dequant(s_x, s_w, bias, M, N)) return rc;
  if (config < -1 || config >= w8a8::gemm_fp8_num_configs()) return W8A8_ERR_CONFIG;
  if (M == 0 || N == 0) return W8A8_OK;
  const int cfg = config >= 0 ? config : w8a8::gemm_fp8_select_config(M, N, K);
  GemmArgs a;
  a.qx = qx;
  a.qw = qw;
  a.sx = s_x;
  a.sw = s_w;
  a.bias = static_cast<const uint16_t*>(bias);
  a.out = y;
  a.M = M;
  a.N = N;
  a.K = K;
  return hip_status(w8a8::launch_gemm_fp8(a, cfg, as_stream(stream)));
}

}  // namespace

extern "C" {

const char* w8a8_status_string(int status) {
  switch (status) {
    case W8A8_OK: return "W8A8_OK";
    case W8A8_ERR_NULL: return "W8A8_ERR_NULL: a required pointer is NULL";
    case W8A8_ERR_SHAPE: return "W8A8_ERR_SHAPE: negative size, K % 16 != 0, or leading dimension < K";
    case W8A8_ERR_ALIGN: return "W8A8_ERR_ALIGN: pointer or row stride not 16-byte aligned";
    case W8A8_ERR_K_OVERFLOW: return "W8A8_ERR_K_OVERFLOW: K > W8A8_MAX_K, int32 accumulation could overflow";
    case W8A8_ERR_WORKSPACE: return "W8A8_ERR_WORKSPACE: workspace NULL or too small";
    case W8A8_ERR_HIP: return "W8A8_ERR_HIP: the HIP runtime rejected a launch";
    case W8A8_ERR_CONFIG: return "W8A8_ERR_CONFIG: unknown GEMM configuration";
    case W8A8_ERR_SCRATCH:
      return "W8A8_ERR_SCRATCH: codes and scales of x exceed the no-alloc entry's static scratch "
             "(w8a8_linear_noalloc_max_bytes)";
    default: return "W8A8: unknown status";
  }
}

int w8a8_quantize_act(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                      int64_t ldq, float* scale, void* stream) {
  if (int rc = check_rows(x_bf16, M, K, ldx, 2, q, ldq, scale)) return rc;
  if (M == 0) return W8A8_OK;
  return hip_status(w8a8::launch_quantize_rows(QuantSrc::kBf16, x_bf16, M, K, ldx, q, ldq, scale,
                                               nullptr, as_stream(stream)));
}

int w8a8_quantize_weight(const float* w, int64_t N, int64_t K, int64_t ldw, int8_t* q,
                         int64_t ldq, float* scale, void* stream) {
  if (int rc = check_rows(w, N, K, ldw, 4, q, ldq, scale)) return rc;
  if (N == 0) return W8A8_OK;
  return hip_status(w8a8::launch_quantize_rows(QuantSrc::kF32, w, N, K, ldw, q, ldq, scale,
                                               nullptr, as_stream(stream)));
}

int w8a8_gelu_quantize_act(const void* y_bf16, int64_t M, int64_t K, int64_t ldy, int8_t* q,
                           int64_t ldq, float* scale, void* h_out_bf16, void* stream) {
  if (int rc = check_rows(y_bf16, M, K, ldy, 2, q, ldq, scale)) return rc;
  if (h_out_bf16 != nullptr && !aligned(h_out_bf16, 16)) return W8A8_ERR_ALIGN;
  if (M == 0) return W8A8_OK;
  return hip_status(w8a8::launch_quantize_rows(QuantSrc::kBf16Gelu, y_bf16, M, K, ldy, q, ldq,
                                               scale, static_cast<uint16_t*>(h_out_bf16),
                                               as_stream(stream)));
}

int w8a8_gemm_i32(const int8_t* q_x, const int8_t* w_q, int64_t M, int64_t N, int64_t K,
                  int32_t* acc, void* stream) {
  return gemm_any(q_x, nullptr, w_q, nullptr, nullptr, M, N, K, acc, true, -1, stream);
}

int w8a8_gemm_dequant(const int8_t* q_x, const float* s_x, const int8_t* w_q, const float* s_w,
                      const void* bias_bf16, int64_t M, int64_t N, int64_t K, void* y_bf16,
                      void* stream) {
  return gemm_any(q_x, s_x, w_q, s_w, bias_bf16, M, N, K, y_bf16, false, -1, stream);
}

int w8a8_gemm_ex(const int8_t* q_x, const float* s_x, const int8_t* w_q, const float* s_w,
                 const void* bias_bf16, int64_t M, int64_t N, int64_t K, void* out, int out_int32,
                 int config, void* stream) {
  return gemm_any(q_x, s_x, w_q, s_w, bias_bf16, M, N, K, out, out_int32 != 0, config, stream);
}

size_t w8a8_linear_workspace_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K < 0) return 0;
  // a size that does not fit in size_t is reported as SIZE_MAX, which no
  // workspace can provide (the fused entry then fails with W8A8_ERR_WORKSPACE)
  const size_t m = static_cast<size_t>(M), k = static_cast<size_t>(K);
  if (m > (SIZE_MAX - 2 * kPad) / (k + 4)) return SIZE_MAX;
  return pad(m * k) + pad(m * 4);
}

int w8a8_linear(const void* x_bf16, const int8_t* w_q, const float* s_w, const void* bias_bf16,
                int64_t M, int64_t N, int64_t K, void* y_bf16, void* workspace,
                size_t workspace_bytes, void* stream) {
  if (M < 0 || N < 0) return W8A8_ERR_SHAPE;
  if (int rc = check_k(K)) return rc;
  if (M == 0 || N == 0) return W8A8_OK;
  const size_t need = w8a8_linear_workspace_bytes(M, K);
  if (workspace == nullptr || workspace_bytes < need) return W8A8_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return W8A8_ERR_ALIGN;
  int8_t* qx = static_cast<int8_t*>(workspace);
  float* sx = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       pad(static_cast<size_t>(M) * static_cast<size_t>(K)));
  // validate both stages before enqueueing either
  if (int rc = check_rows(x_bf16, M, K, K, 2, qx, K, sx)) return rc;
  if (int rc = check_gemm(qx, w_q, M, N, K, y_bf16)) return rc;
  if (int rc = check_dequant(sx, s_w, bias_bf16, M, N)) return rc;
  if (w8a8::linear_few_rows_supported(M, N, K, false)) {
    // a handful of tokens: quantize, GEMM and epilogue in one launch, which
    // also leaves the codes and scales in the workspace
    w8a8::RowsArgs r;
    r.x = static_cast<const uint16_t*>(x_bf16);
    r.qw = w_q;
    r.sw = s_w;
    r.bias = static_cast<const uint16_t*>(bias_bf16);
    r.y = static_cast<uint16_t*>(y_bf16);
    r.qx_out = qx;
    r.sx_out = sx;
    r.M = M;
    r.N = N;
    r.K = K;
    return hip_status(w8a8::launch_linear_few_rows(r, false, as_stream(stream)));
  }
  if (int rc = hip_status(w8a8::launch_quantize_rows(QuantSrc::kBf16, x_bf16, M, K, K, qx, K, sx,
                                                     nullptr, as_stream(stream))))
    return rc;
  return gemm_any(qx, sx, w_q, s_w, bias_bf16, M, N, K, y_bf16, false, -1, stream);
}

int w8a8_linear_noalloc(const void* x_bf16, const int8_t* w_q, const float* s_w,
                        const void* bias_bf16, int64_t M, int64_t N, int64_t K, void* y_bf16,
                        void* stream) {
  if (M < 0 || N < 0) return W8A8_ERR_SHAPE;
  if (int rc = check_k(K)) return rc;
  if (M == 0 || N == 0) return W8A8_OK;
  if (w8a8_linear_workspace_bytes(M, K) > w8a8::kNoAllocScratchBytes) return W8A8_ERR_SCRATCH;
  void* scratch = nullptr;
  if (w8a8::noalloc_scratch(&scratch) != hipSuccess) return W8A8_ERR_HIP;
  return w8a8_linear(x_bf16, w_q, s_w, bias_bf16, M, N, K, y_bf16, scratch,
                     w8a8::kNoAllocScratchBytes, stream);
}

size_t w8a8_linear_noalloc_max_bytes(void) { return w8a8::kNoAllocScratchBytes; }

int w8a8_gemm_dequant_gelu_amax(const int8_t* q_x, const float* s_x, const int8_t* w_q,
                                const float* s_w, const void* bias_bf16, int64_t M, int64_t N,
                                int64_t K, void* h_bf16, uint32_t* amax, void* stream) {
  if (int rc = check_gemm(q_x, w_q, M, N, K, h_bf16)) return rc;
  if (int rc = check_dequant(s_x, s_w, bias_bf16, M, N)) return rc;
  if (M == 0 || N == 0) return W8A8_OK;
  if (amax == nullptr) return W8A8_ERR_NULL;
  if (!aligned(amax, 4)) return W8A8_ERR_ALIGN;
  GemmArgs a;
  a.qx = q_x;
  a.qw = w_q;
  a.sx = s_x;
  a.sw = s_w;
  a.bias = static_cast<const uint16_t*>(bias_bf16);
  a.out = h_bf16;
  a.M = M;
  a.N = N;
  a.K = K;
  a.amax = amax;
  if (!w8a8::gemm_gelu_amax_supported(a)) {
    const bool shape_ok = M % 256 == 0 && N % 256 == 0 && K % 64 == 0 && K >= 256;
    return shape_ok ? W8A8_ERR_ALIGN : W8A8_ERR_SHAPE;
  }
  return hip_status(w8a8::launch_gemm_gelu_amax(a, as_stream(stream)));
}

int w8a8_quantize_act_amax(const void* h_bf16, int64_t M, int64_t K, int64_t ldh,
                           const uint32_t* amax, int8_t* q, int64_t ldq, float* scale,
                           void* stream) {
  if (int rc = check_rows(h_bf16, M, K, ldh, 2, q, ldq, scale)) return rc;
  if (M == 0) return W8A8_OK;
  if (K > 12288) return W8A8_ERR_SHAPE;
  if (amax == nullptr) return W8A8_ERR_NULL;
  if (!aligned(amax, 4)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_quantize_with_amax(h_bf16, M, K, ldh, amax, q, ldq, scale,
                                                    as_stream(stream)));
}

int w8a8_quantize_act_fp8(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                          int64_t ldq, float* scale, void* stream) {
  int8_t* qb = reinterpret_cast<int8_t*>(q);
  if (int rc = check_rows(x_bf16, M, K, ldx, 2, qb, ldq, scale)) return rc;
  if (M == 0) return W8A8_OK;
  return hip_status(w8a8::launch_quantize_rows(QuantSrc::kBf16Fp8, x_bf16, M, K, ldx, qb, ldq,
                                               scale, nullptr, as_stream(stream)));
}

int w8a8_quantize_weight_fp8(const float* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                             int64_t ldq, float* scale, void* stream) {
  int8_t* qb = reinterpret_cast<int8_t*>(q);
  if (int rc = check_rows(w, N, K, ldw, 4, qb, ldq, scale)) return rc;
  if (N == 0) return W8A8_OK;
  return hip_status(w8a8::launch_quantize_rows(QuantSrc::kF32Fp8, w, N, K, ldw, qb, ldq, scale,
                                               nullptr, as_stream(stream)));
}

int w8a8_gelu_quantize_act_fp8(const void* y_bf16, int64_t M, int64_t K, int64_t ldy, uint8_t* q,
                               int64_t ldq, float* scale, void* h_out_bf16, void* stream) {
  int8_t* qb = reinterpret_cast<int8_t*>(q);
  if (int rc = check_rows(y_bf16, M, K, ldy, 2, qb, ldq, scale)) return rc;
  if (h_out_bf16 != nullptr && !aligned(h_out_bf16, 16)) return W8A8_ERR_ALIGN;
  if (M == 0) return W8A8_OK;
  return hip_status(w8a8::launch_quantize_rows(QuantSrc::kBf16GeluFp8, y_bf16, M, K, ldy, qb, ldq,
                                               scale, static_cast<uint16_t*>(h_out_bf16),
                                               as_stream(stream)));
}

int w8a8_gemm_dequant_fp8(const uint8_t* q_x, const float* s_x, const uint8_t* w_q,
                          const float* s_w, const void* bias_bf16, int64_t M, int64_t N, int64_t K,
                          void* y_bf16, void* stream) {
  return gemm_fp8_any(q_x, s_x, w_q, s_w, bias_bf16, M, N, K, y_bf16, -1, stream);
}

int w8a8_gemm_fp8_ex(const uint8_t* q_x, const float* s_x, const uint8_t* w_q, const float* s_w,
                     const void* bias_bf16, int64_t M, int64_t N, int64_t K, void* y_bf16,
                     int config, void* stream) {
  return gemm_fp8_any(q_x, s_x, w_q, s_w, bias_bf16, M, N, K, y_bf16, config, stream);
}

int w8a8_linear_fp8(const void* x_bf16, const uint8_t* w_q, const float* s_w,
                    const void* bias_bf16, int64_t M, int64_t N, int64_t K, void* y_bf16,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || N < 0) return W8A8_ERR_SHAPE;
  if (int rc = check_k(K)) return rc;
  if (M == 0 || N == 0) return W8A8_OK;
  const size_t need = w8a8_linear_workspace_bytes(M, K);
  if (workspace == nullptr || workspace_bytes < need) return W8A8_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return W8A8_ERR_ALIGN;
  int8_t* qx = static_cast<int8_t*>(workspace);
  float* sx = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       pad(static_cast<size_t>(M) * static_cast<size_t>(K)));
  // validate both stages before enqueueing either
  if (int rc = check_rows(x_bf16, M, K, K, 2, qx, K, sx)) return rc;
  if (int rc = check_gemm(qx, reinterpret_cast<const int8_t*>(w_q), M, N, K, y_bf16)) return rc;
  if (int rc = check_dequant(sx, s_w, bias_bf16, M, N)) return rc;
  if (w8a8::linear_few_rows_supported(M, N, K, true)) {
    // a handful of tokens: the e4m3 quantization, GEMM and epilogue in one
    // launch (the same bits as the two launches below)
    w8a8::RowsArgs r;
    r.x = static_cast<const uint16_t*>(x_bf16);
    r.qw = reinterpret_cast<const int8_t*>(w_q);
    r.sw = s_w;
    r.bias = static_cast<const uint16_t*>(bias_bf16);
    r.y = static_cast<uint16_t*>(y_bf16);
    r.qx_out = qx;
    r.sx_out = sx;
    r.M = M;
    r.N = N;
    r.K = K;
    return hip_status(w8a8::launch_linear_few_rows(r, true, as_stream(stream)));
  }
  if (int rc = hip_status(w8a8::launch_quantize_rows(QuantSrc::kBf16Fp8, x_bf16, M, K, K, qx, K,
                                                     sx, nullptr, as_stream(stream))))
    return rc;
  return gemm_fp8_any(reinterpret_cast<const uint8_t*>(qx), sx, w_q, s_w, bias_bf16, M, N, K,
                      y_bf16, -1, stream);
}

int w8a8_gemm_fp8_num_configs(void) { return w8a8::gemm_fp8_num_configs(); }

const char* w8a8_gemm_fp8_config_name(int config) { return w8a8::gemm_fp8_config_name(config); }

int w8a8_gemm_num_configs(void) { return w8a8::gemm_num_configs(); }

const char* w8a8_gemm_config_name(int config) { return w8a8::gemm_config_name(config); }

int w8a8_gemm_select_config(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K < 0) return -1;
  return w8a8::gemm_select_config(M, N, K);
}

}  // extern "C"
