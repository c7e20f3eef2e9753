// Sanitizer build of the C-ABI layer (api.cpp): every entry point is called
// with valid and invalid arguments on the host, with the device-side launch
// functions replaced by stubs that record each launch.  Built with
// -fsanitize=address,undefined by tests/test_host_sanitizers.py; exits 0
// after printing "abi ok" when every check holds.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "internal.h"
#include "w8a8.h"

namespace {
int g_quant = 0, g_gemm = 0, g_gemm_fp8 = 0;
w8a8::GemmArgs g_last{};
int g_last_cfg = -2;
bool g_last_i32 = false;
int g_failures = 0;

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "check failed, line %d: %s\n", __LINE__, #cond); \
      ++g_failures;                                                   \
    }                                                                 \
  } while (0)
}  // namespace

namespace w8a8 {
hipError_t launch_quantize_rows(QuantSrc, const void* x, int64_t M, int64_t K, int64_t ldx,
                                int8_t* q, int64_t ldq, float* scale, uint16_t*, hipStream_t) {
  CHECK(M >= 1 && K >= 0 && ldx >= K && ldq >= K && scale != nullptr);
  CHECK(K == 0 || (x != nullptr && q != nullptr));
  ++g_quant;
  return hipSuccess;
}
int gemm_num_configs() { return 11; }
const char* gemm_config_name(int c) { return (c >= 0 && c < 11) ? "stub" : nullptr; }
int gemm_select_config(int64_t, int64_t, int64_t) { return 3; }
hipError_t launch_gemm(const GemmArgs& a, bool i32, int cfg, hipStream_t) {
  CHECK(a.M >= 1 && a.N >= 1 && a.K >= 0 && cfg >= 0 && cfg < 11 && a.out != nullptr);
  g_last = a;
  g_last_cfg = cfg;
  g_last_i32 = i32;
  ++g_gemm;
  return hipSuccess;
}
alignas(256) unsigned char g_scratch_stub[1024];
hipError_t noalloc_scratch(void** ptr) {
  *ptr = g_scratch_stub;  // stands in for the device scratch
  return hipSuccess;
}
int g_rows = 0, g_rows_fp8 = 0;
bool linear_few_rows_supported(int64_t M, int64_t, int64_t K, bool) { return M <= 2 && K <= 3072; }
hipError_t launch_linear_few_rows(const RowsArgs& a, bool fp8, hipStream_t) {
  CHECK(a.M >= 1 && a.M <= 2 && a.qx_out != nullptr && a.sx_out != nullptr && a.y != nullptr);
  ++(fp8 ? g_rows_fp8 : g_rows);
  return hipSuccess;
}
int g_gelu_gemm = 0, g_quant_amax = 0;
bool gemm_gelu_amax_supported(const GemmArgs& a) { return a.M % 256 == 0 && a.N % 256 == 0 && a.K % 64 == 0 && a.K >= 256; }
hipError_t launch_gemm_gelu_amax(const GemmArgs& a, hipStream_t) {
  CHECK(a.amax != nullptr && a.out != nullptr);
  ++g_gelu_gemm;
  return hipSuccess;
}
hipError_t launch_quantize_with_amax(const void* x, int64_t M, int64_t K, int64_t ldx,
                                     const uint32_t* amax, int8_t* q, int64_t ldq, float* scale,
                                     hipStream_t) {
  CHECK(x != nullptr && M >= 1 && K <= 12288 && ldx >= K && amax != nullptr && q != nullptr && ldq >= K &&
        scale != nullptr);
  ++g_quant_amax;
  return hipSuccess;
}
int gemm_fp8_num_configs() { return 6; }
const char* gemm_fp8_config_name(int c) { return (c >= 0 && c < 6) ? "stub" : nullptr; }
int gemm_fp8_select_config(int64_t, int64_t, int64_t) { return 4; }
hipError_t launch_gemm_fp8(const GemmArgs& a, int cfg, hipStream_t) {
  CHECK(a.M >= 1 && a.N >= 1 && cfg >= 0 && cfg < 6);
  g_last = a;
  g_last_cfg = cfg;
  ++g_gemm_fp8;
  return hipSuccess;
}
}  // namespace w8a8

int main() {
  // heap buffers sized exactly, so that any access past them would be seen
  const int64_t M = 5, N = 24, K = 48;
  std::vector<uint16_t> x(M * K), bias(N);
  std::vector<int8_t> q(M * K), wq(N * K);
  std::vector<float> sx(M), sw(N), wf(N * K);
  std::vector<int32_t> acc(M * N);
  std::vector<uint16_t> y(M * N);
  alignas(16) static unsigned char ws_buf[8192];

  for (int s = 0; s < 9; ++s) CHECK(w8a8_status_string(s) != nullptr);
  CHECK(w8a8_status_string(-1) != nullptr && w8a8_status_string(99) != nullptr);

  // quantize_act
  CHECK(w8a8_quantize_act(x.data(), M, K, K, q.data(), K, sx.data(), nullptr) == W8A8_OK);
  CHECK(g_quant == 1);
  CHECK(w8a8_quantize_act(nullptr, M, K, K, q.data(), K, sx.data(), nullptr) == W8A8_ERR_NULL);
  CHECK(w8a8_quantize_act(x.data(), M, K, K, q.data(), K, nullptr, nullptr) == W8A8_ERR_NULL);
  CHECK(w8a8_quantize_act(x.data(), -1, K, K, q.data(), K, sx.data(), nullptr) == W8A8_ERR_SHAPE);
  CHECK(w8a8_quantize_act(x.data(), M, 40 + 1, K, q.data(), K, sx.data(), nullptr) == W8A8_ERR_SHAPE);
  CHECK(w8a8_quantize_act(x.data(), M, K, K - 16, q.data(), K, sx.data(), nullptr) == W8A8_ERR_SHAPE);
  CHECK(w8a8_quantize_act(x.data(), M, W8A8_MAX_K + 16, W8A8_MAX_K + 16, q.data(), W8A8_MAX_K + 16,
                          sx.data(), nullptr) == W8A8_ERR_K_OVERFLOW);
  CHECK(w8a8_quantize_act(reinterpret_cast<char*>(x.data()) + 2, M, K, K, q.data(), K, sx.data(),
                          nullptr) == W8A8_ERR_ALIGN);
  CHECK(w8a8_quantize_act(x.data(), M, K, K + 4, q.data(), K, sx.data(), nullptr) == W8A8_ERR_ALIGN);
  CHECK(w8a8_quantize_act(x.data(), 0, K, K, nullptr, K, nullptr, nullptr) == W8A8_OK);
  CHECK(g_quant == 1);  // nothing enqueued on errors or empty calls

  // quantize_weight, gelu_quantize_act
  CHECK(w8a8_quantize_weight(wf.data(), N, K, K, wq.data(), K, sw.data(), nullptr) == W8A8_OK);
  CHECK(w8a8_quantize_weight(wf.data(), N, K, K + 2, wq.data(), K, sw.data(), nullptr) == W8A8_ERR_ALIGN);
  CHECK(w8a8_gelu_quantize_act(x.data(), M, K, K, q.data(), K, sx.data(), y.data(), nullptr) == W8A8_OK);
  CHECK(w8a8_gelu_quantize_act(x.data(), M, K, K, q.data(), K, sx.data(),
                               reinterpret_cast<char*>(y.data()) + 2, nullptr) == W8A8_ERR_ALIGN);
  CHECK(g_quant == 3);

  // gemm entries
  CHECK(w8a8_gemm_i32(q.data(), wq.data(), M, N, K, acc.data(), nullptr) == W8A8_OK);
  CHECK(g_gemm == 1 && g_last_i32 && g_last_cfg == 3 && g_last.M == M && g_last.N == N && g_last.K == K);
  CHECK(w8a8_gemm_i32(q.data(), nullptr, M, N, K, acc.data(), nullptr) == W8A8_ERR_NULL);
  CHECK(w8a8_gemm_i32(q.data(), wq.data(), M, N, K, nullptr, nullptr) == W8A8_ERR_NULL);
  CHECK(w8a8_gemm_i32(q.data(), wq.data(), M, N, 40, acc.data(), nullptr) == W8A8_ERR_SHAPE);
  CHECK(w8a8_gemm_i32(q.data() + 1, wq.data(), M, N, K, acc.data(), nullptr) == W8A8_ERR_ALIGN);
  CHECK(w8a8_gemm_i32(q.data(), wq.data(), 0, N, K, acc.data(), nullptr) == W8A8_OK);
  CHECK(w8a8_gemm_dequant(q.data(), sx.data(), wq.data(), sw.data(), bias.data(), M, N, K, y.data(),
                          nullptr) == W8A8_OK);
  CHECK(g_gemm == 2 && !g_last_i32 && g_last.bias == bias.data());
  CHECK(w8a8_gemm_dequant(q.data(), nullptr, wq.data(), sw.data(), nullptr, M, N, K, y.data(),
                          nullptr) == W8A8_ERR_NULL);
  CHECK(w8a8_gemm_dequant(q.data(), sx.data(), wq.data(), sw.data(),
                          reinterpret_cast<char*>(bias.data()) + 1, M, N, K, y.data(),
                          nullptr) == W8A8_ERR_ALIGN);
  CHECK(w8a8_gemm_ex(q.data(), sx.data(), wq.data(), sw.data(), nullptr, M, N, K, y.data(), 0, 10,
                     nullptr) == W8A8_OK);
  CHECK(g_last_cfg == 10);
  CHECK(w8a8_gemm_ex(q.data(), sx.data(), wq.data(), sw.data(), nullptr, M, N, K, y.data(), 0, 11,
                     nullptr) == W8A8_ERR_CONFIG);
  CHECK(w8a8_gemm_ex(q.data(), sx.data(), wq.data(), sw.data(), nullptr, M, N, K, y.data(), 0, -2,
                     nullptr) == W8A8_ERR_CONFIG);
  CHECK(g_gemm == 3);

  // fused linear: workspace size, overflow and validation before any launch
  const size_t need = w8a8_linear_workspace_bytes(M, K);
  CHECK(need == 256 + 256 && need <= sizeof(ws_buf));
  CHECK(w8a8_linear_workspace_bytes(0, K) == 0 && w8a8_linear_workspace_bytes(-1, K) == 0);
  CHECK(w8a8_linear_workspace_bytes(INT64_MAX, W8A8_MAX_K) == SIZE_MAX);  // no wrap-around
  CHECK(w8a8_linear(x.data(), wq.data(), sw.data(), bias.data(), M, N, K, y.data(), ws_buf, need,
                    nullptr) == W8A8_OK);
  CHECK(g_quant == 4 && g_gemm == 4 && g_last.qx == reinterpret_cast<int8_t*>(ws_buf));
  CHECK(w8a8_linear(x.data(), wq.data(), sw.data(), bias.data(), M, N, K, y.data(), ws_buf, need - 1,
                    nullptr) == W8A8_ERR_WORKSPACE);
  CHECK(w8a8_linear(x.data(), wq.data(), sw.data(), bias.data(), M, N, K, y.data(), nullptr, need,
                    nullptr) == W8A8_ERR_WORKSPACE);
  CHECK(w8a8_linear(x.data(), wq.data(), sw.data(), bias.data(), M, N, K, y.data(), ws_buf + 8, need,
                    nullptr) == W8A8_ERR_ALIGN);
  CHECK(w8a8_linear(x.data(), wq.data(), nullptr, bias.data(), M, N, K, y.data(), ws_buf, need,
                    nullptr) == W8A8_ERR_NULL);
  CHECK(w8a8_linear(x.data(), wq.data(), sw.data(), bias.data(), INT64_MAX, N, K, y.data(), ws_buf,
                    sizeof(ws_buf), nullptr) == W8A8_ERR_WORKSPACE);
  CHECK(g_quant == 4 && g_gemm == 4);

  // a handful of tokens: the single-launch fused kernel, codes into the workspace
  CHECK(w8a8_linear(x.data(), wq.data(), sw.data(), bias.data(), 2, N, K, y.data(), ws_buf, need,
                    nullptr) == W8A8_OK);
  CHECK(w8a8::g_rows == 1 && g_quant == 4 && g_gemm == 4);

  // allocation-free fused linear: the static scratch instead of a workspace
  CHECK(w8a8_linear_noalloc_max_bytes() == (size_t{64} << 20));
  CHECK(w8a8_linear_noalloc(x.data(), wq.data(), sw.data(), bias.data(), M, N, K, y.data(), nullptr) ==
        W8A8_OK);
  CHECK(g_quant == 5 && g_gemm == 5 && g_last.qx == reinterpret_cast<int8_t*>(w8a8::g_scratch_stub));
  CHECK(w8a8_linear_noalloc(x.data(), wq.data(), sw.data(), bias.data(), 1 << 20, N, 128, y.data(),
                            nullptr) == W8A8_ERR_SCRATCH);
  CHECK(w8a8_linear_noalloc(x.data(), wq.data(), sw.data(), bias.data(), M, N, 40, y.data(), nullptr) ==
        W8A8_ERR_SHAPE);
  CHECK(w8a8_linear_noalloc(x.data(), wq.data(), sw.data(), bias.data(), 0, N, K, y.data(), nullptr) ==
        W8A8_OK);
  CHECK(g_quant == 5 && g_gemm == 5);

  // FP8 entries
  uint8_t* q8 = reinterpret_cast<uint8_t*>(q.data());
  uint8_t* w8 = reinterpret_cast<uint8_t*>(wq.data());
  CHECK(w8a8_quantize_act_fp8(x.data(), M, K, K, q8, K, sx.data(), nullptr) == W8A8_OK);
  CHECK(w8a8_quantize_weight_fp8(wf.data(), N, K, K, w8, K, sw.data(), nullptr) == W8A8_OK);
  CHECK(w8a8_gelu_quantize_act_fp8(x.data(), M, K, K, q8, K, sx.data(), nullptr, nullptr) == W8A8_OK);
  CHECK(w8a8_gemm_dequant_fp8(q8, sx.data(), w8, sw.data(), nullptr, M, N, K, y.data(), nullptr) ==
        W8A8_OK);
  CHECK(g_gemm_fp8 == 1 && g_last_cfg == 4);
  CHECK(w8a8_gemm_fp8_ex(q8, sx.data(), w8, sw.data(), nullptr, M, N, K, y.data(), 6, nullptr) ==
        W8A8_ERR_CONFIG);
  CHECK(w8a8_linear_fp8(x.data(), w8, sw.data(), nullptr, M, N, K, y.data(), ws_buf, need, nullptr) ==
        W8A8_OK);
  CHECK(w8a8_linear_fp8(x.data(), w8, sw.data(), nullptr, M, N, K, y.data(), ws_buf, 16, nullptr) ==
        W8A8_ERR_WORKSPACE);
  CHECK(g_gemm_fp8 == 2 && g_quant == 9);
  // a handful of tokens: the single-launch fused kernel with e4m3 codes
  CHECK(w8a8_linear_fp8(x.data(), w8, sw.data(), nullptr, 2, N, K, y.data(), ws_buf, need, nullptr) ==
        W8A8_OK);
  CHECK(w8a8::g_rows_fp8 == 1 && w8a8::g_rows == 1 && g_gemm_fp8 == 2 && g_quant == 9);

  // GELU-epilogue GEMM and the absmax-given quantizer (the inter-layer fusion variant)
  {
    const int64_t Mg = 256, Ng = 256, Kg = 256;
    std::vector<int8_t> qg(Mg * Kg), wg(Ng * Kg);
    std::vector<float> sxg(Mg), swg(Ng);
    std::vector<uint16_t> hg(Mg * Ng);
    std::vector<uint32_t> am(Mg);
    CHECK(w8a8_gemm_dequant_gelu_amax(qg.data(), sxg.data(), wg.data(), swg.data(), nullptr, Mg, Ng, Kg,
                                      hg.data(), am.data(), nullptr) == W8A8_OK);
    CHECK(w8a8::g_gelu_gemm == 1);
    CHECK(w8a8_gemm_dequant_gelu_amax(qg.data(), sxg.data(), wg.data(), swg.data(), nullptr, Mg, Ng, Kg,
                                      hg.data(), nullptr, nullptr) == W8A8_ERR_NULL);
    CHECK(w8a8_gemm_dequant_gelu_amax(qg.data(), sxg.data(), wg.data(), swg.data(), nullptr, 128, Ng, Kg,
                                      hg.data(), am.data(), nullptr) == W8A8_ERR_SHAPE);
    CHECK(w8a8::g_gelu_gemm == 1);
    CHECK(w8a8_quantize_act_amax(hg.data(), Mg, Ng, Ng, am.data(), qg.data(), Ng, sxg.data(), nullptr) ==
          W8A8_OK);
    CHECK(w8a8_quantize_act_amax(hg.data(), Mg, Ng, Ng, nullptr, qg.data(), Ng, sxg.data(), nullptr) ==
          W8A8_ERR_NULL);
    CHECK(w8a8::g_quant_amax == 1);
  }

  // configuration tables
  CHECK(w8a8_gemm_num_configs() == 11 && w8a8_gemm_fp8_num_configs() == 6);
  CHECK(w8a8_gemm_config_name(11) == nullptr && w8a8_gemm_config_name(-1) == nullptr);
  CHECK(w8a8_gemm_select_config(0, 1, 16) == -1 && w8a8_gemm_select_config(4, 8, 16) == 3);

  if (g_failures) return 1;
  std::printf("abi ok\n");
  return 0;
}
