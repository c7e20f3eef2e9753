// Row-wise symmetric int8 quantization on gfx950.
//
// Per-token activation quantization and per-channel weight quantization from
// "Realizing Native INT8 Compute for Diffusion Transformers on Consumer GPUs"
// (arXiv 2606.14598), Abstract.  Convention (open on the pages, fixed here):
//   scale = fl32(absmax / 127); code = clamp(rne(fl32(x / scale)), -127, 127);
//   a row whose scale is 0 gets all-zero codes.
// The GELU variant (the activation between the two linears of a DiT MLP, not
// on the pages) first rounds gelu(v) = 0.5 * v * erfc(-v / sqrt(2)) to bf16.
//
// Design: one 64-lane wavefront per row.  Each lane loads 16-byte chunks
// strided by 64 chunks (fully coalesced 1 KiB per wave instruction), keeps
// them in registers, reduces |x| to the row maximum with cross-lane shuffles,
// then divides, rounds and packs the codes into 8-byte (bf16 input) or 4-byte
// (fp32 input) coalesced stores.  The row is read from HBM exactly once.  Rows
// too long for the register budget take a two-pass loop (second read from L2).
//
// Exactness: built with correctly rounded fp32 division, fp32 denormals kept
// and contraction off, so every step matches the IEEE definition bit for bit.
#include "internal.h"

namespace w8a8 {
namespace {

constexpr int kWaves = 4;                 // rows per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int64_t kMaxBlocks = 1 << 20;   // grid cap; rows are grid-strided

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float gelu_bf16(float v) {
  // 0.5 * v * erfc(-v / sqrt(2)); the erfc form keeps relative accuracy in
  // the negative tail, where 1 + erf(.) cancels.
  const float g = 0.5f * v * erfcf(-v * 0.70710678118654752f);
  return static_cast<float>(static_cast<__bf16>(g));  // RNE to bf16
}

__device__ __forceinline__ uint32_t quant_code(float x, float s) {
  const float t = x / s;                               // one IEEE division
  float r = __builtin_rintf(t);                        // half to even
  r = __builtin_fminf(__builtin_fmaxf(r, -127.0f), 127.0f);
  return static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xFFu;
}

template <QuantSrc SRC>
struct Src {
  static constexpr bool kF32 = (SRC == QuantSrc::kF32);
  static constexpr bool kGelu = (SRC == QuantSrc::kBf16Gelu);
  static constexpr int kEpc = kF32 ? 4 : 8;  // elements per 16-byte chunk
  static constexpr int kElemBytes = kF32 ? 4 : 2;

  // Unpack one 16-byte chunk into kEpc floats (GELU applied if requested).
  static __device__ __forceinline__ void unpack(const uint4 raw, float* v) {
    if constexpr (kF32) {
      v[0] = __uint_as_float(raw.x);
      v[1] = __uint_as_float(raw.y);
      v[2] = __uint_as_float(raw.z);
      v[3] = __uint_as_float(raw.w);
    } else {
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
      if constexpr (kGelu) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = gelu_bf16(v[i]);
      }
    }
  }

  // Quantize one chunk and store its codes (and, for GELU, its bf16 values).
  static __device__ __forceinline__ void emit(const float* v, float s, int8_t* qrow,
                                              uint16_t* hrow, int64_t c) {
    uint32_t code[kEpc];
#pragma unroll
    for (int i = 0; i < kEpc; ++i) code[i] = (s == 0.0f) ? 0u : quant_code(v[i], s);
    if constexpr (kF32) {
      const uint32_t p = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
      *reinterpret_cast<uint32_t*>(qrow + c * 4) = p;
    } else {
      uint2 p;
      p.x = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
      p.y = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
      *reinterpret_cast<uint2*>(qrow + c * 8) = p;
      if constexpr (kGelu) {
        if (hrow != nullptr) {
          uint4 h;
          uint32_t hw[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            hw[i] = (__float_as_uint(v[2 * i]) >> 16) | (__float_as_uint(v[2 * i + 1]) & 0xFFFF0000u);
          h.x = hw[0]; h.y = hw[1]; h.z = hw[2]; h.w = hw[3];
          *reinterpret_cast<uint4*>(hrow + c * 8) = h;
        }
      }
    }
  }
};

// CH > 0: each lane holds CH chunks of the row in registers (one HBM read).
template <QuantSrc SRC, int CH>
__global__ __launch_bounds__(kThreads) void quantize_rows_regs(
    const void* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale, uint16_t* __restrict__ h_out) {
  using S = Src<SRC>;
  const int lane = threadIdx.x & 63;
  const int64_t nch = K / S::kEpc;
  for (int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); row < M;
       row += (int64_t)gridDim.x * kWaves) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(x) +
                                                      row * ldx * S::kElemBytes);
    float v[CH][S::kEpc];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int64_t c = lane + 64 * j;
      uint4 raw = make_uint4(0u, 0u, 0u, 0u);
      if (c < nch) raw = src[c];
      S::unpack(raw, v[j]);
#pragma unroll
      for (int i = 0; i < S::kEpc; ++i) amax = fmaxf(amax, fabsf(v[j][i]));
    }
    amax = wave_max(amax);
    const float s = amax / 127.0f;
    if (lane == 0) scale[row] = s;
    int8_t* qrow = q + row * ldq;
    uint16_t* hrow = h_out ? h_out + row * K : nullptr;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int64_t c = lane + 64 * j;
      if (c < nch) S::emit(v[j], s, qrow, hrow, c);
    }
  }
}

// Rows longer than the register budget: pass 1 finds the absmax, pass 2
// re-reads (mostly from L2) and quantizes.  GELU is recomputed identically.
template <QuantSrc SRC>
__global__ __launch_bounds__(kThreads) void quantize_rows_loop(
    const void* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale, uint16_t* __restrict__ h_out) {
  using S = Src<SRC>;
  const int lane = threadIdx.x & 63;
  const int64_t nch = K / S::kEpc;
  for (int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); row < M;
       row += (int64_t)gridDim.x * kWaves) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(x) +
                                                      row * ldx * S::kElemBytes);
    float amax = 0.0f;
    for (int64_t c = lane; c < nch; c += 64) {
      float v[S::kEpc];
      S::unpack(src[c], v);
#pragma unroll
      for (int i = 0; i < S::kEpc; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = wave_max(amax);
    const float s = amax / 127.0f;
    if (lane == 0) scale[row] = s;
    int8_t* qrow = q + row * ldq;
    uint16_t* hrow = h_out ? h_out + row * K : nullptr;
    for (int64_t c = lane; c < nch; c += 64) {
      float v[S::kEpc];
      S::unpack(src[c], v);
      S::emit(v, s, qrow, hrow, c);
    }
  }
}

template <QuantSrc SRC>
hipError_t launch_src(const void* x, int64_t M, int64_t K, int64_t ldx, int8_t* q, int64_t ldq,
                      float* scale, uint16_t* h_out, hipStream_t stream) {
  constexpr int kEpc = Src<SRC>::kEpc;
  const int64_t per_lane = (K / kEpc + 63) / 64;
  int64_t blocks = (M + kWaves - 1) / kWaves;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
#define W8A8_Q_CASE(CHV)                                                                  \
  if (per_lane <= CHV) {                                                                  \
    quantize_rows_regs<SRC, CHV><<<grid, block, 0, stream>>>(x, M, K, ldx, q, ldq, scale, \
                                                             h_out);                      \
    return hipGetLastError();                                                             \
  }
  W8A8_Q_CASE(1)
  W8A8_Q_CASE(2)
  W8A8_Q_CASE(3)
  W8A8_Q_CASE(4)
  W8A8_Q_CASE(6)
  W8A8_Q_CASE(8)
  W8A8_Q_CASE(12)
  W8A8_Q_CASE(16)
  W8A8_Q_CASE(24)
#undef W8A8_Q_CASE
  quantize_rows_loop<SRC><<<grid, block, 0, stream>>>(x, M, K, ldx, q, ldq, scale, h_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_rows(QuantSrc src, const void* x, int64_t M, int64_t K, int64_t ldx,
                                int8_t* q, int64_t ldq, float* scale, uint16_t* h_out,
                                hipStream_t stream) {
  switch (src) {
    case QuantSrc::kBf16:
      return launch_src<QuantSrc::kBf16>(x, M, K, ldx, q, ldq, scale, nullptr, stream);
    case QuantSrc::kF32:
      return launch_src<QuantSrc::kF32>(x, M, K, ldx, q, ldq, scale, nullptr, stream);
    case QuantSrc::kBf16Gelu:
      return launch_src<QuantSrc::kBf16Gelu>(x, M, K, ldx, q, ldq, scale, h_out, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace w8a8
