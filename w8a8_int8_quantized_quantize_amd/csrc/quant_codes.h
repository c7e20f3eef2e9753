// Device helpers of the row quantization shared by the quantize kernels and
// the fused few-row linear: both compute a token's codes with exactly these
// operations, so the codes of one row are the same bits whichever kernel
// computes them.  Convention (open on the pages, fixed here): scale =
// fl32(absmax / 127); code = clamp(rne(fl32(x / scale)), -127, 127); a row
// whose scale is 0 gets all-zero codes.  The e4m3 variant: scale =
// fl32(absmax / 448), code = the nearest e4m3 value (ties to even) of the
// quotient clamped to +-448.  ("Realizing Native INT8 Compute for
// Diffusion Transformers on Consumer GPUs", Abstract: per-token activation
// quantization.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

// Scales from here up take the reciprocal quotient with one Markstein
// correction, which equals the IEEE division's code for every pair of bf16
// values |x| <= absmax (checked exhaustively on the CPU); smaller scales
// take the IEEE division.
constexpr float kFastMinScale = 0x1p-96f;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Packed |x| max of two bf16 values per 32-bit word.
__device__ __forceinline__ u16x2 absmax2(u16x2 m, uint32_t w) {
  const uint32_t a = w & 0x7FFF7FFFu;
  return __builtin_elementwise_max(m, *reinterpret_cast<const u16x2*>(&a));
}

__device__ __forceinline__ float absmax_of(u16x2 m) {
  const uint32_t b = m.x > m.y ? m.x : m.y;
  return __uint_as_float(b << 16);
}
// Maximum over the 64 lanes of a wave (every lane gets it; exact).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Code of x as the low byte of the returned word.  MODE 0: s == 0 (all
// zero); MODE 1: IEEE division, clamped to [-127, 127] (a subnormal scale can
// be far below absmax / 127); MODE 2: reciprocal + Markstein correction, no
// clamp: there s >= 2^-96 is within 2^-24 of absmax / 127, so |x / s| for
// |x| <= absmax stays below 127.5 and rounds into [-127, 127] by itself.
template <int MODE>
__device__ __forceinline__ uint32_t code_word(float x, float s, float r) {
  float t;
  if constexpr (MODE == 0) {
    return 0u;
  } else if constexpr (MODE == 1) {
    t = __builtin_amdgcn_fmed3f(x / s, -127.0f, 127.0f);
  } else {
    const float q = x * r;
    t = __builtin_fmaf(__builtin_fmaf(-q, s, x), r, q);
  }
  return __float_as_uint(t + 12582912.0f);
}

__device__ __forceinline__ uint32_t pack4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// FP8 (OCP e4m3) codes of four quotients: each clamped to the largest finite
// e4m3 magnitude, 448 (so that a quotient inflated by a coarse subnormal
// scale cannot become NaN), then converted two at a time with
// v_cvt_pk_fp8_f32, which rounds to the nearest e4m3 value, ties to even.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
  d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// Largest code magnitude: the row's absmax maps to it.
template <bool FP8>
constexpr float kCodeMax = FP8 ? 448.0f : 127.0f;

// The quotient x / s of the codes: MODE 1 the IEEE division, MODE 2 the
// reciprocal with one Markstein correction.  For scales absmax / 448 the
// latter differs from the division in the last bit on about 0.2% of bf16
// pairs, yet never in the e4m3 code it rounds to (checked over every pair of
// bf16 values with scale >= 2^-96 on the CPU).  The correction turns x = -0
// into +0 (-0 + +0 rounds to +0); s > 0, so the quotient takes the sign of x,
// which keeps e4m3's signed zero (code 0x80) as the division would.
template <int MODE>
__device__ __forceinline__ float quotient(float x, float s, float r) {
  if constexpr (MODE == 1) {
    return x / s;
  } else {
    const float q = x * r;
    return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q, s, x), r, q), x);
  }
}

// Eight codes of a 16-byte chunk of bf16 values.
template <int MODE, bool FP8 = false>
__device__ __forceinline__ uint2 codes_bf16x8(const uint4 raw, float s, float r) {
  uint2 p;
  if constexpr (FP8) {
    p.x = fp8x4(quotient<MODE>(bf_lo(raw.x), s, r), quotient<MODE>(bf_hi(raw.x), s, r),
                quotient<MODE>(bf_lo(raw.y), s, r), quotient<MODE>(bf_hi(raw.y), s, r));
    p.y = fp8x4(quotient<MODE>(bf_lo(raw.z), s, r), quotient<MODE>(bf_hi(raw.z), s, r),
                quotient<MODE>(bf_lo(raw.w), s, r), quotient<MODE>(bf_hi(raw.w), s, r));
  } else {
    p.x = pack4(code_word<MODE>(bf_lo(raw.x), s, r), code_word<MODE>(bf_hi(raw.x), s, r),
                code_word<MODE>(bf_lo(raw.y), s, r), code_word<MODE>(bf_hi(raw.y), s, r));
    p.y = pack4(code_word<MODE>(bf_lo(raw.z), s, r), code_word<MODE>(bf_hi(raw.z), s, r),
                code_word<MODE>(bf_lo(raw.w), s, r), code_word<MODE>(bf_hi(raw.w), s, r));
  }
  return p;
}

}  // namespace w8a8
