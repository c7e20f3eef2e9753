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
// then computes the codes and packs them into 8-byte (bf16 input) or 4-byte
// (fp32 input) coalesced stores.  The row is read from HBM exactly once.  Rows
// too long for the register budget take a two-pass loop (second read from L2).
//
// bf16 rows never leave their packed form until the code is computed: the
// absmax is a packed 16-bit integer max of the magnitude bits (the order of
// non-negative bf16 patterns is the order of their values).
//
// Quotient x / scale, bf16 rows: with r = fl32(1 / s) (one IEEE division per
// row), q = fl32(x * r), e = fma(-q, s, x) (exact) and q' = fma(e, r, q),
// q' = fl32(x / s) -- Markstein's correction of a reciprocal-based quotient.
// It is used for rows with s >= 2^-96, where an exhaustive check over every
// pair of bf16 values |x| <= absmax confirms it (the residual e stays in the
// normal range there); smaller scales, and fp32 rows, use the IEEE division.
// Rounding: adding 1.5 * 2^23 rounds to an integer, half to even, whose
// two's-complement byte is the low byte of the sum's bit pattern; the
// division path clamps to [-127, 127] (v_med3) first, the reciprocal path
// needs no clamp (its quotients stay below 127.5 in magnitude).
//
// GELU: the input is bf16, so gelu is a function on 65536 patterns; its
// correctly rounded bf16 values form a 128 KiB table (written at build time by
// gen_gelu_lut.py in double precision) that every workgroup stages in LDS
// with direct-to-LDS loads.  One workgroup of 16 waves per CU (the table fills
// 128 KiB of the 160 KiB of LDS); each element then costs one LDS gather.
// A workgroup keeps a bounded number of rows in flight, so that rows land one
// after another and their codes overlap the reads of later rows; rows longer
// than 12 chunks per lane are split between two waves.
//
// Exactness: built with correctly rounded fp32 division, fp32 denormals kept
// and contraction off, so every step matches the IEEE definition bit for bit.
#include "internal.h"
#include "quant_codes.h"

#include <atomic>

namespace w8a8 {
namespace {

constexpr int kWaves = 4;                 // rows per workgroup (plain kernels)
constexpr int kThreads = 64 * kWaves;
constexpr int64_t kMaxBlocks = 1 << 20;   // grid cap; rows are grid-strided
constexpr int kLutWaves = 16;             // GELU kernels: one workgroup per CU
constexpr int kLutThreads = 64 * kLutWaves;
constexpr int kLutMaxBlocks = 256;        // persistent: one per compute unit

__device__ const uint16_t kGeluLut[65536] __attribute__((aligned(16))) = {
#include "gelu_lut.inc"
};

typedef __attribute__((address_space(3))) void lds_void;

// Wave index within the workgroup, in a scalar register (so row bases are
// scalar and per-lane addresses are 32-bit offsets from them).
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

// Element c of a row through a 32-bit byte offset from the row's (scalar)
// base, which lets the compiler use the scalar-base + vector-offset form.
template <typename T>
__device__ __forceinline__ T& at(T* base, uint32_t c) {
  return *reinterpret_cast<T*>(reinterpret_cast<char*>(base) + c * static_cast<uint32_t>(sizeof(T)));
}
template <typename T>
__device__ __forceinline__ const T& at(const T* base, uint32_t c) {
  return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) +
                                     c * static_cast<uint32_t>(sizeof(T)));
}

// Loads the CH chunks of a row as exactly CH unconditional load
// instructions: chunk indices past the row's end are clamped to its last
// chunk, so those registers hold a copy of real elements (harmless for the
// absmax; their codes are never stored).  Requires nch > 0.
template <int CH>
__device__ __forceinline__ void load_row(const uint4* src, uint32_t nch, uint32_t ln,
                                         uint4 (&raw)[CH]) {
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const uint32_t c = ln + 64u * j;
    raw[j] = at(src, c < nch ? c : nch - 1);
    __builtin_amdgcn_sched_barrier(0);  // issue order = chunk order
  }
}

template <bool FP8 = false>
__device__ __forceinline__ uint32_t codes_f32x4(const uint4 raw, float s) {
  if (s == 0.0f) return 0u;
  if constexpr (FP8)
    return fp8x4(__uint_as_float(raw.x) / s, __uint_as_float(raw.y) / s,
                 __uint_as_float(raw.z) / s, __uint_as_float(raw.w) / s);
  return pack4(code_word<1>(__uint_as_float(raw.x), s, 0.f), code_word<1>(__uint_as_float(raw.y), s, 0.f),
               code_word<1>(__uint_as_float(raw.z), s, 0.f), code_word<1>(__uint_as_float(raw.w), s, 0.f));
}

// Scale of a bf16 row from its packed absmax; returns the quotient mode.
template <bool FP8 = false>
__device__ __forceinline__ int row_scale(u16x2 m, float& s, float& r) {
  s = wave_max(absmax_of(m)) / kCodeMax<FP8>;
  if (s == 0.0f) return 0;
  if (s >= kFastMinScale) {
    r = 1.0f / s;
    return 2;
  }
  return 1;
}

// Quantize CH register-held bf16 chunks of one row (chunk j is c = lane+64j).
template <int CH, bool FP8 = false>
__device__ __forceinline__ void emit_bf16_row(const uint4 (&raw)[CH], int mode, float s, float r,
                                              uint32_t nch, uint32_t ln, int8_t* qrow) {
  uint2* dst = reinterpret_cast<uint2*>(qrow);
  if (mode == 2) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const uint32_t c = ln + 64u * j;
      if (c < nch) at(dst, c) = codes_bf16x8<2, FP8>(raw[j], s, r);
    }
  } else if (mode == 1) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const uint32_t c = ln + 64u * j;
      if (c < nch) at(dst, c) = codes_bf16x8<1, FP8>(raw[j], s, r);
    }
  } else {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const uint32_t c = ln + 64u * j;
      if (c < nch) at(dst, c) = make_uint2(0u, 0u);
    }
  }
}

// ------------------------------------------------------------ bf16 rows --
template <int CH, bool FP8>
__global__ __launch_bounds__(kThreads) void quantize_bf16_regs(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const uint32_t nch = static_cast<uint32_t>(K / 8);
  for (int64_t row = (int64_t)blockIdx.x * kWaves + wave_id(); row < M;
       row += (int64_t)gridDim.x * kWaves) {
    uint32_t ln = lane;            // opaque per row: keeps per-chunk indices
    asm volatile("" : "+v"(ln));   // from being hoisted into live registers
    uint4 raw[CH];
    load_row<CH>(reinterpret_cast<const uint4*>(x + row * ldx), nch, ln, raw);
    u16x2 m = {0, 0};
#pragma unroll
    for (int j = 0; j < CH; ++j)
      m = absmax2(absmax2(absmax2(absmax2(m, raw[j].x), raw[j].y), raw[j].z), raw[j].w);
    float s, r = 0.0f;
    const int mode = row_scale<FP8>(m, s, r);
    if (lane == 0) scale[row] = s;
    emit_bf16_row<CH, FP8>(raw, mode, s, r, nch, ln, q + row * ldq);
  }
}

// Long rows (13-24 chunks per lane: K up to 12288): two waves per row (the
// workgroup's waves w and w + 2 take its row w's two halves), so that a wave
// has at most 12 loads per lane in flight; the halves' maxima meet in LDS.
template <int CHH, bool FP8>
__global__ __launch_bounds__(kThreads) void quantize_bf16_halves(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale) {
  constexpr int R = kWaves / 2;  // rows per workgroup and round
  __shared__ float hmax[2][kWaves];  // alternating rounds: no overwrite before a read
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int slot = wave % R, half = wave / R;
  const uint32_t nch = static_cast<uint32_t>(K / 8);
  const uint32_t hch = (nch + 1) / 2;    // chunks of the first half (<= 64 CHH)
  const uint32_t c0 = half * hch;        // this wave's first chunk
  const uint32_t c1 = half ? nch : hch;  // one past its last (c1 > c0: nch >= 2)
  int par = 0;
  // every wave runs the same rounds (the bound depends on the workgroup only)
  for (int64_t base = (int64_t)blockIdx.x * R; base < M; base += (int64_t)gridDim.x * R, par ^= 1) {
    const int64_t row = base + slot;
    const bool active = row < M;  // wave-uniform
    uint32_t ln = lane;            // opaque per row: keeps per-chunk indices
    asm volatile("" : "+v"(ln));   // from being hoisted into live registers
    uint4 raw[CHH];
    u16x2 m = {0, 0};
    if (active) {
      // chunks past the half's end are clamped to its last one (copies of
      // real elements: the maximum is unchanged, their codes not stored)
      const uint4* src = reinterpret_cast<const uint4*>(x + row * ldx);
#pragma unroll
      for (int j = 0; j < CHH; ++j) {
        const uint32_t c = c0 + ln + 64u * j;
        raw[j] = at(src, c < c1 ? c : c1 - 1);
        __builtin_amdgcn_sched_barrier(0);  // issue order = chunk order
      }
#pragma unroll
      for (int j = 0; j < CHH; ++j)
        m = absmax2(absmax2(absmax2(absmax2(m, raw[j].x), raw[j].y), raw[j].z), raw[j].w);
    }
    const float wm = wave_max(absmax_of(m));
    if (lane == 0) hmax[par][wave] = wm;
    __syncthreads();
    if (!active) continue;
    // the row's scale and quotient mode, as row_scale computes them
    const float s = fmaxf(hmax[par][slot], hmax[par][slot + R]) / kCodeMax<FP8>;
    float r = 0.0f;
    const int mode = s == 0.0f ? 0 : (s >= kFastMinScale ? 2 : 1);
    if (mode == 2) r = 1.0f / s;
    if (lane == 0 && half == 0) scale[row] = s;
    uint2* dst = reinterpret_cast<uint2*>(q + row * ldq);
#pragma unroll
    for (int j = 0; j < CHH; ++j) {
      const uint32_t c = c0 + ln + 64u * j;
      if (c < c1)
        at(dst, c) = mode == 2 ? codes_bf16x8<2, FP8>(raw[j], s, r)
                               : (mode == 1 ? codes_bf16x8<1, FP8>(raw[j], s, r)
                                            : make_uint2(0u, 0u));
    }
  }
}

template <bool FP8>
__global__ __launch_bounds__(kThreads) void quantize_bf16_loop(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const uint32_t nch = static_cast<uint32_t>(K / 8);
  for (int64_t row = (int64_t)blockIdx.x * kWaves + wave_id(); row < M;
       row += (int64_t)gridDim.x * kWaves) {
    uint32_t ln = lane;            // opaque per row: keeps per-chunk indices
    asm volatile("" : "+v"(ln));   // from being hoisted into live registers
    const uint4* src = reinterpret_cast<const uint4*>(x + row * ldx);
    u16x2 m = {0, 0};
    for (uint32_t c = ln; c < nch; c += 64) {
      const uint4 v = at(src, c);
      m = absmax2(absmax2(absmax2(absmax2(m, v.x), v.y), v.z), v.w);
    }
    float s, r = 0.0f;
    const int mode = row_scale<FP8>(m, s, r);
    if (lane == 0) scale[row] = s;
    uint2* dst = reinterpret_cast<uint2*>(q + row * ldq);
    for (uint32_t c = ln; c < nch; c += 64) {
      const uint4 v = at(src, c);
      at(dst, c) = mode == 2 ? codes_bf16x8<2, FP8>(v, s, r)
                             : (mode == 1 ? codes_bf16x8<1, FP8>(v, s, r) : make_uint2(0u, 0u));
    }
  }
}

// Rows whose absmax is known (amax[row]: fp32 bits), e.g. raised by the
// GEMM's GELU epilogue: the same scale and codes as quantize_bf16_regs on
// the same row (its absmax is the same value), without the reduction.
template <int CH>
__global__ __launch_bounds__(kThreads) void quantize_bf16_amax_regs(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
    const uint32_t* __restrict__ amax, int8_t* __restrict__ q, int64_t ldq,
    float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const uint32_t nch = static_cast<uint32_t>(K / 8);
  for (int64_t row = (int64_t)blockIdx.x * kWaves + wave_id(); row < M;
       row += (int64_t)gridDim.x * kWaves) {
    uint32_t ln = lane;            // opaque per row: keeps per-chunk indices
    asm volatile("" : "+v"(ln));   // from being hoisted into live registers
    uint4 raw[CH];
    load_row<CH>(reinterpret_cast<const uint4*>(x + row * ldx), nch, ln, raw);
    const float s = __uint_as_float(amax[row]) / 127.0f;
    float r = 0.0f;
    int mode = 0;
    if (s >= kFastMinScale) {
      r = 1.0f / s;
      mode = 2;
    } else if (s != 0.0f) {
      mode = 1;
    }
    if (lane == 0) scale[row] = s;
    emit_bf16_row<CH, false>(raw, mode, s, r, nch, ln, q + row * ldq);
  }
}

// ----------------------------------------------------------- GELU rows --
// GELU of 8 packed bf16 values through the table: issue() starts the 8
// gathers, pack() joins the halves.  The packed words are made opaque: the
// compiler would otherwise keep the 16-bit halves apart until their use,
// doubling the registers a register-held row needs.
struct Gather8 {
  uint32_t h[8];
  __device__ __forceinline__ void issue(const uint16_t* lut, const uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[2 * i] = lut[w[i] & 0xFFFFu];
      h[2 * i + 1] = lut[w[i] >> 16];
    }
  }
  __device__ __forceinline__ uint4 pack() const {
    uint4 p = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                         h[6] | (h[7] << 16));
    asm volatile("" : "+v"(p.x), "+v"(p.y), "+v"(p.z), "+v"(p.w));
    return p;
  }
};

__device__ __forceinline__ uint4 gelu_chunk(const uint16_t* lut, uint4 v) {
  Gather8 g;
  g.issue(lut, v);
  return g.pack();
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit field");
  // gfx9 s_waitcnt: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt
  // (bits 6:4) and lgkmcnt (bits 11:8) left at their maxima (no wait).
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Stage the table: 8192 16-byte pieces, 8 per lane, straight into LDS.
__device__ __forceinline__ void stage_lut(uint16_t* lut) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8192 / kLutThreads; ++i) {
    const int piece = (i * kLutWaves + wave) * 64;  // first piece of this wave instruction
    const uint16_t* g = kGeluLut + (piece + lane) * 8;
    lds_void* d = (lds_void*)(lut + piece * 8);
    __builtin_amdgcn_global_load_lds(g, d, 16, 0, 0);
  }
}

// Rows of a workgroup in flight: the wave holding the workgroup's i-th row
// (i = wave + 16 n for its n-th row) issues that row's loads once at least
// i - depth + 1 of the workgroup's rows have arrived, as counted in LDS.
// Rows increase with i, so every row before a waiting one exists and is
// counted once its own (earlier) wait has ended: every wait ends.  The wait
// only paces the loads (the row's data and codes do not depend on it), so it
// also ends after kMaxRowWaits polls (tens of milliseconds), whatever the
// count: a wave that stopped counting can slow its workgroup, never hang it.
constexpr int kMaxRowWaits = 1 << 20;
__device__ __forceinline__ void wait_rows_arrived(const int* arrived, int need) {
  for (int i = 0; i < kMaxRowWaits; ++i) {
    if (__hip_atomic_load(arrived, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= need) break;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// GELU through the staged table, absmax (counting the row as arrived once
// its last chunk has been read), optional h copy, codes.
template <int CH, bool FP8>
__device__ __forceinline__ void gelu_finish_row(const uint16_t* lut, uint4 (&raw)[CH], int64_t row,
                                                int64_t K, uint32_t nch, uint32_t ln, int lane,
                                                int8_t* q, int64_t ldq, float* scale,
                                                uint16_t* h_out, int* arrived) {
  u16x2 m = {0, 0};
  Gather8 cur;
  cur.issue(lut, raw[0]);
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    Gather8 nxt;
    if (j + 1 < CH) nxt.issue(lut, raw[j + 1]);  // next chunk's gathers in flight
    raw[j] = cur.pack();
    m = absmax2(absmax2(absmax2(absmax2(m, raw[j].x), raw[j].y), raw[j].z), raw[j].w);
    cur = nxt;
    __builtin_amdgcn_sched_barrier(0);  // at most two chunks' gathers at a time
  }
  if (lane == 0) __hip_atomic_fetch_add(arrived, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  if (h_out != nullptr) {
    uint4* hrow = reinterpret_cast<uint4*>(h_out + row * K);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const uint32_t c = ln + 64u * j;
      if (c < nch) at(hrow, c) = raw[j];
    }
  }
  float s, r = 0.0f;
  const int mode = row_scale<FP8>(m, s, r);
  if (lane == 0) scale[row] = s;
  emit_bf16_row<CH, FP8>(raw, mode, s, r, nch, ln, q + row * ldq);
}

// depth: rows of the workgroup in flight (1..16).  At most `depth` rows
// per compute unit are being read at a time, so rows arrive one after
// another and their codes are computed while later rows stream in, instead
// of every row's data landing at the end of one long read phase.
template <int CH, bool FP8>
__global__ __launch_bounds__(kLutThreads) void gelu_quantize_regs(
    const uint16_t* __restrict__ y, int64_t M, int64_t K, int64_t ldy, int8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale, uint16_t* __restrict__ h_out, int depth) {
  __shared__ __attribute__((aligned(1024))) uint16_t lut[65536];
  __shared__ int arrived;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const uint32_t nch = static_cast<uint32_t>(K / 8);  // K >= 16: nch >= 2
  const int64_t stride = (int64_t)gridDim.x * kLutWaves;
  int64_t row = (int64_t)blockIdx.x * kLutWaves + wave;
  int item = wave;  // position of `row` in the workgroup's row sequence
  if (wave == 0) {
    if (lane == 0) arrived = 0;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the store is in LDS before the barrier
  }
  stage_lut(lut);
  if (row < M && wave < depth) {
    // First rows, peeled: their loads go out while the table pieces are in
    // flight.  Every wave reaches the barrier, also one without a row.
    uint4 raw[CH];
    __builtin_amdgcn_sched_barrier(0);
    load_row<CH>(reinterpret_cast<const uint4*>(y + row * ldy), nch, lane, raw);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<CH>();   // loads complete in order: the older table pieces have landed
    __builtin_amdgcn_s_barrier();  // ... and so have every other wave's
    __builtin_amdgcn_sched_barrier(0);
    gelu_finish_row<CH, FP8>(lut, raw, row, K, nch, lane, lane, q, ldq, scale, h_out, &arrived);
    row += stride;
    item += kLutWaves;
  } else {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  }
  for (; row < M; row += stride, item += kLutWaves) {
    wait_rows_arrived(&arrived, item - depth + 1);
    uint32_t ln = lane;            // opaque per row: keeps per-chunk indices
    asm volatile("" : "+v"(ln));   // from being hoisted into live registers
    uint4 raw[CH];
    load_row<CH>(reinterpret_cast<const uint4*>(y + row * ldy), nch, ln, raw);
    gelu_finish_row<CH, FP8>(lut, raw, row, K, nch, ln, lane, q, ldq, scale, h_out, &arrived);
  }
}

// Long rows (13-24 chunks per lane: K up to 12288): two waves per row, wave
// w and w + 8 taking its two halves, so that a wave has at most 12 loads in
// flight (a streaming probe of 256 workgroups ran ~25% slower with 21-42
// 16-byte loads per lane in flight than with 6-14).  The halves' maxima meet
// in LDS, and the workgroup takes rows in rounds of 8 (one barrier each).
// For 4096 rows of 12288: 33.8-34.0 us against 35.7-36.2 us for one wave per
// row with 8 rows in flight.
template <int CHH, bool FP8>
__global__ __launch_bounds__(kLutThreads) void gelu_quantize_pairs(
    const uint16_t* __restrict__ y, int64_t M, int64_t K, int64_t ldy, int8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale, uint16_t* __restrict__ h_out) {
  __shared__ __attribute__((aligned(1024))) uint16_t lut[65536];
  __shared__ float pmax[2][kLutWaves];  // alternating rounds: no overwrite before a read
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int pair = wave % 8, half = wave / 8;
  const uint32_t nch = static_cast<uint32_t>(K / 8);
  const uint32_t hch = (nch + 1) / 2;    // chunks of the first half (<= 64 CHH)
  const uint32_t c0 = half * hch;        // this wave's first chunk
  const uint32_t c1 = half ? nch : hch;  // one past its last (c1 > c0: nch >= 2)
  stage_lut(lut);
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  int par = 0;
  // every wave runs the same rounds (the bound depends on the workgroup only)
  for (int64_t base = (int64_t)blockIdx.x * 8; base < M; base += (int64_t)gridDim.x * 8, par ^= 1) {
    const int64_t row = base + pair;
    const bool active = row < M;  // wave-uniform
    uint32_t ln = lane;            // opaque per row: keeps per-chunk indices
    asm volatile("" : "+v"(ln));   // from being hoisted into live registers
    uint4 raw[CHH];
    u16x2 m = {0, 0};
    if (active) {
      // chunks past the half's end are clamped to its last one (copies of
      // real elements: the maximum is unchanged, their codes not stored)
      const uint4* src = reinterpret_cast<const uint4*>(y + row * ldy);
#pragma unroll
      for (int j = 0; j < CHH; ++j) {
        const uint32_t c = c0 + ln + 64u * j;
        raw[j] = at(src, c < c1 ? c : c1 - 1);
        __builtin_amdgcn_sched_barrier(0);  // issue order = chunk order
      }
      Gather8 cur;
      cur.issue(lut, raw[0]);
#pragma unroll
      for (int j = 0; j < CHH; ++j) {
        Gather8 nxt;
        if (j + 1 < CHH) nxt.issue(lut, raw[j + 1]);  // next chunk's gathers in flight
        raw[j] = cur.pack();
        m = absmax2(absmax2(absmax2(absmax2(m, raw[j].x), raw[j].y), raw[j].z), raw[j].w);
        cur = nxt;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const float hmax = wave_max(absmax_of(m));
    if (lane == 0) pmax[par][wave] = hmax;
    __syncthreads();
    if (!active) continue;
    // the row's scale and quotient mode, as row_scale computes them
    const float s = fmaxf(pmax[par][pair], pmax[par][pair + 8]) / kCodeMax<FP8>;
    float r = 0.0f;
    const int mode = s == 0.0f ? 0 : (s >= kFastMinScale ? 2 : 1);
    if (mode == 2) r = 1.0f / s;
    if (lane == 0 && half == 0) scale[row] = s;
    if (h_out != nullptr) {
      uint4* hrow = reinterpret_cast<uint4*>(h_out + row * K);
#pragma unroll
      for (int j = 0; j < CHH; ++j) {
        const uint32_t c = c0 + ln + 64u * j;
        if (c < c1) at(hrow, c) = raw[j];
      }
    }
    uint2* dst = reinterpret_cast<uint2*>(q + row * ldq);
#pragma unroll
    for (int j = 0; j < CHH; ++j) {
      const uint32_t c = c0 + ln + 64u * j;
      if (c < c1)
        at(dst, c) = mode == 2 ? codes_bf16x8<2, FP8>(raw[j], s, r)
                               : (mode == 1 ? codes_bf16x8<1, FP8>(raw[j], s, r)
                                            : make_uint2(0u, 0u));
    }
  }
}

template <bool FP8>
__global__ __launch_bounds__(kLutThreads) void gelu_quantize_loop(
    const uint16_t* __restrict__ y, int64_t M, int64_t K, int64_t ldy, int8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale, uint16_t* __restrict__ h_out) {
  __shared__ __attribute__((aligned(1024))) uint16_t lut[65536];
  const int lane = threadIdx.x & 63;
  const uint32_t nch = static_cast<uint32_t>(K / 8);
  stage_lut(lut);
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  for (int64_t row = (int64_t)blockIdx.x * kLutWaves + wave_id(); row < M;
       row += (int64_t)gridDim.x * kLutWaves) {
    uint32_t ln = lane;            // opaque per row: keeps per-chunk indices
    asm volatile("" : "+v"(ln));   // from being hoisted into live registers
    const uint4* src = reinterpret_cast<const uint4*>(y + row * ldy);
    u16x2 m = {0, 0};
    for (uint32_t c = ln; c < nch; c += 64) {
      const uint4 v = gelu_chunk(lut, at(src, c));
      m = absmax2(absmax2(absmax2(absmax2(m, v.x), v.y), v.z), v.w);
    }
    float s, r = 0.0f;
    const int mode = row_scale<FP8>(m, s, r);
    if (lane == 0) scale[row] = s;
    uint2* dst = reinterpret_cast<uint2*>(q + row * ldq);
    uint4* hrow = h_out ? reinterpret_cast<uint4*>(h_out + row * K) : nullptr;
    for (uint32_t c = ln; c < nch; c += 64) {
      const uint4 v = gelu_chunk(lut, at(src, c));
      if (hrow != nullptr) at(hrow, c) = v;
      at(dst, c) = mode == 2 ? codes_bf16x8<2, FP8>(v, s, r)
                             : (mode == 1 ? codes_bf16x8<1, FP8>(v, s, r) : make_uint2(0u, 0u));
    }
  }
}

// ------------------------------------------------------------ fp32 rows --
__device__ __forceinline__ float absmax4(float m, const uint4 v) {
  m = fmaxf(m, fabsf(__uint_as_float(v.x)));
  m = fmaxf(m, fabsf(__uint_as_float(v.y)));
  m = fmaxf(m, fabsf(__uint_as_float(v.z)));
  return fmaxf(m, fabsf(__uint_as_float(v.w)));
}

template <int CH, bool FP8>
__global__ __launch_bounds__(kThreads) void quantize_f32_regs(
    const float* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const uint32_t nch = static_cast<uint32_t>(K / 4);
  for (int64_t row = (int64_t)blockIdx.x * kWaves + wave_id(); row < M;
       row += (int64_t)gridDim.x * kWaves) {
    uint32_t ln = lane;            // opaque per row: keeps per-chunk indices
    asm volatile("" : "+v"(ln));   // from being hoisted into live registers
    uint4 raw[CH];
    load_row<CH>(reinterpret_cast<const uint4*>(x + row * ldx), nch, ln, raw);
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < CH; ++j) m = absmax4(m, raw[j]);
    const float s = wave_max(m) / kCodeMax<FP8>;
    if (lane == 0) scale[row] = s;
    uint32_t* dst = reinterpret_cast<uint32_t*>(q + row * ldq);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const uint32_t c = ln + 64u * j;
      if (c < nch) at(dst, c) = codes_f32x4<FP8>(raw[j], s);
    }
  }
}

template <bool FP8>
__global__ __launch_bounds__(kThreads) void quantize_f32_loop(
    const float* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const uint32_t nch = static_cast<uint32_t>(K / 4);
  for (int64_t row = (int64_t)blockIdx.x * kWaves + wave_id(); row < M;
       row += (int64_t)gridDim.x * kWaves) {
    uint32_t ln = lane;            // opaque per row: keeps per-chunk indices
    asm volatile("" : "+v"(ln));   // from being hoisted into live registers
    const uint4* src = reinterpret_cast<const uint4*>(x + row * ldx);
    float m = 0.0f;
    for (uint32_t c = ln; c < nch; c += 64) m = absmax4(m, at(src, c));
    const float s = wave_max(m) / kCodeMax<FP8>;
    if (lane == 0) scale[row] = s;
    uint32_t* dst = reinterpret_cast<uint32_t*>(q + row * ldq);
    for (uint32_t c = ln; c < nch; c += 64) at(dst, c) = codes_f32x4<FP8>(at(src, c), s);
  }
}

// --------------------------------------------------------------- launch --
// Register-held chunk counts per lane; longer rows, and K == 0 (scales 0,
// no loads), take the loop kernels.
#define W8A8_FOR_CH(X) X(1) X(2) X(3) X(4) X(6) X(8) X(12) X(16) X(24)

template <bool FP8>
hipError_t launch_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                       int64_t ldq, float* scale, hipStream_t stream) {
  const int64_t per_lane = (K / 8 + 63) / 64;
  const int64_t blocks = std::min<int64_t>((M + kWaves - 1) / kWaves, kMaxBlocks);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
#define W8A8_Q_CASE(CHV)                                                                  \
  if (K > 0 && per_lane <= CHV) {                                                                  \
    quantize_bf16_regs<CHV, FP8><<<grid, block, 0, stream>>>(x, M, K, ldx, q, ldq, scale); \
    return hipGetLastError();                                                             \
  }
  W8A8_Q_CASE(1) W8A8_Q_CASE(2) W8A8_Q_CASE(3) W8A8_Q_CASE(4) W8A8_Q_CASE(6) W8A8_Q_CASE(8)
  W8A8_Q_CASE(12)
#undef W8A8_Q_CASE
  if (K > 0 && per_lane <= 24) {
    // two waves per row, two rows per workgroup and round
    const dim3 grid2(static_cast<unsigned>(std::min<int64_t>((M + 1) / 2, kMaxBlocks)));
    if (per_lane <= 16)
      quantize_bf16_halves<8, FP8><<<grid2, block, 0, stream>>>(x, M, K, ldx, q, ldq, scale);
    else
      quantize_bf16_halves<12, FP8><<<grid2, block, 0, stream>>>(x, M, K, ldx, q, ldq, scale);
    return hipGetLastError();
  }
  quantize_bf16_loop<FP8><<<grid, block, 0, stream>>>(x, M, K, ldx, q, ldq, scale);
  return hipGetLastError();
}

// Rows per GELU workgroup in flight (one wave per row, rows of up to 12
// chunks per lane): about 192 KiB of row data per compute unit, at least 4
// rows and at most one per wave.  (When K = 12288 rows took this kernel, 8
// in flight measured 31.9 us for 4096 rows against 34.3 us with all 16 and
// 32.0-34.4 us with 3, 4 or 6.)
int gelu_rows_in_flight(int64_t K) {
  const int64_t row_bytes = 2 * K;
  const int64_t d = (192 * 1024 + row_bytes - 1) / row_bytes;
  return static_cast<int>(std::max<int64_t>(4, std::min<int64_t>(d, kLutWaves)));
}

template <bool FP8>
hipError_t launch_gelu(const uint16_t* y, int64_t M, int64_t K, int64_t ldy, int8_t* q,
                       int64_t ldq, float* scale, uint16_t* h_out, hipStream_t stream) {
  const int64_t per_lane = (K / 8 + 63) / 64;
  const int64_t blocks = std::min<int64_t>((M + kLutWaves - 1) / kLutWaves, kLutMaxBlocks);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kLutThreads);
  const int depth = gelu_rows_in_flight(K);
#define W8A8_G_CASE(CHV)                                                                     \
  if (K > 0 && per_lane <= CHV) {                                                            \
    gelu_quantize_regs<CHV, FP8>                                                             \
        <<<grid, block, 0, stream>>>(y, M, K, ldy, q, ldq, scale, h_out, depth);            \
    return hipGetLastError();                                                                \
  }
  W8A8_G_CASE(1) W8A8_G_CASE(2) W8A8_G_CASE(3) W8A8_G_CASE(4) W8A8_G_CASE(6) W8A8_G_CASE(8)
  W8A8_G_CASE(12)
#undef W8A8_G_CASE
  if (per_lane <= 24) {
    // two waves per row, rows in rounds of 8 per workgroup
    const dim3 grid2(static_cast<unsigned>(std::min<int64_t>((M + 7) / 8, kLutMaxBlocks)));
    if (per_lane <= 16)
      gelu_quantize_pairs<8, FP8><<<grid2, block, 0, stream>>>(y, M, K, ldy, q, ldq, scale, h_out);
    else
      gelu_quantize_pairs<12, FP8><<<grid2, block, 0, stream>>>(y, M, K, ldy, q, ldq, scale, h_out);
    return hipGetLastError();
  }
  gelu_quantize_loop<FP8><<<grid, block, 0, stream>>>(y, M, K, ldy, q, ldq, scale, h_out);
  return hipGetLastError();
}

template <bool FP8>
hipError_t launch_f32(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* q, int64_t ldq,
                      float* scale, hipStream_t stream) {
  const int64_t per_lane = (K / 4 + 63) / 64;
  const int64_t blocks = std::min<int64_t>((M + kWaves - 1) / kWaves, kMaxBlocks);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
#define W8A8_F_CASE(CHV)                                                                  \
  if (K > 0 && per_lane <= CHV) {                                                                  \
    quantize_f32_regs<CHV, FP8><<<grid, block, 0, stream>>>(x, M, K, ldx, q, ldq, scale); \
    return hipGetLastError();                                                             \
  }
  W8A8_FOR_CH(W8A8_F_CASE)
#undef W8A8_F_CASE
  quantize_f32_loop<FP8><<<grid, block, 0, stream>>>(x, M, K, ldx, q, ldq, scale);
  return hipGetLastError();
}

#undef W8A8_FOR_CH

}  // namespace

hipError_t launch_quantize_with_amax(const void* x, int64_t M, int64_t K, int64_t ldx,
                                     const uint32_t* amax, int8_t* q, int64_t ldq, float* scale,
                                     hipStream_t stream) {
  const int64_t per_lane = (K / 8 + 63) / 64;
  const int64_t blocks = std::min<int64_t>((M + kWaves - 1) / kWaves, kMaxBlocks);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
#define W8A8_A_CASE(CHV)                                                                        \
  if (K > 0 && per_lane <= CHV) {                                                               \
    quantize_bf16_amax_regs<CHV><<<grid, block, 0, stream>>>(xb, M, K, ldx, amax, q, ldq, scale); \
    return hipGetLastError();                                                                   \
  }
  W8A8_A_CASE(1) W8A8_A_CASE(2) W8A8_A_CASE(3) W8A8_A_CASE(4) W8A8_A_CASE(6) W8A8_A_CASE(8)
  W8A8_A_CASE(12) W8A8_A_CASE(16) W8A8_A_CASE(24)
#undef W8A8_A_CASE
  return hipErrorInvalidValue;  // rows longer than 24 chunks per lane (K > 12288)
}

hipError_t launch_quantize_rows(QuantSrc src, const void* x, int64_t M, int64_t K, int64_t ldx,
                                int8_t* q, int64_t ldq, float* scale, uint16_t* h_out,
                                hipStream_t stream) {
  switch (src) {
    case QuantSrc::kBf16:
      return launch_bf16<false>(static_cast<const uint16_t*>(x), M, K, ldx, q, ldq, scale, stream);
    case QuantSrc::kF32:
      return launch_f32<false>(static_cast<const float*>(x), M, K, ldx, q, ldq, scale, stream);
    case QuantSrc::kBf16Fp8:
      return launch_bf16<true>(static_cast<const uint16_t*>(x), M, K, ldx, q, ldq, scale, stream);
    case QuantSrc::kF32Fp8:
      return launch_f32<true>(static_cast<const float*>(x), M, K, ldx, q, ldq, scale, stream);
    case QuantSrc::kBf16Gelu:
      return launch_gelu<false>(static_cast<const uint16_t*>(x), M, K, ldx, q, ldq, scale, h_out,
                         stream);
    case QuantSrc::kBf16GeluFp8:
      return launch_gelu<true>(static_cast<const uint16_t*>(x), M, K, ldx, q, ldq, scale, h_out,
                               stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace w8a8
