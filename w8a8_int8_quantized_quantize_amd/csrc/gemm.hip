// int8 x int8 -> int32 GEMM on the gfx950 integer matrix cores, with the
// per-token x per-channel dequantization and the bias fused into the epilogue.
//
// Operation: "Realizing Native INT8 Compute for Diffusion Transformers on
// Consumer GPUs" (arXiv 2606.14598), Abstract -- the fused INT8 GEMM whose
// epilogue folds the two scales and the bias, autotuned per GEMM shape.  The
// paper's kernel targets Ampere tensor cores; this one is designed for CDNA4:
//
//  * MFMA v_mfma_i32_16x16x64_i8.  The weight tile is the MFMA "A" operand and
//    the activation tile the "B" operand, so the 16x16 result block holds
//    D[n][m]: each lane owns four consecutive output columns n of one row m,
//    which the epilogue writes as one 8-byte bf16 store (16 bytes for int32).
//  * Both operands are K-contiguous ([M,K] and [N,K] row-major), which is
//    exactly what the MFMA operand layout wants: every lane reads 16
//    consecutive k of one row with a single ds_read_b128, no transposes.
//  * LDS: BK = 128 bytes of K per stage, double buffered.  Each tile row is
//    128 B; its eight 16-byte chunks are XOR-swizzled by the row index so that
//    both the global->LDS writes (8 lanes per row) and the MFMA operand reads
//    (16 rows at one chunk) hit distinct banks.
//  * Global loads are 16 B per lane, 8 lanes covering one 128-byte row segment.
//  * Tile order: the dispatcher deals workgroups round-robin to the 8 XCDs,
//    each with its own L2.  Tile ids are remapped so that each XCD receives a
//    contiguous range, walked in groups of 8 M-tiles ("grouped" order), so the
//    workgroups sharing an L2 also share activation and weight panels.
//  * Epilogue in fp32, no contraction: (s_x[m] * s_w[n]) * float(acc) + bias[n],
//    rounded once to bf16 (v_cvt_pk_bf16_f32, round to nearest even).  The
//    int32 accumulators never touch memory unless the int32 debug output is
//    requested.
//
// Ragged edges: rows beyond M / N and chunks beyond K are zero-filled in LDS;
// out-of-range outputs are never stored.  K is a multiple of 16 (API contract),
// so a 16-byte chunk is either entirely inside K or entirely outside.
#include "internal.h"

namespace w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kGroupM = 8;  // M-tiles per group in the grouped tile order

// XOR swizzle of the 16-byte chunk index inside a 128-byte LDS row.  Rows r and
// r+8 differ as well, so 16 consecutive rows read at one logical chunk land in
// 16 distinct bank groups even when two rows share a 256-byte bank line.
__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ ((row ^ (row >> 3)) & 7);
}

template <int BM_, int BN_, int WM_, int WN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int BK = 128;                    // bytes of K per stage
  static constexpr int kSlots = BK / 16;            // 16-byte chunks per row
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;  // per-wave tile
  static constexpr int FM = TM / 16, FN = TN / 16;  // 16x16 MFMA blocks per wave
  static constexpr int kWChunks = BN * kSlots;
  static constexpr int kXChunks = BM * kSlots;
  static constexpr int kWPer = (kWChunks + kThreads - 1) / kThreads;
  static constexpr int kXPer = (kXChunks + kThreads - 1) / kThreads;
  static constexpr int kStage = (BM + BN) * BK;     // LDS bytes per stage
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be whole MFMA blocks");
  static_assert(2 * kStage <= 160 * 1024, "LDS budget");
};

// Map a linear tile index to (tile_m, tile_n): XCD-contiguous ranges, then
// grouped order inside a range.
__device__ __forceinline__ void tile_coords(int t, int T, int MT, int NT, int& tm, int& tn) {
  const int per = T / 8;
  if (t < per * 8) t = (t % 8) * per + t / 8;
  const int width = kGroupM * NT;
  const int group = t / width;
  const int first_m = group * kGroupM;
  const int gsz = min(MT - first_m, kGroupM);
  const int r = t - group * width;
  tm = first_m + r % gsz;
  tn = r / gsz;
}

template <class C>
struct Stage {
  uint4 w[C::kWPer];
  uint4 x[C::kXPer];
};

// Global -> registers for one K stage (zero-filled outside the matrices).
template <class C>
__device__ __forceinline__ void load_stage(Stage<C>& st, const int8_t* __restrict__ qw,
                                           const int8_t* __restrict__ qx, int64_t n0, int64_t m0,
                                           int64_t k0, int64_t M, int64_t N, int64_t K) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < C::kWPer; ++j) {
    const int i = t + j * C::kThreads;
    const int r = i / C::kSlots, c = i % C::kSlots;
    const int64_t n = n0 + r, k = k0 + c * 16;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (i < C::kWChunks && n < N && k < K) v = *reinterpret_cast<const uint4*>(qw + n * K + k);
    st.w[j] = v;
  }
#pragma unroll
  for (int j = 0; j < C::kXPer; ++j) {
    const int i = t + j * C::kThreads;
    const int r = i / C::kSlots, c = i % C::kSlots;
    const int64_t m = m0 + r, k = k0 + c * 16;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (i < C::kXChunks && m < M && k < K) v = *reinterpret_cast<const uint4*>(qx + m * K + k);
    st.x[j] = v;
  }
}

// Registers -> LDS (swizzled).  sW: BN rows, sX: BM rows, 128 B each.
template <class C>
__device__ __forceinline__ void store_stage(const Stage<C>& st, int8_t* sW, int8_t* sX) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < C::kWPer; ++j) {
    const int i = t + j * C::kThreads;
    if (i < C::kWChunks) {
      const int r = i / C::kSlots, c = i % C::kSlots;
      *reinterpret_cast<uint4*>(sW + r * C::BK + swz(r, c) * 16) = st.w[j];
    }
  }
#pragma unroll
  for (int j = 0; j < C::kXPer; ++j) {
    const int i = t + j * C::kThreads;
    if (i < C::kXChunks) {
      const int r = i / C::kSlots, c = i % C::kSlots;
      *reinterpret_cast<uint4*>(sX + r * C::BK + swz(r, c) * 16) = st.x[j];
    }
  }
}

// MFMAs over one LDS stage.
template <class C>
__device__ __forceinline__ void compute_stage(const int8_t* sW, const int8_t* sX, int wn, int wm,
                                              v4i (&acc)[C::FN][C::FM]) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < C::BK / 64; ++kk) {
    const int c = kk * 4 + lq;
    v4i a[C::FN], b[C::FM];
#pragma unroll
    for (int f = 0; f < C::FN; ++f) {
      const int r = wn * C::TN + f * 16 + lr;
      a[f] = *reinterpret_cast<const v4i*>(sW + r * C::BK + swz(r, c) * 16);
    }
#pragma unroll
    for (int f = 0; f < C::FM; ++f) {
      const int r = wm * C::TM + f * 16 + lr;
      b[f] = *reinterpret_cast<const v4i*>(sX + r * C::BK + swz(r, c) * 16);
    }
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
      for (int j = 0; j < C::FM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)));
}

// (s_x * s_w) * float(acc) [+ bias]: each step one IEEE fp32 operation.
__device__ __forceinline__ float dequant(int32_t acc, float sx, float sw, float b, bool has_bias) {
  const float f = sx * sw;
  const float v = f * static_cast<float>(acc);
  return has_bias ? v + b : v;
}

template <class C, bool OUT_I32>
__global__ __launch_bounds__(C::kThreads) void gemm_kernel(GemmArgs a, int T, int MT, int NT) {
  __shared__ __attribute__((aligned(16))) int8_t smem[2 * C::kStage];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wn = wave % C::WN, wm = wave / C::WN;
  const int64_t M = a.M, N = a.N, K = a.K;
  const int KT = static_cast<int>((K + C::BK - 1) / C::BK);

  for (int t = blockIdx.x; t < T; t += gridDim.x) {
    int tm, tn;
    tile_coords(t, T, MT, NT, tm, tn);
    const int64_t m0 = static_cast<int64_t>(tm) * C::BM;
    const int64_t n0 = static_cast<int64_t>(tn) * C::BN;

    v4i acc[C::FN][C::FM];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
      for (int j = 0; j < C::FM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    if (KT > 0) {
      Stage<C> st;
      load_stage<C>(st, a.qw, a.qx, n0, m0, 0, M, N, K);
      store_stage<C>(st, smem, smem + C::BN * C::BK);
      __syncthreads();
      for (int kt = 0; kt < KT; ++kt) {
        int8_t* cur = smem + (kt & 1) * C::kStage;
        int8_t* nxt = smem + ((kt + 1) & 1) * C::kStage;
        const bool more = (kt + 1 < KT);
        if (more) load_stage<C>(st, a.qw, a.qx, n0, m0, static_cast<int64_t>(kt + 1) * C::BK, M, N, K);
        compute_stage<C>(cur, cur + C::BN * C::BK, wn, wm, acc);
        if (more) store_stage<C>(st, nxt, nxt + C::BN * C::BK);
        __syncthreads();
      }
    }

    // Epilogue: lane owns D[n = 4*lq + i][m = lr] of each 16x16 block.
    const int lr = lane & 15, lq = lane >> 4;
    const bool vec_ok = (N % 4) == 0;
#pragma unroll
    for (int fi = 0; fi < C::FN; ++fi) {
      const int64_t n = n0 + wn * C::TN + fi * 16 + lq * 4;
      float sw[4], bv[4];
      if constexpr (!OUT_I32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sw[i] = (n + i < N) ? a.sw[n + i] : 0.0f;
          bv[i] = (a.bias != nullptr && n + i < N) ? __uint_as_float(static_cast<uint32_t>(a.bias[n + i]) << 16) : 0.0f;
        }
      }
#pragma unroll
      for (int fj = 0; fj < C::FM; ++fj) {
        const int64_t m = m0 + wm * C::TM + fj * 16 + lr;
        if (m >= M || n >= N) continue;
        const v4i d = acc[fi][fj];
        if constexpr (OUT_I32) {
          int32_t* out = static_cast<int32_t*>(a.out) + m * N + n;
          if (vec_ok && n + 3 < N) {
            *reinterpret_cast<v4i*>(out) = d;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (n + i < N) out[i] = d[i];
          }
        } else {
          const float sx = a.sx[m];
          const bool hb = a.bias != nullptr;
          uint32_t h[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) h[i] = bf16_bits(dequant(d[i], sx, sw[i], bv[i], hb));
          uint16_t* out = static_cast<uint16_t*>(a.out) + m * N + n;
          if (vec_ok && n + 3 < N) {
            uint2 p;
            p.x = h[0] | (h[1] << 16);
            p.y = h[2] | (h[3] << 16);
            *reinterpret_cast<uint2*>(out) = p;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (n + i < N) out[i] = static_cast<uint16_t>(h[i]);
          }
        }
      }
    }
    // the next tile's prologue overwrites stage 0 of the LDS
    __syncthreads();
  }
}

// ------------------------------------------------------- configurations --
struct ConfigInfo {
  const char* name;
  int BM, BN, threads;
  int wg_per_cu;   // workgroups that fit on one CU (LDS / register bound)
  float rel_speed; // relative per-CU throughput when the chip is full
};

using T256x256 = Tile<256, 256, 2, 4>;  // 8 waves, wave tile 128(m) x 64(n)
using T256x128 = Tile<256, 128, 4, 2>;  // 8 waves, wave tile 64 x 64
using T128x256 = Tile<128, 256, 2, 4>;  // 8 waves, wave tile 64 x 64
using T128x128 = Tile<128, 128, 2, 2>;  // 4 waves, wave tile 64 x 64
using T64x64 = Tile<64, 64, 2, 2>;      // 4 waves, wave tile 32 x 32
using T16x64 = Tile<16, 64, 1, 4>;      // 4 waves, wave tile 16 x 16 (skinny M)

const ConfigInfo kConfigs[] = {
    {"bm256_bn256_bk128_w2x4", 256, 256, 512, 1, 1.00f},
    {"bm256_bn128_bk128_w4x2", 256, 128, 512, 1, 0.90f},
    {"bm128_bn256_bk128_w2x4", 128, 256, 512, 1, 0.90f},
    {"bm128_bn128_bk128_w2x2", 128, 128, 256, 2, 0.80f},
    {"bm64_bn64_bk128_w2x2", 64, 64, 256, 4, 0.45f},
    {"bm16_bn64_bk128_w1x4", 16, 64, 256, 4, 0.20f},
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);
constexpr int kNumCU = 256;
constexpr int kMaxGrid = 1 << 20;

template <class C, bool I32>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
  const int64_t MT = (a.M + C::BM - 1) / C::BM;
  const int64_t NT = (a.N + C::BN - 1) / C::BN;
  const int64_t T = MT * NT;
  if (T > INT32_MAX || MT > INT32_MAX || NT > INT32_MAX) return hipErrorInvalidValue;
  const int grid = static_cast<int>(T < kMaxGrid ? T : kMaxGrid);
  gemm_kernel<C, I32><<<dim3(grid), dim3(C::kThreads), 0, stream>>>(a, static_cast<int>(T),
                                                                   static_cast<int>(MT),
                                                                   static_cast<int>(NT));
  return hipGetLastError();
}

template <class C>
hipError_t launch_cfg_out(const GemmArgs& a, bool i32, hipStream_t stream) {
  return i32 ? launch_cfg<C, true>(a, stream) : launch_cfg<C, false>(a, stream);
}

}  // namespace

int gemm_num_configs() { return kNumConfigs; }

const char* gemm_config_name(int cfg) {
  return (cfg >= 0 && cfg < kNumConfigs) ? kConfigs[cfg].name : nullptr;
}

// Per-shape choice: the configuration with the least estimated time, where a
// configuration's time is (number of full-chip waves of tiles) x (tile area)
// / (its relative per-CU throughput).  Skinny M (<= 16) takes the narrow tile.
int gemm_select_config(int64_t M, int64_t N, int64_t K) {
  (void)K;
  if (M <= 16) return 5;
  int best = 0;
  double best_cost = 1e300;
  for (int c = 0; c < kNumConfigs - 1; ++c) {
    const ConfigInfo& ci = kConfigs[c];
    const double tiles = static_cast<double>((M + ci.BM - 1) / ci.BM) * ((N + ci.BN - 1) / ci.BN);
    const double slots = static_cast<double>(kNumCU) * ci.wg_per_cu;
    const double waves = static_cast<double>(static_cast<int64_t>((tiles + slots - 1) / slots));
    // workgroups resident on one CU share its matrix-core throughput
    const double cost = waves * ci.BM * ci.BN * ci.wg_per_cu / ci.rel_speed;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = c;
    }
  }
  return best;
}

hipError_t launch_gemm(const GemmArgs& a, bool out_int32, int cfg, hipStream_t stream) {
  switch (cfg) {
    case 0: return launch_cfg_out<T256x256>(a, out_int32, stream);
    case 1: return launch_cfg_out<T256x128>(a, out_int32, stream);
    case 2: return launch_cfg_out<T128x256>(a, out_int32, stream);
    case 3: return launch_cfg_out<T128x128>(a, out_int32, stream);
    case 4: return launch_cfg_out<T64x64>(a, out_int32, stream);
    case 5: return launch_cfg_out<T16x64>(a, out_int32, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w8a8
