// int8 x int8 -> int32 GEMM on the gfx950 integer matrix cores, with the
// per-token x per-channel dequantization and the bias fused into the epilogue.
//
// Operation: "Realizing Native INT8 Compute for Diffusion Transformers on
// Consumer GPUs" (arXiv 2606.14598), Abstract -- the fused INT8 GEMM whose
// epilogue folds the two scales and the bias, autotuned per GEMM shape.  The
// paper's kernel targets Ampere tensor cores; this one is designed for CDNA4:
//
//  * MFMA v_mfma_i32_32x32x32_i8 or v_mfma_i32_16x16x64_i8.  The weight tile
//    is the MFMA "A" operand and the activation tile the "B" operand, so a
//    result block holds D[n][m]: each lane owns runs of four consecutive
//    output columns n of one row m; the epilogue joins two such runs held by
//    different lanes (v_permlane32_swap for 32x32 blocks, v_permlane16_swap
//    across two 16x16 blocks) into one 16-byte bf16 store per lane.  The
//    16x16x64 form moves half the accumulator bytes per operation of the
//    32x32x32 one and draws less power per operation; under the chip's power
//    limit its 256 x 256 tile runs at a higher clock and is the faster one on
//    the large shapes.
//  * Both operands are K-contiguous ([M,K] and [N,K] row-major), which is what
//    the MFMA operand layout wants: every lane reads 16 consecutive k of one
//    row with a single ds_read_b128, no transposes anywhere.
//  * Global -> LDS with global_load_lds_dwordx4: each wave instruction moves
//    1 KiB straight into LDS (lane i fills bytes 16i..16i+15 of the block), so
//    no staging registers and no ds_write instructions.  The XOR swizzle of
//    the 16-byte chunks inside a row is applied on the global side: a lane
//    loads the logical chunk that belongs in its fixed LDS slot, and the
//    fragment reads are free of bank conflicts.
//  * LDS pipeline of STAGES buffers of BK bytes of K.  One wave per SIMD
//    (a 256 x 256 tile's 128 x 128 wave tiles fill the accumulator file), so
//    nothing may stall the wave between MFMAs: fragment reads and refill
//    loads are woven in one instruction at a time, and every wait uses an
//    exact vmcnt / lgkmcnt count (see Sched and wait_next_stage).
//  * Persistent workgroups: the grid is as many workgroups as fit on the
//    device at once (a multiple of the 8 XCDs); each walks tiles t, t + grid,
//    ...  Consecutive interior tiles of a workgroup are chained: the refills
//    of a tile's last stages already load the next tile's first stages, so
//    the pipeline never drains between tiles and the epilogue's stores
//    overlap the next tile's loads.
//  * Tile order: the dispatcher deals workgroups round-robin to the 8 XCDs,
//    each with its own L2.  Tile ids are remapped so each XCD receives a
//    contiguous range, walked in groups of 8 M-tiles, so the workgroups
//    sharing an L2 also share activation and weight panels, and all walk K
//    in the same order.
//  * A handful of token rows (M <= 16) is weight-streaming bound and has its
//    own split-K kernel (gemm_few_rows) with register-direct loads.
//  * Epilogue in fp32, no contraction: (s_x[m] * s_w[n]) * float(acc) + bias[n],
//    rounded once to bf16 (v_cvt_pk_bf16_f32, round to nearest even).  The
//    int32 accumulators never touch memory unless the int32 debug output is
//    requested.
//
// Ragged edges: operand rows beyond M / N are clamped to the last row (their
// results are never stored); 16-byte chunks beyond K are clamped in address
// and zeroed in the activation fragment before the MFMA.  K is a multiple of
// 16 (API contract), so a chunk is entirely inside or outside K.
#include "internal.h"
#include "quant_codes.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) int8_t global_i8;

constexpr int kGroupM = 8;  // M-tiles per group in the grouped tile order

// Swizzled slot of logical 16-byte chunk c in LDS row r.  The pattern
// depends on r & 15 only, so every fragment of a tile shares it and fragment
// addresses differ by compile-time offsets.  128-byte rows (8 chunks): any 8
// aligned consecutive rows read at one chunk hit 8 distinct 16-byte bank
// groups, and any 16 rows hit 16 distinct (row parity, slot) pairs.  64-byte
// rows (4 chunks), 32x32 operands (lane l: row l % 32, chunk l / 32): the same
// for 2 and 4 rows per bank line.  64-byte rows read as 16x16x64 operands
// (lane l: row l % 16, chunk l / 16) take R1 = true, c ^ ((r >> 1) & 3): which
// lanes the LDS serves together for a 16-byte read is not documented, and
// measured on gfx950 (SQ_LDS_BANK_CONFLICT of one wave reading each layout,
// a probe outside this library) the 64-byte-row form above costs that read 4
// conflict cycles (8 LDS cycles instead of 4) whatever the chunk order,
// while this one costs none.
template <int SLOTS, bool R1 = false>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (SLOTS == 8) return c ^ ((r & 7) ^ ((r >> 3) & 1));
  else if constexpr (R1) return c ^ ((r >> 1) & 3);
  else return c ^ (((r >> 1) & 3) ^ ((r >> 3) & 1));
}

// MFMA shapes.  MF = 32: v_mfma_i32_32x32x32_i8, 32 bytes of K per step; lane
// l holds row l % 32 of a 32-row fragment, K bytes 16 (l / 32) .. +15, and the
// result D[i][j] sits in lane j + 32 ((i / 4) % 2), register (i % 4) + 4 (i / 8).
// MF = 16: v_mfma_i32_16x16x64_i8, 64 bytes of K per step; lane l holds row
// l % 16, K bytes 16 (l / 16) .. +15, and D[i][j] sits in lane j + 16 (i / 4),
// register i % 4.  (Which K bytes of a step feed which of these positions is
// set by piece_chunk below: any assignment shared by both operands gives the
// same sums.)
template <int MF, bool FP8 = false>
struct Mfma;
// kStepBytes: K bytes of one MFMA; Frag: one lane's operand, read from LDS
// as kReads 16-byte pieces.
template <>
struct Mfma<32, false> {
  using Acc = v16i;
  using Frag = v4i;
  static constexpr int kStepBytes = 32, kGroups = 4, kReads = 1;
  static __device__ __forceinline__ Acc run(Frag a, Frag b, Acc c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mfma<16, false> {
  using Acc = v4i;
  using Frag = v4i;
  static constexpr int kStepBytes = 64, kGroups = 1, kReads = 1;
  static __device__ __forceinline__ Acc run(Frag a, Frag b, Acc c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  }
};
// FP8 (OCP e4m3) operands, fp32 accumulation: v_mfma_scale_f32_32x32x64_f8f6f4
// with both block scales 2^0 (E8M0 code 127) and e4m3 for both operands.  Same
// result layout as the int8 32x32 MFMA; a lane supplies 32 consecutive K
// bytes of its row (two 16-byte LDS reads).
template <>
struct Mfma<32, true> {
  using Acc = v16f;
  using Frag = v8i;
  static constexpr int kStepBytes = 64, kGroups = 4, kReads = 2;
  static __device__ __forceinline__ Acc run(Frag a, Frag b, Acc c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// Which 16-byte chunk of a k-step piece h of a lane holds, for lane group
// q = lane / MF.  The K positions inside one MFMA are summed in any order, so
// the lane -> chunk assignment is free as long as both operands use the same
// one; it is chosen with the LDS swizzle (see swz) so that fragment reads are
// free of bank conflicts:
//   int8 32x32x32: q
//   int8 16x16x64, 64-byte rows (swizzle R1): q
//   int8 16x16x64, 128-byte rows: q = 0, 1, 2, 3 -> 0, 2, 1, 3
//   FP8 32x32x64:  pieces q and q + 2
template <int MF, bool FP8, bool R1 = false>
__device__ __forceinline__ int piece_chunk(int q, int h) {
  if constexpr (FP8) return q + 2 * h;
  else if constexpr (MF == 16 && !R1) return ((q & 1) << 1) | (q >> 1);
  else return q;
}

template <int BM_, int BN_, int WM_, int WN_, int BK_, int STAGES_, int MF_, bool FP8_ = false>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, STAGES = STAGES_;
  static constexpr int MF = MF_;
  static constexpr bool kFp8 = FP8_;
  // 16x16x64 int8 operands in 64-byte LDS rows take the R1 swizzle (see swz)
  static constexpr bool kSwzR1 = MF_ == 16 && !FP8_ && BK_ == 64;
  using Op = Mfma<MF, FP8_>;
  using Acc = typename Op::Acc;
  static constexpr int kSlots = BK / 16;            // 16-byte chunks per LDS row
  static constexpr int kSteps = BK / Op::kStepBytes;
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int TM = BM / WM, TN = BN / WN;  // per-wave tile
  static constexpr int FM = TM / MF, FN = TN / MF;  // MFMA blocks per wave
  static constexpr int kRowsPerLoad = 1024 / BK;    // rows one wave instruction fills
  static constexpr int kLoads = (BM + BN) / kRowsPerLoad;  // per stage, whole workgroup
  static constexpr int kLoadsPerWave = (kLoads + kWaves - 1) / kWaves;
  static constexpr int kStage = (BM + BN) * BK;     // LDS bytes per stage
  // 3+ stages: refill loads are spread over the stage after the one whose
  // buffer they refill (one slice per MFMA row)
  static constexpr bool kSpread = STAGES >= 3;
  // Large tiles stage their epilogue's scales and bias in LDS (after the
  // stages: s_w [BN] fp32, s_x [BM] fp32, bias [BN] bf16), loaded early in
  // the tile's K loop, so the epilogue does not wait on global loads queued
  // behind the next tile's first stages.
  static constexpr bool kEpiLds = BM >= 128 && BN >= 128;
  static constexpr int kEpiBytes = kEpiLds ? ((BN * 6 + BM * 4 + 255) / 256) * 256 : 0;
  static constexpr int kEpiOffset = STAGES * kStage;
  static_assert(BK == 64 || BK == 128, "BK");
  static_assert(kSteps == 1 || kSteps % 2 == 0, "fragment sets alternate per k-step");
  static_assert(TM % MF == 0 && TN % MF == 0, "wave tile must be whole MFMA blocks");
  static_assert(BN % 16 == 0 && BM % 16 == 0 && BM % kRowsPerLoad == 0, "load blocks");
  static_assert((BN / kRowsPerLoad) % kWaves == 0 || kLoads <= kWaves,
                "a load slot of a wave is all weight rows or all activation rows");
  // deeper pipelines count each wave's own loads in vmcnt waits, so every
  // wave must issue the same number per stage; 2-stage pipelines wait for 0
  static_assert(STAGES == 2 || kLoads % kWaves == 0, "uneven loads need a 2-stage pipeline");
  static_assert(STAGES >= 2 && STAGES * kStage + kEpiBytes <= 160 * 1024, "LDS budget");
  // one 1 KiB load per wave: s_w on wave 0 (and wave 3 past 256 columns),
  // s_x on wave 1, the bias on wave 2
  static_assert(!kEpiLds || (kWaves >= (BN * 4 > 1024 ? 4 : 3) && BN * 4 <= 2048 && BM * 4 <= 1024),
                "epilogue vectors: one load per wave");
};

// Store instructions one wave of the interior-tile bf16 epilogue issues: one
// 16-byte store per pair of 4-column groups (32x32 blocks: the block's own
// groups pair up; 16x16 blocks: two blocks of adjacent rows pair up).
template <class C>
constexpr int kFastStores = (C::Op::kGroups % 2 == 0 || (C::MF == 16 && C::FM % 2 == 0))
                                ? C::FM * C::FN * C::Op::kGroups / 2
                                : C::FM * C::FN * C::Op::kGroups;

// Map a linear tile index to (tile_m, tile_n): XCD-contiguous ranges, then
// grouped order inside a range (groups of GM M-tiles).
template <int GM = kGroupM>
__device__ __forceinline__ void tile_coords(int t, int T, int MT, int NT, int& tm, int& tn) {
  const int per = T / 8;
  if (t < per * 8) t = (t % 8) * per + t / 8;
  const int width = GM * NT;
  const int group = t / width;
  const int first_m = group * GM;
  const int gsz = min(MT - first_m, GM);
  const int r = t - group * width;
  tm = first_m + r % gsz;
  tn = r / gsz;
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8).  Issued through the builtin so that the compiler's own
// wait insertion knows about them and does not add conservative waits.
template <int VM, int LGKM>
constexpr int waitcnt_imm() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "counter range");
  return (VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (LGKM << 8);
}

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(waitcnt_imm<0, 15>()); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm<N, 15>());
}

// Wait until at most `ahead` stages of this wave's loads are outstanding.
template <class C>
__device__ __forceinline__ void wait_stages(int ahead) {
  constexpr int L = C::kLoadsPerWave;
  if constexpr (C::STAGES >= 3) {
    if (ahead >= 1) {
      if constexpr (C::STAGES >= 4) {
        if (ahead >= 2) {
          if constexpr (C::STAGES >= 5) {
            if (ahead >= 3) { wait_vm<3 * L>(); return; }
          }
          wait_vm<2 * L>();
          return;
        }
      }
      wait_vm<L>();
      return;
    }
  }
  wait_vm0();
}

// All waves of the workgroup: this wave's LDS reads done, then everyone
// arrives.  (No vmcnt wait: later stages stay in flight.)
__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm<63, 0>());
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A uniform 64-bit address forced into scalar registers, as a global-address-
// space pointer: its loads then take the scalar-base + 32-bit vector-offset
// form, and the compiler cannot fold per-lane offsets into hoisted 64-bit
// vector addresses.
__device__ __forceinline__ const global_i8* sgpr_gptr(const int8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const global_i8*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Stage loads.  Block j of a stage covers rows [j R, (j+1) R) of the
// concatenated [BN weight rows | BM activation rows] tile, R = 1024 / BK;
// lane i fills row j R + i / SLOTS at physical slot i % SLOTS, i.e. it loads
// logical chunk swz(row, slot) (the swizzle is an involution).  FAST (interior
// tile, K a multiple of BK): a scalar base per block plus one per-lane
// offset.  Otherwise rows and chunks are clamped into the operands per lane
// (clamped data only feeds outputs that are never stored, or meets a zeroed
// activation fragment).
template <class C, bool FAST>
struct Loader {
  static constexpr int R = C::kRowsPerLoad;
  static constexpr int kWBlocksPerWave = C::BN / R / C::kWaves;  // leading weight slots
  const int8_t* qw;
  const int8_t* qx;
  int64_t n0, m0, M, N, K;
  uint32_t lane_off;

  __device__ __forceinline__ Loader(const GemmArgs& a, int64_t n0_, int64_t m0_, int wave, int lane)
      : qw(a.qw), qx(a.qx), n0(n0_), m0(m0_), M(a.M), N(a.N), K(a.K) {
    const int lr = lane / C::kSlots, p = lane % C::kSlots;
    // row & 15 of this wave's blocks: (j R) & 15 + lr, j = wave + jj kWaves
    const int rbase = (R == 8) ? ((wave & 1) * 8) : 0;
    lane_off = static_cast<uint32_t>(lr * K + swz<C::kSlots, C::kSwzR1>(rbase + lr, p) * 16);
  }


  __device__ __forceinline__ void issue(int s, int8_t* dst, int wave, int lane) const {
    issue_part<0, C::kLoadsPerWave>(s, dst, wave, lane);
  }

  // This wave's loads [J0, J1) of stage s of its own tile.
  template <int J0, int J1>
  __device__ __forceinline__ void issue_part(int s, int8_t* dst, int wave, int lane) const {
    issue_part_at<J0, J1>(n0, m0, s, dst, wave, lane);
  }

  // This wave's loads [J0, J1) of stage s of the tile at (n0t, m0t).  The
  // fast path may load for another interior tile than the loader's own (the
  // next tile of a persistent workgroup); the guarded path is only ever used
  // with its own tile.
  template <int J0, int J1>
  __device__ __forceinline__ void issue_part_at(int64_t n0t, int64_t m0t, int s, int8_t* dst,
                                                int wave, int lane) const {
    if constexpr (J0 >= J1) return;
    const int64_t k0 = static_cast<int64_t>(s) * C::BK;
#pragma unroll
    for (int jj = J0; jj < J1; ++jj) {
      const int j = wave + jj * C::kWaves;
      if (C::kLoads % C::kWaves != 0 && j >= C::kLoads) break;
      const bool is_w = jj < kWBlocksPerWave;  // compile-time after unrolling
      const int row0 = is_w ? j * R : j * R - C::BN;
      const int8_t* op = is_w ? qw : qx;
      const int64_t g0 = (is_w ? n0t : m0t) + row0;
      lds_void* d = (lds_void*)(dst + j * 1024);
      if constexpr (FAST) {
        // opaque lane offset: keeps the address a scalar base plus a 32-bit
        // vector offset (the scalar-base form of the load) instead of letting
        // the compiler hoist one 64-bit vector address per load slot
        uint32_t off = lane_off;
        asm volatile("" : "+v"(off));
        const global_i8* g = sgpr_gptr(op + g0 * K + k0) + off;
        __builtin_amdgcn_global_load_lds(g, d, 16, 0, 0);
      } else {
        const int lr = lane / C::kSlots, p = lane % C::kSlots;
        int64_t row = g0 + lr;
        const int64_t lim = is_w ? N : M;
        if (row > lim - 1) row = lim - 1;
        int64_t k = k0 + swz<C::kSlots, C::kSwzR1>(row0 + lr, p) * 16;
        if (k > K - 16) k = K - 16;
        const int8_t* g = op + row * K + k;
        __builtin_amdgcn_global_load_lds(g, d, 16, 0, 0);
      }
    }
  }
};

template <class C>
struct Frags {
  typename C::Op::Frag w[C::FN];
  typename C::Op::Frag x[C::FM];
};

// One lane's operand at byte offset `off` of an LDS stage.  A two-piece
// (32-byte) operand is the logical 16-byte chunks c and c + 2 of its row (c
// even modulo 4, see piece_chunk); the chunk swizzle is an XOR on the chunk
// index, so their slots differ only in bit 1: offsets off and off ^ 32.
template <class C>
__device__ __forceinline__ typename C::Op::Frag load_frag(const int8_t* stage, uint32_t off) {
  if constexpr (C::Op::kReads == 1) {
    return *reinterpret_cast<const v4i*>(stage + off);
  } else {
    const v4i lo = *reinterpret_cast<const v4i*>(stage + off);
    const v4i hi = *reinterpret_cast<const v4i*>(stage + (off ^ 32u));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// Fragments of one k-step: lane reads row (MF f + lane % MF) of its wave tile
// at the lane's chunk; lw / lx: lane + wave part of the address.
template <class C>
__device__ __forceinline__ void read_frags(Frags<C>& fr, const int8_t* stage, uint32_t lw,
                                           uint32_t lx) {
  // same order as the interleaved schedule: activation fragments first
#pragma unroll
  for (int f = 0; f < C::FM; ++f) fr.x[f] = load_frag<C>(stage, lx + f * C::MF * C::BK);
#pragma unroll
  for (int f = 0; f < C::FN; ++f) fr.w[f] = load_frag<C>(stage, lw + f * C::MF * C::BK);
}

// MFMAs of one k-step, weight-fragment rows [I0, I1).
template <class C, int I0, int I1>
__device__ __forceinline__ void mfma_rows(const Frags<C>& fr, typename C::Acc (&acc)[C::FN][C::FM]) {
#pragma unroll
  for (int i = I0; i < I1; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = C::Op::run(fr.w[i], fr.x[j], acc[i][j]);
}

template <class C>
__device__ __forceinline__ void mfma_step(const Frags<C>& fr, typename C::Acc (&acc)[C::FN][C::FM]) {
  mfma_rows<C, 0, C::FN>(fr, acc);
}

// Keep the compiler's scheduler from moving instructions across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// All of this wave's LDS reads have landed.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(waitcnt_imm<63, 0>()); }

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)));
}

// Two floats to a packed pair of bf16 (round to nearest even), low half first:
// one v_cvt_pk_bf16_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  const bf16x2 h = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// The bias term of one output: bias[n] as fp32, or -0.0 without a bias.
// Adding -0.0 is the identity for every fp32 value (including -0.0), so the
// epilogue adds unconditionally and a missing bias still adds nothing.
__device__ __forceinline__ float bias_term(const uint16_t* bias, int64_t n) {
  return bias ? __uint_as_float(static_cast<uint32_t>(bias[n]) << 16) : -0.0f;
}

// (s_x * s_w) * float(acc) + b: each step one IEEE fp32 operation.
__device__ __forceinline__ float dequant(int32_t acc, float sx, float sw, float b) {
  const float f = sx * sw;
  const float v = f * static_cast<float>(acc);
  return v + b;
}
// fp32 accumulator (FP8 operands): the same order without the conversion
__device__ __forceinline__ float dequant(float acc, float sx, float sw, float b) {
  const float f = sx * sw;
  const float v = f * acc;
  return v + b;
}

// Lane owns, in each MFMA block, output row m = lane % MF and four runs of
// four consecutive columns (one run for MF = 16).
template <class C, bool OUT_I32, bool GUARD>
__device__ __forceinline__ void epilogue(const GemmArgs& a, int64_t m0, int64_t n0, int wn, int wm,
                                         int lane, const typename C::Acc (&acc)[C::FN][C::FM]) {
  constexpr int MF = C::MF;
  constexpr int G = C::Op::kGroups;
  const int64_t M = a.M, N = a.N;
  const int lr = lane % MF, lq = lane / MF;
#pragma unroll
  for (int fi = 0; fi < C::FN; ++fi) {
    const int64_t nb = n0 + wn * C::TN + fi * MF + lq * 4;
    float sw[G][4], bv[G][4];
    if constexpr (!OUT_I32) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t n = nb + g * 8 + e;
          const bool in = !GUARD || n < N;
          sw[g][e] = in ? a.sw[n] : 0.0f;
          bv[g][e] = in ? bias_term(a.bias, n) : 0.0f;
        }
    }
#pragma unroll
    for (int fj = 0; fj < C::FM; ++fj) {
      // one block at a time: keeps the scheduler from pulling every
      // accumulator out of the AGPRs at once
      __builtin_amdgcn_sched_barrier(0);
      const int64_t m = m0 + wm * C::TM + fj * MF + lr;
      if (GUARD && m >= M) continue;
      const typename C::Acc d = acc[fi][fj];
      const float sx = OUT_I32 ? 0.0f : a.sx[m];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int64_t n = nb + g * 8;
        if (GUARD && n >= N) continue;
        const bool vec = !GUARD || ((N % 4) == 0 && n + 3 < N);
        if constexpr (OUT_I32) {
          int32_t* out = static_cast<int32_t*>(a.out) + m * N + n;
          if (vec) {
            *reinterpret_cast<v4i*>(out) = v4i{d[4 * g], d[4 * g + 1], d[4 * g + 2], d[4 * g + 3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) out[e] = d[4 * g + e];
          }
        } else {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = dequant(d[4 * g + e], sx, sw[g][e], bv[g][e]);
          uint16_t* out = static_cast<uint16_t*>(a.out) + m * N + n;
          if (vec) {
            uint2 pk;
            pk.x = bf16_pair(v[0], v[1]);
            pk.y = bf16_pair(v[2], v[3]);
            *reinterpret_cast<uint2*>(out) = pk;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) out[e] = static_cast<uint16_t>(bf16_bits(v[e]));
          }
        }
      }
    }
  }
}

// The 65536-entry table of correctly rounded bf16 GELU values (written at
// build time by gen_gelu_lut.py, the same table the GELU quantizer uses).
// The kernels reference it by name in device code: a constant device array
// like this one is not registered as a host-visible symbol, so its device
// address cannot be asked of the runtime.
__device__ const uint16_t kGeluTable[65536] __attribute__((aligned(16))) = {
#include "gelu_lut.inc"
};

// GELU of 8 packed bf16 outputs through the table (global memory,
// L2-resident): one gather each.
__device__ __forceinline__ uint4 gelu8(uint4 o) {
  const uint32_t w[4] = {o.x, o.y, o.z, o.w};
  uint32_t h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    h[i] = static_cast<uint32_t>(kGeluTable[w[i] & 0xFFFFu]) |
           (static_cast<uint32_t>(kGeluTable[w[i] >> 16]) << 16);
  return make_uint4(h[0], h[1], h[2], h[3]);
}

// Interior-tile bf16 epilogue, stored straight from the MFMA layout.  All
// scales and biases the lane needs are fetched up front (four consecutive
// columns at a time), then each accumulator block is dequantized and
// written in 16-byte runs (8-byte runs for 16x16 blocks without a partner
// row block).
// EPI: the tile's scales and bias were staged in LDS (stage_epilogue_vectors)
// and are read from there; otherwise from global memory, with 16-byte s_w
// and 8-byte bias loads when VEC (the vectors are aligned for them), else
// element by element (any alignment the ABI accepts).
// GELU: instead of y, store h = bf16(gelu(y)) (kGeluTable) and raise a.amax[m]
// (fp32 bits of max |h| over the row; atomic max, exact in any order) to
// each row's largest |h| over this wave's columns.  16x16 tiles only.
template <class C, bool EPI = false, bool GELU = false, bool VEC = true>
__device__ __forceinline__ void epilogue_fast(const GemmArgs& a, int64_t m0, int64_t n0, int wn,
                                              int wm, int lane,
                                              const typename C::Acc (&acc)[C::FN][C::FM],
                                              const int8_t* smem = nullptr) {
  constexpr int MF = C::MF;
  constexpr int G = C::Op::kGroups;
  static_assert(!GELU || (MF == 16 && C::FM % 2 == 0), "GELU epilogue: 16x16 blocks");
  const int lr = lane % MF, lq = lane / MF;
  // opaque bases: the scale / bias loads below must not be hoisted above the
  // K loop, where their ~100 registers would crowd out the loop's
  const float* sxp = a.sx;
  const float* swp = a.sw;
  const uint16_t* bp = a.bias;
  asm volatile("" : "+s"(sxp), "+s"(swp), "+s"(bp));
  float sx[C::FM];
  float4 sw[C::FN][G];
  uint2 bb[C::FN][G];
  // no bias: every term is -0.0 (bf16 0x8000)
  const uint2 nobias = make_uint2(0x80008000u, 0x80008000u);
  if constexpr (EPI) {
    typedef __attribute__((address_space(3))) const int8_t lds_i8;
    lds_i8* epi = (lds_i8*)(smem + C::kEpiOffset);  // address-space cast
    typedef __attribute__((address_space(3))) const float lds_f32;
    typedef __attribute__((address_space(3))) const v4f lds_f32x4;
    typedef unsigned int v2u __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) const v2u lds_u32x2;
    lds_f32* lsx = reinterpret_cast<lds_f32*>(epi + C::BN * 4);
    // the bias words are read whether or not there is a bias (the area then
    // holds stale bytes) and replaced by -0.0 with a bit mask: a choice
    // between loading and not loading would become a choice of address,
    // which loses the LDS address space
    const uint32_t keep = bp ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int fj = 0; fj < C::FM; ++fj) sx[fj] = lsx[wm * C::TM + fj * MF + lr];
#pragma unroll
    for (int fi = 0; fi < C::FN; ++fi)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int c = wn * C::TN + fi * MF + lq * 4 + g * 8;
        const v4f w = *reinterpret_cast<lds_f32x4*>(epi + c * 4);
        sw[fi][g] = make_float4(w[0], w[1], w[2], w[3]);
        const v2u v = *reinterpret_cast<lds_u32x2*>(epi + C::BN * 4 + C::BM * 4 + c * 2);
        bb[fi][g] = make_uint2((v[0] & keep) | (nobias.x & ~keep), (v[1] & keep) | (nobias.y & ~keep));
      }
  } else {
#pragma unroll
    for (int fj = 0; fj < C::FM; ++fj) sx[fj] = sxp[m0 + wm * C::TM + fj * MF + lr];
#pragma unroll
    for (int fi = 0; fi < C::FN; ++fi)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int64_t n = n0 + wn * C::TN + fi * MF + lq * 4 + g * 8;
        if constexpr (VEC) {
          sw[fi][g] = *reinterpret_cast<const float4*>(swp + n);
          bb[fi][g] = bp ? *reinterpret_cast<const uint2*>(bp + n) : nobias;
        } else {
          sw[fi][g] = make_float4(swp[n], swp[n + 1], swp[n + 2], swp[n + 3]);
          bb[fi][g] = bp ? make_uint2(bp[n] | (static_cast<uint32_t>(bp[n + 1]) << 16),
                                      bp[n + 2] | (static_cast<uint32_t>(bp[n + 3]) << 16))
                         : nobias;
        }
      }
  }
  uint16_t* y = static_cast<uint16_t*>(a.out);
  // group g of block (fi, fj), dequantized and packed to 4 bf16
  auto pack = [&](int fi, int fj, int g) {
    const typename C::Acc& d = acc[fi][fj];
    const float swv[4] = {sw[fi][g].x, sw[fi][g].y, sw[fi][g].z, sw[fi][g].w};
    const float bv[4] = {__uint_as_float(bb[fi][g].x << 16), __uint_as_float(bb[fi][g].x & 0xFFFF0000u),
                         __uint_as_float(bb[fi][g].y << 16), __uint_as_float(bb[fi][g].y & 0xFFFF0000u)};
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = dequant(d[4 * g + e], sx[fj], swv[e], bv[e]);
    return make_uint2(bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3]));
  };
  if constexpr (MF == 16 && C::FM % 2 == 0) {
    // 16x16 blocks: lane l holds columns 4 (l / 16) .. +3 of row l % 16.
    // v_permlane16_swap exchanges the odd 16-lane rows of its first operand
    // with the even rows of its second; applied to blocks fj and fj + 1 (the
    // next 16 output rows), every lane then holds 8 consecutive columns of
    // one row: lane row r = l / 16 stores row (fj + (r & 1)) 16 + l % 16,
    // columns 8 (r >> 1) .. +7 of the block, in one 16-byte store.
#pragma unroll
    for (int fj = 0; fj < C::FM; fj += 2) {
      u16x2 hmax = {0, 0};
#pragma unroll
      for (int fi = 0; fi < C::FN; ++fi) {
        __builtin_amdgcn_sched_barrier(0);
        const uint2 pa = pack(fi, fj, 0), pb = pack(fi, fj + 1, 0);
        const auto sx2 = __builtin_amdgcn_permlane16_swap(pa.x, pb.x, false, false);
        const auto sy2 = __builtin_amdgcn_permlane16_swap(pa.y, pb.y, false, false);
        uint4 o = make_uint4(sx2[0], sy2[0], sx2[1], sy2[1]);
        const int64_t m = m0 + wm * C::TM + (fj + (lq & 1)) * MF + lr;
        const int64_t n = n0 + wn * C::TN + fi * MF + (lq >> 1) * 8;
        if constexpr (GELU) {
          o = gelu8(o);
          hmax = absmax2(absmax2(absmax2(absmax2(hmax, o.x), o.y), o.z), o.w);
        }
        *reinterpret_cast<uint4*>(y + m * a.N + n) = o;
      }
      if constexpr (GELU) {
        // lanes l and l ^ 32 hold the two column halves of the same row
        float hm = absmax_of(hmax);
        hm = fmaxf(hm, __shfl_xor(hm, 32));
        if (lq < 2) {
          const int64_t m = m0 + wm * C::TM + (fj + (lq & 1)) * MF + lr;
          atomicMax(a.amax + m, __float_as_uint(hm));
        }
      }
    }
    return;
  }
  // row blocks outermost: the 16 stores of one row block complete its
  // output rows' 256-byte runs back to back, so L2 merges whole lines
  // before it writes them back (interleaving row blocks left half-written
  // lines to be written back twice)
#pragma unroll
  for (int fj = 0; fj < C::FM; ++fj) {
#pragma unroll
    for (int fi = 0; fi < C::FN; ++fi) {
      __builtin_amdgcn_sched_barrier(0);
      const int64_t m = m0 + wm * C::TM + fj * MF + lr;
      uint2 pk[G];
#pragma unroll
      for (int g = 0; g < G; ++g) pk[g] = pack(fi, fj, g);
      const int64_t nb = n0 + wn * C::TN + fi * MF;
      if constexpr (G % 2 == 0) {
        // Lanes l and l + 32 hold the two 4-column halves of each 8-column
        // group of row m.  Swap so that lane l holds group 2p whole and lane
        // l + 32 group 2p + 1 (v_permlane32_swap exchanges the upper half of
        // the first operand with the lower half of the second): one 16-byte
        // store per lane and pair of groups.
#pragma unroll
        for (int p = 0; p < G / 2; ++p) {
          const auto sx2 = __builtin_amdgcn_permlane32_swap(pk[2 * p].x, pk[2 * p + 1].x, false, false);
          const auto sy2 = __builtin_amdgcn_permlane32_swap(pk[2 * p].y, pk[2 * p + 1].y, false, false);
          const uint4 o = make_uint4(sx2[0], sy2[0], sx2[1], sy2[1]);
          const int64_t n = nb + (2 * p + lq) * 8;
          *reinterpret_cast<uint4*>(y + m * a.N + n) = o;
        }
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g)
          *reinterpret_cast<uint2*>(y + m * a.N + nb + lq * 4 + g * 8) = pk[g];
      }
    }
  }
}

template <class C>
__device__ __forceinline__ void zero_tail(Frags<C>& fr, int64_t kstep0, int64_t K, int lane) {
  constexpr int RD = C::Op::kReads;
  const int q = lane / C::MF;
#pragma unroll
  for (int h = 0; h < RD; ++h)
    if (kstep0 + 16 * piece_chunk<C::MF, C::kFp8, C::kSwzR1>(q, h) >= K) {  // piece h lies past K
#pragma unroll
      for (int f = 0; f < C::FM; ++f)
#pragma unroll
        for (int e = 0; e < 4; ++e) fr.x[f][4 * h + e] = 0;
    }
}

// Wait for the next stage's loads (this wave's) at the end of a stage.
// `ahead` whole later stages may stay in flight; with spread refills the
// last of them is only partly issued at this point.
// XST: the previous tile's epilogue stores (kFastStores of them) were issued
// after stage st + 1's loads and may stay in flight too.
template <class C, bool REFILL, bool XST = false>
__device__ __forceinline__ void wait_next_stage(int ahead) {
  if constexpr (C::kSpread && REFILL) {
    // after stage st + 1's loads: stages st + 2 .. st + S - 2 whole, and the
    // part of stage st + S - 1 issued in this stage's earlier k-steps
    constexpr int L = C::kLoadsPerWave;
    constexpr int P = L * (C::kSteps - 1) / C::kSteps;
    wait_vm<(C::STAGES - 3) * L + P + (XST ? kFastStores<C> : 0)>();
  } else {
    wait_stages<C>(ahead);
  }
}

// Interleaved k-step schedule.  A k-step is FN x FM MFMAs, row-major (row i
// uses weight fragment i with every activation fragment).  Its fragments are
// read during the previous k-step, one ds_read_b128 at a time between MFMAs,
// in the order x[0..FM-1], w[0..FN-1]; the refill loads go out one slice per
// row.  Issuing LDS reads and loads in bursts stalls the issuing wave (the
// LDS and address queues fill up) and, with one wave per SIMD, the matrix
// core with it; spread out, they overlap the MFMAs.
//   * a k-step that is not the last of its stage issues the next k-step's
//     reads over its first half, so they have all landed when the stage ends;
//   * the last k-step opens the next stage (wait for its loads, barrier) and
//     issues the next stage's first reads over its first three quarters, so
//     they have landed when the next stage starts.
template <class C>
struct Sched {
  static constexpr int R = C::FM + C::FN;  // fragment reads per k-step
  static constexpr int NM = C::FN * C::FM; // MFMAs per k-step
  // MFMA index after which read r is issued
  static constexpr int read_after(bool last, int r) {
    return last ? r * (3 * NM / 4 > 0 ? 3 * NM / 4 : 1) / R : r * (NM / 2 > 0 ? NM / 2 : 1) / R;
  }
  // reads of a `last`-type schedule issued before MFMA index j
  static constexpr int reads_before(bool last, int j) {
    int n = 0;
    for (int r = 0; r < R; ++r) n += read_after(last, r) < j ? 1 : 0;
    return n;
  }
  // lgkmcnt that guarantees row i's fragments (x[0..FM-1], w[i]) of a
  // non-last k-step have landed: the reads issued after w[i] (rest of the
  // previous step's reads, then this step's reads so far) may stay pending
  static constexpr int row_wait(int i) {
    const int n = ((R - 1 - (C::FM + i)) + reads_before(false, i * C::FM)) * C::Op::kReads;
    return n > 15 ? 15 : n;
  }
  // MFMA index after which the refill slice of row i goes out
  static constexpr int dma_after(int i) { return i * C::FM + (C::FM - 1) / 2; }
};

template <class C>
__device__ __forceinline__ void read_frag(Frags<C>& fr, int r, const int8_t* stage, uint32_t lw,
                                          uint32_t lx) {
  if (r < C::FM)
    fr.x[r] = load_frag<C>(stage, lx + r * C::MF * C::BK);
  else
    fr.w[r - C::FM] = load_frag<C>(stage, lw + (r - C::FM) * C::MF * C::BK);
}

template <int N>
__device__ __forceinline__ void wait_lgkm() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm<63, N>());
}

// Where one stage's refill loads go: stage `s` of the tile at (n0, m0)
// into LDS buffer `buf`.
struct Refill {
  int64_t n0, m0;
  int s;
  int8_t* buf;
};

// MFMAs J.. of k-step KS with the reads of the following k-step (into fn,
// from stage `rstage`; none if !READ) and the refill slices woven in.
template <class C, bool FAST, bool READ, bool EXT, int KS, int J>
__device__ __forceinline__ void step_mfmas(const Loader<C, FAST>& ld, const Frags<C>& fc,
                                           Frags<C>& fn, typename C::Acc (&acc)[C::FN][C::FM],
                                           const int8_t* rstage, uint32_t rlw, uint32_t rlx,
                                           const Refill& rf, int wave, int lane) {
  using Sc = Sched<C>;
  constexpr bool LAST = KS + 1 == C::kSteps;
  if constexpr (J < Sc::NM) {
    constexpr int i = J / C::FM, jj = J % C::FM;
    if constexpr (!LAST && jj == 0) wait_lgkm<Sc::row_wait(i)>();  // row i's fragments landed
    sched_fence();
    acc[i][jj] = C::Op::run(fc.w[i], fc.x[jj], acc[i][jj]);
    sched_fence();
    if constexpr (READ) {
#pragma unroll
      for (int r = 0; r < Sc::R; ++r)
        if (Sc::read_after(LAST, r) == J) read_frag<C>(fn, r, rstage, rlw, rlx);
    }
    if constexpr (C::kSpread) {
      if constexpr (Sc::dma_after(i) == J) {
        constexpr int Q = C::kSteps * C::FN;
        constexpr int q = KS * C::FN + i;
        constexpr int L = C::kLoadsPerWave;
        if constexpr (EXT)
          ld.template issue_part_at<q * L / Q, (q + 1) * L / Q>(rf.n0, rf.m0, rf.s, rf.buf, wave,
                                                                 lane);
        else
          ld.template issue_part<q * L / Q, (q + 1) * L / Q>(rf.s, rf.buf, wave, lane);
      }
    } else {
      constexpr int FQ = (C::FN >= 4) ? C::FN / 4 : 1;
      if constexpr (LAST && J == FQ * C::FM - 1)
        ld.template issue_part<0, C::kLoadsPerWave>(rf.s, rf.buf, wave, lane);
    }
    sched_fence();
    step_mfmas<C, FAST, READ, EXT, KS, J + 1>(ld, fc, fn, acc, rstage, rlw, rlx, rf, wave, lane);
  }
}

// k-steps KS .. KSEND-1 of one full stage.  With OPEN, the last k-step first
// opens the next stage: its loads landed everywhere (wait, barrier), which
// also means every wave's reads of this stage are done, freeing its buffer
// for a refill; and it reads the next stage's first fragments.  Without
// OPEN (a tile's last stage) it only waits for its own fragments.
// PAR: which of the two fragment sets k-step 0 of this stage uses.  A stage
// of an even number of k-steps starts and ends on set 0.  With one k-step per
// stage the steady-state loop alternates the sets (PAR 0, then 1); every other
// stage runs with PAR 0 and then moves the next stage's fragments into set 0
// (next_to_current), so a stage always begins with its fragments in set 0.
template <class C, bool FAST, bool OPEN, bool EXT, int KS, int KSEND, bool XST = false, int PAR = 0>
__device__ __forceinline__ void stage_steps(const Loader<C, FAST>& ld, Frags<C> (&f)[2],
                                            typename C::Acc (&acc)[C::FN][C::FM], const int8_t* cur,
                                            const int8_t* next, const uint32_t* lw,
                                            const uint32_t* lx, const Refill& rf, int ahead,
                                            int wave, int lane) {
  if constexpr (KS < KSEND) {
    Frags<C>& fc = f[(KS + PAR) & 1];
    Frags<C>& fn = f[(KS + 1 + PAR) & 1];
    sched_fence();
    if constexpr (KS + 1 < C::kSteps) {
      step_mfmas<C, FAST, true, EXT, KS, 0>(ld, fc, fn, acc, cur, lw[KS + 1], lx[KS + 1], rf, wave,
                                            lane);
    } else if constexpr (OPEN) {
      wait_next_stage<C, true, XST>(ahead);  // next stage landed (this wave's loads)
      block_barrier();                  // ... everywhere; this step's fragments too
      step_mfmas<C, FAST, true, EXT, KS, 0>(ld, fc, fn, acc, next, lw[0], lx[0], rf, wave, lane);
    } else {
      wait_lds();
      step_mfmas<C, FAST, false, EXT, KS, 0>(ld, fc, fn, acc, next, lw[0], lx[0], rf, wave, lane);
    }
    stage_steps<C, FAST, OPEN, EXT, KS + 1, KSEND, XST, PAR>(ld, f, acc, cur, next, lw, lx, rf, ahead,
                                                             wave, lane);
  }
}


// The tile's epilogue vectors into LDS, one direct-to-LDS load per wave
// (16 bytes per lane): wave 0 the BN scales s_w, wave 1 the BM scales s_x,
// wave 2 the BN bf16 biases (none without a bias).  Issued after the tile's
// first barrier (every wave is done with the previous tile's epilogue) and
// before the loads of its stage S - 1 (spread) or 2 (two stages), so the
// K loop's wait for those loads and its next barrier also make these visible
// to every wave; tiles with too few stages for that wait explicitly.
template <class C>
__device__ __forceinline__ void stage_epilogue_vectors(const GemmArgs& a, int8_t* smem, int64_t m0,
                                                       int64_t n0, int wave, int lane) {
  int8_t* epi = smem + C::kEpiOffset;
  const int8_t* src = nullptr;
  int bytes = 0, dst = 0;
  if (wave == 0) {
    src = reinterpret_cast<const int8_t*>(a.sw + n0);
    bytes = C::BN * 4 > 1024 ? 1024 : C::BN * 4;
  } else if (C::BN * 4 > 1024 && wave == 3) {
    src = reinterpret_cast<const int8_t*>(a.sw + n0) + 1024;
    bytes = C::BN * 4 - 1024;
    dst = 1024;
  } else if (wave == 1) {
    src = reinterpret_cast<const int8_t*>(a.sx + m0);
    bytes = C::BM * 4;
    dst = C::BN * 4;
  } else if (wave == 2 && a.bias != nullptr) {
    src = reinterpret_cast<const int8_t*>(a.bias + n0);
    bytes = C::BN * 2;
    dst = C::BN * 4 + C::BM * 4;
  }
  if (lane * 16 < bytes) {
    const global_i8* g = sgpr_gptr(src) + lane * 16;
    __builtin_amdgcn_global_load_lds(g, (lds_void*)(epi + dst), 16, 0, 0);
  }
}

// Stages the prologue of a tile loads before its K loop.  Every wave issues
// the same load sequence whatever KST is: the prologue stages and each
// stage's refill always go out.  Spread pipelines prefetch S - 1 stages
// (stage st refills stage st + S - 1 into the buffer freed just before it);
// others prefetch S.  Refills past a tile's last stage load the first stages
// of the workgroup's next tile when both are interior tiles (so that tile
// needs no prologue); otherwise they repeat the last stage, into buffers
// that are never read again.  The uniform sequence makes every vmcnt wait
// exact.
template <class C>
constexpr int kPrologue = C::kSpread ? C::STAGES - 1 : C::STAGES;

// A tile's prologue loads (all LDS buffers must be free), stage s into
// buffer s.
template <class C, bool FAST>
__device__ __forceinline__ void tile_prologue(const GemmArgs& a, int8_t* smem, int64_t m0,
                                              int64_t n0, int wave, int lane) {
  const int KST = static_cast<int>((a.K + C::BK - 1) / C::BK);
  if (KST > 0) {
    Loader<C, FAST> ld(a, n0, m0, wave, lane);
#pragma unroll
    for (int s = 0; s < kPrologue<C>; ++s)
      ld.issue(min(s, KST - 1), smem + s * C::kStage, wave, lane);
  }
}

// A tile's K loop, from its first stages' loads to the accumulators.  The
// tile's stage st lives in LDS buffer (ph + st) % S.  With `chain` (spread
// pipelines, this and the next tile both interior) the last refills load the
// next tile at (n1, m1), whose phase is then (ph + KST) % S.  All tiles walk
// K in the same order: the tiles of one XCD that share an operand panel then
// ask for the same K slice at about the same time, so L2 needs to hold only
// a few stages of each panel.  (Starting tiles at different K stages instead
// was measured slower: more L2 misses.)  Loads and stores return in issue
// order, so the first wait below also covers stores the previous tile's
// epilogue issued after this tile's first loads.
template <class C, bool FAST, bool EPI = false>
__device__ __forceinline__ void tile_mainloop(const GemmArgs& a, int8_t* smem, int64_t m0,
                                              int64_t n0, int ph, bool chain, int64_t m1,
                                              int64_t n1, bool stored, int wave, int lane,
                                              typename C::Acc (&acc)[C::FN][C::FM]) {
  constexpr int S = C::STAGES;
  constexpr int NS = C::kSteps;
  constexpr int SB = C::Op::kStepBytes;
  constexpr int PRO = kPrologue<C>;
  const int wn = wave % C::WN, wm = wave / C::WN;
  const int KST = static_cast<int>((a.K + C::BK - 1) / C::BK);  // stages
  Loader<C, FAST> ld(a, n0, m0, wave, lane);
  auto buf = [&](int st) { return smem + ((ph + st) % S) * C::kStage; };

  // fragment addressing: row (MF f + lane % MF), chunk (step SB/16 + piece_chunk(lane / MF, 0))
  uint32_t lw[NS], lx[NS];
  {
    const int fr = lane % C::MF, fq = lane / C::MF;
#pragma unroll
    for (int ks = 0; ks < NS; ++ks) {
      const uint32_t l = static_cast<uint32_t>(
          fr * C::BK + swz<C::kSlots, C::kSwzR1>(fr, ks * (SB / 16) + piece_chunk<C::MF, C::kFp8, C::kSwzR1>(fq, 0)) * 16);
      lw[ks] = l + static_cast<uint32_t>(wn * C::TN * C::BK);
      lx[ks] = l + static_cast<uint32_t>(C::BN * C::BK + wm * C::TM * C::BK);
    }
  }

#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = typename C::Acc{};

  if (KST > 0) {
    // stage 0 landed; with `stored`, the previous tile's epilogue issued
    // kFastStores stores after this tile's first PRO stages, which need not
    // have completed
    if constexpr (C::kSpread) {
      if (stored)
        wait_vm<(PRO - 1) * C::kLoadsPerWave + kFastStores<C>>();
      else
        wait_stages<C>(PRO - 1);
    } else {
      wait_stages<C>(PRO - 1);
    }
    block_barrier();
    if constexpr (EPI) stage_epilogue_vectors<C>(a, smem, m0, n0, wave, lane);
    Frags<C> f[2];
    read_frags<C>(f[0], buf(0), lw[0], lx[0]);
    // nothing in flight on the LDS / scalar-load counter when the K loop
    // starts, so the row waits inside it are exact
    wait_lds();
    // Stage st's k-steps run as a head (steps 0 .. NS-2) and a tail (the
    // last step, which opens stage st + 1).  The loop body is one stage's
    // tail followed by the next stage's head, so the fragment reads that
    // cross the loop back edge are always waited for by the tail's barrier
    // and the row waits inside the body are exact.
    // A stage refills stage st + S - 1 (spread; st + S otherwise) of this
    // tile while that exists ("own": addresses from per-tile bases the
    // compiler keeps across the loop); past the end it loads the next
    // tile's first stages when chained, else it repeats the last stage
    // ("ext": addresses from a run-time origin, only in the last stages).
    auto refill_of = [&](int st) {
      Refill r;
      const int rs = C::kSpread ? st + S - 1 : st + S;
      r.buf = C::kSpread ? buf(st + S - 1) : buf(st);  // freed just before / once the next is open
      if (rs < KST) {
        r.n0 = n0; r.m0 = m0; r.s = rs;
      } else if (chain) {
        r.n0 = n1; r.m0 = m1; r.s = rs - KST;
      } else {
        r.n0 = n0; r.m0 = m0; r.s = KST - 1;
      }
      return r;
    };
    auto head = [&](auto ext, int st) {
      if constexpr (NS > 1) {
        const Refill r = refill_of(st);
        stage_steps<C, FAST, true, decltype(ext)::value, 0, NS - 1>(ld, f, acc, buf(st), buf(st + 1),
                                                                   lw, lx, r, S - 2, wave, lane);
      }
    };
    // one k-step per stage: the next stage's fragments were read into set 1
    auto next_to_current = [&]() {
      if constexpr (NS == 1) f[0] = f[1];
    };
    auto tail = [&](auto ext, int st) {
      const Refill r = refill_of(st);
      stage_steps<C, FAST, true, decltype(ext)::value, NS - 1, NS>(ld, f, acc, buf(st), buf(st + 1),
                                                                  lw, lx, r, S - 2, wave, lane);
      next_to_current();
    };
    // a tail whose wait also lets the previous epilogue's stores stay in
    // flight (the next stage was loaded before them)
    auto tail_xst = [&](int st) {
      const Refill r = refill_of(st);
      stage_steps<C, FAST, true, false, NS - 1, NS, true>(ld, f, acc, buf(st), buf(st + 1), lw, lx, r,
                                                          S - 2, wave, lane);
      next_to_current();
    };
    using Own = std::false_type;
    using Ext = std::true_type;
    // stages [0, own_end) refill from this tile
    const int own_end = KST - (C::kSpread ? S - 1 : S);
    if constexpr (FAST && C::kSpread) {
      // every stage is whole: the last one runs as a head and a closing
      // tail that still issues its refills (the next tile's first stages)
      if (own_end > 0) head(Own{}, 0); else head(Ext{}, 0);
      int st = 0;
      // stages 1 .. S-2 were loaded before the previous tile's epilogue
      // stores: their waits need not wait for the stores
      if (stored && own_end >= S - 1) {
        for (; st < S - 2; ++st) {
          tail_xst(st);
          head(Own{}, st + 1);
        }
      }
      if constexpr (NS == 1) {
        // one k-step per stage: the fragment sets alternate with the stage,
        // so the steady-state loop runs two stages per iteration with
        // compile-time sets (st is even here)
        for (; st + 2 < own_end; st += 2) {
          const Refill r0 = refill_of(st);
          stage_steps<C, FAST, true, false, 0, 1, false, 0>(ld, f, acc, buf(st), buf(st + 1), lw, lx,
                                                            r0, S - 2, wave, lane);
          const Refill r1 = refill_of(st + 1);
          stage_steps<C, FAST, true, false, 0, 1, false, 1>(ld, f, acc, buf(st + 1), buf(st + 2), lw,
                                                            lx, r1, S - 2, wave, lane);
        }
      }
      for (; st + 1 < own_end; ++st) {
        tail(Own{}, st);
        head(Own{}, st + 1);
      }
      if (st + 1 < KST && st < own_end) {
        tail(Own{}, st);
        head(Ext{}, st + 1);
        ++st;
      }
      for (; st + 1 < KST; ++st) {
        tail(Ext{}, st);
        head(Ext{}, st + 1);
      }
      const Refill r = refill_of(KST - 1);
      stage_steps<C, FAST, false, true, NS - 1, NS>(ld, f, acc, buf(KST - 1), buf(KST), lw, lx, r,
                                                    S - 2, wave, lane);
      // repeated stages must land before the buffers are reused; chained
      // loads are the next tile's
      if (!chain) wait_vm0();
    } else {
      // own-tile refills only (repeats clamp the stage index); the last
      // (possibly partial) stage is peeled below
      const int nfull = KST - 1;
      if (nfull > 0) {
        head(Own{}, 0);
        for (int st = 0; st + 1 < nfull; ++st) {
          tail(Own{}, st);
          head(Own{}, st + 1);
        }
        tail(Own{}, nfull - 1);
      }
      {
        constexpr int P = 0;
        const int st = KST - 1;
        const int8_t* cur = buf(st);
        const int64_t k0 = static_cast<int64_t>(st) * C::BK;
#pragma unroll
        for (int ks = 0; ks < NS; ++ks) {
          const int64_t ksk = k0 + ks * SB;
          if (!FAST && ksk >= a.K) break;
          sched_fence();
          wait_lds();
          if (ks + 1 < NS && (FAST || ksk + SB < a.K))
            read_frags<C>(f[(ks + 1 + P) & 1], cur, lw[ks + 1], lx[ks + 1]);
          if (!FAST && ksk + SB > a.K) zero_tail<C>(f[(ks + P) & 1], ksk, a.K, lane);
          sched_fence();
          mfma_step<C>(f[(ks + P) & 1], acc);
        }
      }
      // the repeated loads past the last stage must land before the buffers
      // are reused by a next tile or the workgroup ends
      wait_vm0();
    }
  }
}

template <class C, bool FAST, bool OUT_I32, bool EPI = false, bool VEC = true>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& a, int64_t m0, int64_t n0, int wave,
                                              int lane, const typename C::Acc (&acc)[C::FN][C::FM],
                                              const int8_t* smem = nullptr) {
  const int wn = wave % C::WN, wm = wave / C::WN;
  if constexpr (FAST && !OUT_I32)
    epilogue_fast<C, EPI, false, VEC>(a, m0, n0, wn, wm, lane, acc, smem);
  else
    epilogue<C, OUT_I32, !FAST>(a, m0, n0, wn, wm, lane, acc);
}

// Tiles of the edge kernel, e in [0, E): the last row of tiles when M is
// ragged (every column), then the last column when N is ragged (the rows
// above it); or, with `all`, every tile (row-major) when no tile can take the
// unguarded path.
__device__ __forceinline__ void edge_coords(int e, int MT, int NT, int MTi, int NTi, bool all,
                                            int& tm, int& tn) {
  if (all) {
    tm = e / NT;
    tn = e - tm * NT;
    return;
  }
  const int nrow = MT > MTi ? NT : 0;
  if (e < nrow) {
    tm = MTi;
    tn = e;
    return;
  }
  tm = e - nrow;
  tn = NTi;
}

// Persistent workgroups: workgroup b takes tiles b, b + G, b + 2G, ... (G =
// grid size, a multiple of 8 when there are more tiles than workgroups, so
// each workgroup stays on one XCD's tile range).  The next tile's prologue
// loads go out before the current tile's epilogue, so their latency hides
// behind its arithmetic and stores.
// Two kernels per configuration: the interior one (EDGE = false) takes the
// MTi x NTi tiles that lie wholly inside M and N -- the host launches it only
// when K is a whole number of stages and output rows are multiples of 16
// bytes -- with unguarded loads, chained tiles and the vector epilogue (its
// VEC form when the scales / bias are vector aligned, else reading them
// element by element); the edge one takes the remaining tiles with
// clamped loads and guarded stores.  Kept apart, the interior kernel holds no
// registers for the guarded code: it does not spill, so no reload (and no
// wait for all outstanding loads that a reload implies) sits between a tile's
// K loop and its epilogue while the next tile's first stages are in flight.
template <class C, bool OUT_I32, bool EDGE, bool VEC = true>
__global__ __launch_bounds__(C::kThreads) void gemm_kernel(GemmArgs a, int T, int MT, int NT,
                                                           int MTi, int NTi, int all) {
  constexpr bool FAST = !EDGE;
  // interior bf16 tiles of large configurations stage their epilogue vectors
  // (VEC: the vectors are aligned for it; otherwise the epilogue reads them
  // from global memory element by element)
  constexpr bool EPI = FAST && !OUT_I32 && C::kEpiLds && VEC;
  __shared__ __attribute__((aligned(1024))) int8_t smem[C::STAGES * C::kStage + (EPI ? C::kEpiBytes : 0)];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  int t = blockIdx.x;
  if (t >= T) return;
  auto origin = [&](int tt, int64_t& m, int64_t& n) {
    int tm, tn;
    if constexpr (EDGE)
      edge_coords(tt, MT, NT, MTi, NTi, all != 0, tm, tn);
    else
      tile_coords(tt, T, MTi, NTi, tm, tn);
    m = static_cast<int64_t>(tm) * C::BM;
    n = static_cast<int64_t>(tn) * C::BN;
  };
  int64_t m0, n0;
  origin(t, m0, n0);
  tile_prologue<C, FAST>(a, smem, m0, n0, wave, lane);
  const int KST = static_cast<int>((a.K + C::BK - 1) / C::BK);
  int ph = 0;       // LDS buffer of the current tile's stage 0
  bool stored = false;  // see tile_mainloop
  typename C::Acc acc[C::FN][C::FM];
  for (;;) {
    const int tnext = t + static_cast<int>(gridDim.x);
    const bool more = tnext < T;
    int64_t m1 = 0, n1 = 0;
    if (more) origin(tnext, m1, n1);
    // interior tiles chain: this tile's last refills are the next one's
    // first stages.  Stage st refills stage st + S - 1, so the refills reach
    // the next tile's stages 0 .. S - 2 only when the tile has at least S - 1
    // stages; shorter tiles load the next tile's prologue after their K loop
    // (with clamped stage indices) instead.
    const bool chain = FAST && C::kSpread && more && KST >= C::STAGES - 1;
    // opaque per tile: lane- and wave-derived offsets are recomputed for
    // each tile instead of being hoisted out of the tile loop, where their
    // registers would be held through every K loop
    int ln = lane, wv = wave;
    asm volatile("" : "+v"(ln), "+s"(wv));
    tile_mainloop<C, FAST, EPI>(a, smem, m0, n0, ph, chain, m1, n1, stored, wv, ln, acc);
    if constexpr (EPI) {
      // too few stages for the K loop's waits and barriers to cover the
      // epilogue vectors: wait for them explicitly (K <= STAGES x BK)
      if (KST <= C::STAGES) {
        wait_vm0();
        block_barrier();
      }
    }
    if (chain) {
      ph = (ph + KST) % C::STAGES;
    } else if (more) {
      ph = 0;
      block_barrier();  // every wave is done reading this tile's LDS buffers
      int ln1 = lane, wv1 = wave;
      asm volatile("" : "+v"(ln1), "+s"(wv1));
      tile_prologue<C, FAST>(a, smem, m1, n1, wv1, ln1);
    }
    int ln2 = lane, wv2 = wave;
    asm volatile("" : "+v"(ln2), "+s"(wv2));
    tile_epilogue<C, FAST, OUT_I32, EPI, VEC>(a, m0, n0, wv2, ln2, acc, smem);
    // the next tile's first stages went out before these stores; the
    // interior bf16 epilogue issues exactly kFastStores of them
    stored = FAST && !OUT_I32;
    if (!more) break;
    t = tnext;
    m0 = m1;
    n0 = n1;
  }
}

// ------------------------------------------------------------ ping-pong --
// Interior tiles with two waves per SIMD that take turns on the matrix core.
// The 8 waves form two groups of four (one wave of each group per SIMD):
// group 0 owns output rows [0, BM/2) of the tile, group 1 rows [BM/2, BM);
// within a group wave w owns columns [w TN, (w+1) TN).  Every k-step of a
// wave is a memory phase (its fragments for the step read from LDS into
// registers, its share of a refill stage issued global -> LDS) followed by
// a compute phase (the step's MFMAs back to back from registers), and the
// phases are separated by workgroup barriers.  Group 1 starts one barrier
// late, so while one group's wave on a SIMD runs its compute phase the other
// group's wave runs its memory phase: the matrix core is fed by one wave
// without LDS reads, loads or address arithmetic between its MFMAs (issued
// from a single wave, those cost the 16x16x64 MFMA stream about a third of
// its rate).  A tile's epilogue runs in the group's memory slot, alongside
// the other group's MFMAs.
//
// Interval k lies between the k-th and (k+1)-th barrier; group 0 runs the
// memory phase of step i in interval 2i and its compute phase in 2i + 1,
// group 1 one interval later.  Hence:
//  * stage i's buffer is read in intervals 2i (group 0) and 2i + 1 (group
//    1); the refill issued in step i + 1's memory phase (interval >= 2i + 2)
//    overwrites it only after every wave passed the barrier that ends 2i + 1
//    (block_barrier waits for the wave's own LDS reads first);
//  * stage i + 1 is first read in interval 2i + 2, so every wave waits for
//    its own loads of that stage before the barrier that opens it: group 0
//    at the end of its compute phase of step i, group 1 at the end of its
//    memory phase of step i.
// Loads and stores of a wave retire in issue order; a wave's loads of stage
// i + 1 are followed by the refills of S - 2 later steps (L loads each), and
// for the first S - 2 steps of a tile also by the previous tile's epilogue
// stores, which fixes each wait count at compile time.  (Waves 0-2, and 3
// on 384-column tiles, also load the tile's epilogue vectors at step 0, one
// load each, after those stages: their waits then cover one load more than
// needed.)  The refills of a
// tile's last S - 1 steps load the workgroup's next tile's first stages
// (consecutive tiles chain, so a tile needs K >= S x BK), or repeat the last
// stage after the workgroup's last tile.  The epilogue vectors (scales, bias)
// alternate between two LDS buffers from tile to tile: group 0 loads the next
// tile's while group 1 may still read the previous ones.
template <class C, bool OUT_I32, bool GELU = false>
__global__ __launch_bounds__(C::kThreads) void gemm_pp_kernel(GemmArgs a, int T, int MTi, int NTi) {
  static_assert(C::kWaves == 8 && C::WM == 2 && C::WN == 4 && C::kSteps == 1 && C::kSpread,
                "ping-pong tiles: 2 x 4 waves, one k-step per stage, 3+ stages");
  constexpr int S = C::STAGES;
  constexpr int L = C::kLoadsPerWave;
  constexpr bool EPI = !OUT_I32 && C::kEpiLds;
  constexpr int kStores = OUT_I32 ? C::FM * C::FN * C::Op::kGroups : kFastStores<C>;
  static_assert((S - 2) * L + kStores <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) int8_t smem[S * C::kStage + (EPI ? 2 * C::kEpiBytes : 0)];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int grp = wave / C::WN;  // = wm
  const int wn = wave % C::WN;
  int t = blockIdx.x;
  if (t >= T) return;
  const int KST = static_cast<int>(a.K / C::BK);  // >= S (host condition)
  auto origin = [&](int tt, int64_t& m, int64_t& n) {
    int tm, tn;
    tile_coords(tt, T, MTi, NTi, tm, tn);
    m = static_cast<int64_t>(tm) * C::BM;
    n = static_cast<int64_t>(tn) * C::BN;
  };
  int64_t m0, n0;
  origin(t, m0, n0);
  // fragment addresses: row MF f + lane % MF of the wave's tile, chunk
  // piece_chunk(lane / MF) of the 64-byte k-step
  uint32_t lw, lx;
  {
    const int fr = lane % C::MF, fq = lane / C::MF;
    const uint32_t l = static_cast<uint32_t>(fr * C::BK + swz<C::kSlots, C::kSwzR1>(fr, piece_chunk<C::MF, false, C::kSwzR1>(fq, 0)) * 16);
    lw = l + static_cast<uint32_t>(wn * C::TN * C::BK);
    lx = l + static_cast<uint32_t>(C::BN * C::BK + grp * C::TM * C::BK);
  }
  {
    Loader<C, true> ld(a, n0, m0, wave, lane);
#pragma unroll
    for (int s = 0; s < S - 1; ++s) ld.template issue_part_at<0, L>(n0, m0, s, smem + s * C::kStage, wave, lane);
  }
  wait_vm<(S - 2) * L>();  // this wave's stage 0
  block_barrier();         // everyone's
  if (grp == 1) block_barrier();  // group 1 runs one interval behind
  int ph = 0;        // LDS buffer of the current tile's stage 0
  int par = 0;       // epilogue-vector buffer of the current tile
  bool stored = false;
  typename C::Acc acc[C::FN][C::FM];
  Frags<C> f;
  for (;;) {
    const int tnext = t + static_cast<int>(gridDim.x);
    const bool more = tnext < T;
    int64_t m1 = m0, n1 = n0;
    if (more) origin(tnext, m1, n1);
    int ln = lane, wv = wave;
    asm volatile("" : "+v"(ln), "+s"(wv));
    Loader<C, true> ld(a, n0, m0, wv, ln);
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
      for (int j = 0; j < C::FM; ++j) acc[i][j] = typename C::Acc{};
    int8_t* epi = smem + par * C::kEpiBytes;  // epilogue vectors at epi + kEpiOffset
    for (int i = 0; i < KST; ++i) {
      // ---- memory phase of step i
      sched_fence();
      const int8_t* cur = smem + ((ph + i) % S) * C::kStage;
#pragma unroll
      for (int q = 0; q < C::FM; ++q) f.x[q] = load_frag<C>(cur, lx + q * C::MF * C::BK);
#pragma unroll
      for (int q = 0; q < C::FN; ++q) f.w[q] = load_frag<C>(cur, lw + q * C::MF * C::BK);
      if constexpr (EPI) {
        if (i == 0 && grp == 0) stage_epilogue_vectors<C>(a, epi, m0, n0, wv, ln);
      }
      {
        const int rs = i + S - 1;  // refill: stage rs, into the buffer stage i - 1 used
        int8_t* dst = smem + ((ph + rs) % S) * C::kStage;
        if constexpr (C::BN > 256) {
          // one call site (scalar selects): on the 256 x 384 tile the three
          // cases' load addresses overflowed the scalar registers, and the
          // spill's reload made the compiler drain every load at each tile's
          // first k-steps
          const bool own = rs < KST, nxt = !own && more;
          ld.template issue_part_at<0, L>(nxt ? n1 : n0, nxt ? m1 : m0,
                                          own ? rs : (nxt ? rs - KST : KST - 1), dst, wv, ln);
        } else {
          if (rs < KST)
            ld.template issue_part_at<0, L>(n0, m0, rs, dst, wv, ln);
          else if (more)
            ld.template issue_part_at<0, L>(n1, m1, rs - KST, dst, wv, ln);
          else
            ld.template issue_part_at<0, L>(n0, m0, KST - 1, dst, wv, ln);
        }
      }
      const bool xst = stored && i <= S - 3;  // previous epilogue's stores after stage i + 1
      if (grp == 1) {
        if (xst) wait_vm<(S - 2) * L + kStores>(); else wait_vm<(S - 2) * L>();
      }
      block_barrier();
      // ---- compute phase of step i
      sched_fence();
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int fi = 0; fi < C::FN; ++fi)
#pragma unroll
        for (int fj = 0; fj < C::FM; ++fj) acc[fi][fj] = C::Op::run(f.w[fi], f.x[fj], acc[fi][fj]);
      __builtin_amdgcn_s_setprio(0);
      sched_fence();
      if (grp == 0) {
        if (xst) wait_vm<(S - 2) * L + kStores>(); else wait_vm<(S - 2) * L>();
      }
      block_barrier();
    }
    ph = (ph + KST) % S;
    // after the last tile the repeated stages must land before the
    // workgroup's LDS is released
    if (!more) wait_vm0();
    int ln2 = lane, wv2 = wave;
    asm volatile("" : "+v"(ln2), "+s"(wv2));
    if constexpr (OUT_I32)
      epilogue<C, true, false>(a, m0, n0, wv2 % C::WN, wv2 / C::WN, ln2, acc);
    else
      epilogue_fast<C, EPI, GELU>(a, m0, n0, wv2 % C::WN, wv2 / C::WN, ln2, acc, epi);
    stored = true;
    par ^= 1;
    if (!more) break;
    t = tnext;
    m0 = m1;
    n0 = n1;
  }
  // group 1 passed one barrier more than group 0
  if (grp == 0) block_barrier();
}

// Ping-pong over K (configuration 15, the 1024px down-projection).  Two groups
// of four waves each hold the whole BM x BN tile (wave tiles TM x TN, as in
// the 4-wave kernel) and take alternate k-steps: interval t is group t % 2's
// memory phase for k-step t (its fragment reads, and its refill of stage
// t + S - 1 into the buffer stage t - 1 used) while the other group runs the
// MFMAs of k-step t - 1.  The ring has an odd number of stages S, so the group
// that refills a buffer is the group that reads it next and each wave waits
// for its own loads only.  At the end of a tile (no chaining: every load is
// drained) group 1 hands its partial sums to group 0 through LDS, and group 0
// writes the epilogue.  Shapes of whole tiles with K a multiple of 2 BK and at
// least 4 BK; int32 sums are exact, so the output bits equal the 4-wave
// kernel's.
template <class C>
__global__ __launch_bounds__(2 * C::kThreads) void gemm_ppk_kernel(GemmArgs a, int T, int MTi, int NTi) {
  static_assert(C::kWaves == 4 && C::WN == 2 && C::kSteps == 1 && C::MF == 16 && C::kEpiLds &&
                C::STAGES % 2 == 1 && C::FM % 2 == 0, "K-split ping-pong tile");
  constexpr int S = C::STAGES;
  constexpr int L = C::kLoadsPerWave;
  static_assert(4 * C::FN * 2 * 1024 <= S * C::kStage, "exchange area");
  __shared__ __attribute__((aligned(1024))) int8_t smem[S * C::kStage + C::kEpiBytes];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int grp = wave / 4, w4 = wave % 4;
  const int wm = w4 / C::WN, wn = w4 % C::WN;
  int t = blockIdx.x;
  if (t >= T) return;
  const int KST = static_cast<int>(a.K / C::BK);  // even, >= 4 (host)
  const int KH = KST / 2;
  // fragment addresses: lx per lane; the weight fragments sit a uniform
  // distance below (one register fewer across the K loop)
  uint32_t lx;
  {
    const int fr = lane % C::MF, fq = lane / C::MF;
    const uint32_t l = static_cast<uint32_t>(fr * C::BK + swz<C::kSlots, C::kSwzR1>(fr, piece_chunk<C::MF, false, C::kSwzR1>(fq, 0)) * 16);
    lx = l + static_cast<uint32_t>(C::BN * C::BK + wm * C::TM * C::BK);
  }
  const uint32_t dwx = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(C::BN * C::BK + wm * C::TM * C::BK - wn * C::TN * C::BK));
  typename C::Acc acc[C::FN][C::FM];
  Frags<C> f;
  for (; t < T; t += static_cast<int>(gridDim.x)) {
    int tm, tn;
    // groups of 4 M-tiles: on the 1024px down-projection (16 x 16 tiles, one
    // per workgroup) each XCD takes a 4 x 8 block, whose 4 activation and 8
    // weight panels (31.5 MB at K = 12288) are fewer bytes than the 8 x 4
    // block's (34.6 MB); measured 2% faster than groups of 8, same bits
    tile_coords<4>(t, T, MTi, NTi, tm, tn);
    const int64_t m0 = static_cast<int64_t>(tm) * C::BM, n0 = static_cast<int64_t>(tn) * C::BN;
    // stage loads: block j of a stage (as in Loader) from two scalar bases,
    // the row and k offsets added per load (no per-block 64-bit addresses
    // kept across the K loop)
    const global_i8* bw = sgpr_gptr(a.qw + n0 * a.K);
    const global_i8* bx = sgpr_gptr(a.qx + m0 * a.K);
    auto dma = [&](int st, int8_t* dst) {
      // the lane's offset, recomputed per call (not kept across the K loop)
      int lnr = lane;
      asm volatile("" : "+v"(lnr));
      const uint32_t loff = static_cast<uint32_t>((lnr / C::kSlots) * a.K +
                                                  swz<C::kSlots, C::kSwzR1>(lnr / C::kSlots, lnr % C::kSlots) * 16);
#pragma unroll
      for (int jj = 0; jj < L; ++jj) {
        const int j = w4 + jj * C::kWaves;
        constexpr int KWB = C::BN / C::kRowsPerLoad / C::kWaves;
        const bool is_w = jj < KWB;  // compile-time after unrolling
        const int row0 = is_w ? j * C::kRowsPerLoad : j * C::kRowsPerLoad - C::BN;
        uint32_t off = loff + static_cast<uint32_t>(row0 * a.K + st * C::BK);
        asm volatile("" : "+v"(off));
        __builtin_amdgcn_global_load_lds((is_w ? bw : bx) + off, (lds_void*)(dst + j * 1024), 16, 0, 0);
      }
    };
    // prologue: this group's stages grp and grp + 2 (of the first S - 1)
#pragma unroll
    for (int p = 0; p < (S - 1) / 2; ++p) {
      const int st = grp + 2 * p;
      dma(st < KST ? st : KST - 1, smem + __builtin_amdgcn_readfirstlane((st % S) * C::kStage));
    }
    wait_vm<((S - 1) / 2 - 1) * L>();  // this wave's first stage
    block_barrier();                    // everyone's
    if (grp == 1) block_barrier();      // group 1 runs one interval behind
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
      for (int j = 0; j < C::FM; ++j) acc[i][j] = typename C::Acc{};
    for (int i = 0; i < KH; ++i) {
      const int j = 2 * i + grp;  // this group's k-step
      // ---- memory phase
      sched_fence();
      // buffer offsets as scalars: computed as vector values they took the
      // registers the K loop does not have
      const int8_t* cur = smem + __builtin_amdgcn_readfirstlane((j % S) * C::kStage);
#pragma unroll
      for (int q = 0; q < C::FM; ++q) f.x[q] = load_frag<C>(cur, lx + q * C::MF * C::BK);
#pragma unroll
      for (int q = 0; q < C::FN; ++q) f.w[q] = load_frag<C>(cur, lx - dwx + q * C::MF * C::BK);
      if (i == 0 && grp == 0) stage_epilogue_vectors<C>(a, smem, m0, n0, w4, lane);
      {
        const int rs = j + S - 1;  // this group's stage, into the buffer stage j - 1 used
        dma(rs < KST ? rs : KST - 1, smem + __builtin_amdgcn_readfirstlane((rs % S) * C::kStage));
      }
      block_barrier();
      // ---- compute phase
      sched_fence();
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int fi = 0; fi < C::FN; ++fi)
#pragma unroll
        for (int fj = 0; fj < C::FM; ++fj) acc[fi][fj] = C::Op::run(f.w[fi], f.x[fj], acc[fi][fj]);
      __builtin_amdgcn_s_setprio(0);
      sched_fence();
      // this group's next stage (j + 2, issued one own step earlier) landed
      wait_vm<((S - 1) / 2 - 1) * L>();
      block_barrier();
    }
    if (grp == 0) block_barrier();  // group 1 passed one barrier more
    wait_vm0();                     // the trailing repeated stages
    block_barrier();
    // group 1 hands its partial sums to group 0 (the wave at the same tile
    // position) through LDS, two activation blocks at a time
#pragma unroll
    for (int r = 0; r < C::FM / 2; ++r) {
      if (grp == 1) {
        v4i* mine = reinterpret_cast<v4i*>(smem + w4 * (C::FN * 2 * 1024));
#pragma unroll
        for (int fi = 0; fi < C::FN; ++fi)
#pragma unroll
          for (int fj = 0; fj < 2; ++fj)
            mine[(fi * 2 + fj) * 64 + lane] = __builtin_bit_cast(v4i, acc[fi][2 * r + fj]);
      }
      block_barrier();
      if (grp == 0) {
        const v4i* theirs = reinterpret_cast<const v4i*>(smem + w4 * (C::FN * 2 * 1024));
#pragma unroll
        for (int fi = 0; fi < C::FN; ++fi)
#pragma unroll
          for (int fj = 0; fj < 2; ++fj) {
            const v4i o = theirs[(fi * 2 + fj) * 64 + lane];
            acc[fi][2 * r + fj] += __builtin_bit_cast(typename C::Acc, o);
          }
      }
      block_barrier();
    }
    if (grp == 0) {
      int ln2 = lane, wv2 = w4;
      asm volatile("" : "+v"(ln2), "+s"(wv2));
      epilogue_fast<C, true>(a, m0, n0, wv2 % C::WN, wv2 / C::WN, ln2, acc, smem);
    }
    block_barrier();  // the epilogue vectors and stages are free again
  }
}

// ----------------------------------------------------------- few tokens --
// A GEMM with a handful of token rows is bound by streaming the weights from
// HBM once (M = 1 .. 16: 2 .. 32 ops per weight byte).  Each workgroup owns
// NB blocks of 16 output columns and MB blocks of 16 token rows; its NW waves
// split K, each loading its weight and activation fragments straight into
// registers (ST 64-byte K steps in flight per wave -- or two chunks of ST
// steps, one loading while the other multiplies (PIPE) -- no LDS staging),
// accumulating with v_mfma_i32_16x16x64_i8, then the waves' partial sums
// meet in LDS and the MB x NB result blocks are shared out over the waves
// for the reduction and the epilogue.  grid.y covers M in steps of 16 x MB
// rows, so any M works.  MB = 1 is the few-row kernel proper; MB = 4 (64
// rows) serves a few hundred tokens, where the tiled kernel's large tiles
// would leave most CUs idle: 64 x 48 blocks make 256 workgroups of a
// 256 x 3072 output.  The int8 configurations load coalesced (COAL, below)
// and permute into the MFMA layout: loaded in that layout, every four
// consecutive lanes read four different rows, which measured 5-9% slower on
// the weight-streaming shapes (1 and 16 rows) and 1.8x slower at 256 rows
// than the coalesced load plus the permute.
//   MFMA 16x16x64 layout: lane l holds row l % 16 of a 16-row operand, K
//   bytes 16 (l / 16) .. +15 of a 64-byte step; D[i][j] (i: weight row n,
//   j: token m) sits in lane j + 16 (i / 4), register i % 4.
//   FP8 operands: v_mfma_scale_f32_16x16x128_f8f6f4 (unit block scales), a
//   128-byte K step, lane l holding 32 bytes (two 16-byte loads) of row l % 16
//   at K bytes 32 (l / 16) .. +31, fp32 accumulators, same result layout.
// A 16-byte fragment moved between lanes: lane d receives the fragment of
// lane perm / 4 (perm: byte address as ds_bpermute takes it).
__device__ __forceinline__ v4i to_mfma_layout(v4i v, int perm) {
  v4i o;
  o[0] = __builtin_amdgcn_ds_bpermute(perm, v[0]);
  o[1] = __builtin_amdgcn_ds_bpermute(perm, v[1]);
  o[2] = __builtin_amdgcn_ds_bpermute(perm, v[2]);
  o[3] = __builtin_amdgcn_ds_bpermute(perm, v[3]);
  return o;
}

template <int NW, int NB, bool OUT_I32, int ST, bool LOOP, bool FP8 = false, int MB = 1,
          bool COAL = false, bool PIPE = false>
__global__ __launch_bounds__(64 * NW) void gemm_few_rows(GemmArgs a) {
  static_assert(!(FP8 && OUT_I32), "FP8 products accumulate in fp32: bf16 output only");
  static_assert(!(FP8 && COAL), "coalesced loads: int8 operands");
  using Frag = std::conditional_t<FP8, v8i, v4i>;
  using Acc = std::conditional_t<FP8, v4f, v4i>;
  constexpr int SB = FP8 ? 128 : 64;  // K bytes of one MFMA
  constexpr int PB = SB / 4;          // K bytes one lane supplies per step
  constexpr int NBLK = MB * NB;       // result blocks of the workgroup
  __shared__ Acc part[NW][NBLK][64];
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int64_t M = a.M, N = a.N, K = a.K;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16 * NB;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 16 * MB;
  const int r = lane % 16, kq = lane / 16;
  // COAL: each lane loads row lane / 4, piece lane % 4 (four consecutive lanes
  // read one 64-byte run of a row; the instruction reads the same 16 rows x
  // 64 bytes as in the MFMA layout), and a ds_bpermute then moves every
  // fragment into the MFMA layout above (lane d takes lane 4 (d % 16) +
  // d / 16's piece)
  const int lr = COAL ? lane / 4 : r, lq = COAL ? lane % 4 : kq;
  const int perm = 4 * (4 * (lane % 16) + lane / 16);  // bpermute byte address
  const int64_t steps = (K + SB - 1) / SB;
  const int64_t per = (steps + NW - 1) / NW;
  const int64_t s0 = wave * per, s1 = min(steps, s0 + per);
  const int8_t* xrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t mr = m0 + 16 * mb + lr;
    xrow[mb] = a.qx + (mr < M ? mr : 0) * K;
  }
  const int8_t* wrow[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int64_t nr = n0 + 16 * b + lr;
    wrow[b] = a.qw + (nr < N ? nr : 0) * K;
  }
  // The epilogue's scales and biases are loaded first, so that their latency
  // hides behind the weight stream instead of following it.
  // (Indices are clamped rather than tested, so that the loads are
  // unconditional and all go out before the first wait.)
  float sxe[MB], swe[NB][4];
  uint32_t braw[NB][4];  // bf16 bias bits, widened in the epilogue
  // (Every wave loads them all, though each uses only its own blocks': a
  // branch here would make the waits after it conservative.)
  if constexpr (!OUT_I32) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) sxe[mb] = a.sx[min(m0 + 16 * mb + lane % 16, M - 1)];
    // no bias: read any valid 16-bit word, replaced by -0.0 in the epilogue
    const uint16_t* bsrc = a.bias ? a.bias : reinterpret_cast<const uint16_t*>(a.sw);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t n = min(n0 + 16 * b + 4 * (lane / 16) + e, N - 1);
        swe[b][e] = a.sw[n];
        braw[b][e] = bsrc[n];
      }
  }
  Acc acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[mb][b] = Acc{};
  // one lane's operand at K byte k of a row (kc2: its second 16-byte piece,
  // clamped into the row when it lies past K)
  auto load_op = [&](const int8_t* row, int64_t kc, int64_t kc2) {
    if constexpr (FP8) {
      const v4i lo = *reinterpret_cast<const v4i*>(row + kc);
      const v4i hi = *reinterpret_cast<const v4i*>(row + kc2);
      return Frag(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      (void)kc2;
      return Frag(*reinterpret_cast<const v4i*>(row + kc));
    }
  };
  // The loads of ST steps from step c0 (addresses clamped into the operands
  // past the wave's share or past K): loads only, since a test on loaded
  // data here would make each load wait for the one before.  Rows beyond M
  // or N only feed outputs that are never stored, so they need no zeroing.
  auto load_chunk = [&](int64_t c0, Frag (&xf)[ST][MB], Frag (&wf)[ST][NB]) {
#pragma unroll
    for (int i = 0; i < ST; ++i) {
      const int64_t k = (c0 + i) * SB + lq * PB;  // this lane's load
      const bool in = (c0 + i) < s1 && k < K;
      const int64_t kc = in ? k : 0;
      const int64_t kc2 = (in && k + 16 < K) ? k + 16 : kc;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) xf[i][mb] = load_op(xrow[mb], kc, kc2);
#pragma unroll
      for (int b = 0; b < NB; ++b) wf[i][b] = load_op(wrow[b], kc, kc2);
      __builtin_amdgcn_sched_barrier(0);  // issue order = step order
    }
  };
  // The products of those steps (steps past the share skipped).
  auto mma_chunk = [&](int64_t c0, Frag (&xf)[ST][MB], Frag (&wf)[ST][NB]) {
#pragma unroll
    for (int i = 0; i < ST; ++i) {
      if (c0 + i >= s1) break;  // wave-uniform
      // the 16-byte pieces of a step past K (K not a multiple of SB) are zeroed
      const int64_t k = (c0 + i) * SB + kq * PB;  // the piece this lane multiplies
      if constexpr (COAL) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) xf[i][mb] = to_mfma_layout(xf[i][mb], perm);
#pragma unroll
        for (int b = 0; b < NB; ++b) wf[i][b] = to_mfma_layout(wf[i][b], perm);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        Frag xv = xf[i][mb];
        if (!(k < K)) xv = Frag{};
        if constexpr (FP8) {
          if (!(k + 16 < K)) xv = __builtin_shufflevector(xv, Frag{}, 0, 1, 2, 3, 12, 13, 14, 15);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if constexpr (FP8)
            acc[mb][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[i][b], xv, acc[mb][b], 0,
                                                                         0, 0, 127, 0, 127);
          else
            acc[mb][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[i][b], xv, acc[mb][b], 0, 0, 0);
        }
      }
    }
  };
  // (An empty share -- K == 0, or more waves than 64-byte steps -- loads
  // nothing: with K == 0 the operand pointers need not be valid.)
  if constexpr (PIPE) {
    // Two chunk buffers: the next chunk's loads are in flight while this
    // one's products run (the loads past the share are clamped, unused).
    // With 64-row blocks (7 fragments a step) one step per chunk measured
    // 7% faster than the whole share in flight at once (14.8 against
    // 15.9 us at M = 256, N = K = 3072); chunks without the overlap, 15.1.
    if (s0 < s1) {
      Frag xa[ST][MB], wa[ST][NB], xb[ST][MB], wb[ST][NB];
      load_chunk(s0, xa, wa);
      for (int64_t c0 = s0; c0 < s1; c0 += 2 * ST) {
        __builtin_amdgcn_sched_barrier(0);
        load_chunk(c0 + ST, xb, wb);
        __builtin_amdgcn_sched_barrier(0);
        mma_chunk(c0, xa, wa);
        __builtin_amdgcn_sched_barrier(0);
        if (c0 + ST >= s1) break;  // wave-uniform
        load_chunk(c0 + 2 * ST, xa, wa);
        __builtin_amdgcn_sched_barrier(0);
        mma_chunk(c0 + ST, xb, wb);
      }
    }
  } else if constexpr (LOOP) {
    // chunks one after the other (shares longer than ST steps)
    for (int64_t c0 = s0; c0 < s1; c0 += ST) {
      Frag xf[ST][MB], wf[ST][NB];
      load_chunk(c0, xf, wf);
      __builtin_amdgcn_sched_barrier(0);
      mma_chunk(c0, xf, wf);
    }
  } else {
    // the whole share in one chunk, every load in flight before the first
    // product; straight code (a loop header would make the waits inside it
    // conservative)
    if (s0 < s1) {
      Frag xf[ST][MB], wf[ST][NB];
      load_chunk(s0, xf, wf);
      __builtin_amdgcn_sched_barrier(0);
      mma_chunk(s0, xf, wf);
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int b = 0; b < NB; ++b) part[wave][mb * NB + b][lane] = acc[mb][b];
  __syncthreads();
  // result block j (row block j / NB, column block j % NB) goes to wave j % NW
  const int nq = 4 * (lane / 16);
#pragma unroll
  for (int j = 0; j < NBLK; ++j) {
    if (j % NW != wave) continue;  // wave-uniform
    const int mb = j / NB, b = j % NB;
    const int64_t m = m0 + 16 * mb + lane % 16;
    if (m >= M) continue;
    Acc t = part[0][j][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) t += part[w][j][lane];
    const int64_t nb = n0 + 16 * b + nq;
    if constexpr (OUT_I32) {
      int32_t* out = static_cast<int32_t*>(a.out) + m * N + nb;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (nb + e < N) out[e] = static_cast<int32_t>(t[e]);
    } else {
      uint16_t* out = static_cast<uint16_t*>(a.out) + m * N + nb;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float bv = a.bias ? __uint_as_float(braw[b][e] << 16) : -0.0f;
        v[e] = dequant(t[e], sxe[mb], swe[b][e], bv);
      }
      if (N % 4 == 0 && nb + 3 < N) {
        // the lane's 4 columns in one 8-byte store (rows start 8-byte aligned)
        *reinterpret_cast<uint2*>(out) = make_uint2(bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3]));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (nb + e < N) out[e] = static_cast<uint16_t>(bf16_bits(v[e]));
      }
    }
  }
}

// ------------------------------------------- few tokens, fused quantize --
// The whole fused linear for M <= 16 token rows in one launch.  Each
// workgroup owns 16 output columns; its 4 or 8 waves split K for the MFMAs
// as in gemm_few_rows.  Before them, the workgroup quantizes the M x K
// activations itself, one wave per row as the row quantizer does (wave w
// takes rows w, w + NW, ...): each lane loads 16-byte chunks lane,
// lane + 64, ... of the row, the wave reduces the row's absmax with
// cross-lane maxima, and the codes, computed with the row quantizer's own
// operations (quant_codes.h, the same bits w8a8_quantize_act writes), go
// into an LDS copy of the codes; each lane then reads its MFMA operand from
// there.  The activations are
// loaded before the weight fragments (loads complete in issue order), so
// they are quantized while the weights stream in.  Every workgroup reads all
// of x (at most 16 x 3072 bf16, L2-resident after the first), in place of a
// separate quantize launch and the gap before the GEMM's.  Column block 0
// also writes the codes and scales to the workspace, as the two-launch path
// does.
// LDS copy of the codes: row stride K + 16 bytes, so that the 16 rows of a
// fragment read fall in 16 different 16-byte bank groups.
constexpr int kRowsMaxK = 3072;  // codes of 16 rows of up to this K fit the LDS copy
// Every workgroup quantizes all M rows, so the redundant work grows with M
// and with the number of column blocks: the single launch is taken for up to
// 16 rows while there are no more column blocks than CUs, up to 12 above
// (measured against the two launches at K = 3072: M = 4, N = 3072 9.2 ->
// 7.8 us, N = 18432 20.2 -> 16.9 us; M = 8 11.2 -> 8.4 and 20.8 -> 19.6 us;
// M = 12 11.8 -> 8.7 and 23.4 -> 21.8 us; M = 16, N = 3072 12.2 -> 10.5 us,
// N = 18432 25.2 -> 25.1 us, FP8 24.3 -> 27.8 us).
constexpr int kRowsMaxM = 16;
constexpr int kRowsMaxMWide = 12;  // above kNumCU column blocks
// FP8: the fp32 partial sums of the K shares are added in wave order, so the
// single launch gives the two-launch path's bits only with the same 4-wave K
// split: 4 waves (two rows each above 4 rows), up to 8 rows (measured against
// the two launches at K = 3072: M = 8, N = 3072 11.4 -> 9.9 us, N = 18432
// 21.4 -> 21.0 us).
constexpr int kRowsMaxMFp8 = 8;
// K runs in 128-byte steps; lane l holds 32 bytes of row l % 16, K bytes
// 32 (l / 16) .. +31 of a step (two 16-byte loads straight from the row).
// int8: each step is two v_mfma_i32_16x16x64_i8, one on every lane's first
// 16 bytes and one on its second (the K positions of an int32 sum may be
// split among MFMAs in any way both operands share); measured 5-8% faster
// than 64-byte steps loaded coalesced and permuted into the MFMA layout.
// FP8: e4m3 codes (scale absmax / 448) and one
// v_mfma_scale_f32_16x16x128_f8f6f4 per step, fp32 partial sums added in
// wave order; the weights are loaded and the pieces past K zeroed exactly as
// the FP8 few-row GEMM does, so the output is the same bits as the two-launch
// path (e4m3 quantizer + FP8 few-row GEMM).
// Rows over the NW waves: WPR waves share a row when there are fewer rows
// than waves (each wave a 64-lane slice of every 64 WPR chunks, maxima
// joined in LDS); otherwise wave w takes rows w, w + NW, ... (RPW of them).
template <int WPR, int RPW, int ST, bool FP8 = false, int NW = 4>
__global__ __launch_bounds__(64 * NW) void linear_few_rows(RowsArgs a) {
  static_assert(WPR == 1 || RPW == 1, "shared rows: one per wave group");
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int SB = 128;  // K bytes of one step
  constexpr int PB = 32;   // K bytes of one lane's operand in a step
  // chunks of a row per lane: NW ST 128-byte steps cover K, so a row's K / 8
  // chunks are at most 64 ST NW / 4
  constexpr int CHR = (ST * NW / 4 + WPR - 1) / WPR;
  using Acc = std::conditional_t<FP8, v4f, v4i>;
  constexpr int ROWS = NW / WPR * RPW;  // rows this launch shape holds (>= M)
  static_assert(ROWS <= 16, "one 16-row MFMA block");
  __shared__ __attribute__((aligned(16))) int8_t codes[ROWS * (kRowsMaxK + 16)];
  __shared__ Acc part[NW][64];
  __shared__ float srow[16];
  __shared__ float wmax[NW];
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int64_t M = a.M, N = a.N, K = a.K;
  const int64_t ldc = K + 16;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int r = lane % 16, kq = lane / 16;
  const int64_t steps = (K + SB - 1) / SB;
  const int64_t per = (steps + NW - 1) / NW;
  const int64_t s0 = wave * per, s1 = min(steps, s0 + per);
  // epilogue scales and bias (clamped columns past N)
  float swe[4];
  uint32_t braw[4];
  {
    const uint16_t* bsrc = a.bias ? a.bias : reinterpret_cast<const uint16_t*>(a.sw);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t n = min(n0 + 4 * kq + e, N - 1);
      swe[e] = a.sw[n];
      braw[e] = bsrc[n];
    }
  }
  // this wave's rows (row g + (NW / WPR) i, where it exists): chunks
  // li + 64 WPR j of each (li: the lane's place in its row's WPR waves),
  // clamped past the row's end to its last chunk (a copy of real elements,
  // which leaves the absmax unchanged; its codes are not stored)
  const int ck = static_cast<int>(K / 8);  // chunks per row, <= 64 ST
  const int g = wave / WPR;
  const int li = (wave % WPR) * 64 + lane;
  uint4 xv[RPW][CHR];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int row = g + (NW / WPR) * i;
    if (row >= M) break;  // wave-uniform
    const uint4* src = reinterpret_cast<const uint4*>(a.x) + static_cast<int64_t>(row) * ck;
#pragma unroll
    for (int j = 0; j < CHR; ++j) {
      const int c = li + 64 * WPR * j;
      xv[i][j] = src[c < ck ? c : ck - 1];
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the weight pieces of this wave's K share (past the share or past K:
  // clamped into the row, and met by zeroed activation pieces)
  const int8_t* wrow = a.qw + min(n0 + r, N - 1) * K;
  v8i wf[ST];
#pragma unroll
  for (int i = 0; i < ST; ++i) {
    const int64_t k = (s0 + i) * SB + kq * PB;
    const bool in = (s0 + i) < s1 && k < K;
    const int64_t kc = in ? k : 0;
    const int64_t kc2 = (in && k + 16 < K) ? k + 16 : kc;
    const v4i lo = *reinterpret_cast<const v4i*>(wrow + kc);
    const v4i hi = *reinterpret_cast<const v4i*>(wrow + kc2);
    wf[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    __builtin_amdgcn_sched_barrier(0);
  }
  // per row: absmax (the magnitude bits of the largest element: non-negative
  // values order as their bit patterns), scale, codes into the LDS copy
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int row = g + (NW / WPR) * i;
    float amax = 0.0f;
    if (row < M) {  // wave-uniform
      u16x2 m2 = {0, 0};
#pragma unroll
      for (int j = 0; j < CHR; ++j)
        m2 = absmax2(absmax2(absmax2(absmax2(m2, xv[i][j].x), xv[i][j].y), xv[i][j].z), xv[i][j].w);
      amax = wave_max(absmax_of(m2));
    }
    if constexpr (WPR > 1) {
      // the row's maxima from its WPR waves (every wave passes the barrier)
      if (lane == 0) wmax[wave] = amax;
      __syncthreads();
#pragma unroll
      for (int v = 0; v < WPR; ++v) amax = fmaxf(amax, wmax[g * WPR + v]);
    }
    if (row >= M) break;  // wave-uniform
    const float s = amax / kCodeMax<FP8>;
    if (lane == 0 && wave % WPR == 0) {
      srow[row] = s;
      if (blockIdx.x == 0 && a.sx_out != nullptr) a.sx_out[row] = s;
    }
    const int mode = s >= kFastMinScale ? 2 : (s != 0.0f ? 1 : 0);
    const float rs = mode == 2 ? 1.0f / s : 0.0f;
    int8_t* crow = codes + row * ldc;
    int8_t* qrow = a.qx_out + static_cast<int64_t>(row) * K;
    const bool out_codes = blockIdx.x == 0 && a.qx_out != nullptr;
#pragma unroll
    for (int j = 0; j < CHR; ++j) {
      const int c = li + 64 * WPR * j;
      if (c < ck) {
        uint2 p = make_uint2(0u, 0u);
        if (mode == 2)
          p = codes_bf16x8<2, FP8>(xv[i][j], s, rs);
        else if (mode == 1)
          p = codes_bf16x8<1, FP8>(xv[i][j], s, 0.0f);
        *reinterpret_cast<uint2*>(crow + c * 8) = p;
        if (out_codes) *reinterpret_cast<uint2*>(qrow + c * 8) = p;
      }
    }
  }
  __syncthreads();
  // MFMAs over the wave's K share; rows past M read row M - 1 of the copy
  const int8_t* crow_l = codes + min<int64_t>(r, M - 1) * ldc;
  Acc acc = {};
#pragma unroll
  for (int i = 0; i < ST; ++i) {
    if (s0 + i >= s1) break;  // wave-uniform
    const int64_t k = (s0 + i) * SB + kq * PB;
    // pieces past K are zero (the copy's row padding is never used)
    v4i lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
    if (k < K) lo = *reinterpret_cast<const v4i*>(crow_l + k);
    if (k + 16 < K) hi = *reinterpret_cast<const v4i*>(crow_l + k + 16);
    if constexpr (FP8) {
      const v8i xq = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[i], xq, acc, 0, 0, 0, 127, 0, 127);
    } else {
      const v4i wlo = __builtin_shufflevector(wf[i], wf[i], 0, 1, 2, 3);
      const v4i whi = __builtin_shufflevector(wf[i], wf[i], 4, 5, 6, 7);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wlo, lo, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(whi, hi, acc, 0, 0, 0);
    }
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave != 0 || r >= M) return;
  Acc tt = part[0][lane];
#pragma unroll
  for (int w = 1; w < NW; ++w) tt += part[w][lane];
  const float s = srow[r];
  const int64_t nb = n0 + 4 * kq;
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float bv = a.bias ? __uint_as_float(braw[e] << 16) : -0.0f;
    v[e] = dequant(tt[e], s, swe[e], bv);
  }
  uint16_t* out = a.y + r * N + nb;
  if (N % 4 == 0 && nb + 3 < N) {
    *reinterpret_cast<uint2*>(out) = make_uint2(bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3]));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (nb + e < N) out[e] = static_cast<uint16_t>(bf16_bits(v[e]));
  }
}

template <int NW, int NB, bool I32, int ST, bool LOOP = false, bool FP8 = false, int MB = 1,
          bool COAL = false, bool PIPE = false>
hipError_t launch_few_rows_st(const GemmArgs& a, hipStream_t stream) {
  const int64_t gx = (a.N + 16 * NB - 1) / (16 * NB), gy = (a.M + 16 * MB - 1) / (16 * MB);
  if (gx > INT32_MAX || gy > 65535) return hipErrorInvalidValue;
  gemm_few_rows<NW, NB, I32, ST, LOOP, FP8, MB, COAL, PIPE>
      <<<dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)), dim3(64 * NW), 0, stream>>>(a);
  return hipGetLastError();
}

// Steps in flight per wave: the smallest of 1, 2, 3, 4, 6, 8, 12 (at most
// STMAX, which bounds the fragment registers) that covers the wave's share
// of K (no load is wasted on a step past the share), else a loop of
// STLOOP-step chunks (the loop's own registers leave room for fewer).
template <int NW, int NB, bool I32, bool FP8 = false, int MB = 1, int STMAX = 12,
          int STLOOP = STMAX, bool COAL = false>
hipError_t launch_few_rows(const GemmArgs& a, hipStream_t stream) {
  constexpr int64_t SB = FP8 ? 128 : 64;
  const int64_t per = ((a.K + SB - 1) / SB + NW - 1) / NW;
#define W8A8_ST_CASE(STV)                                                                   \
  if constexpr (STV <= STMAX) {                                                             \
    if (per <= STV) return launch_few_rows_st<NW, NB, I32, STV, false, FP8, MB, COAL>(a, stream); \
  }
  W8A8_ST_CASE(1) W8A8_ST_CASE(2) W8A8_ST_CASE(3) W8A8_ST_CASE(4) W8A8_ST_CASE(6)
  W8A8_ST_CASE(8) W8A8_ST_CASE(12)
#undef W8A8_ST_CASE
  return launch_few_rows_st<NW, NB, I32, STLOOP, true, FP8, MB, COAL>(a, stream);
}

template <int WPR, int RPW, int ST, bool FP8, int NW = 4>
hipError_t launch_linear_few_rows_st(const RowsArgs& a, hipStream_t stream) {
  const int64_t gx = (a.N + 15) / 16;
  if (gx > INT32_MAX) return hipErrorInvalidValue;
  linear_few_rows<WPR, RPW, ST, FP8, NW>
      <<<dim3(static_cast<unsigned>(gx)), dim3(64 * NW), 0, stream>>>(a);
  return hipGetLastError();
}

// 4 waves for up to 4 rows (4 or 2 waves per row for 1 or 2 rows, else one
// row per wave), 8 waves for 5-16 int8 rows (one or two rows per wave, K in
// 8 shares): more waves hide more of the quantization's latency there, but at
// 1-4 rows on wide N the 4-wave form measured faster (M = 1, N = 18432:
// 14.6 against 15.5 us).  FP8 keeps 4 waves (two rows each for 5-8 rows).
template <int ST, bool FP8>
hipError_t launch_linear_few_rows_w4(const RowsArgs& a, hipStream_t stream) {
  if (a.M == 1) return launch_linear_few_rows_st<4, 1, ST, FP8>(a, stream);
  if (a.M == 2) return launch_linear_few_rows_st<2, 1, ST, FP8>(a, stream);
  if (a.M <= 4) return launch_linear_few_rows_st<1, 1, ST, FP8>(a, stream);
  if (FP8 && a.M <= kRowsMaxMFp8) return launch_linear_few_rows_st<1, 2, ST, FP8>(a, stream);
  return hipErrorInvalidValue;
}
template <int ST, bool FP8>
hipError_t launch_linear_few_rows_w8(const RowsArgs& a, hipStream_t stream) {
  if (a.M <= 8) return launch_linear_few_rows_st<1, 1, ST, FP8, 8>(a, stream);
  if (a.M <= 16) return launch_linear_few_rows_st<1, 2, ST, FP8, 8>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_few_rows_any(const GemmArgs& a, bool i32, hipStream_t stream) {
  return i32 ? launch_few_rows<4, 1, true, false, 1, 12, 12, true>(a, stream)
             : launch_few_rows<4, 1, false, false, 1, 12, 12, true>(a, stream);
}

// ------------------------------------------------------- configurations --
struct ConfigInfo {
  const char* name;
  int BM, BN, threads;
  int wg_per_cu;   // workgroups resident per CU (LDS / register bound)
  float rel_speed; // relative per-CU throughput with the chip full
};

//             BM   BN  WM WN  BK  STAGES MFMA
using C0 = Tile<256, 256, 2, 2, 64, 4, 32>;   // 4 waves, wave tile 128 x 128
using C1 = Tile<256, 256, 2, 2, 128, 2, 32>;  // same, 2 deep stages
using C2 = Tile<256, 128, 2, 2, 128, 3, 32>;  // wave tile 128(m) x 64(n), 3 deep stages
using C3 = Tile<128, 256, 2, 2, 128, 3, 32>;  // wave tile 64(m) x 128(n), 3 deep stages
using C4 = Tile<128, 128, 2, 2, 64, 4, 32>;   // wave tile 64 x 64
using C5 = Tile<64, 64, 2, 2, 128, 2, 32>;    // wave tile 32 x 32
using C6 = Tile<16, 64, 1, 4, 128, 2, 16>;    // wave tile 16 x 16 (skinny M)
using C7 = Tile<256, 192, 2, 2, 64, 4, 32>;   // wave tile 128(m) x 96(n)
using C9 = Tile<256, 256, 2, 2, 64, 4, 16>;   // C0 on 16x16x64 blocks, one k-step per stage
using C10 = Tile<256, 192, 2, 2, 64, 4, 16>;  // C7 on 16x16x64 blocks
using C11 = Tile<256, 256, 2, 4, 64, 4, 16>;  // C9 with 8 waves (2 per SIMD), wave tile 128 x 64
using C14 = Tile<256, 384, 2, 4, 64, 3, 16>;  // 8 waves, wave tile 128 x 96, 3 stages of 40 KiB
using C15 = Tile<256, 192, 2, 2, 64, 5, 16>;  // C10's wave tiles, 5 stages, twice the waves (K split)
// configuration 12: C11's tile on the ping-pong kernel (gemm_pp_kernel) for
// interior tiles; its edge tiles, and shapes with K < STAGES x BK, take C11's
// own kernels
// configuration 13: the split-K register kernel (gemm_few_rows) with blocks
// of 64 token rows and 48 columns, for a few hundred tokens: 256 workgroups
// on a 256 x 3072 output, where the tiled kernels' large tiles would leave
// most CUs idle; each wave's K share runs one 64-byte step at a time with
// the next step's loads in flight (PIPE)
// configuration 14: the ping-pong kernel on 256 x 384 tiles (C14): each
// wave's 128 x 96 accumulator tile reads 22% fewer LDS bytes per MFMA than
// C11's 128 x 64 (224 against 192 bytes of fragments for 48 against 32
// MFMAs per k-step), and a tile loads 17% fewer operand bytes per operation;
// it fills the 256 registers two waves per SIMD allow.  Shapes of whole
// tiles (M a multiple of 256, N of 384, K of 64 with at least 3 stages,
// aligned vectors) with bf16 output; anything else, int32 output included,
// takes configuration 12's path.
// configuration 15: the K-split ping-pong kernel (gemm_ppk_kernel) on C10's
// 256 x 192 tile: two groups of four 128 x 96 wave tiles take alternate
// k-steps, so that one wave per SIMD issues MFMAs while the other loads; for
// the 1024px down-projection (one tile per workgroup), a measured choice only

const ConfigInfo kConfigs[] = {
    {"bm256_bn256_bk64_s4_mf32", 256, 256, 256, 1, 0.97f},
    {"bm256_bn256_bk128_s2_mf32", 256, 256, 256, 1, 0.98f},
    {"bm256_bn128_bk128_s3_mf32", 256, 128, 256, 1, 0.85f},
    {"bm128_bn256_bk128_s3_mf32", 128, 256, 256, 1, 0.85f},
    {"bm128_bn128_bk64_s4_mf32", 128, 128, 256, 2, 0.70f},
    {"bm64_bn64_bk128_s2_mf32", 64, 64, 256, 4, 0.40f},
    {"bm16_bn64_bk128_s2_mf16", 16, 64, 256, 4, 0.15f},
    {"bm256_bn192_bk64_s4_mf32", 256, 192, 256, 1, 0.92f},
    {"few_rows_splitk4_mf16", 16, 16, 256, 8, 0.10f},
    {"bm256_bn256_bk64_s4_mf16", 256, 256, 256, 1, 1.00f},
    {"bm256_bn192_bk64_s4_mf16", 256, 192, 256, 1, 0.93f},
    {"bm256_bn256_bk64_s4_mf16_w8", 256, 256, 512, 1, 0.99f},
    {"bm256_bn256_bk64_s4_mf16_pp", 256, 256, 512, 1, 1.05f},
    {"rows64_bn48_splitk8_mf16", 64, 48, 512, 1, 0.30f},
    {"bm256_bn384_bk64_s3_mf16_pp", 256, 384, 512, 1, 1.14f},
    {"bm256_bn192_bk64_s5_mf16_ppk", 256, 192, 512, 1, 0.95f},
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);
constexpr int kSkinny = 6;    // 16-row tiled kernel
constexpr int kFewRows = 8;   // split-K few-row kernel
constexpr int kRowBlocks = 13;  // split-K kernel on 64-row blocks
constexpr int kPpWide = 14;     // 256 x 384 ping-pong tile, whole tiles only
constexpr int kPpK = 15;        // K-split ping-pong on 256 x 192 tiles
constexpr int kNumCU = 256;  // MI355X compute units (tile-wave estimate)

// Persistent grid: as many workgroups of `kernel` as fit on the device at
// once (a multiple of the 8 XCDs), or one per tile if there are fewer tiles.
// The resident count depends only on the device and the kernel, so it is
// asked of the runtime once per (kernel, device) and kept: the occupancy
// query costs microseconds of host time, which the launch-bound small shapes
// would otherwise pay on every call.  (Racing first calls store the same
// value.)
constexpr int kMaxDevices = 64;
template <auto Kernel>
hipError_t persistent_grid(int threads, int64_t tiles, int& grid) {
  static std::atomic<int> cache[kMaxDevices];  // per kernel; 0: not known yet
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int resident = (dev >= 0 && dev < kMaxDevices) ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (resident == 0) {
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, Kernel, threads, 0);
    if (e != hipSuccess) return e;
    int64_t r = static_cast<int64_t>(cus) * (per_cu > 0 ? per_cu : 1);
    r = r >= 8 ? (r / 8) * 8 : r;
    resident = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(r, INT32_MAX)));
    if (dev >= 0 && dev < kMaxDevices) cache[dev].store(resident, std::memory_order_relaxed);
  }
  grid = static_cast<int>(tiles < resident ? tiles : resident);
  return hipSuccess;
}

template <class C, bool I32, bool VEC>
hipError_t launch_interior(const GemmArgs& a, int64_t Ti, int64_t MT, int64_t NT, int64_t MTi,
                           int64_t NTi, hipStream_t stream) {
  int grid = 0;
  hipError_t e = persistent_grid<gemm_kernel<C, I32, false, VEC>>(C::kThreads, Ti, grid);
  if (e != hipSuccess) return e;
  gemm_kernel<C, I32, false, VEC><<<dim3(grid), dim3(C::kThreads), 0, stream>>>(
      a, static_cast<int>(Ti), static_cast<int>(MT), static_cast<int>(NT), static_cast<int>(MTi),
      static_cast<int>(NTi), 0);
  return hipGetLastError();
}

template <class C, bool I32>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
  const int64_t MT = (a.M + C::BM - 1) / C::BM;
  const int64_t NT = (a.N + C::BN - 1) / C::BN;
  if (MT * NT > INT32_MAX) return hipErrorInvalidValue;
  // the interior kernel's conditions: whole stages in K and 16-byte output
  // rows; then every tile wholly inside M and N takes it, and the edge
  // kernel the rest.  Its vector form (VEC) also needs 16-byte aligned s_w
  // and 8-byte aligned bias, and configurations that stage their epilogue
  // vectors in LDS K > 0 and 16-byte aligned s_x and bias (16-byte
  // direct-to-LDS loads); otherwise the interior tiles read the vectors
  // element by element
  const bool epi = C::kEpiLds && !I32;
  const bool interior = (a.N % 8 == 0) && (a.K % C::BK == 0);
  const bool vec = I32 || ((reinterpret_cast<uintptr_t>(a.sw) % 16 == 0) &&
                           (reinterpret_cast<uintptr_t>(a.bias) % 8 == 0) &&
                           (!epi || (a.K > 0 && reinterpret_cast<uintptr_t>(a.sx) % 16 == 0 &&
                                     reinterpret_cast<uintptr_t>(a.bias) % 16 == 0)));
  const int64_t MTi = interior ? a.M / C::BM : 0;
  const int64_t NTi = interior ? a.N / C::BN : 0;
  const int64_t Ti = MTi * NTi;
  const int64_t E = interior ? (MT > MTi ? NT : 0) + (NT > NTi ? MTi : 0) : MT * NT;
  int grid = 0;
  if (Ti > 0) {
    hipError_t e = vec ? launch_interior<C, I32, true>(a, Ti, MT, NT, MTi, NTi, stream)
                       : launch_interior<C, I32, false>(a, Ti, MT, NT, MTi, NTi, stream);
    if (e != hipSuccess) return e;
  }
  if (E > 0) {
    hipError_t e = persistent_grid<gemm_kernel<C, I32, true>>(C::kThreads, E, grid);
    if (e != hipSuccess) return e;
    gemm_kernel<C, I32, true><<<dim3(grid), dim3(C::kThreads), 0, stream>>>(
        a, static_cast<int>(E), static_cast<int>(MT), static_cast<int>(NT), static_cast<int>(MTi),
        static_cast<int>(NTi), interior ? 0 : 1);
    return hipGetLastError();
  }
  return hipSuccess;
}

// Ping-pong launch: interior tiles (whole stages in K, at least STAGES of
// them, aligned vectors) on gemm_pp_kernel, the ragged edge on the tile
// configuration's own edge kernel; shapes that do not meet the interior
// conditions run wholly on the configuration's own kernels.
template <class C, bool I32>
hipError_t launch_pp(const GemmArgs& a, hipStream_t stream) {
  const int64_t MT = (a.M + C::BM - 1) / C::BM;
  const int64_t NT = (a.N + C::BN - 1) / C::BN;
  if (MT * NT > INT32_MAX) return hipErrorInvalidValue;
  const bool epi = C::kEpiLds && !I32;
  const bool interior = (a.N % 8 == 0) && (a.K % C::BK == 0) && (a.K / C::BK >= C::STAGES) &&
                        (reinterpret_cast<uintptr_t>(a.sw) % 16 == 0) &&
                        (reinterpret_cast<uintptr_t>(a.bias) % 8 == 0) &&
                        (!epi || (reinterpret_cast<uintptr_t>(a.sx) % 16 == 0 &&
                                  reinterpret_cast<uintptr_t>(a.bias) % 16 == 0));
  const int64_t MTi = a.M / C::BM, NTi = a.N / C::BN, Ti = MTi * NTi;
  if (!interior || Ti == 0) return launch_cfg<C, I32>(a, stream);
  int grid = 0;
  hipError_t e = persistent_grid<gemm_pp_kernel<C, I32>>(C::kThreads, Ti, grid);
  if (e != hipSuccess) return e;
  gemm_pp_kernel<C, I32><<<dim3(grid), dim3(C::kThreads), 0, stream>>>(
      a, static_cast<int>(Ti), static_cast<int>(MTi), static_cast<int>(NTi));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t E = (MT > MTi ? NT : 0) + (NT > NTi ? MTi : 0);
  if (E > 0) {
    e = persistent_grid<gemm_kernel<C, I32, true>>(C::kThreads, E, grid);
    if (e != hipSuccess) return e;
    gemm_kernel<C, I32, true><<<dim3(grid), dim3(C::kThreads), 0, stream>>>(
        a, static_cast<int>(E), static_cast<int>(MT), static_cast<int>(NT), static_cast<int>(MTi),
        static_cast<int>(NTi), 0);
    return hipGetLastError();
  }
  return hipSuccess;
}

// Configuration 15, bf16 output: the K-split ping-pong kernel when the shape
// is whole 256 x 192 tiles with K a multiple of 128 and at least 256 (and
// aligned vectors), else configuration 10's path (the same output bits).
hipError_t launch_ppk(const GemmArgs& a, hipStream_t stream) {
  using C = C15;
  const bool ok = a.M > 0 && a.N > 0 && a.M % C::BM == 0 && a.N % C::BN == 0 &&
                  a.K % (2 * C::BK) == 0 && a.K >= 4 * C::BK &&
                  reinterpret_cast<uintptr_t>(a.sw) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(a.sx) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(a.bias) % 16 == 0;
  if (!ok) return launch_cfg<C10, false>(a, stream);
  const int64_t MTi = a.M / C::BM, NTi = a.N / C::BN, Ti = MTi * NTi;
  if (Ti > INT32_MAX) return hipErrorInvalidValue;
  int grid = 0;
  hipError_t e = persistent_grid<gemm_ppk_kernel<C>>(2 * C::kThreads, Ti, grid);
  if (e != hipSuccess) return e;
  gemm_ppk_kernel<C><<<dim3(grid), dim3(2 * C::kThreads), 0, stream>>>(
      a, static_cast<int>(Ti), static_cast<int>(MTi), static_cast<int>(NTi));
  return hipGetLastError();
}

// Whole 256 x 384 tiles for the wide ping-pong configuration (vector
// alignment is checked at launch).
bool pp_wide_covers(int64_t M, int64_t N, int64_t K) {
  return M > 0 && N > 0 && M % C14::BM == 0 && N % C14::BN == 0 && K % C14::BK == 0 &&
         K / C14::BK >= C14::STAGES;
}

// Configuration 14, bf16 output: the wide ping-pong tile when it covers the
// shape, else configuration 12's path (same output bits either way).
hipError_t launch_pp_wide(const GemmArgs& a, hipStream_t stream) {
  const bool aligned = reinterpret_cast<uintptr_t>(a.sw) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(a.sx) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(a.bias) % 16 == 0;
  if (!aligned || !pp_wide_covers(a.M, a.N, a.K)) return launch_pp<C11, false>(a, stream);
  const int64_t MTi = a.M / C14::BM, NTi = a.N / C14::BN, Ti = MTi * NTi;
  if (Ti > INT32_MAX) return hipErrorInvalidValue;
  int grid = 0;
  hipError_t e = persistent_grid<gemm_pp_kernel<C14, false>>(C14::kThreads, Ti, grid);
  if (e != hipSuccess) return e;
  gemm_pp_kernel<C14, false><<<dim3(grid), dim3(C14::kThreads), 0, stream>>>(
      a, static_cast<int>(Ti), static_cast<int>(MTi), static_cast<int>(NTi));
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
// x (workgroups sharing a CU) / (relative per-CU throughput).  Workgroups
// share a CU only when there are more tiles than CUs: with fewer, each tile
// has a CU to itself and small tiles finish sooner.  A handful of
// tokens (M <= 16) takes the split-K few-row kernel (also with 16 rows and
// enough 64-column tiles to give every CU one, where the 16-row tiled kernel
// was the faster one before the few-row kernel's coalesced loads: 21.2
// against 23.7 us on 16 x 18432 x 3072).
// Measured choices for the workload shapes: the fastest configuration of a
// full sweep on MI355X (bench.py --sweep, median of 20 calls on the shape's
// own seeded codes, weights rotated past the last-level cache), with close
// calls settled by interleaved rounds.  Other shapes take the cost model
// below, which on these 15 shapes picks the measured choice on 11, is within
// 1.6% of it on one (the 4608-token down-projection) and 3.1-3.3% on two (the
// 64 x 128 x 256 unit shape, the 768px attention projection), and misses the
// 256 x 3072 shape by 22%, whose 64-row split-K configuration is a measured
// choice only.
namespace {
struct MeasuredChoice {
  int64_t M, N, K;
  int cfg;
};
const MeasuredChoice kMeasured[] = {
    {64, 128, 256, 8},         // unit: few_rows_splitk4_mf16
    {2304, 3072, 3072, 3},     // 768px attention projection: bm128_bn256_bk128_s3_mf32
    {2304, 9216, 3072, 14},    // 768px fused QKV: bm256_bn384_bk64_s3_mf16_pp
    {4096, 12288, 3072, 14},   // 1024px MLP up: bm256_bn384_bk64_s3_mf16_pp
    {4096, 3072, 12288, 15},   // 1024px MLP down: bm256_bn192_bk64_s5_mf16_ppk
    {1, 18432, 3072, 8},       // few_rows_splitk4_mf16
    {1, 3072, 3072, 8},
    {16, 18432, 3072, 8},
    {16, 3072, 3072, 8},
    {256, 18432, 3072, 2},     // bm256_bn128_bk128_s3_mf32
    {256, 3072, 3072, 13},     // rows64_bn48_splitk8_mf16
    {4608, 9216, 3072, 14},    // 1024px block chain: the wide ping-pong tile on the QKV
    {4608, 3072, 3072, 12},    // projection, the 256 x 256 one on the out- and up-projections
    {4608, 12288, 3072, 12},   // (576 wide tiles fill 2.25 rounds of the CUs: a tie), and the
    {4608, 3072, 12288, 11},   // 8-wave generic tile on the down-projection, faster in three
                               // interleaved rounds of 100 calls (162-164 against 165-167 us)
};
const MeasuredChoice kFp8Measured[] = {
    {64, 128, 256, 3},         // fp8_few_rows_splitk4_mf16
    {2304, 3072, 3072, 1},     // fp8_bm128_bn256_bk128_s3_mf32
    {2304, 9216, 3072, 5},     // fp8_bm256_bn192_bk64_s4_mf32
    {4096, 12288, 3072, 4},    // fp8_bm256_bn256_bk64_s4_mf32
    {4096, 3072, 12288, 5},
    {256, 18432, 3072, 0},     // fp8_bm256_bn128_bk128_s3_mf32
    {256, 3072, 3072, 2},      // fp8_bm128_bn128_bk128_s4_mf32
    {4608, 9216, 3072, 4},
    {4608, 3072, 3072, 4},
    {4608, 12288, 3072, 4},
    {4608, 3072, 12288, 4},
};

template <size_t N>
int measured_choice(const MeasuredChoice (&t)[N], int64_t M, int64_t Nn, int64_t K) {
  for (const MeasuredChoice& c : t)
    if (c.M == M && c.N == Nn && c.K == K) return c.cfg;
  return -1;
}
}  // namespace

int gemm_select_config(int64_t M, int64_t N, int64_t K) {
  if (int c = measured_choice(kMeasured, M, N, K); c >= 0) return c;
  if (M <= 16) return kFewRows;
  int best = 0;
  double best_cost = 1e300;
  for (int c = 0; c < kNumConfigs; ++c) {
    if (c == kSkinny || c == kFewRows) continue;  // chosen above for M <= 16
    if (c == kRowBlocks || c == kPpK) continue;  // measured choices only
    if (c == kPpWide && !pp_wide_covers(M, N, K)) continue;  // else configuration 12's path
    const ConfigInfo& ci = kConfigs[c];
    const int64_t tiles = ((M + ci.BM - 1) / ci.BM) * ((N + ci.BN - 1) / ci.BN);
    // workgroups resident on one CU share its matrix-core throughput
    const int64_t share = std::min<int64_t>(ci.wg_per_cu, (tiles + kNumCU - 1) / kNumCU);
    const int64_t slots = static_cast<int64_t>(kNumCU) * share;
    const double waves = static_cast<double>((tiles + slots - 1) / slots);
    const double cost = waves * ci.BM * ci.BN * static_cast<double>(share) / ci.rel_speed;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = c;
    }
  }
  return best;
}

// ------------------------------------------------------------------ FP8 --
// Tile configurations of the e4m3 GEMM: 64-byte K steps, so BK = 128 keeps
// two steps per stage; bf16 output only.
namespace {
// (A 32-byte operand doubles the fragment registers: with two 64-byte k-steps
// per stage the wave tiles are limited to 128 x 64 / 64 x 128 / 64 x 64; with
// one k-step per 64-deep stage the int8 kernel's 128 x 128 wave tile fits.)
using F0 = Tile<256, 128, 2, 2, 128, 3, 32, true>;  // 3 x 48 KiB stages, spread refills
using F1 = Tile<128, 256, 2, 2, 128, 3, 32, true>;  // 3 x 48 KiB stages
using F2 = Tile<128, 128, 2, 2, 128, 4, 32, true>;  // 4 x 32 KiB stages
using F3 = Tile<256, 256, 2, 2, 64, 4, 32, true>;   // 4 x 32 KiB stages, one k-step each
using F4 = Tile<256, 192, 2, 2, 64, 4, 32, true>;   // 4 x 28 KiB stages, wave tile 128 x 96
// (256 x 192 makes one full wave of 256 tiles of the 4096 x 3072 down-projection: 138.5 us
// against 145.0 us with 256 x 256, and 77.1 against 81.8 us on the 2304 x 9216 QKV projection;
// where both take the same number of waves the cost ties and the lower index, 256 x 256, wins)
const ConfigInfo kFp8Configs[] = {
    {"fp8_bm256_bn128_bk128_s3_mf32", 256, 128, 256, 1, 1.00f},
    {"fp8_bm128_bn256_bk128_s3_mf32", 128, 256, 256, 1, 1.00f},
    {"fp8_bm128_bn128_bk128_s4_mf32", 128, 128, 256, 1, 0.80f},
    {"fp8_few_rows_splitk4_mf16", 16, 16, 256, 8, 0.10f},
    {"fp8_bm256_bn256_bk64_s4_mf32", 256, 256, 256, 1, 1.03f},
    {"fp8_bm256_bn192_bk64_s4_mf32", 256, 192, 256, 1, 1.03f},
};
constexpr int kFp8FewRows = 3;
constexpr int kNumFp8Configs = sizeof(kFp8Configs) / sizeof(kFp8Configs[0]);
}  // namespace

int gemm_fp8_num_configs() { return kNumFp8Configs; }

const char* gemm_fp8_config_name(int cfg) {
  return (cfg >= 0 && cfg < kNumFp8Configs) ? kFp8Configs[cfg].name : nullptr;
}

// Least (full-chip waves of tiles) x (tile area) / (relative throughput); a
// handful of tokens (M <= 16) takes the split-K few-row kernel.
int gemm_fp8_select_config(int64_t M, int64_t N, int64_t K) {
  if (int c = measured_choice(kFp8Measured, M, N, K); c >= 0) return c;
  if (M <= 16) return kFp8FewRows;
  int best = 0;
  double best_cost = 1e300;
  for (int c = 0; c < kNumFp8Configs; ++c) {
    if (c == kFp8FewRows) continue;
    const ConfigInfo& ci = kFp8Configs[c];
    const int64_t tiles = ((M + ci.BM - 1) / ci.BM) * ((N + ci.BN - 1) / ci.BN);
    const double waves = static_cast<double>((tiles + kNumCU - 1) / kNumCU);
    const double cost = waves * ci.BM * ci.BN / ci.rel_speed;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = c;
    }
  }
  return best;
}

hipError_t launch_gemm_fp8(const GemmArgs& a, int cfg, hipStream_t stream) {
  switch (cfg) {
    case 0: return launch_cfg<F0, false>(a, stream);
    case 1: return launch_cfg<F1, false>(a, stream);
    case 2: return launch_cfg<F2, false>(a, stream);
    case 3: return launch_few_rows<4, 1, false, true>(a, stream);
    case 4: return launch_cfg<F3, false>(a, stream);
    case 5: return launch_cfg<F4, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

namespace {
__global__ __launch_bounds__(256) void zero_u32(uint32_t* p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0u;
}
}  // namespace

// The up-projection with GELU and the row absmax in its epilogue: the
// ping-pong tile on interior tiles only (M, N multiples of 256, K a multiple
// of 64 with at least 4 stages, aligned vectors).
bool gemm_gelu_amax_supported(const GemmArgs& a) {
  using C = C11;
  return a.M % C::BM == 0 && a.N % C::BN == 0 && a.K % C::BK == 0 && a.K / C::BK >= C::STAGES &&
         a.M > 0 && a.N > 0 && reinterpret_cast<uintptr_t>(a.sw) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(a.sx) % 16 == 0 && reinterpret_cast<uintptr_t>(a.bias) % 16 == 0;
}

hipError_t launch_gemm_gelu_amax(const GemmArgs& a, hipStream_t stream) {
  using C = C11;
  if (!gemm_gelu_amax_supported(a) || a.amax == nullptr) return hipErrorInvalidValue;
  // the row maxima start from zero (|h| >= 0): a fill kernel, graph-capturable
  const int64_t zb = std::min<int64_t>((a.M + 255) / 256, 1024);
  zero_u32<<<dim3(static_cast<unsigned>(zb)), dim3(256), 0, stream>>>(a.amax, a.M);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t MTi = a.M / C::BM, NTi = a.N / C::BN, Ti = MTi * NTi;
  if (Ti > INT32_MAX) return hipErrorInvalidValue;
  int grid = 0;
  e = persistent_grid<gemm_pp_kernel<C, false, true>>(C::kThreads, Ti, grid);
  if (e != hipSuccess) return e;
  gemm_pp_kernel<C, false, true><<<dim3(grid), dim3(C::kThreads), 0, stream>>>(
      a, static_cast<int>(Ti), static_cast<int>(MTi), static_cast<int>(NTi));
  return hipGetLastError();
}

// The single-launch fused linear takes up to kRowsMaxM rows (kRowsMaxMWide
// above kNumCU column blocks) whose codes fit the LDS copy (K <= 3072: at
// most 6 128-byte steps per wave), where the library would run the few-row
// GEMM.
bool linear_few_rows_supported(int64_t M, int64_t N, int64_t K, bool fp8) {
  if (M < 1 || M > (fp8 ? kRowsMaxMFp8 : kRowsMaxM) || N < 1 || K < 16 || K % 16 != 0 ||
      K > kRowsMaxK)
    return false;
  if (M > kRowsMaxMWide && (N + 15) / 16 > kNumCU) return false;
  return fp8 ? gemm_fp8_select_config(M, N, K) == kFp8FewRows
             : gemm_select_config(M, N, K) == kFewRows;
}

template <bool FP8>
hipError_t launch_linear_few_rows_fmt(const RowsArgs& a, hipStream_t stream) {
  const int64_t steps = (a.K + 127) / 128;  // 128-byte steps of K
  if (a.M > 4 && !FP8) {
    switch ((steps + 7) / 8) {  // per wave of 8
      case 1: return launch_linear_few_rows_w8<1, FP8>(a, stream);
      case 2: return launch_linear_few_rows_w8<2, FP8>(a, stream);
      case 3: return launch_linear_few_rows_w8<3, FP8>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch ((steps + 3) / 4) {  // per wave of 4
    case 1: return launch_linear_few_rows_w4<1, FP8>(a, stream);
    case 2: return launch_linear_few_rows_w4<2, FP8>(a, stream);
    case 3: case 4: return launch_linear_few_rows_w4<4, FP8>(a, stream);
    case 5: case 6: return launch_linear_few_rows_w4<6, FP8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_linear_few_rows(const RowsArgs& a, bool fp8, hipStream_t stream) {
  return fp8 ? launch_linear_few_rows_fmt<true>(a, stream) : launch_linear_few_rows_fmt<false>(a, stream);
}

hipError_t launch_gemm(const GemmArgs& a, bool out_int32, int cfg, hipStream_t stream) {
  if (cfg < 0 || cfg >= kNumConfigs) return hipErrorInvalidValue;
  switch (cfg) {
    case 0: return launch_cfg_out<C0>(a, out_int32, stream);
    case 1: return launch_cfg_out<C1>(a, out_int32, stream);
    case 2: return launch_cfg_out<C2>(a, out_int32, stream);
    case 3: return launch_cfg_out<C3>(a, out_int32, stream);
    case 4: return launch_cfg_out<C4>(a, out_int32, stream);
    case 5: return launch_cfg_out<C5>(a, out_int32, stream);
    case 6: return launch_cfg_out<C6>(a, out_int32, stream);
    case 7: return launch_cfg_out<C7>(a, out_int32, stream);
    case 8: return launch_few_rows_any(a, out_int32, stream);
    case 9: return launch_cfg_out<C9>(a, out_int32, stream);
    case 10: return launch_cfg_out<C10>(a, out_int32, stream);
    case 11: return launch_cfg_out<C11>(a, out_int32, stream);
    case 12: return out_int32 ? launch_pp<C11, true>(a, stream) : launch_pp<C11, false>(a, stream);
    case 13: return out_int32 ? launch_few_rows_st<8, 3, true, 1, false, false, 4, true, true>(a, stream)
                              : launch_few_rows_st<8, 3, false, 1, false, false, 4, true, true>(a, stream);
    case 14: return out_int32 ? launch_pp<C11, true>(a, stream) : launch_pp_wide(a, stream);
    case 15: return out_int32 ? launch_cfg<C10, true>(a, stream) : launch_ppk(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w8a8
