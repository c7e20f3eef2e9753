// Measurement probe, not part of the W8A8 library: how many int8 (or e4m3)
// matrix-core operations per second the chip sustains on given operand codes
// when nothing else runs -- no HBM, L2 or global-to-LDS traffic and no
// epilogue.  Under sustained MFMA load the MI355X shader clock is set by the
// power limit, and the power drawn per operation depends on the operand bits
// that toggle, so this rate (not the 2.4 GHz spec peak) is the ceiling a GEMM
// on the same codes can approach.  Built into its own libw8a8_probe.so and
// driven by bench.py --mfma-ceiling.
//
// Each workgroup is 4 waves (one per SIMD, 256 CUs x 1 workgroup), each wave
// holding two sets of 8 operand fragments (16 bytes per lane each) read once
// from `a` (weight-like, MFMA "A") and `b` (activation-like, MFMA "B") and a
// 128 x 128 accumulator tile, and issuing MFMAs in the GEMM's k-loop order
// (fragment set 0, then set 1, so the operands change from one k-step to the
// next as in a GEMM).  Modes:
//   0  int8 v_mfma_i32_32x32x32_i8, 4 x 4 blocks, operands in registers
//   1  int8 v_mfma_i32_16x16x64_i8, 8 x 8 blocks, operands in registers
//   2  mode 0 plus the LDS fragment reads of the 256 x 256 GEMM tile: every
//      k-step re-reads its 8 fragments from LDS (one 16-byte read per lane
//      per 2 MFMAs), so the LDS read energy is included; as in the GEMM the
//      reads of the next k-step go out before the current k-step's MFMAs
//      (two fragment sets), so their latency is hidden
//   3  FP8 v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3, unit block scales),
//      4 x 2 blocks of 32-byte operands (the same operations per k-step)
//   4  mode 1 plus the LDS fragment reads of the 256 x 256 GEMM tile on
//      16x16x64 blocks (its 16 fragments re-read per 64-byte k-step: one
//      16-byte read per lane per 4 MFMAs, the same bytes per operation),
//      read one k-step ahead into a second set of 16 fragments
// Lane 0 of wave 0 of every workgroup writes its shader-clock cycles
// (s_memtime) and 100 MHz real-time ticks (s_memrealtime) across the loop to
// stamps[2 b], stamps[2 b + 1], giving the clock the loop ran at.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kFrags = 8;  // per operand and lane: two k-step sets of 4

__device__ __forceinline__ void stamp(unsigned long long* st, unsigned long long cyc,
                                      unsigned long long rt) {
  int l = threadIdx.x;
  asm volatile("" : "+v"(l));  // per-lane address: a vector store
  if (l == 0) {
    st[2 * blockIdx.x + l] = cyc;
    st[2 * blockIdx.x + 1 + l] = rt;
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void mfma_ceiling(const v4i* a, const v4i* b, int iters,
                                                         int* sink, unsigned long long* st) {
  __shared__ v4i lds[2 * kFrags * kThreads];
  const int gid = blockIdx.x * kThreads + threadIdx.x;
  v4i fa[kFrags], fb[kFrags];
#pragma unroll
  for (int i = 0; i < kFrags; ++i) {
    fa[i] = a[gid * kFrags + i];
    fb[i] = b[gid * kFrags + i];
  }
  if constexpr (MODE == 2 || MODE == 4) {
#pragma unroll
    for (int i = 0; i < kFrags; ++i) {
      lds[i * kThreads + threadIdx.x] = fa[i];
      lds[(kFrags + i) * kThreads + threadIdx.x] = fb[i];
    }
    __syncthreads();
  }
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  int sum = 0;
  if constexpr (MODE == 0 || MODE == 2) {
    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v16i{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if constexpr (MODE == 2) {
          // the next k-step's fragments (the other set) from LDS, rotating
          // slots so that the reads cannot be hoisted out of the loop
          const int n = 4 * (s ^ 1);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            fa[n + i] = lds[((n + i + it) & (kFrags - 1)) * kThreads + threadIdx.x];
            fb[n + i] = lds[(kFrags + ((n + i + it) & (kFrags - 1))) * kThreads + threadIdx.x];
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[4 * s + i], fb[4 * s + j], acc[i][j], 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) sum += acc[i][j][e];
  } else if constexpr (MODE == 1 || MODE == 4) {
    // a 64-byte k-step: 16x16x64 blocks over the lane's 8 A and 8 B fragments
    v4i acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = v4i{};
    if constexpr (MODE == 1) {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
    } else {
      // two sets of 16 fragments: the next k-step's are read from LDS during
      // the current k-step's MFMAs, one read after every 4 MFMAs as in the
      // GEMM (a burst of reads stalls the issuing wave); iterations run in
      // pairs (iters is even)
      v4i ga[kFrags], gb[kFrags];
      for (int it = 0; it < iters; it += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          v4i(&ca)[kFrags] = h ? ga : fa;
          v4i(&cb)[kFrags] = h ? gb : fb;
          v4i(&na)[kFrags] = h ? fa : ga;
          v4i(&nb)[kFrags] = h ? fb : gb;
#pragma unroll
          for (int r = 0; r < 2 * kFrags; ++r) {
            const int slot = ((r & (kFrags - 1)) + it + h + 1) & (kFrags - 1);
            __builtin_amdgcn_sched_barrier(0);
            if (r < kFrags)
              na[r] = lds[slot * kThreads + threadIdx.x];
            else
              nb[r - kFrags] = lds[(kFrags + slot) * kThreads + threadIdx.x];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int i = (4 * r + q) / 8, j = (4 * r + q) % 8;
              acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ca[i], cb[j], acc[i][j], 0, 0, 0);
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) sum += acc[i][j][e];
  } else {
    // e4m3: a 64-byte k-step per MFMA, 32-byte operands from two fragments
    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const v8i av = __builtin_shufflevector(fa[4 * s + i], fa[4 * s + ((i + 1) & 3)], 0, 1, 2, 3, 4, 5, 6, 7);
            const v8i bv = __builtin_shufflevector(fb[4 * s + 2 * j], fb[4 * s + 2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], 0, 0, 0, 127, 0, 127);
          }
    }
    float fs = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) fs += acc[i][j][e];
    sum = static_cast<int>(fs);
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  sink[gid] = sum;  // keeps the products live
  stamp(st, c1 - c0, r1 - r0);
}

}  // namespace

// Operations one launch performs: 4 waves x iters x 2 097 152 per workgroup
// (every mode issues 2^20 multiply-adds, 2^21 operations, per wave and
// iteration).
extern "C" double w8a8_probe_mfma_ops(int grid, int iters) {
  return static_cast<double>(grid) * 4.0 * iters * 2097152.0;
}

// a, b: device buffers of at least grid * 256 * 8 * 16 bytes; sink: grid *
// 256 ints; stamps: 2 * grid 64-bit values.  Returns 0, or a HIP error code,
// or -1 for invalid arguments (nothing launched).
extern "C" int w8a8_probe_mfma_ceiling(int mode, const void* a, const void* b, int64_t bytes,
                                       int grid, int iters, void* sink, void* stamps,
                                       void* stream) {
  if (!a || !b || !sink || !stamps || grid <= 0 || iters <= 0 || mode < 0 || mode > 4) return -1;
  if (bytes < static_cast<int64_t>(grid) * kThreads * kFrags * 16) return -1;
  if (mode == 4 && iters % 2 != 0) return -1;  // iterations run in pairs
  const v4i* pa = static_cast<const v4i*>(a);
  const v4i* pb = static_cast<const v4i*>(b);
  int* ps = static_cast<int*>(sink);
  unsigned long long* pt = static_cast<unsigned long long*>(stamps);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (mode) {
    case 0: mfma_ceiling<0><<<grid, kThreads, 0, s>>>(pa, pb, iters, ps, pt); break;
    case 1: mfma_ceiling<1><<<grid, kThreads, 0, s>>>(pa, pb, iters, ps, pt); break;
    case 2: mfma_ceiling<2><<<grid, kThreads, 0, s>>>(pa, pb, iters, ps, pt); break;
    case 3: mfma_ceiling<3><<<grid, kThreads, 0, s>>>(pa, pb, iters, ps, pt); break;
    default: mfma_ceiling<4><<<grid, kThreads, 0, s>>>(pa, pb, iters, ps, pt); break;
  }
  return static_cast<int>(hipGetLastError());
}
