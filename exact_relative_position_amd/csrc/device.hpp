// device.hpp -- gfx950 building blocks: 32x32 MFMA traits per element type,
// the lane layout of the MFMA operands and results, XCD-aware block order.
//
// MFMA lane layout (CDNA, 32x32 output tiles, 64-wide wavefront):
//  * operand A (M x K) and operand B (K x N) have the same per-lane shape:
//    lane l holds index l % 32 of its free dimension and E consecutive
//    k-indices starting at E * (l / 32) of each k-step of KS = 2E values;
//  * result element e (0..15) of lane l sits at row 8*(e/4) + 4*(l/32) + e%4,
//    column l % 32.
// fp16 / bf16 use v_mfma_f32_32x32x16_{f16,bf16} (KS = 16, E = 8); fp32 uses
// v_mfma_f32_32x32x2_f32 (KS = 2, E = 1).
//
// Row permutation: the rows of a score tile come out of the MFMA as result
// elements, and the next MFMA consumes the same registers as its k-operand.
// Loading A-row m from tile row sigma(m) makes result element e of lane-half h
// hold tile row kappa(h, e) = KS*(e/E) + E*h + e%E, which is exactly the
// k-index the next MFMA expects there, so no data moves between the two.
#pragma once
#include <hip/hip_runtime.h>

#include "geometry.hpp"

namespace relpos {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <typename T>
struct MT;

template <>
struct MT<_Float16> {
  using frag = f16x8;
  static constexpr int KS = 16, E = 8;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag zero() {
    frag z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (_Float16)0.f;
    return z;
  }
  __device__ static inline frag pack(const float* p) {
    frag r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (_Float16)p[i];
    return r;
  }
  __device__ static inline float to_f(_Float16 x) { return (float)x; }
  __device__ static inline _Float16 from_f(float x) { return (_Float16)x; }
  // acc + sum of the 8 elements of a fragment (v_dot2 against ones)
  __device__ static inline float sum_acc(frag f, float acc) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 one = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(h2{f[2 * i], f[2 * i + 1]}, one, acc, false);
    return acc;
  }
};

template <>
struct MT<__bf16> {
  using frag = bf16x8;
  static constexpr int KS = 16, E = 8;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag zero() {
    frag z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.f;
    return z;
  }
  __device__ static inline frag pack(const float* p) {
    frag r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (__bf16)p[i];
    return r;
  }
  __device__ static inline float to_f(__bf16 x) { return (float)x; }
  __device__ static inline __bf16 from_f(float x) { return (__bf16)x; }
  __device__ static inline float sum_acc(frag f, float acc) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 one = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(b2{f[2 * i], f[2 * i + 1]}, one, acc, false);
    return acc;
  }
};

template <>
struct MT<float> {
  using frag = float;
  static constexpr int KS = 2, E = 1;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag zero() { return 0.f; }
  __device__ static inline frag pack(const float* p) { return p[0]; }
  __device__ static inline float to_f(float x) { return x; }
  __device__ static inline float from_f(float x) { return x; }
  __device__ static inline float sum_acc(frag f, float acc) { return acc + f; }
};

// Tile row held by result element e of lane-half h (see header comment).
template <typename T>
__device__ inline int kappa(int h, int e) {
  constexpr int KS = MT<T>::KS, E = MT<T>::E;
  return KS * (e / E) + E * h + (e % E);
}
// Tile row that lane-row m of an A operand loads.
template <typename T>
__device__ inline int sigma(int m) {
  int h = (m >> 2) & 1;
  int e = 4 * (m >> 3) + (m & 3);
  return kappa<T>(h, e);
}
// Row of result element e of lane-half h (plain MFMA result layout).
__device__ inline int res_row(int h, int e) { return 8 * (e >> 2) + 4 * h + (e & 3); }

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Index of this thread's wavefront in the workgroup, as a wave-uniform value
// (readfirstlane), so that the compiler keeps everything derived from it --
// tile kinds, mask decisions, segment bounds -- in scalar registers and
// branches on it with scalar branches.
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Blocks are dealt to the 8 XCDs round-robin; renumber them so that blocks
// consecutive in the logical order run on the same XCD (and share its L2).
__device__ inline int xcd_remap(int bid, int total) {
  int q = total >> 3;
  if (bid >= (q << 3)) return bid;
  return (bid & 7) * q + (bid >> 3);
}

// Block of a launch over (B*H) x nblk blocks -> (bh, rank): equal-work
// launches use xcd_remap (the blocks of one head consecutive on one XCD);
// causal launches number the blocks rank-major (rank 0 = the longest block of
// every head first, so that the dispatch order is longest first over the
// whole grid), and with B*H a multiple of 8 block b still runs on XCD
// b % 8 = bh % 8, so that a head's blocks share one L2.
__device__ inline void block_of(int bid, int total, int nblk, bool causal, int& bh, int& rank) {
  if (causal) {
    const int nbh = total / nblk;
    rank = bid / nbh;
    bh = bid - rank * nbh;
  } else {
    const int lid = xcd_remap(bid, total);
    bh = lid / nblk;
    rank = lid - bh * nblk;
  }
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a value with the one of lane l ^ 32 (v_permlane32_swap: one VALU
// operation, no trip through the LDS crossbar).
__device__ inline float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16-byte store to an address that is only 4-byte aligned (global memory
// accepts unaligned vector accesses; the type's alignment tells the compiler
// so, which keeps it one dwordx4 store).
typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ void store_f32x4_a4(float* p, f32x4 v) {
  *reinterpret_cast<f32x4_a4*>(p) = v;
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Four 16-byte LDS reads at byte offsets O0..O3 from p, issued in one asm
// block that also waits for them (the results are early-clobber operands,
// so that no read lands in the address register of a later one).  For LDS areas that the kernel fills with
// direct-to-LDS loads and waits for itself (explicit vmcnt and a barrier):
// the compiler cannot tell such an area from the ones whose loads are still
// in flight and would otherwise wait for every outstanding global access
// (the prefetch of the next tile, the stores of this one) before the read.
template <int O0, int O1, int O2, int O3>
__device__ __forceinline__ void lds_read4x16(const float* p, f32x4& a, f32x4& b, f32x4& c,
                                             f32x4& d) {
  const uint32_t ad = lds_addr(p);
  asm volatile(
      "ds_read_b128 %0, %4 offset:%5\n\t"
      "ds_read_b128 %1, %4 offset:%6\n\t"
      "ds_read_b128 %2, %4 offset:%7\n\t"
      "ds_read_b128 %3, %4 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d)
      : "v"(ad), "i"(O0), "i"(O1), "i"(O2), "i"(O3)
      : "memory");
}

// s_waitcnt immediate for "vmcnt(0)" with the other counters left alone
// (gfx9 encoding: vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8]).
constexpr int kWaitVmcnt0 = 0x0F70;

}  // namespace relpos
