// prep.hip -- per-query row terms prepared once per backward.
//
//  * rowterm_kernel: the backward's per-query terms, padded to Np:
//    L2[i] = LSE_i * log2(e) (+inf for a row whose keys are all masked, and
//    for padding, so that P = exp2(s - L2) = 0 there) and
//    D[i] = sum_d dO_id O_id (0 for padding), the row term of
//    dS = P (dP - D) in the FlashAttention backward; and the per-query seeds
//    of the key pass, which start its score accumulator at the row's
//    -LSE (plus, on saturated tiles, the query-side saturated relation
//    scalar) and its dP accumulator at -D (at -D (1 - p) under attention
//    dropout, where the key pass rescales the kept entries by 1 / (1 - p)).
#include "device.hpp"
#include "tiles.hpp"
#include "qside.hpp"

namespace relpos {

// 8 lanes per row; rows [r0, r1) of each of the B*H sequences (padded to Np).
template <typename T>
__global__ __launch_bounds__(kThreads) void rowterm_kernel(RowTermArgs a) {
  constexpr float kLog2e = 1.4426950408889634f;
  const int nr = a.r1 - a.r0;
  const int64_t rows = (int64_t)a.B * a.H * a.Np;  // stride between the seed vectors
  const int64_t todo = (int64_t)a.B * a.H * nr;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / 8) + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  float acc = 0.f;
  int i = 0;
  int64_t bh = 0, row = 0;
  if (t < todo) {
    bh = t / nr;
    i = a.r0 + (int)(t - bh * nr);
    row = bh * a.Np + i;
    if (i < a.N) {
      const int b = (int)(bh / a.H), h = (int)(bh % a.H);
      const T* o = (const T*)a.o + b * a.so.b + h * a.so.h + (int64_t)i * a.so.n + 8 * part;
      const T* d = (const T*)a.dO + b * a.sdo.b + h * a.sdo.h + (int64_t)i * a.sdo.n + 8 * part;
#pragma unroll
      for (int u = 0; u < 8; ++u) acc = fmaf(MT<T>::to_f(o[u]), MT<T>::to_f(d[u]), acc);
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (t < todo && part == 0) {
    a.D[row] = acc;
    float l2 = INFINITY;
    if (i < a.N) {
      const float L = a.lse[bh * a.N + i];
      l2 = L == -INFINITY ? INFINITY : L * kLog2e;
    }
    a.L2[row] = l2;
    const float base = -(l2 / a.scale2);
    float zlo = 0.f, zhi = 0.f;
    if (a.zq) {
      const float* zqb = a.zq + zq_off(a.geo, bh, 0);
      const float* p0 = qside_sat_ptr(a.geo, zqb, i, 0);
      const float* p1 = qside_sat_ptr(a.geo, zqb, i, 1);
      if (p0) zlo = *p0;
      if (p1) zhi = *p1;
    }
    a.kseed[row] = zlo + base;
    a.kseed[rows + row] = zhi + base;
    a.kseed[2 * rows + row] = base;
    a.kseed[3 * rows + row] = -acc * a.dseed_scale;
  }
}

hipError_t launch_rowterm(int dtype, const RowTermArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.H * (a.r1 - a.r0);
  const int blocks = (int)((rows + kThreads / 8 - 1) / (kThreads / 8));
  if (blocks <= 0) return hipSuccess;
  switch (dtype) {
    case 0: hipLaunchKernelGGL(rowterm_kernel<float>, dim3(blocks), dim3(kThreads), 0, st, a); break;
    case 1: hipLaunchKernelGGL(rowterm_kernel<_Float16>, dim3(blocks), dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL(rowterm_kernel<__bf16>, dim3(blocks), dim3(kThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace relpos
