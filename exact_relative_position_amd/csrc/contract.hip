// contract.hip -- final contraction of the per-offset relation gradients.
//
// Source: "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (nanless.github.io digest), end of the backward section: the table
// gradients are matrix products, dZ^T times Q (or K) gives the gradient of the
// relation table, and dZ times the table gives the extra term of dQ (dK);
// copied bucket columns are summed back into their bucket in a fixed order.
// The scalar-bias gradient is read here as the column sums of dZ^Q
// (db[r] = tau * sum over all pairs with phi = r of dS, from Eq. 1 and 4).
//
// All three kernels use v_mfma_f32_32x32x2_f32 on fp32 data and fixed
// summation orders (no atomics):
//  * rows_kernel:  dX[i] = dX_part[i] + sum_c dZ[i][c] tab[fold(ws + c)]
//  * cols_kernel:  part[s][h][u] = sum over the rows i of split s of dZ[i][u - ws(i)] x_i
//                  (and the column sums for db), window-aware;
//  * fold_kernel:  out[h][k] = sum over splits and over the unfolded rows u of k.
#include "device.hpp"
#include "tiles.hpp"

namespace relpos {

__device__ inline f32x16 mma32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// One block: 128 rows of one (b, h) (one group); 4 waves x 32 rows x 64 d.
template <typename T>
__global__ __launch_bounds__(kThreads) void rows_kernel(RowsArgs a) {
  constexpr int P = 65;
  __shared__ float sZ[kBlockRows * P];
  __shared__ float sT[64 * P];
  const Geo g = a.geo;
  const int N = g.N;
  const int total = a.B * a.H * a.nblk;
  const int lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / a.nblk, rb = lid - bh * a.nblk;
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int i0 = rb * kBlockRows;
  int cb, ce, ws;
  if (a.key_side) {
    cols_k(g, rb, cb, ce);
    ws = win_k(g, rb);
  } else {
    cols_q(g, rb, cb, ce);
    ws = win_q(g, rb);
  }
  const float* dzb = a.dz + (int64_t)bh * N * g.W;
  const T* tab = (const T*)a.tab + hh * a.tab_hs;

  f32x16 acc[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = i0 + 32 * w + res_row(hl, e);
      acc[nt][e] = i < N ? a.part[((int64_t)bh * N + i) * kHeadDim + 32 * nt + l32] : 0.f;
    }

  for (int c0 = cb; c0 < ce; c0 += 64) {
    // stage dZ[i0 .. i0+127][c0 .. c0+63] and the 64 table rows (as fp32);
    // all loads of a thread are issued before its LDS stores
    {
      float zv[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int idx = tid + kThreads * u;
        const int r = idx >> 6, cc = idx & 63;
        const int i = i0 + r, col = c0 + cc;
        zv[u] = (i < N && col < ce) ? dzb[(int64_t)i * g.W + col] : 0.f;
      }
      float tv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int idx = tid + kThreads * u;
        const int cc = idx >> 6, d = idx & 63;
        const int col = c0 + cc;
        float v = 0.f;
        if (col < ce) {
          const int uu = ws + col;
          const int r = a.fold ? a.fold[uu] : uu;
          v = MT<T>::to_f(tab[(int64_t)r * kHeadDim + d]);
        }
        tv[u] = v;
      }
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int idx = tid + kThreads * u;
        sZ[(idx >> 6) * P + (idx & 63)] = zv[u];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int idx = tid + kThreads * u;
        sT[(idx >> 6) * P + (idx & 63)] = tv[u];
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int ks = 0; ks < 32; ++ks) {
      const float av = sZ[(32 * w + l32) * P + 2 * ks + hl];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[nt] = mma32(av, sT[(2 * ks + hl) * P + 32 * nt + l32], acc[nt]);
    }
    __syncthreads();
  }

  T* ob = (T*)a.out + bb * a.sout.b + hh * a.sout.h;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = i0 + 32 * w + res_row(hl, e);
      if (i < N) ob[(int64_t)i * a.sout.n + 32 * nt + l32] = MT<T>::from_f(acc[nt][e]);
    }
}

// Block (rt, s, ho): unfolded rows u in [32 rt, 32 rt + 32), all 64 d, over
// the rows of split s.  The 4 waves take interleaved pairs of rows (one MFMA
// k-step each) and are summed in LDS in wave order.
template <typename T>
__global__ __launch_bounds__(kThreads) void cols_kernel(ColsArgs a) {
  __shared__ float sAcc[4][32 * 64];
  __shared__ float sSum[4][32];
  const Geo g = a.geo;
  const int N = g.N;
  const int rt = blockIdx.x, sp = blockIdx.y, ho = blockIdx.z;
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int u = 32 * rt + l32;  // unfolded row of this lane (operand A row)
  const int nseg = a.shared ? a.B * a.H : a.B;
  const int64_t nrows = (int64_t)nseg * N;
  const int64_t per = (nrows + a.splits - 1) / a.splits;
  const int64_t f0 = (int64_t)sp * per;
  const int64_t f1 = f0 + per < nrows ? f0 + per : nrows;

  f32x16 acc[2];
  acc[0] = zero16();
  acc[1] = zero16();
  float csum = 0.f;

  int64_t f = f0;
  while (f < f1) {
    const int seg = (int)(f / N);
    const int i_start = (int)(f - (int64_t)seg * N);
    const int grp = grouped(g) ? i_start / kGroup : 0;
    const int i_gend = grouped(g) ? imin(N, (grp + 1) * kGroup) : N;
    const int64_t fend0 = (int64_t)seg * N + i_gend;
    const int64_t fend = fend0 < f1 ? fend0 : f1;
    int cb, ce, ws;
    if (a.key_side) {
      cols_k(g, grp, cb, ce);
      ws = win_k(g, grp);
    } else {
      cols_q(g, grp, cb, ce);
      ws = win_q(g, grp);
    }
    // skip the chunk when its live columns miss this block's rows
    if (ws + ce > 32 * rt && ws + cb < 32 * rt + 32) {
      const int b_ = a.shared ? seg / a.H : seg;
      const int h_ = a.shared ? seg % a.H : ho;
      const int bh = b_ * a.H + h_;
      const float* dzb = a.dz + (int64_t)bh * N * g.W;
      const T* xb = (const T*)a.x + b_ * a.sx.b + h_ * a.sx.h;
      const int col = u - ws;
      const bool colv = col >= cb && col < ce;
      const int i_end = (int)(fend - (int64_t)seg * N);
      // each wave takes 16 consecutive rows (8 MFMA k-steps) per round, loads first
      for (int ib = i_start + 16 * w; ib < i_end; ib += 64) {
        float av[8], bv[8][2];
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          const int i = ib + 2 * s2 + hl;
          const bool rv = i < i_end;
          av[s2] = (rv && colv) ? dzb[(int64_t)i * g.W + col] : 0.f;
          const T* xr = xb + (int64_t)i * a.sx.n;
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            bv[s2][nt] = (rv && a.want_x) ? MT<T>::to_f(xr[32 * nt + l32]) : 0.f;
        }
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          csum += av[s2];
          if (a.want_x) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) acc[nt] = mma32(av[s2], bv[s2][nt], acc[nt]);
          }
        }
      }
    }
    f = fend;
  }

  csum += __shfl_xor(csum, 32);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int e = 0; e < 16; ++e) sAcc[w][res_row(hl, e) * 64 + 32 * nt + l32] = acc[nt][e];
  if (hl == 0) sSum[w][l32] = csum;
  __syncthreads();
  float* outp = a.part + (((int64_t)sp * gridDim.z + ho) * a.Rpad + 32 * rt) * 64;
  for (int idx = tid; idx < 32 * 64; idx += kThreads) {
    const float v = ((sAcc[0][idx] + sAcc[1][idx]) + sAcc[2][idx]) + sAcc[3][idx];
    if (a.want_x) outp[idx] = v;
  }
  if (a.partb && tid < 32) {
    const float v = ((sSum[0][tid] + sSum[1][tid]) + sSum[2][tid]) + sSum[3][tid];
    a.partb[((int64_t)sp * gridDim.z + ho) * a.Rpad + 32 * rt + tid] = v;
  }
}

// out[ho][k][d] = sum_{u in [ub[k], ue[k])} sum_s part[s][ho][u][d], u ascending.
__global__ void fold_kernel(FoldArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)a.Ho * a.R * 65;
  if (idx >= n) return;
  const int d = (int)(idx % 65);
  const int64_t hk = idx / 65;
  const int k = (int)(hk % a.R), ho = (int)(hk / a.R);
  const int b = a.ub ? a.ub[k] : k;
  const int e = a.ub ? a.ue[k] : k + 1;
  if (d < 64) {
    if (!a.out) return;
    float s = 0.f;
    for (int u = b; u < e; ++u)
      for (int sp = 0; sp < a.splits; ++sp)
        s += a.part[(((int64_t)sp * a.Ho + ho) * a.Rpad + u) * 64 + d];
    a.out[((int64_t)ho * a.R + k) * 64 + d] = s;
  } else {
    if (!a.outb) return;
    float s = 0.f;
    for (int u = b; u < e; ++u)
      for (int sp = 0; sp < a.splits; ++sp) s += a.partb[((int64_t)sp * a.Ho + ho) * a.Rpad + u];
    a.outb[(int64_t)ho * a.R + k] = s;
  }
}

hipError_t launch_rows(int dtype, const RowsArgs& a, hipStream_t st) {
  const int total = a.B * a.H * a.nblk;
  if (total <= 0) return hipSuccess;
  switch (dtype) {
    case 0: hipLaunchKernelGGL(rows_kernel<float>, dim3(total), dim3(kThreads), 0, st, a); break;
    case 1: hipLaunchKernelGGL(rows_kernel<_Float16>, dim3(total), dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL(rows_kernel<__bf16>, dim3(total), dim3(kThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_cols(int dtype, const ColsArgs& a, int Ho, hipStream_t st) {
  dim3 grid(a.rtiles, a.splits, Ho);
  switch (dtype) {
    case 0: hipLaunchKernelGGL(cols_kernel<float>, grid, dim3(kThreads), 0, st, a); break;
    case 1: hipLaunchKernelGGL(cols_kernel<_Float16>, grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL(cols_kernel<__bf16>, grid, dim3(kThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_fold(const FoldArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.Ho * a.R * 65;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fold_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace relpos
