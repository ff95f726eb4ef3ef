// proj.hip -- offset-map tables and the relation projection.
//
// Source: "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (nanless.github.io digest):
//  * Eq. (3): Z^Q[i, r] = q_i . aQ[r] and Z^K[j, r] = k_j . aK[r];
//  * grouped reachable range: each group of G = 128 queries (keys) projects
//    only the contiguous window of rows it can reach (N + G - 1 rows), or all
//    rows when the table is shorter; with a causal mask only offsets <= 0 are
//    live, so only those columns are computed;
//  * constant tiles: a bucketed map is unfolded into a truncated map by
//    copying each bucket row once per offset it covers (here the copy is an
//    index table `fold`: unfolded row u reads table row fold[u]).
//
// The projection is an HBM-write-bound GEMM: 128 rows x 64 columns per
// workgroup, fp16/bf16 (or fp32) MFMA with fp32 accumulation, coalesced fp32
// stores of the window.  When the scalar bias b sits next to a query-side
// table it is added here, so the score needs one lookup instead of two.
#include <math.h>

#include "device.hpp"
#include "tiles.hpp"
#include "buckets.hpp"

namespace relpos {

__device__ inline int phi_row(const PhiArgs& p, int o) {
  switch (p.kind) {
    case 0: return imin(imax(o, p.lo), p.hi) - p.lo;
    case 1: return t5_bucket_dev(o, p.num_buckets, p.max_exact, p.max_distance, p.bidirectional);
    case 3: return log_bucket_dev(o, p.num_buckets, p.max_distance);
    default: return o + p.N - 1;
  }
}

// rows[t] = phi(t - (N - 1)), t in [0, 2N - 1)
__global__ void phi_rows_kernel(PhiArgs p, int32_t* rows) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < 2LL * p.N - 1) rows[t] = phi_row(p, (int)(t - (p.N - 1)));
}

// fold[u] = phi(u + lo_unf), u in [0, R_unf)
__global__ void phi_fold_kernel(PhiArgs p, int32_t* fold) {
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  const int R = p.hi_unf - p.lo_unf + 1;
  if (u < R) fold[u] = phi_row(p, u + p.lo_unf);
}

// For each table row k: the unfolded rows [ub[k], ue[k]) that copy it.  Each
// bucket covers one contiguous offset range, so the unfolded row u that
// starts (ends) a run of equal rows writes its row's ub (ue); buckets with no
// unfolded row keep ub = ue = 0 from fold_range_clear_kernel (launched
// first: a fill kernel rather than a memset, so the sequence can be
// captured in a graph).
__global__ void fold_range_clear_kernel(int R, int32_t* ub, int32_t* ue) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k < R) {
    ub[k] = 0;
    ue[k] = 0;
  }
}

__global__ void fold_range_kernel(const int32_t* fold, int Runf, int32_t* ub, int32_t* ue) {
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= Runf) return;
  const int k = fold[u];
  if (u == 0 || fold[u - 1] != k) ub[k] = u;
  if (u == Runf - 1 || fold[u + 1] != k) ue[k] = u + 1;
}

// bunf[h][u] = b[h][fold[u]] as fp32 (fold null: identity)
template <typename T>
__global__ void bias_unfold_kernel(BiasArgs a) {
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  const int h = blockIdx.y;
  if (u >= a.Runf) return;
  const int r = a.fold ? a.fold[u] : u;
  a.bunf[(int64_t)h * a.Runf + u] = MT<T>::to_f(((const T*)a.b)[h * a.b_hs + r]);
}

// Z[bh][i][c] = x_i . tab[fold(ws + c)] (+ bias[fold(ws + c)]) for c in the
// group's live columns [cb, ce), for the groups [g0, g0 + ngroups).  Block:
// 128 rows x proj_cols() columns (256 for windows of 2048 columns and more,
// else 128); wave w owns rows 32w..32w+31, keeps their X fragments in
// registers and walks the block's 32-column MFMA tiles, loading the next
// tile's table fragments before it computes and stores the current one, so
// that the loads overlap the stores (each store instruction writes 128-byte
// runs of two rows).
//
// Every iteration issues the same memory instructions whatever its lanes
// hold: lanes past the window's end load table row 0, and the stores are
// buffer stores whose out-of-range lanes (rows beyond N, columns beyond the
// window) carry an offset past the buffer's end, which the hardware drops.
// With fixed counts the compiler's wait for the prefetched fragments leaves
// the previous tile's stores in flight.  (Conditional loads or stores would
// make it wait for every outstanding access.)  BUF: the (b, h) slab of Z is
// below 2 GiB, as 32-bit buffer offsets need; otherwise plain stores.
__host__ __device__ inline int proj_cols(const ProjArgs& a) { return a.ncol_tiles >= 32 ? 256 : 128; }

// FOLD: bucketed map (table rows through the fold table); BIAS: b is folded
// into the projection.
template <typename T, bool FOLD, bool BIAS, bool BUF>
__global__ __launch_bounds__(kThreads) void proj_kernel(ProjArgs a) {
  using M = MT<T>;
  using frag = typename M::frag;
  constexpr int KS = M::KS, E = M::E, NSD = kHeadDim / KS;
  const Geo g = a.geo;
  const int N = g.N;
  const int pc = proj_cols(a);
  const int nch = (a.ncol_tiles + pc / 64 - 1) / (pc / 64);  // chunks per group
  const int per_bh = a.ngroups * nch;
  const int total = a.B * a.H * per_bh;
  const int lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / per_bh;
  const int rem = lid - bh * per_bh;
  const int grp = a.g0 + rem / nch, ch = rem - (rem / nch) * nch;
  const int bb = bh / a.H, hh = bh - bb * a.H;
  int cb, ce, ws;
  if (a.key_side) {
    cols_k(g, grp, cb, ce);
    ws = win_k(g, grp);
  } else {
    cols_q(g, grp, cb, ce);
    ws = win_q(g, grp);
  }
  const int c0 = cb + ch * pc;
  if (c0 >= ce) return;
  const int nsub = (imin(ce - c0, pc) + 31) / 32;
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int i = grp * kBlockRows + 32 * w + l32;  // row loaded by this lane (operand A)

  const T* xrow = (const T*)a.x + bb * a.sx.b + hh * a.sx.h + (int64_t)i * a.sx.n;
  frag xf[NSD];
#pragma unroll
  for (int ks = 0; ks < NSD; ++ks) xf[ks] = i < N ? frag_g<T>(xrow, KS * ks + E * hl) : M::zero();

  // the fold rows of the block's columns, looked up once (a lookup inside
  // the loop would be a dependent global load)
  __shared__ int sfold[FOLD ? 256 : 1];
  if constexpr (FOLD) {
    for (int c = tid; c < pc; c += kThreads) {
      const int cc = c0 + c;
      sfold[c] = cc < ce ? a.fold[ws + cc] : 0;
    }
    __syncthreads();
  }

  const T* tab = (const T*)a.tab + hh * a.tab_hs;
  const T* bias = BIAS ? (const T*)a.bias + hh * a.bias_hs : nullptr;
  // rows addressed by token: every key row (key side), the held query rows
  // [first, first + nrows)
  const int first = a.key_side ? 0 : g.z0;
  const int nrows = a.key_side ? N : zq_last(g) + 1 - g.z0;
  float* zb = a.key_side ? a.z + (int64_t)bh * N * g.Wp : a.z + zq_off(g, bh, g.z0);
  const int row0 = grp * kBlockRows + 32 * w - first;  // this wave's first row in the slab
  const int rlim = imin(N - first, nrows);             // rows of the slab that exist
  __amdgpu_buffer_rsrc_t zr;
  if constexpr (BUF) zr = __builtin_amdgcn_make_buffer_rsrc(zb, 0, nrows * g.Wp * 4, 0x00020000);

  // table fragments (operand B: the lane's column) and bias of tile n; the
  // bias stays in the input type until it is used
  auto load_tile = [&](int n, frag (&tf)[NSD], T& braw, int& col) {
    col = c0 + 32 * n + l32;
    // (n < nsub keeps the fold lookup inside the block's own columns: the
    // window can go on beyond them, into the next block's chunk)
    const bool cv = n < nsub && col < ce;
    const int r = cv ? (FOLD ? sfold[col - c0] : ws + col) : 0;
    const T* trow = tab + (int64_t)r * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < NSD; ++ks) tf[ks] = frag_g<T>(trow, KS * ks + E * hl);
    if constexpr (BIAS) braw = bias[r];
  };
  frag tf[NSD];
  T braw = MT<T>::from_f(0.f);
  int col;
  load_tile(0, tf, braw, col);
#pragma unroll 1
  for (int n = 0; n < nsub; ++n) {
    // (past the last tile this loads row 0 again: a fixed count per iteration)
    frag tn[NSD];
    T bn = MT<T>::from_f(0.f);
    int coln;
    load_tile(n + 1, tn, bn, coln);
    f32x16 acc = zero16();
#pragma unroll
    for (int ks = 0; ks < NSD; ++ks) acc = M::mma(xf[ks], tf[ks], acc);
    const float badd = BIAS ? MT<T>::to_f(braw) : 0.f;
    if constexpr (BUF) {
      const bool cv = col < ce;  // (n < nsub here)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = row0 + res_row(hl, e);
        const uint32_t off = (cv && row < rlim) ? (uint32_t)(row * g.Wp + col) * 4u : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[e] + badd), zr, off, 0, 0);
      }
    } else if (col < ce) {
      float* zc = zb + col;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = row0 + res_row(hl, e);
        if (row < rlim) zc[(int64_t)row * g.Wp] = acc[e] + badd;
      }
    }
#pragma unroll
    for (int ks = 0; ks < NSD; ++ks) tf[ks] = tn[ks];
    braw = bn;
    col = coln;
  }
}

template <typename T, bool FOLD, bool BIAS>
static void launch_proj_b(const ProjArgs& a, int total, bool buf, hipStream_t st) {
  if (buf) hipLaunchKernelGGL((proj_kernel<T, FOLD, BIAS, true>), dim3(total), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL((proj_kernel<T, FOLD, BIAS, false>), dim3(total), dim3(kThreads), 0, st, a);
}
template <typename T>
static void launch_proj_t(const ProjArgs& a, int total, bool buf, hipStream_t st) {
  if (a.fold) {
    if (a.bias) launch_proj_b<T, true, true>(a, total, buf, st);
    else launch_proj_b<T, true, false>(a, total, buf, st);
  } else {
    if (a.bias) launch_proj_b<T, false, true>(a, total, buf, st);
    else launch_proj_b<T, false, false>(a, total, buf, st);
  }
}

hipError_t launch_phi_rows(const PhiArgs& p, int32_t* rows, hipStream_t st) {
  const int64_t n = 2LL * p.N - 1;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(phi_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, rows);
  return hipGetLastError();
}

hipError_t launch_phi_fold(const PhiArgs& p, int32_t* fold, int32_t* ub, int32_t* ue, int R,
                           hipStream_t st) {
  const int Runf = p.hi_unf - p.lo_unf + 1;
  hipLaunchKernelGGL(phi_fold_kernel, dim3((Runf + 255) / 256), dim3(256), 0, st, p, fold);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !ub) return e;
  hipLaunchKernelGGL(fold_range_clear_kernel, dim3((R + 255) / 256), dim3(256), 0, st, R, ub, ue);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fold_range_kernel, dim3((Runf + 255) / 256), dim3(256), 0, st,
                     (const int32_t*)fold, Runf, ub, ue);
  return hipGetLastError();
}

hipError_t launch_bias_unfold(int dtype, const BiasArgs& a, hipStream_t st) {
  dim3 grid((a.Runf + 255) / 256, a.Hb);
  switch (dtype) {
    case 0: hipLaunchKernelGGL(bias_unfold_kernel<float>, grid, dim3(256), 0, st, a); break;
    case 1: hipLaunchKernelGGL(bias_unfold_kernel<_Float16>, grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL(bias_unfold_kernel<__bf16>, grid, dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_proj(int dtype, const ProjArgs& a, hipStream_t st) {
  const int pc = proj_cols(a);
  const int nch = (a.ncol_tiles + pc / 64 - 1) / (pc / 64);
  const int total = a.B * a.H * a.ngroups * nch;
  if (total <= 0) return hipSuccess;
  // the (b, h) slab of Z must be below 2 GiB for 32-bit buffer offsets
  const int64_t slab_rows = a.key_side ? a.geo.N : a.geo.zr;
  const bool buf = slab_rows * a.geo.Wp * 4 < ((int64_t)1 << 31);
  switch (dtype) {
    case 0: launch_proj_t<float>(a, total, buf, st); break;
    case 1: launch_proj_t<_Float16>(a, total, buf, st); break;
    default: launch_proj_t<__bf16>(a, total, buf, st); break;
  }
  return hipGetLastError();
}

}  // namespace relpos
