// attn_bwd_q.hip -- backward preprocess D and the query-parallel backward pass.
//
// Source: "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (nanless.github.io digest), section on the backward pass: a
// query-parallel pass recomputes the scores and accumulates the query
// gradient and the query-side relation gradient; for a fixed query, keys and
// offsets correspond one to one, so the per-row sum of Eq. (4),
// dZ^Q[i, r] = tau * sum_{j: phi(i,j) = r} dS_ij, is stored per offset by the
// block that owns the query (single writer, no atomics, fixed order); the two
// saturated rows collect into two on-chip sums per query.
//
// D_i = sum_d dO_id O_id (the row term of dS = P (dP - D)) is the standard
// FlashAttention backward preprocess, computed by pre_kernel.
#include "qside.hpp"

namespace relpos {

// D[bh][i] = sum_d dO[i][d] * O[i][d]; 8 lanes per row.
template <typename T>
__global__ __launch_bounds__(kThreads) void pre_kernel(PreArgs a) {
  using C = TileCfg<T>;
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 8) + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  float acc = 0.f;
  if (row < rows) {
    const int i = (int)(row % a.N);
    const int64_t bh = row / a.N;
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);
    const T* o = (const T*)a.o + b * a.so.b + h * a.so.h + (int64_t)i * a.so.n + 8 * part;
    const T* d = (const T*)a.dO + b * a.sdo.b + h * a.sdo.h + (int64_t)i * a.sdo.n + 8 * part;
    if constexpr (C::kHalf) {
      typename MT<T>::frag x = *reinterpret_cast<const typename MT<T>::frag*>(o);
      typename MT<T>::frag y = *reinterpret_cast<const typename MT<T>::frag*>(d);
#pragma unroll
      for (int t = 0; t < 8; ++t) acc = fmaf(MT<T>::to_f(x[t]), MT<T>::to_f(y[t]), acc);
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) acc = fmaf(o[t], d[t], acc);
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < rows && part == 0) a.D[row] = acc;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_q_kernel(AttnArgs a) {
  using M = MT<T>;
  using frag = typename M::frag;
  using C = TileCfg<T>;
  constexpr int KS = M::KS, E = M::E, NSD = kHeadDim / KS, NSK = kTile / KS;
  constexpr float kLog2e = 1.4426950408889634f;

  __shared__ __align__(16) T sK[2][C::ELEMS];
  __shared__ __align__(16) T sKt[C::kHalf ? 2 : 1][C::kHalf ? C::ELEMS : 1];
  __shared__ __align__(16) T sV[2][C::ELEMS];
  __shared__ __align__(16) float sZK[2][2 * kTile];

  const Geo g = a.geo;
  const int N = g.N;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int total = a.B * a.H * a.nblk;
  const int lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / a.nblk;
  int qb = lid - bh * a.nblk;
  if (g.causal) qb = a.nblk - 1 - qb;
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int i0 = qb * kBlockRows, iw0 = i0 + 32 * w, iq = iw0 + l32;

  int kv_end = N;
  if (a.flags & F_KEYPAD) kv_end = imax(0, imin(N, a.key_len[bb]));
  int kv_blk = kv_end;
  if (g.causal) kv_blk = imin(kv_blk, i0 + kBlockRows);
  const int nkt = kv_blk > 0 ? (kv_blk + kTile - 1) / kTile : 0;
  const int kv_lim = imin(N, nkt * kTile);  // keys written by the band stores

  const T* Qp = (const T*)a.q + bb * a.sq.b + hh * a.sq.h;
  const T* Kp = (const T*)a.k + bb * a.sk.b + hh * a.sk.h;
  const T* Vp = (const T*)a.v + bb * a.sv.b + hh * a.sv.h;
  const T* dOp = (const T*)a.dO + bb * a.sdo.b + hh * a.sdo.h;

  QCtx c;
  c.iq = iq;
  c.hl = hl;
  c.sig = sigma<T>(l32);
  c.kv_end = kv_end;
  c.has_zq = a.flags & F_ZQ;
  c.has_zk = a.flags & F_ZK;
  c.has_b = a.flags & F_B;
  c.wsq = win_q(g, qb);
  c.zq_row = c.has_zq ? a.zq + ((int64_t)bh * N + iq) * g.W : nullptr;
  c.zkb = c.has_zk ? a.zk + (int64_t)bh * N * g.W : nullptr;
  c.bun = c.has_b ? a.bunf + hh * a.bunf_hs : nullptr;
  const bool need_dz = a.flags & F_ZQ_NEEDED;
  float cst_lo, cst_hi;
  qside_consts(g, c, qb, cst_lo, cst_hi);

  frag qf[NSD], df[NSD];
  float lse2 = INFINITY, Dl = 0.f;
  {
    const T* qrow = Qp + (int64_t)iq * a.sq.n;
    const T* drow = dOp + (int64_t)iq * a.sdo.n;
#pragma unroll
    for (int ks = 0; ks < NSD; ++ks) {
      qf[ks] = iq < N ? frag_g<T>(qrow, KS * ks + E * hl) : M::zero();
      df[ks] = iq < N ? frag_g<T>(drow, KS * ks + E * hl) : M::zero();
    }
    if (iq < N) {
      const float L = a.lse[(int64_t)bh * N + iq];
      lse2 = L == -INFINITY ? INFINITY : L * kLog2e;  // a dead row gives P = 0
      Dl = a.D[(int64_t)bh * N + iq];
    }
  }
  float* dz_row = need_dz ? a.dzq + ((int64_t)bh * N + iq) * g.W : nullptr;

  Chunk rk[C::NCH], rv[C::NCH];
  float rz0 = 0.f, rz1 = 0.f;
  auto gload = [&](int t) {
    const int j0 = t * kTile;
    tile_load<T, C::kHalf>(rk, Kp, a.sk.n, j0, N, tid);
    tile_load<T, false>(rv, Vp, a.sv.n, j0, N, tid);
    if (c.has_zk && tid < kTile) kside_sat(g, c.zkb, j0 + tid, rz0, rz1);
  };
  auto sstore = [&](int buf) {
    tile_store_rm<T, C::kHalf>(sK[buf], rk, tid);
    if constexpr (C::kHalf) tile_store_tr<T>(sKt[buf], rk, tid);
    tile_store_rm<T, false>(sV[buf], rv, tid);
    if (c.has_zk && tid < kTile) {
      sZK[buf][tid] = rz0;
      sZK[buf][kTile + tid] = rz1;
    }
  };

  f32x16 dq[2];
  dq[0] = zero16();
  dq[1] = zero16();
  float acc_lo = 0.f, acc_hi = 0.f;
  const float sc2 = a.scale2;

  if (nkt > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  for (int t = 0; t < nkt; ++t) {
    const int buf = t & 1;
    if (t + 1 < nkt) gload(t + 1);
    const int j0 = t * kTile;
    const bool active = iw0 < N && !(g.causal && j0 > iw0 + 31);
    if (active) {
      const int kind = tile_kind_q(g, j0, iw0);
      const bool needmask = (j0 + kTile > kv_end) || (g.causal && j0 + kTile - 1 > iw0);
      f32x16 s[2];
      qside_scores<T>(s, g, c, sK[buf], sZK[buf], qf, kind, j0, needmask);
      const float cst = kind == KIND_LO ? cst_lo : (kind == KIND_HI ? cst_hi : 0.f);
      const float off = cst * sc2 - lse2;

      f32x16 dp[2];
      dp[0] = zero16();
      dp[1] = zero16();
#pragma unroll
      for (int ks = 0; ks < NSD; ++ks)
#pragma unroll
        for (int st = 0; st < 2; ++st)
          dp[st] = M::mma(frag_rm<T>(sV[buf], 32 * st + c.sig, KS * ks + E * hl), df[ks], dp[st]);

      float ds[2][16];
      float tsum = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2_fast(fmaf(s[st][e], sc2, off));
          ds[st][e] = p * (dp[st][e] - Dl);
          tsum += ds[st][e];
        }

      if (need_dz) {
        if (kind == KIND_LO) {
          acc_lo += tsum;
        } else if (kind == KIND_HI) {
          acc_hi += tsum;
        } else {
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int j = j0 + 32 * st + kappa<T>(hl, e);
              const int o = j - iq;
              if (o <= g.lo) {
                acc_lo += ds[st][e];
              } else if (o >= g.hi) {
                acc_hi += ds[st][e];
              } else if (iq < N && j < N && !(g.causal && j > iq)) {
                dz_row[o - g.lo - c.wsq] = a.tau * ds[st][e];
              }
            }
        }
      }

      frag sf[NSK];
#pragma unroll
      for (int ks = 0; ks < NSK; ++ks) {
        const int st = (ks * KS) / 32, e0 = ((ks * KS) % 32) / KS * E;
        sf[ks] = M::pack(&ds[st][e0]);
      }
      const T* kt = C::kHalf ? sKt[C::kHalf ? buf : 0] : sK[buf];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int ks = 0; ks < NSK; ++ks)
          dq[dt] = M::mma(frag_t<T>(kt, 32 * dt + l32, KS * ks + E * hl), sf[ks], dq[dt]);
    }
    if (t + 1 < nkt) sstore(buf ^ 1);
    __syncthreads();
  }

  if (iq < N) {
    // dQ = tau * dS K  (plus dZ^Q aQ added by the contraction when aQ is present)
    if (a.flags & F_ZQ) {
      float* prow = (float*)a.dq + ((int64_t)bh * N + iq) * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int d = 32 * dt + 8 * e4 + 4 * hl;
          store4<float>(prow + d, a.tau * dq[dt][4 * e4], a.tau * dq[dt][4 * e4 + 1],
                        a.tau * dq[dt][4 * e4 + 2], a.tau * dq[dt][4 * e4 + 3]);
        }
    } else {
      T* orow = (T*)a.dq + bb * a.sdq.b + hh * a.sdq.h + (int64_t)iq * a.sdq.n;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int d = 32 * dt + 8 * e4 + 4 * hl;
          store4<T>(orow + d, a.tau * dq[dt][4 * e4], a.tau * dq[dt][4 * e4 + 1],
                    a.tau * dq[dt][4 * e4 + 2], a.tau * dq[dt][4 * e4 + 3]);
        }
    }
  }

  if (need_dz) {
    acc_lo += __shfl_xor(acc_lo, 32);
    acc_hi += __shfl_xor(acc_hi, 32);
    if (iq < N) {
      int cb, ce;
      cols_q(g, qb, cb, ce);
      const int ws = c.wsq;
      const int c0 = 0 - ws, c1 = g.R - 1 - ws;
      if (hl == 0) {
        if (g.R == 1) {
          if (c0 >= cb && c0 < ce) dz_row[c0] = a.tau * (acc_lo + acc_hi);
        } else {
          if (c0 >= cb && c0 < ce) dz_row[c0] = a.tau * acc_lo;
          if (c1 >= cb && c1 < ce) dz_row[c1] = a.tau * acc_hi;
        }
      }
      // Interior columns whose key was never visited (j < 0 or j >= kv_lim)
      // hold no gradient: write zeros so the whole live window is defined.
      const int ib = imax(cb, 1 - ws), ie = imin(ce, g.R - 1 - ws);
      const int shift = iq + g.lo + ws;  // key of column col is col + shift
      const int a_end = imin(ie, -shift);
      for (int col = ib + hl; col < a_end; col += 2) dz_row[col] = 0.f;
      for (int col = imax(ib, kv_lim - shift) + hl; col < ie; col += 2) dz_row[col] = 0.f;
    }
  }
}

template <typename T>
static hipError_t launch_pre_t(const PreArgs& p, hipStream_t st) {
  const int64_t rows = (int64_t)p.B * p.H * p.N;
  const int pre_blocks = (int)((rows + kThreads / 8 - 1) / (kThreads / 8));
  hipLaunchKernelGGL(pre_kernel<T>, dim3(pre_blocks), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_bwd_q_t(const AttnArgs& a, hipStream_t st) {
  const int total = a.B * a.H * a.nblk;
  hipLaunchKernelGGL(bwd_q_kernel<T>, dim3(total), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pre(int dtype, const PreArgs& p, hipStream_t st) {
  switch (dtype) {
    case 0: return launch_pre_t<float>(p, st);
    case 1: return launch_pre_t<_Float16>(p, st);
    default: return launch_pre_t<__bf16>(p, st);
  }
}

hipError_t launch_bwd_q(int dtype, const AttnArgs& a, hipStream_t st) {
  switch (dtype) {
    case 0: return launch_bwd_q_t<float>(a, st);
    case 1: return launch_bwd_q_t<_Float16>(a, st);
    default: return launch_bwd_q_t<__bf16>(a, st);
  }
}

}  // namespace relpos
