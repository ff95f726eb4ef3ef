// attn_bwd_k.hip -- key-parallel backward pass.
//
// Source: "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (nanless.github.io digest), section on the backward pass: the
// key-parallel pass recomputes the scores and accumulates dK, dV and the
// key-side relation gradient dZ^K[j, r] = tau * sum_{i: phi(i,j) = r} dS_ij
// (Eq. 4), stored per offset by the block that owns the key (for a fixed key,
// queries and offsets correspond one to one); the saturated rows collect in
// two on-chip sums per key.
//
// One workgroup = one (batch, head, 128-key block); 4 waves x 32 keys; inner
// loop over 64-query tiles.  Orientation S = Q K^T: lane l owns key l % 32.
// Q and dO are staged both row-major (operands of S = Q K^T and dP = dO V^T,
// contracted over d) and transposed (operands of dV^T = dO^T P and
// dK^T = Q^T dS, contracted over the queries).
#include "qside.hpp"

namespace relpos {

__device__ inline int tile_kind_k(const Geo& g, int qt0, int jw0) {
  int omax = jw0 + 31 - qt0;
  int omin = jw0 - (qt0 + kTile - 1);
  return omax <= g.lo ? KIND_LO : (omin >= g.hi ? KIND_HI : KIND_BAND);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_k_kernel(AttnArgs a) {
  using M = MT<T>;
  using frag = typename M::frag;
  using C = TileCfg<T>;
  constexpr int KS = M::KS, E = M::E, NSD = kHeadDim / KS, NSK = kTile / KS;
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr int NT = C::kHalf ? 2 : 1;
  constexpr int TE = C::kHalf ? C::ELEMS : 1;

  __shared__ __align__(16) T sQ[2][C::ELEMS];
  __shared__ __align__(16) T sQt[NT][TE];
  __shared__ __align__(16) T sO[2][C::ELEMS];
  __shared__ __align__(16) T sOt[NT][TE];
  __shared__ __align__(16) float sL[2][kTile];
  __shared__ __align__(16) float sD[2][kTile];
  __shared__ __align__(16) float sZQ[2][2 * kTile];

  const Geo g = a.geo;
  const int N = g.N;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int total = a.B * a.H * a.nblk;
  const int lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / a.nblk;
  const int kb = lid - bh * a.nblk;  // causal: early key blocks have the most queries
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int j0b = kb * kBlockRows, jw0 = j0b + 32 * w, jk = jw0 + l32;
  const bool has_zq = a.flags & F_ZQ, has_zk = a.flags & F_ZK, has_b = a.flags & F_B;

  int kv_end = N;
  if (a.flags & F_KEYPAD) kv_end = imax(0, imin(N, a.key_len[bb]));
  const int qt_begin = g.causal ? j0b / kTile : 0;
  const int ntq = (N + kTile - 1) / kTile;
  // Whole block padded away: nothing to recompute, every output is zero.
  const int t_begin = (j0b >= kv_end) ? ntq : qt_begin;

  const T* Qp = (const T*)a.q + bb * a.sq.b + hh * a.sq.h;
  const T* Kp = (const T*)a.k + bb * a.sk.b + hh * a.sk.h;
  const T* Vp = (const T*)a.v + bb * a.sv.b + hh * a.sv.h;
  const T* dOp = (const T*)a.dO + bb * a.sdo.b + hh * a.sdo.h;
  const float* lse_bh = a.lse + (int64_t)bh * N;
  const float* D_bh = a.D + (int64_t)bh * N;
  const float* zq_bh = has_zq ? a.zq + (int64_t)bh * N * g.W : nullptr;
  const float* bun = has_b ? a.bunf + hh * a.bunf_hs : nullptr;
  const int wsk = win_k(g, kb);
  const float* zk_row = has_zk ? a.zk + ((int64_t)bh * N + jk) * g.W : nullptr;
  float* dz_row = has_zk ? a.dzk + ((int64_t)bh * N + jk) * g.W : nullptr;
  const int sig = sigma<T>(l32);

  // Key-side constants of saturated tiles: Z^K[j, first/last row] + b.
  float cst_lo = 0.f, cst_hi = 0.f;
  if (has_zk && jk < N) {
    int cb, ce;
    cols_k(g, kb, cb, ce);
    const int c0 = 0 - wsk, c1 = g.R - 1 - wsk;
    if (c0 >= cb && c0 < ce) cst_lo += zk_row[c0];
    if (c1 >= cb && c1 < ce) cst_hi += zk_row[c1];
  }
  if (has_b) {
    cst_lo += bun[0];
    cst_hi += bun[g.R - 1];
  }

  frag kf[NSD], vf[NSD];
  {
    const T* krow = Kp + (int64_t)jk * a.sk.n;
    const T* vrow = Vp + (int64_t)jk * a.sv.n;
#pragma unroll
    for (int ks = 0; ks < NSD; ++ks) {
      kf[ks] = jk < N ? frag_g<T>(krow, KS * ks + E * hl) : M::zero();
      vf[ks] = jk < N ? frag_g<T>(vrow, KS * ks + E * hl) : M::zero();
    }
  }

  Chunk rq[C::NCH], ro[C::NCH];
  float rl = 0.f, rd = 0.f, rz0 = 0.f, rz1 = 0.f;
  auto gload = [&](int t) {
    const int q0 = t * kTile;
    tile_load<T, C::kHalf>(rq, Qp, a.sq.n, q0, N, tid);
    tile_load<T, C::kHalf>(ro, dOp, a.sdo.n, q0, N, tid);
    if (tid < kTile) {
      const int i = q0 + tid;
      rl = INFINITY;
      rd = 0.f;
      if (i < N) {
        const float L = lse_bh[i];
        rl = L == -INFINITY ? INFINITY : L * kLog2e;
        rd = D_bh[i];
      }
      rz0 = 0.f;
      rz1 = 0.f;
      if (has_zq && i < N) {
        const int grp = i / kGroup;
        const int wq = win_q(g, grp);
        int cb, ce;
        cols_q(g, grp, cb, ce);
        const float* zr = zq_bh + (int64_t)i * g.W;
        const int c0 = 0 - wq, c1 = g.R - 1 - wq;
        if (c0 >= cb && c0 < ce) rz0 = zr[c0];
        if (c1 >= cb && c1 < ce) rz1 = zr[c1];
      }
    }
  };
  auto sstore = [&](int buf) {
    tile_store_rm<T, C::kHalf>(sQ[buf], rq, tid);
    tile_store_rm<T, C::kHalf>(sO[buf], ro, tid);
    if constexpr (C::kHalf) {
      tile_store_tr<T>(sQt[buf], rq, tid);
      tile_store_tr<T>(sOt[buf], ro, tid);
    }
    if (tid < kTile) {
      sL[buf][tid] = rl;
      sD[buf][tid] = rd;
      sZQ[buf][tid] = rz0;
      sZQ[buf][kTile + tid] = rz1;
    }
  };

  f32x16 dk[2], dv[2];
  dk[0] = zero16();
  dk[1] = zero16();
  dv[0] = zero16();
  dv[1] = zero16();
  float acc_lo = 0.f, acc_hi = 0.f;
  const float sc2 = a.scale2;

  if (t_begin < ntq) {
    gload(t_begin);
    sstore(0);
  }
  __syncthreads();

  for (int t = t_begin; t < ntq; ++t) {
    const int buf = (t - t_begin) & 1;
    if (t + 1 < ntq) gload(t + 1);
    const int qt0 = t * kTile;
    const bool active = jw0 < imin(N, kv_end) && !(g.causal && qt0 + kTile - 1 < jw0);
    if (active) {
      const int kind = tile_kind_k(g, qt0, jw0);
      const bool needmask = (qt0 + kTile > N) || (jw0 + 32 > kv_end) ||
                            (g.causal && jw0 + 31 > qt0);
      f32x16 s[2];
      if (kind != KIND_BAND) {
        if (has_zq) {
          const float* z = sZQ[buf] + (kind == KIND_LO ? 0 : kTile);
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            float v[16];
            lds_rows16<T>(z + 32 * st, hl, v);
#pragma unroll
            for (int e = 0; e < 16; ++e) s[st][e] = v[e];
          }
        } else {
          s[0] = zero16();
          s[1] = zero16();
        }
      } else {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int i = qt0 + 32 * st + kappa<T>(hl, e);
            const bool live = i < N && jk < kv_end && !(g.causal && jk > i);
            float v = 0.f;
            if (live) {
              const int r = rrow(g, jk - i);
              if (has_zq) v += zq_bh[(int64_t)i * g.W + r - win_q(g, i / kGroup)];
              if (has_zk) v += zk_row[r - wsk];
              if (has_b) v += bun[r];
            }
            s[st][e] = v;
          }
      }
#pragma unroll
      for (int ks = 0; ks < NSD; ++ks)
#pragma unroll
        for (int st = 0; st < 2; ++st)
          s[st] = M::mma(frag_rm<T>(sQ[buf], 32 * st + sig, KS * ks + E * hl), kf[ks], s[st]);
      if (needmask) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int i = qt0 + 32 * st + kappa<T>(hl, e);
            if (i >= N || jk >= kv_end || (g.causal && jk > i)) s[st][e] = -INFINITY;
          }
      }
      const float cst = kind == KIND_LO ? cst_lo : (kind == KIND_HI ? cst_hi : 0.f);
      const float off = cst * sc2;

      f32x16 dp[2];
      dp[0] = zero16();
      dp[1] = zero16();
#pragma unroll
      for (int ks = 0; ks < NSD; ++ks)
#pragma unroll
        for (int st = 0; st < 2; ++st)
          dp[st] = M::mma(frag_rm<T>(sO[buf], 32 * st + sig, KS * ks + E * hl), vf[ks], dp[st]);

      float p[2][16], ds[2][16];
      float tsum = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float L[16], Dv[16];
        lds_rows16<T>(sL[buf] + 32 * st, hl, L);
        lds_rows16<T>(sD[buf] + 32 * st, hl, Dv);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          p[st][e] = exp2_fast(fmaf(s[st][e], sc2, off - L[e]));
          ds[st][e] = p[st][e] * (dp[st][e] - Dv[e]);
          tsum += ds[st][e];
        }
      }

      if (has_zk) {
        if (kind == KIND_LO) {
          acc_lo += tsum;
        } else if (kind == KIND_HI) {
          acc_hi += tsum;
        } else {
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int i = qt0 + 32 * st + kappa<T>(hl, e);
              const int o = jk - i;
              if (o <= g.lo) {
                acc_lo += ds[st][e];
              } else if (o >= g.hi) {
                acc_hi += ds[st][e];
              } else if (i < N && jk < N && !(g.causal && jk > i)) {
                dz_row[o - g.lo - wsk] = a.tau * ds[st][e];
              }
            }
        }
      }

      frag pf[NSK], sf[NSK];
#pragma unroll
      for (int ks = 0; ks < NSK; ++ks) {
        const int st = (ks * KS) / 32, e0 = ((ks * KS) % 32) / KS * E;
        pf[ks] = M::pack(&p[st][e0]);
        sf[ks] = M::pack(&ds[st][e0]);
      }
      const T* ot = C::kHalf ? sOt[C::kHalf ? buf : 0] : sO[buf];
      const T* qt = C::kHalf ? sQt[C::kHalf ? buf : 0] : sQ[buf];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int ks = 0; ks < NSK; ++ks) {
          dv[dt] = M::mma(frag_t<T>(ot, 32 * dt + l32, KS * ks + E * hl), pf[ks], dv[dt]);
          dk[dt] = M::mma(frag_t<T>(qt, 32 * dt + l32, KS * ks + E * hl), sf[ks], dk[dt]);
        }
    }
    if (t + 1 < ntq) sstore(buf ^ 1);
    __syncthreads();
  }

  if (jk < N) {
    T* vrow = (T*)a.dv + bb * a.sdv.b + hh * a.sdv.h + (int64_t)jk * a.sdv.n;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = 32 * dt + 8 * e4 + 4 * hl;
        store4<T>(vrow + d, dv[dt][4 * e4], dv[dt][4 * e4 + 1], dv[dt][4 * e4 + 2],
                  dv[dt][4 * e4 + 3]);
      }
    if (has_zk) {
      float* prow = (float*)a.dk + ((int64_t)bh * N + jk) * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int d = 32 * dt + 8 * e4 + 4 * hl;
          store4<float>(prow + d, a.tau * dk[dt][4 * e4], a.tau * dk[dt][4 * e4 + 1],
                        a.tau * dk[dt][4 * e4 + 2], a.tau * dk[dt][4 * e4 + 3]);
        }
    } else {
      T* krow = (T*)a.dk + bb * a.sdk.b + hh * a.sdk.h + (int64_t)jk * a.sdk.n;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int d = 32 * dt + 8 * e4 + 4 * hl;
          store4<T>(krow + d, a.tau * dk[dt][4 * e4], a.tau * dk[dt][4 * e4 + 1],
                    a.tau * dk[dt][4 * e4 + 2], a.tau * dk[dt][4 * e4 + 3]);
        }
    }
  }

  if (has_zk) {
    acc_lo += __shfl_xor(acc_lo, 32);
    acc_hi += __shfl_xor(acc_hi, 32);
    if (jk < N) {
      int cb, ce;
      cols_k(g, kb, cb, ce);
      const int c0 = 0 - wsk, c1 = g.R - 1 - wsk;
      if (hl == 0) {
        if (g.R == 1) {
          if (c0 >= cb && c0 < ce) dz_row[c0] = a.tau * (acc_lo + acc_hi);
        } else {
          if (c0 >= cb && c0 < ce) dz_row[c0] = a.tau * acc_lo;
          if (c1 >= cb && c1 < ce) dz_row[c1] = a.tau * acc_hi;
        }
      }
      // Queries written by the band stores: [q_lo, q_hi).  Interior columns
      // of any other query carry no gradient and are zeroed.
      const bool wave_ran = jw0 < imin(N, kv_end) && t_begin < ntq;
      const int q_lo = t_begin * kTile;
      const int q_hi = wave_ran ? N : q_lo;
      const int ib = imax(cb, 1 - wsk), ie = imin(ce, g.R - 1 - wsk);
      // query of column col is jk - (col + wsk + lo) = shift - col
      const int shift = jk - wsk - g.lo;
      // i < q_lo  <=>  col > shift - q_lo
      for (int col = imax(ib, shift - q_lo + 1) + hl; col < ie; col += 2) dz_row[col] = 0.f;
      // i >= q_hi <=>  col <= shift - q_hi
      const int b_end = imin(ie, shift - q_hi + 1);
      for (int col = ib + hl; col < b_end; col += 2) dz_row[col] = 0.f;
    }
  }
}

template <typename T>
static hipError_t launch_bwd_k_t(const AttnArgs& a, hipStream_t st) {
  const int total = a.B * a.H * a.nblk;
  hipLaunchKernelGGL(bwd_k_kernel<T>, dim3(total), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_k(int dtype, const AttnArgs& a, hipStream_t st) {
  switch (dtype) {
    case 0: return launch_bwd_k_t<float>(a, st);
    case 1: return launch_bwd_k_t<_Float16>(a, st);
    default: return launch_bwd_k_t<__bf16>(a, st);
  }
}

}  // namespace relpos
