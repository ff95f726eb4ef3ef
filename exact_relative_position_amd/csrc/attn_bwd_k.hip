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
// Q and dO tiles go into LDS both row-major (operands of S = Q K^T and
// dP = dO V^T, contracted over d) and transposed from query-contiguous
// copies (operands of dV^T = dO^T P and dK^T = Q^T dS, contracted over the
// queries), all by direct loads; the query loop runs in three segments.
#include "qside.hpp"

namespace relpos {

__device__ inline int tile_kind_k(const Geo& g, int qt0, int jw0) {
  int omax = jw0 + 31 - qt0;
  int omin = jw0 - (qt0 + kTile - 1);
  return omax <= g.lo ? KIND_LO : (omin >= g.hi ? KIND_HI : KIND_BAND);
}

__device__ inline int floor_div_k(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
__device__ inline int ceil_div_k(int a, int b) { return -floor_div_k(-a, b); }

template <typename T>
struct BwdK {
  using M = MT<T>;
  using frag = typename M::frag;
  static constexpr bool kHalf = sizeof(T) == 2;
  static constexpr int KS = M::KS, E = M::E, NSD = kHeadDim / KS;
  static constexpr int KPS = 32 / KS;  // MFMA k-steps per 32-query half
  static constexpr int TB = DTile<T>::BYTES;

  char* sQ;     // [2][TB] Q rows
  char* sQt;    // [2][TB] Q^T (16-bit)
  char* sO;     // [2][TB] dO rows
  char* sOt;    // [2][TB] dO^T (16-bit)
  float* sL;    // [2][kTile] padded log2-domain LSE of the tile's queries
  float* sD;    // [2][kTile]
  float* sZQ;   // [2][2 * kTile]

  Geo g;
  int w, lane, hl, l32, jw0, jk, sig, ntq, N, kv_end, wsk;
  bool has_zq, has_zk, has_b;
  float cst_lo, cst_hi, sc2, tau;
  const T* Qb;
  const T* Qtb;
  const T* Ob;
  const T* Otb;
  const float* L2b;
  const float* Db;
  const float* zq_bh;
  const float* zk_row;
  const float* bun;
  float* dz_row;
  int64_t sq, so, Np;
  DLoader<T> ldQ, ldQt, ldO, ldOt;
  frag kf[NSD], vf[NSD];
  f32x16 dk[2], dv[2];
  float acc_lo, acc_hi;

  __device__ __forceinline__ void issue(int t, int buf) {
    const int q0 = t * kTile;
    ldQ.load(sQ + buf * TB, Qb + (int64_t)q0 * sq, N - q0, lane);
    ldO.load(sO + buf * TB, Ob + (int64_t)q0 * so, N - q0, lane);
    if constexpr (kHalf) {
      ldQt.load(sQt + buf * TB, Qtb + q0, 64, lane);
      ldOt.load(sOt + buf * TB, Otb + q0, 64, lane);
    }
    if (w == 0) {
      dword_direct((char*)(sL + buf * kTile), L2b + q0 + lane, true, lane);
    } else if (w == 1) {
      dword_direct((char*)(sD + buf * kTile), Db + q0 + lane, true, lane);
    } else if (has_zq) {
      const float* p = qside_sat_ptr(g, zq_bh, q0 + lane, w - 2);
      dword_direct((char*)(sZQ + buf * 2 * kTile + (w - 2) * kTile), p, p != nullptr, lane);
    }
  }

  template <int SEG>
  __device__ __forceinline__ void tile(int t, int buf) {
    const int qt0 = t * kTile;
    if (jw0 >= imin(N, kv_end) || (g.causal && qt0 + kTile - 1 < jw0)) return;
    const int kind = SEG == KIND_BAND ? tile_kind_k(g, qt0, jw0) : SEG;
    const bool needmask = (qt0 + kTile > N) || (jw0 + 32 > kv_end) || (g.causal && jw0 + 31 > qt0);
    const char* tQ = sQ + buf * TB;
    const char* tO = sO + buf * TB;
    const char* tQt = kHalf ? sQt + buf * TB : tQ;
    const char* tOt = kHalf ? sOt + buf * TB : tO;
    const float cst = kind == KIND_LO ? cst_lo : (kind == KIND_HI ? cst_hi : 0.f);
    const float off = cst * sc2;
    // the two 32-query halves of the tile, one after the other
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x16 s;
      int ks0 = 0;
      if (kind != KIND_BAND && !has_zq) {
        s = M::mma(dfrag<T>(tQ, 32 * st + sig, E * hl), kf[0], zero16());
        ks0 = 1;
      } else if (kind != KIND_BAND) {
        float v[16];
        lds_rows16<T>(sZQ + buf * 2 * kTile + (kind == KIND_LO ? 0 : kTile) + 32 * st, hl, v);
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = v[e];
      } else {
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
          s[e] = v;
        }
      }
#pragma unroll
      for (int ks = 0; ks < NSD; ++ks) {
        if (ks < ks0) continue;
        s = M::mma(dfrag<T>(tQ, 32 * st + sig, KS * ks + E * hl), kf[ks], s);
      }
      if (needmask) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int i = qt0 + 32 * st + kappa<T>(hl, e);
          if (i >= N || jk >= kv_end || (g.causal && jk > i)) s[e] = -INFINITY;
        }
      }
      f32x16 dp = M::mma(dfrag<T>(tO, 32 * st + sig, E * hl), vf[0], zero16());
#pragma unroll
      for (int ks = 1; ks < NSD; ++ks)
        dp = M::mma(dfrag<T>(tO, 32 * st + sig, KS * ks + E * hl), vf[ks], dp);

      float p[16], ds[16];
      {
        float L[16], Dv[16];
        lds_rows16<T>(sL + buf * kTile + 32 * st, hl, L);
        lds_rows16<T>(sD + buf * kTile + 32 * st, hl, Dv);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          p[e] = exp2_fast(fmaf(s[e], sc2, off - L[e]));
          ds[e] = p[e] * (dp[e] - Dv[e]);
        }
      }
      if (has_zk) {
        if (SEG != KIND_BAND || kind != KIND_BAND) {
          float tsum = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) tsum += ds[e];
          if (kind == KIND_LO) acc_lo += tsum; else acc_hi += tsum;
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int i = qt0 + 32 * st + kappa<T>(hl, e);
            const int o = jk - i;
            if (o <= g.lo) {
              acc_lo += ds[e];
            } else if (o >= g.hi) {
              acc_hi += ds[e];
            } else if (i < N && jk < N && !(g.causal && jk > i)) {
              dz_row[o - g.lo - wsk] = tau * ds[e];
            }
          }
        }
      }
      frag pf[KPS], sf[KPS];
#pragma unroll
      for (int kk = 0; kk < KPS; ++kk) {
        pf[kk] = M::pack(&p[kk * E]);
        sf[kk] = M::pack(&ds[kk * E]);
      }
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int kk = 0; kk < KPS; ++kk) {
          const int col = KS * (KPS * st + kk) + E * hl;
          frag of, qf;
          if constexpr (kHalf) {
            of = dfrag<T>(tOt, 32 * dt + l32, col);
            qf = dfrag<T>(tQt, 32 * dt + l32, col);
          } else {
            of = dfrag_t32(tO, 32 * dt + l32, col);
            qf = dfrag_t32(tQ, 32 * dt + l32, col);
          }
          dv[dt] = M::mma(of, pf[kk], dv[dt]);
          dk[dt] = M::mma(qf, sf[kk], dk[dt]);
        }
    }
  }

  template <int SEG>
  __device__ __forceinline__ void segment(int tb, int te) {
    for (int t = tb; t < te; ++t) {
      const int buf = t & 1;
      if (t + 1 < ntq) issue(t + 1, buf ^ 1);
      tile<SEG>(t, buf);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
    }
  }
};

template <typename T>
__global__ __launch_bounds__(kThreads, 2) void bwd_k_kernel(AttnArgs a) {
  using M = MT<T>;
  using K = BwdK<T>;
  constexpr int TB = DTile<T>::BYTES;
  __shared__ __align__(16) char sQ[2 * TB];
  __shared__ __align__(16) char sQt[K::kHalf ? 2 * TB : 16];
  __shared__ __align__(16) char sO[2 * TB];
  __shared__ __align__(16) char sOt[K::kHalf ? 2 * TB : 16];
  __shared__ __align__(16) float sL[2 * kTile];
  __shared__ __align__(16) float sD[2 * kTile];
  __shared__ __align__(16) float sZQ[2 * 2 * kTile];

  K k;
  k.sQ = sQ;
  k.sQt = sQt;
  k.sO = sO;
  k.sOt = sOt;
  k.sL = sL;
  k.sD = sD;
  k.sZQ = sZQ;
  k.g = a.geo;
  const Geo& g = k.g;
  const int N = g.N;
  k.N = N;
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  k.w = w;
  k.lane = lane;
  k.hl = hl;
  k.l32 = l32;
  const int total = a.B * a.H * a.nblk;
  const int lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / a.nblk;
  const int kb = lid - bh * a.nblk;  // causal: early key blocks have the most queries
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int j0b = kb * kBlockRows, jw0 = j0b + 32 * w, jk = jw0 + l32;
  k.jw0 = jw0;
  k.jk = jk;
  k.sig = sigma<T>(l32);
  k.has_zq = a.flags & F_ZQ;
  k.has_zk = a.flags & F_ZK;
  k.has_b = a.flags & F_B;

  int kv_end = N;
  if (a.flags & F_KEYPAD) kv_end = imax(0, imin(N, a.key_len[bb]));
  k.kv_end = kv_end;
  const int qt_begin = g.causal ? j0b / kTile : 0;
  const int ntq = (N + kTile - 1) / kTile;
  k.ntq = ntq;
  // Whole block padded away: nothing to recompute, every output is zero.
  const int t_begin = (j0b >= kv_end) ? ntq : qt_begin;

  k.Qb = (const T*)a.q + bb * a.sq.b + hh * a.sq.h;
  k.Ob = (const T*)a.dO + bb * a.sdo.b + hh * a.sdo.h;
  k.sq = a.sq.n;
  k.so = a.sdo.n;
  k.Np = a.Np;
  k.ldQ.init(a.sq.n, w, lane);
  k.ldO.init(a.sdo.n, w, lane);
  if constexpr (K::kHalf) {
    k.Qtb = (const T*)a.qt + (int64_t)bh * kHeadDim * a.Np;
    k.Otb = (const T*)a.dot + (int64_t)bh * kHeadDim * a.Np;
    k.ldQt.init(a.Np, w, lane);
    k.ldOt.init(a.Np, w, lane);
  }
  k.L2b = a.L2 + (int64_t)bh * a.Np;
  k.Db = a.D + (int64_t)bh * a.Np;
  k.zq_bh = k.has_zq ? a.zq + (int64_t)bh * N * g.W : nullptr;
  k.bun = k.has_b ? a.bunf + hh * a.bunf_hs : nullptr;
  k.wsk = win_k(g, kb);
  k.zk_row = k.has_zk ? a.zk + ((int64_t)bh * N + jk) * g.W : nullptr;
  k.dz_row = k.has_zk ? a.dzk + ((int64_t)bh * N + jk) * g.W : nullptr;
  k.sc2 = a.scale2;
  k.tau = a.tau;

  // Key-side constants of saturated tiles: Z^K[j, first/last row] + b.
  k.cst_lo = 0.f;
  k.cst_hi = 0.f;
  if (k.has_zk && jk < N) {
    int cb, ce;
    cols_k(g, kb, cb, ce);
    const int c0 = 0 - k.wsk, c1 = g.R - 1 - k.wsk;
    if (c0 >= cb && c0 < ce) k.cst_lo += k.zk_row[c0];
    if (c1 >= cb && c1 < ce) k.cst_hi += k.zk_row[c1];
  }
  if (k.has_b) {
    k.cst_lo += k.bun[0];
    k.cst_hi += k.bun[g.R - 1];
  }
  {
    const T* krow = (const T*)a.k + bb * a.sk.b + hh * a.sk.h + (int64_t)jk * a.sk.n;
    const T* vrow = (const T*)a.v + bb * a.sv.b + hh * a.sv.h + (int64_t)jk * a.sv.n;
#pragma unroll
    for (int ks = 0; ks < K::NSD; ++ks) {
      k.kf[ks] = jk < N ? frag_g<T>(krow, K::KS * ks + K::E * hl) : M::zero();
      k.vf[ks] = jk < N ? frag_g<T>(vrow, K::KS * ks + K::E * hl) : M::zero();
    }
  }
  k.dk[0] = zero16();
  k.dk[1] = zero16();
  k.dv[0] = zero16();
  k.dv[1] = zero16();
  k.acc_lo = 0.f;
  k.acc_hi = 0.f;

  // segments over the query tiles [t_begin, ntq): all offsets >= hi first,
  // band, then all offsets <= lo
  const int tA = imin(ntq, imax(t_begin, floor_div_k(j0b - (kTile - 1) - g.hi, kTile) + 1));
  const int tB = imin(ntq, imax(tA, ceil_div_k(j0b + kBlockRows - 1 - g.lo, kTile)));

  if (t_begin < ntq) k.issue(t_begin, t_begin & 1);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  k.template segment<KIND_HI>(t_begin, tA);
  k.template segment<KIND_BAND>(tA, tB);
  k.template segment<KIND_LO>(tB, ntq);

  if (jk < N) {
    T* vrow = (T*)a.dv + bb * a.sdv.b + hh * a.sdv.h + (int64_t)jk * a.sdv.n;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = 32 * dt + 8 * e4 + 4 * hl;
        store4<T>(vrow + d, k.dv[dt][4 * e4], k.dv[dt][4 * e4 + 1], k.dv[dt][4 * e4 + 2],
                  k.dv[dt][4 * e4 + 3]);
      }
    if (k.has_zk) {
      float* prow = (float*)a.dk + ((int64_t)bh * N + jk) * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int d = 32 * dt + 8 * e4 + 4 * hl;
          store4<float>(prow + d, a.tau * k.dk[dt][4 * e4], a.tau * k.dk[dt][4 * e4 + 1],
                        a.tau * k.dk[dt][4 * e4 + 2], a.tau * k.dk[dt][4 * e4 + 3]);
        }
    } else {
      T* krow = (T*)a.dk + bb * a.sdk.b + hh * a.sdk.h + (int64_t)jk * a.sdk.n;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int d = 32 * dt + 8 * e4 + 4 * hl;
          store4<T>(krow + d, a.tau * k.dk[dt][4 * e4], a.tau * k.dk[dt][4 * e4 + 1],
                    a.tau * k.dk[dt][4 * e4 + 2], a.tau * k.dk[dt][4 * e4 + 3]);
        }
    }
  }

  if (k.has_zk) {
    const float acc_lo = k.acc_lo + __shfl_xor(k.acc_lo, 32);
    const float acc_hi = k.acc_hi + __shfl_xor(k.acc_hi, 32);
    float* dz_row = k.dz_row;
    const int wsk = k.wsk;
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
