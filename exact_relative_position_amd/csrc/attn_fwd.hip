// attn_fwd.hip -- fused forward of relative-position attention on gfx950.
//
// Source: "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (nanless.github.io digest): pipeline section (FlashAttention outer
// loop over query blocks, inner loop over key blocks, online softmax, the
// relation response added on chip), score formula Eq. (2), constant tiles and
// the three-segment key loop.
//
// One workgroup = one (batch, head, 128-query block); 4 waves x 32 queries.
// Per 64-key tile: K and V^T (read from a key-contiguous copy of V) go from
// HBM straight into LDS with global_load_lds_dwordx4 (no staging registers),
// double buffered; S^T = K Q^T and O^T += V^T P^T run on
// v_mfma_f32_32x32x16_{f16,bf16} (32x32x2_f32 for fp32 inputs, whose V tile
// is read transposed from its row-major copy).
//
// Three-segment key loop: two comparisons per tile against the thresholds
// split the block's key tiles into a left-saturated run, a band run and a
// right-saturated run.  Each run is its own loop, compiled for its kind, so
// the saturated loops contain no per-score lookup and no gather (and the
// next tile's prefetch is never held up behind one).  Inside the band run
// each wave refines the kind for its own 32 queries.
//
// Softmax: base-2 with tau*log2(e) folded into one FMA per score; the
// reference maximum is only moved when a row's maximum grows by more than
// 2^8, so most tiles skip the rescaling of the accumulator (exact: the final
// division uses the same reference).
#include "qside.hpp"

namespace relpos {

__device__ inline int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
__device__ inline int ceil_div(int a, int b) { return -floor_div(-a, b); }

template <typename T>
struct Fwd {
  using M = MT<T>;
  using frag = typename M::frag;
  static constexpr bool kHalf = sizeof(T) == 2;
  static constexpr int KS = M::KS, E = M::E, NSD = kHeadDim / KS;
  static constexpr int KPS = 32 / KS;  // MFMA k-steps per 32-key half
  static constexpr int TB = DTile<T>::BYTES;

  char* sK;    // [2][TB]
  char* sV;    // [2][TB]  V^T (16-bit) or V (fp32)
  float* sZK;  // [2][2 * kTile]

  Geo g;
  QCtx c;
  int tid, w, lane, hl, l32, iw0, nkt, N;
  float cst_lo, cst_hi, sc2;
  const T* Kb;   // K of this (b, h)
  const T* Vb;   // V^T copy (16-bit, row stride Np) or V (fp32)
  int64_t sk, Np;
  DLoader<T> ldK, ldV;
  frag qf[NSD];
  f32x16 oacc[2];
  float m_used, lsum;

  // Issue the loads of tile t into LDS buffer buf (asynchronous).
  __device__ __forceinline__ void issue(int t, int buf) {
    const int j0 = t * kTile;
    ldK.load(sK + buf * TB, Kb + (int64_t)j0 * sk, N - j0, lane);
    if constexpr (kHalf) {
      ldV.load(sV + buf * TB, Vb + j0, 64, lane);
    } else {
      ldV.load(sV + buf * TB, Vb + (int64_t)j0 * Np, N - j0, lane);
    }
    if (c.has_zk && w < 2) {
      const float* p = kside_sat_ptr(g, c.zkb, j0 + lane, w);
      dword_direct((char*)(sZK + buf * 2 * kTile + w * kTile), p, p != nullptr, lane);
    }
  }

  // One 64-key tile for this wave; SEG is the block-level kind of the tile.
  template <int SEG>
  __device__ __forceinline__ void tile(int t, int buf) {
    const int j0 = t * kTile;
    if (iw0 >= N || (g.causal && j0 > iw0 + 31)) return;
    const int kind = SEG == KIND_BAND ? tile_kind_q(g, j0, iw0) : SEG;
    const bool needmask = (j0 + kTile > c.kv_end) || (g.causal && j0 + kTile - 1 > iw0);
    const char* tK = sK + buf * TB;
    const char* tV = sV + buf * TB;
    const float* zk = sZK + buf * 2 * kTile;
    const float cst = kind == KIND_LO ? cst_lo : (kind == KIND_HI ? cst_hi : 0.f);
    // the two 32-key halves of the tile, one after the other (each its own
    // online-softmax step)
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x16 s;
      if (SEG == KIND_BAND && kind == KIND_BAND)
        s = qside_scores<T>(g, c, tK, zk, qf, KIND_BAND, j0, st, needmask);
      else
        s = qside_scores<T>(g, c, tK, zk, qf, kind == KIND_HI ? KIND_HI : KIND_LO, j0, st,
                            needmask);
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mt = (mx + cst) * sc2;
      const bool need = mt > m_used + 8.f;
      if (__any(need)) {
        const float alpha = need ? exp2_fast(m_used - mt) : 1.f;
        if (need) m_used = mt;
        lsum *= alpha;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          oacc[0][e] *= alpha;
          oacc[1][e] *= alpha;
        }
      }
      const float off = cst * sc2 - (m_used == -INFINITY ? 0.f : m_used);
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) p[e] = exp2_fast(fmaf(s[e], sc2, off));
      // P is rounded to the input type for P V; the normaliser sums the same
      // rounded values
      frag pf[KPS];
      float part[KPS];
#pragma unroll
      for (int kk = 0; kk < KPS; ++kk) {
        pf[kk] = M::pack(&p[kk * E]);
        part[kk] = M::sum_acc(pf[kk], 0.f);
      }
#pragma unroll
      for (int kk = 0; kk < KPS; ++kk) lsum += part[kk];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int kk = 0; kk < KPS; ++kk) {
          const int col = KS * (KPS * st + kk) + E * hl;
          frag vf;
          if constexpr (kHalf) {
            vf = dfrag<T>(tV, 32 * dt + l32, col);
          } else {
            vf = dfrag_t32(tV, 32 * dt + l32, col);
          }
          oacc[dt] = M::mma(vf, pf[kk], oacc[dt]);
        }
    }
  }

  template <int SEG>
  __device__ __forceinline__ void segment(int tb, int te) {
    for (int t = tb; t < te; ++t) {
      const int buf = t & 1;
      if (t + 1 < nkt) issue(t + 1, buf ^ 1);
      tile<SEG>(t, buf);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's loads of tile t+1 landed
      __syncthreads();
    }
  }
};

template <typename T>
__global__ __launch_bounds__(kThreads, 3) void fwd_kernel(AttnArgs a) {
  using M = MT<T>;
  constexpr float kLn2 = 0.693147180559945309f;
  constexpr int TB = DTile<T>::BYTES;

  __shared__ __align__(16) char sK[2 * TB];
  __shared__ __align__(16) char sV[2 * TB];
  __shared__ __align__(16) float sZK[2 * 2 * kTile];

  Fwd<T> f;
  f.sK = sK;
  f.sV = sV;
  f.sZK = sZK;
  f.g = a.geo;
  const Geo& g = f.g;
  const int N = g.N;
  f.N = N;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  f.tid = tid;
  f.w = w;
  f.lane = lane;
  f.hl = hl;
  f.l32 = l32;
  const int total = a.B * a.H * a.nblk;
  const int lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / a.nblk;
  int qb = lid - bh * a.nblk;
  if (g.causal) qb = a.nblk - 1 - qb;  // longest rows first
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int i0 = qb * kBlockRows, iw0 = i0 + 32 * w, iq = iw0 + l32;
  f.iw0 = iw0;

  int kv_end = N;
  if (a.flags & F_KEYPAD) kv_end = imax(0, imin(N, a.key_len[bb]));
  int kv_blk = kv_end;
  if (g.causal) kv_blk = imin(kv_blk, i0 + kBlockRows);
  const int nkt = kv_blk > 0 ? (kv_blk + kTile - 1) / kTile : 0;
  f.nkt = nkt;

  const T* Qp = (const T*)a.q + bb * a.sq.b + hh * a.sq.h;
  f.Kb = (const T*)a.k + bb * a.sk.b + hh * a.sk.h;
  f.sk = a.sk.n;
  f.Np = a.Np;
  if constexpr (Fwd<T>::kHalf) {
    f.Vb = (const T*)a.vt + (int64_t)bh * kHeadDim * a.Np;
    f.ldV.init(a.Np, w, lane);
  } else {
    f.Vb = (const T*)a.v + bb * a.sv.b + hh * a.sv.h;
    f.Np = a.sv.n;
    f.ldV.init(a.sv.n, w, lane);
  }
  f.ldK.init(a.sk.n, w, lane);

  QCtx& c = f.c;
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
  qside_consts(g, c, qb, f.cst_lo, f.cst_hi);
  f.sc2 = a.scale2;

  {
    const T* qrow = Qp + (int64_t)iq * a.sq.n;
#pragma unroll
    for (int ks = 0; ks < Fwd<T>::NSD; ++ks)
      f.qf[ks] = iq < N ? frag_g<T>(qrow, Fwd<T>::KS * ks + Fwd<T>::E * hl) : M::zero();
  }
  f.oacc[0] = zero16();
  f.oacc[1] = zero16();
  f.m_used = -INFINITY;
  f.lsum = 0.f;

  // segment bounds of this block's key tiles: [0, t1) all offsets <= lo,
  // [t2, nkt) all offsets >= hi, band in between
  const int t1 = imin(nkt, imax(0, floor_div(g.lo + i0 - (kTile - 1), kTile) + 1));
  const int t2 = imin(nkt, imax(t1, ceil_div(g.hi + i0 + kBlockRows - 1, kTile)));

  if (nkt > 0) f.issue(0, 0);
  // every load issued so far (Q fragments, tile 0) has landed: inside the
  // loops a wave only waits for its own next-tile loads, before the barrier
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  f.template segment<KIND_LO>(0, t1);
  f.template segment<KIND_BAND>(t1, t2);
  f.template segment<KIND_HI>(t2, nkt);

  const float ltot = f.lsum + __shfl_xor(f.lsum, 32);
  if (iq < N) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    T* orow = (T*)a.o_out + bb * a.so.b + hh * a.so.h + (int64_t)iq * a.so.n;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = 32 * dt + 8 * e4 + 4 * hl;
        store4<T>(orow + d, f.oacc[dt][4 * e4] * inv, f.oacc[dt][4 * e4 + 1] * inv,
                  f.oacc[dt][4 * e4 + 2] * inv, f.oacc[dt][4 * e4 + 3] * inv);
      }
    if (hl == 0)
      a.lse[(int64_t)bh * N + iq] = ltot > 0.f ? (f.m_used + __log2f(ltot)) * kLn2 : -INFINITY;
  }
}

template <typename T>
static hipError_t launch_fwd_t(const AttnArgs& a, hipStream_t st) {
  const int total = a.B * a.H * a.nblk;
  hipLaunchKernelGGL(fwd_kernel<T>, dim3(total), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fwd(int dtype, const AttnArgs& a, hipStream_t st) {
  switch (dtype) {
    case 0: return launch_fwd_t<float>(a, st);
    case 1: return launch_fwd_t<_Float16>(a, st);
    default: return launch_fwd_t<__bf16>(a, st);
  }
}

}  // namespace relpos
