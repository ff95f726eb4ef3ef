// attn_fwd.hip -- fused forward of relative-position attention on gfx950.
//
// Source: "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (nanless.github.io digest): pipeline section (FlashAttention outer
// loop over query blocks, inner loop over key blocks, online softmax, the
// relation response added on chip), score formula Eq. (2), constant tiles and
// the three-segment key loop.
//
// One workgroup = one (batch, head, 128-query block); 4 waves x 32 queries.
// Per 64-key tile: K (row-major) and V (transposed) are staged in LDS, double
// buffered; S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16_{f16,bf16}
// (32x32x2_f32 for fp32 inputs).  The tile kind (LO / BAND / HI) is decided
// per wave with two comparisons; the key tiles of a block fall into three
// consecutive segments LO, BAND, HI in ascending order.
//
// Softmax: base-2 with tau*log2(e) folded into one FMA per score; the
// reference maximum is only moved when a row's maximum grows by more than
// 2^8, so most tiles skip the rescaling of the accumulator (exact: the final
// division uses the same reference).
#include "qside.hpp"

namespace relpos {

template <typename T>
__global__ __launch_bounds__(kThreads) void fwd_kernel(AttnArgs a) {
  using M = MT<T>;
  using frag = typename M::frag;
  using C = TileCfg<T>;
  constexpr int KS = M::KS, E = M::E, NSD = kHeadDim / KS, NSK = kTile / KS;
  constexpr float kLn2 = 0.693147180559945309f;

  __shared__ __align__(16) T sK[2][C::ELEMS];
  __shared__ __align__(16) T sV[2][C::ELEMS];
  __shared__ __align__(16) float sZK[2][2 * kTile];

  const Geo g = a.geo;
  const int N = g.N;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int total = a.B * a.H * a.nblk;
  const int lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / a.nblk;
  int qb = lid - bh * a.nblk;
  if (g.causal) qb = a.nblk - 1 - qb;  // longest rows first
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int i0 = qb * kBlockRows, iw0 = i0 + 32 * w, iq = iw0 + l32;

  int kv_end = N;
  if (a.flags & F_KEYPAD) kv_end = imax(0, imin(N, a.key_len[bb]));
  int kv_blk = kv_end;
  if (g.causal) kv_blk = imin(kv_blk, i0 + kBlockRows);
  const int nkt = kv_blk > 0 ? (kv_blk + kTile - 1) / kTile : 0;

  const T* Qp = (const T*)a.q + bb * a.sq.b + hh * a.sq.h;
  const T* Kp = (const T*)a.k + bb * a.sk.b + hh * a.sk.h;
  const T* Vp = (const T*)a.v + bb * a.sv.b + hh * a.sv.h;

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
  float cst_lo, cst_hi;
  qside_consts(g, c, qb, cst_lo, cst_hi);

  frag qf[NSD];
  {
    const T* qrow = Qp + (int64_t)iq * a.sq.n;
#pragma unroll
    for (int ks = 0; ks < NSD; ++ks) qf[ks] = iq < N ? frag_g<T>(qrow, KS * ks + E * hl) : M::zero();
  }

  Chunk rk[C::NCH], rv[C::NCH];
  float rz0 = 0.f, rz1 = 0.f;
  auto gload = [&](int t) {
    const int j0 = t * kTile;
    tile_load<T, false>(rk, Kp, a.sk.n, j0, N, tid);
    tile_load<T, C::kHalf>(rv, Vp, a.sv.n, j0, N, tid);
    if (c.has_zk && tid < kTile) kside_sat(g, c.zkb, j0 + tid, rz0, rz1);
  };
  auto sstore = [&](int buf) {
    tile_store_rm<T, false>(sK[buf], rk, tid);
    if constexpr (C::kHalf) {
      tile_store_tr<T>(sV[buf], rv, tid);
    } else {
      tile_store_rm<T, false>(sV[buf], rv, tid);
    }
    if (c.has_zk && tid < kTile) {
      sZK[buf][tid] = rz0;
      sZK[buf][kTile + tid] = rz1;
    }
  };

  f32x16 oacc[2];
  oacc[0] = zero16();
  oacc[1] = zero16();
  float m_used = -INFINITY, lsum = 0.f;
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

      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[st][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float cst = kind == KIND_LO ? cst_lo : (kind == KIND_HI ? cst_hi : 0.f);
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
      float p[2][16];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) p[st][e] = exp2_fast(fmaf(s[st][e], sc2, off));
      // P is rounded to the input type for P V; the normaliser sums the same
      // rounded values, in independent chains per fragment
      frag pf[NSK];
      float part[NSK];
#pragma unroll
      for (int ks = 0; ks < NSK; ++ks) {
        const int st = (ks * KS) / 32, e0 = ((ks * KS) % 32) / KS * E;
        pf[ks] = M::pack(&p[st][e0]);
        part[ks] = M::sum_acc(pf[ks], 0.f);
      }
#pragma unroll
      for (int ks = 0; ks < NSK; ++ks) lsum += part[ks];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int ks = 0; ks < NSK; ++ks)
          oacc[dt] = M::mma(frag_t<T>(sV[buf], 32 * dt + l32, KS * ks + E * hl), pf[ks], oacc[dt]);
    }
    if (t + 1 < nkt) sstore(buf ^ 1);
    __syncthreads();
  }

  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (iq < N) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    T* orow = (T*)a.o_out + bb * a.so.b + hh * a.so.h + (int64_t)iq * a.so.n;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = 32 * dt + 8 * e4 + 4 * hl;
        store4<T>(orow + d, oacc[dt][4 * e4] * inv, oacc[dt][4 * e4 + 1] * inv,
                  oacc[dt][4 * e4 + 2] * inv, oacc[dt][4 * e4 + 3] * inv);
      }
    if (hl == 0)
      a.lse[(int64_t)bh * N + iq] = ltot > 0.f ? (m_used + __log2f(ltot)) * kLn2 : -INFINITY;
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
