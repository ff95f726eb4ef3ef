// attn_fwd.hip -- fused forward of relative-position attention on gfx950.
//
// Source: "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (nanless.github.io digest): pipeline section (FlashAttention outer
// loop over query blocks, inner loop over key blocks, online softmax, the
// relation response added on chip), score formula Eq. (2), constant tiles and
// the three-segment key loop.
//
// One workgroup = one (batch, head, 128-query block); 4 waves x 32 queries.
// Per 64-key tile: the K and V rows go from HBM straight into LDS with
// global_load_lds_dwordx4 (no staging registers), double buffered;
// S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16_{f16,bf16}
// (32x32x2_f32 for fp32 inputs).  The V^T operand is read from the V row
// tile with ds_read_b64_tr_b16 transpose reads (fp32: element reads).
//
// Three-segment key loop: two comparisons per tile against the thresholds
// split each wave's key tiles (for its own 32 queries) into a left-saturated
// run, a band run and a right-saturated run.  The saturated runs take a body
// compiled without per-score lookup, gather or mask code (and the next
// tile's prefetch is never held up behind one); the band run and the tiles
// with masked entries take the general body.
//
// Softmax: base-2 with tau*log2(e) folded into one FMA per score; the
// reference maximum is only moved when a row's maximum grows by more than
// 2^8, so most tiles skip the rescaling of the accumulator (exact: the final
// division uses the same reference).
//
// Attention dropout (16-bit inputs): the P V operand takes the kept weights
// only, the normaliser sums all of them, and the final division carries the
// 1 / (1 - p) factor; the keep bits come from dropout.hpp.
#include "dropout.hpp"
#include "inblock.hpp"
#include "qside.hpp"

namespace relpos {

__device__ inline int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
__device__ inline int ceil_div(int a, int b) { return -floor_div(-a, b); }

// Groups of 4 waves per workgroup: for a causal 16-bit launch whose blocks all
// fit on the device at once (the longest block bounds it) two
// groups take alternate key tiles of the 128-query block and merge their
// softmax states through LDS at the end, which halves the longest (last)
// blocks; otherwise one.
template <typename T, bool GRP>
constexpr int fwd_groups() {
  return (GRP && sizeof(T) == 2) ? 2 : 1;
}
// Ways the band tiles get the query-side relation: gathered per score from
// the stored Z^Q, staged from it in LDS by row DMA (wide bands), or computed
// in the block (no stored Z^Q; inblock.hpp).
enum : int { ZM_GATHER = 0, ZM_STAGED = 1, ZM_INBLOCK = 2 };

// Waves per SIMD the forward is compiled for: 16-bit inputs without a
// key-side term, staged rows, in-block relation or groups fit 3 (168 VGPRs),
// which hides more latency than operand prefetch (with dropout too: its few
// spills cost less than the third wave gains); the others keep 2.
template <typename T, bool ZK, int ZM, bool GRP, bool DROP>
constexpr int fwd_occupancy() {
  return (sizeof(T) == 2 && !ZK && ZM == ZM_GATHER && !GRP) ? 3 : (sizeof(T) == 2 ? 2 : 1);
}
template <typename T, bool GRP>
constexpr int fwd_threads() {
  return kThreads * fwd_groups<T, GRP>();
}
template <typename T, bool ZK, int ZM, bool GRP, bool DROP>
constexpr int fwd_blocks_per_cu() {
  return fwd_occupancy<T, ZK, ZM, GRP, DROP>() / fwd_groups<T, GRP>();
}

struct NoInBlock {};

// ZM: how band tiles get the query-side relation (ZM_*).
// OCC3: compiled for 3 waves per SIMD: each subtile reads its own operand
// fragments (instead of the whole tile's up front), which keeps fewer
// registers live.  DROP: attention dropout.
template <typename T, int ZM, bool OCC3, bool GRP, bool DROP>
struct Fwd {
  using M = MT<T>;
  using frag = typename M::frag;
  static constexpr bool ZQS = ZM == ZM_STAGED;
  static constexpr bool ZIB = ZM == ZM_INBLOCK;
  static constexpr bool kHalf = sizeof(T) == 2;
  static constexpr bool kOcc3 = OCC3;
  static constexpr int kGroups = fwd_groups<T, GRP>();
  static constexpr int KS = M::KS, E = M::E, NSD = kHeadDim / KS;
  static constexpr int KPS = 32 / KS;  // MFMA k-steps per 32-key half
  static constexpr int TB = DTile<T>::BYTES;

  // LDS buffers, two of each (separate arrays, so that the compiler can tell
  // the asynchronous loads into one buffer from the reads of the other)
  char* sK[2];    // K tile (group 0's buffers; this group's start goff bytes in)
  char* sV[2];    // V tile
  float* sZK[2];  // saturated Z^K scalars of the tile's keys [group][2][kTile]
  int grp, goff;  // this wave's group, byte offset of its K / V buffers

  Geo g;
  QCtx c;
  int tid, w, lane, hl, l32, i0, iw0, nkt, N;
  float cst_lo, cst_hi, sc2;
  const T* Kb;   // K of this (b, h)
  const T* Vb;   // V of this (b, h)
  int64_t sk, sv;
  DLoader<T> ldK, ldV;
  // per-lane LDS byte offsets of the 16-bit operand fragments (buffer 0):
  // K row sigma(l32) at k-step ks
  int kofs[kHalf ? NSD : 1];
  // V^T (contracted over the keys in P V) comes from the V row tile through
  // transpose reads
  TrReader<std::conditional_t<kHalf, T, _Float16>> tr;
  frag qf[NSD];
  f32x16 oacc[2];
  float m_used, lsum;
  RowStage zs;  // Z^Q band rows of this wave, staged per subtile
  DropCtx dr;   // DROP only
  // in-block relation (ZIB only): the ring of table rows, and whether b is
  // present
  std::conditional_t<ZIB, InBlock<T>, NoInBlock> ib;
  char* ring;
  bool ib_b;

  // Issue the loads of tile t into LDS buffer BUF (asynchronous).
  template <int BUF>
  __device__ __forceinline__ void issue(int t) {
    const int j0 = t * kTile;
    ldK.load(sK[BUF] + goff, Kb + (int64_t)j0 * sk, N - j0, lane);
    ldV.load(sV[BUF] + goff, Vb + (int64_t)j0 * sv, N - j0, lane);
    if constexpr (ZIB) ib.load_block(g, ring, j0 - i0);  // the tile's 64 new offsets
    if (c.has_zk && w < 2) {
      const float* p = kside_sat_ptr(g, c.zkb, j0 + lane, w);
      dword_direct((char*)(sZK[BUF] + (2 * grp + w) * kTile), p, p != nullptr, lane);
    }
  }

  // Whether this wave takes the band path with a Z^Q lookup on tile t (the
  // tile's Z^Q rows are then staged in LDS).
  __device__ __forceinline__ bool band_here(int t) const {
    if constexpr (!ZQS) return false;
    const int j0 = t * kTile;
    return c.has_zq && t < nkt && iw0 < N && !(g.causal && j0 > iw0 + 31) &&
           tile_kind_q(g, j0, iw0) == KIND_BAND;
  }
  template <int ST>
  __device__ __forceinline__ void stage(int t) {
    zs.template issue_q<ST>(g, c, iw0, t * kTile + 32 * ST, lane);
  }

  // V^T fragment (rows d = 32 dt + l32, keys of chunk column c4) of P V.
  __device__ __forceinline__ frag vfrag(const char* tV, int dt, int c4) const {
    if constexpr (kHalf) {
      return tr.read(tV, dt, c4);
    } else {
      return dfrag_t32(tV, 32 * dt + l32, KS * c4 + E * hl);
    }
  }

  // One 64-key tile for this wave, read from LDS buffer BUF.  BAND: the
  // block's tile crosses the band (each wave refines the kind for its own
  // queries); otherwise the whole tile is saturated on side `sat`.
  // stage_next: this wave stages the Z^Q rows of tile t + 1 from its band
  // path here, each subtile's rows once its own have been read.
  template <bool BAND, int BUF>
  __device__ __forceinline__ void tile(int t, int sat, bool stage_next) {
    const int j0 = t * kTile;
    // (a saturated body also runs for a wave whose queries are all beyond N:
    // its results are discarded, and skipping would cost a branch and
    // register copies in every tile)
    if (BAND && (iw0 >= N || (g.causal && j0 > iw0 + 31))) return;
    const int kind = BAND ? tile_kind_q(g, j0, iw0) : sat;
    // masks are only applied in the band body (a saturated body is only
    // used for tiles that need no mask anywhere in the block)
    const bool needmask = BAND && ((j0 + kTile > c.kv_end) || (g.causal && j0 + kTile - 1 > iw0));
    const char* tK = sK[BUF];
    const char* tV = sV[BUF];
    const float* zk = sZK[BUF] + 2 * grp * kTile;
    const float cst = kind == KIND_LO ? cst_lo : (kind == KIND_HI ? cst_hi : 0.f);
    // 16-bit types at occupancy 2: every operand fragment of the tile is read
    // from LDS up front (one batch), so the reads of the second half overlap
    // the first half's MFMAs and softmax; at occupancy 3 (and for fp32) each
    // subtile reads its own
    frag kf[2][NSD], vf[2][2 * KPS];
    // in-block relation: offset tiles U = 0, 1, 2 start at j0 - iw0 - 31 + 32 U;
    // subtile st takes its seeds from tiles st and st + 1
    f32x16 tprev;
    int ob = 0;
    T bv[3] = {};
    if constexpr (ZIB) {
      if (BAND && kind == KIND_BAND) {
        ob = j0 - iw0 - 31;
        if (ib_b) {
#pragma unroll
          for (int u = 0; u < 3; ++u) bv[u] = ib.b_of(g, ob + 32 * u);
        }
        tprev = ib.tmm(ob, qf, ib_b, bv[0], hl);
      }
    }
    if constexpr (kHalf && !kOcc3) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int ks = 0; ks < NSD; ++ks) kf[st][ks] = kfrag<T>(tK, kofs, c, st, ks);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int kk = 0; kk < KPS; ++kk) vf[st][dt * KPS + kk] = vfrag(tV, dt, KPS * st + kk);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if constexpr (!kHalf || kOcc3) {
#pragma unroll
        for (int ks = 0; ks < NSD; ++ks) kf[st][ks] = kfrag<T>(tK, kofs, c, st, ks);
      }
      if constexpr (kHalf && kOcc3) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int kk = 0; kk < KPS; ++kk) vf[st][dt * KPS + kk] = vfrag(tV, dt, KPS * st + kk);
      }
      f32x16 s;
      if (ZIB && BAND && kind == KIND_BAND) {
        if constexpr (ZIB) {
          const f32x16 tn = ib.tmm(ob + 32 * (st + 1), qf, ib_b, bv[st + 1], hl);
          float v[16];
          ib.seeds(tprev, tn, v);
          tprev = tn;
          s = seeded_scores<T>(g, c, kf[st], qf, v, j0, st, needmask);
        }
      } else if (BAND && kind == KIND_BAND) {
        s = qside_scores<T, ZQS>(g, c, kf[st], zk, qf, KIND_BAND, j0, st, needmask,
                            ZQS ? zs.row(st, l32) + E * hl : nullptr);
        if (stage_next) {
          if (st == 0) stage<0>(t + kGroups); else stage<1>(t + kGroups);
        }
      } else
        s = qside_scores<T>(g, c, kf[st], zk, qf, kind == KIND_HI ? KIND_HI : KIND_LO, j0, st,
                            needmask);
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
      mx = max_xor32(mx);
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
#pragma unroll
      for (int kk = 0; kk < KPS; ++kk) {
        pf[kk] = M::pack(&p[kk * E]);
        lsum = M::sum_acc(pf[kk], lsum);
      }
      if constexpr (DROP) {
        // the dropped weights go into P V (the normaliser above keeps all)
        const uint32_t kb = drop_bits<T, true>(dr, c.iq, j0 + 32 * st, hl);
#pragma unroll
        for (int e = 0; e < 16; ++e) p[e] = keep_or_zero(kb, e, p[e]);
#pragma unroll
        for (int kk = 0; kk < KPS; ++kk) pf[kk] = M::pack(&p[kk * E]);
      }
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int kk = 0; kk < KPS; ++kk)
          oacc[dt] = M::mma(kHalf ? vf[st][dt * KPS + kk] : vfrag(tV, dt, KPS * st + kk), pf[kk],
                            oacc[dt]);
    }
  }

  // Key tile t (none once t >= nkt) from buffer BUF, with the loads of the
  // group's next tile into the other buffer in flight.  Tiles [0, t1) are
  // left-saturated, [t2, nkt) right-saturated, the rest cross the band;
  // tiles with masked entries (the key-length edge, the causal diagonal)
  // also take the band body.
  template <int BUF>
  __device__ __forceinline__ void step(int t, int t1, int t2) {
    const int tn = t + kGroups;
    if (tn < nkt) issue<BUF ^ 1>(tn);
    // Z^Q rows of the group's next tile: staged now when tile t leaves the
    // buffers free, else from tile t's band path
    const bool bn = band_here(tn), bc = band_here(t);
    if (bn && !bc) {
      stage<0>(tn);
      stage<1>(tn);
    }
    if (kGroups == 1 || t < nkt) {  // (one group: t < nkt always holds)
      const int j0 = t * kTile;
      const bool masked = (j0 + kTile > c.kv_end) || (g.causal && j0 + kTile - 1 > iw0);
      if ((t >= t1 && t < t2) || masked)
        tile<true, BUF>(t, KIND_BAND, bn && bc);
      else
        tile<false, BUF>(t, t < t1 ? KIND_LO : KIND_HI, false);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's loads of its next tile landed
    __syncthreads();
  }

  // Group grp takes key tiles grp, grp + kGroups, ...; every group runs the
  // same number of steps (one workgroup barrier each), step m in buffer m & 1.
  __device__ __forceinline__ void run(int t1, int t2) {
    const int t0 = grp;
    if (t0 < nkt) {
      issue<0>(t0);
      if constexpr (ZIB) {
        // the two blocks of offsets below the first tile's own
        ib.load_block(g, ring, t0 * kTile - i0 - 128);
        ib.load_block(g, ring, t0 * kTile - i0 - 64);
      }
    }
    if (band_here(t0)) {
      stage<0>(t0);
      stage<1>(t0);
    }
    // every load issued so far (Q fragments, the first tile) has landed:
    // inside the loop a wave only waits for its own next-tile loads, before
    // the barrier
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    const int nsteps = (nkt + kGroups - 1) / kGroups;
    for (int m = 0; m < nsteps; m += 2) {
      step<0>(t0 + kGroups * m, t1, t2);
      if (m + 1 < nsteps) step<1>(t0 + kGroups * (m + 1), t1, t2);
    }
  }
};

// ZK: whether the key-side relation term is present (a compile-time switch, so
// that saturated tiles without it seed their MFMA accumulators with zero and
// carry no branch); ZM: how band tiles get the query-side relation (ZM_*);
// GRP: grouped workgroup; DROP: attention dropout.
template <typename T, bool ZK, int ZM, bool GRP, bool DROP>
__global__ __launch_bounds__((fwd_threads<T, GRP>()), (fwd_blocks_per_cu<T, ZK, ZM, GRP, DROP>()))
    void fwd_kernel(AttnArgs a) {
  using M = MT<T>;
  constexpr float kLn2 = 0.693147180559945309f;
  constexpr int TB = DTile<T>::BYTES;
  constexpr int G = fwd_groups<T, GRP>();
  constexpr bool ZQS = ZM == ZM_STAGED;

  __shared__ __align__(16) char sK0[G * TB], sK1[G * TB], sV0[G * TB], sV1[G * TB];

  using F = Fwd<T, ZM, fwd_occupancy<T, ZK, ZM, GRP, DROP>() == 3, GRP, DROP>;
  F f;
  f.sK[0] = sK0;
  f.sK[1] = sK1;
  f.sV[0] = sV0;
  f.sV[1] = sV1;
  // (the in-block kernel has neither Z^K scalars nor staged rows: its ring
  // and skew tiles take that LDS, 80 KB per block in all, two blocks per CU)
  float* zq_stage[2];
  if constexpr (ZM == ZM_INBLOCK) {
    __shared__ __align__(128) char sRing[kRingBytes];
    __shared__ __align__(128) float sSkew[4 * kSkewFloats];
    f.ring = sRing;
    f.ib.init(lds_addr(sRing), lds_addr(sSkew + wave_id() * kSkewFloats), wave_id(),
              threadIdx.x & 63);
    f.sZK[0] = f.sZK[1] = reinterpret_cast<float*>(sK0);
    zq_stage[0] = zq_stage[1] = reinterpret_cast<float*>(sK0);
  } else {
    __shared__ __align__(16) float sZK0[G * 2 * kTile], sZK1[G * 2 * kTile];
    constexpr int kZQ = ZQS ? 4 * G * RowStage::kFloats : 4;
    __shared__ __align__(16) float sZQ0[kZQ], sZQ1[kZQ];
    f.sZK[0] = sZK0;
    f.sZK[1] = sZK1;
    zq_stage[0] = ZQS ? sZQ0 + wave_id() * RowStage::kFloats : sZQ0;
    zq_stage[1] = ZQS ? sZQ1 + wave_id() * RowStage::kFloats : sZQ1;
  }
  f.g = a.geo;
  const Geo& g = f.g;
  const int N = g.N;
  f.N = N;
  const int tid = threadIdx.x, wall = wave_id(), lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int grp = G == 2 ? wall >> 2 : 0, w = wall & 3;
  f.grp = grp;
  // the group offset goes into the per-lane fragment offsets, so that the
  // LDS reads keep compile-time buffer bases
  f.goff = grp * TB;
  f.tid = tid;
  f.w = w;
  f.lane = lane;
  f.hl = hl;
  f.l32 = l32;
  // this launch covers the query blocks [qb0, qb0 + nqb) of every (b, h)
  const int total = a.B * a.H * a.nqb;
  int bh, qb;
  block_of(blockIdx.x, total, a.nqb, g.causal, bh, qb);
  if (g.causal) qb = a.nqb - 1 - qb;  // longest rows first
  qb += a.qb0;
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int i0 = qb * kBlockRows, iw0 = i0 + 32 * w, iq = iw0 + l32;
  f.i0 = i0;
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
  f.Vb = (const T*)a.v + bb * a.sv.b + hh * a.sv.h;
  f.sv = a.sv.n;
  f.ldV.init(a.sv.n, w, lane);
  f.ldK.init(a.sk.n, w, lane);
  if constexpr (F::kHalf) {
    const int sig = sigma<T>(l32);
#pragma unroll
    for (int ks = 0; ks < F::NSD; ++ks)
      f.kofs[ks] = f.goff + dt_off<T>(sig, F::KS * ks + F::E * hl);
    f.tr.init(lane, f.goff);
  }

  QCtx& c = f.c;
  c.iq = iq;
  c.hl = hl;
  c.sig = sigma<T>(l32);
  c.kv_end = kv_end;
  // (an in-block kernel reads no Z^Q; b is part of its relation term)
  c.has_zq = ZM != ZM_INBLOCK && (a.flags & F_ZQ);
  c.has_zk = ZK;
  // (a staged kernel has a query-side table, into which b is folded: no
  // lookup of its own, and no code for one)
  c.has_b = ZM == ZM_GATHER && (a.flags & F_B);
  c.wsq = win_q(g, qb);
  c.zq_row = c.has_zq ? a.zq + zq_off(g, bh, imin(iq, zq_last(g))) : nullptr;
  c.zkb = c.has_zk ? a.zk + (int64_t)bh * N * g.Wp : nullptr;
  c.bun = c.has_b ? a.bunf + hh * a.bunf_hs : nullptr;
  f.zs.buf[0] = zq_stage[0];
  f.zs.buf[1] = zq_stage[1];
  f.zs.init(g, c.has_zq ? a.zq + zq_off(g, bh, 0) : nullptr, -1, lane);
  f.sc2 = a.scale2;
  if constexpr (DROP) f.dr = drop_ctx(a, bh, lane);

  {
    const T* qrow = Qp + (int64_t)iq * a.sq.n;
#pragma unroll
    for (int ks = 0; ks < F::NSD; ++ks)
      f.qf[ks] = iq < N ? frag_g<T>(qrow, F::KS * ks + F::E * hl) : M::zero();
  }
  if constexpr (ZM == ZM_INBLOCK) {
    f.ib.tab = (const T*)a.tabq + hh * a.tabq_hs;
    // (b is part of the relation term here whenever it is present)
    f.ib.bt = a.tabb ? (const T*)a.tabb + hh * a.tabb_hs : nullptr;
    f.ib.fold = a.fold;
    f.ib_b = a.tabb != nullptr;
    f.ib.consts(g, f.qf, hl, f.cst_lo, f.cst_hi);
  } else {
    qside_consts(g, c, qb, f.cst_lo, f.cst_hi);
  }
  f.oacc[0] = zero16();
  f.oacc[1] = zero16();
  f.m_used = -INFINITY;
  f.lsum = 0.f;

  // this wave's segments: key tiles [0, t1) have all offsets <= lo for its
  // 32 queries, [t2, nkt) all offsets >= hi, the band in between (a tile
  // goes through the band body only for the waves that need it)
  const int t1 = imin(nkt, imax(0, floor_div(g.lo + iw0 - (kTile - 1), kTile) + 1));
  const int t2 = imin(nkt, imax(t1, ceil_div(g.hi + iw0 + 31, kTile)));

  f.run(t1, t2);

  if constexpr (G == 2) {
    // group 1 hands its softmax state (O accumulator, reference maximum,
    // partial sum) to group 0 through the K / V buffers; group 0 rescales
    // both to the larger maximum and adds them
    const int t = tid & (4 * 64 - 1);
    float* x0 = reinterpret_cast<float*>(sK0);
    float* x1 = reinterpret_cast<float*>(sK1);
    float* x2 = reinterpret_cast<float*>(sV0);
    static_assert(G * TB >= 16 * 256 * 4, "combine buffers");
    if (grp == 1) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        x0[e * 256 + t] = f.oacc[0][e];
        x1[e * 256 + t] = f.oacc[1][e];
      }
      x2[t] = f.m_used;
      x2[256 + t] = f.lsum;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = x2[t], l1 = x2[256 + t];
    const float m = fmaxf(f.m_used, m1);
    const float a0 = f.m_used == -INFINITY ? 0.f : exp2_fast(f.m_used - m);
    const float a1 = m1 == -INFINITY ? 0.f : exp2_fast(m1 - m);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      f.oacc[0][e] = f.oacc[0][e] * a0 + x0[e * 256 + t] * a1;
      f.oacc[1][e] = f.oacc[1][e] * a0 + x1[e * 256 + t] * a1;
    }
    f.lsum = f.lsum * a0 + l1 * a1;
    f.m_used = m;
  }

  const float ltot = sum_xor32(f.lsum);
  if (iq < N) {
    const float inv = ltot > 0.f ? (DROP ? a.drop_scale : 1.f) / ltot : 0.f;
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

template <typename T, bool GRP, bool DROP>
static hipError_t launch_fwd_g(const AttnArgs& a, hipStream_t st) {
  const int total = a.B * a.H * a.nqb;
  const bool zk = a.flags & F_ZK, zqs = (a.flags & F_ZQ) && wide_band(a.geo);
  const int nt = fwd_threads<T, GRP>();
  if (zk && zqs)
    hipLaunchKernelGGL((fwd_kernel<T, true, ZM_STAGED, GRP, DROP>), dim3(total), dim3(nt), 0, st,
                       a);
  else if (zk)
    hipLaunchKernelGGL((fwd_kernel<T, true, ZM_GATHER, GRP, DROP>), dim3(total), dim3(nt), 0, st,
                       a);
  else if (zqs)
    hipLaunchKernelGGL((fwd_kernel<T, false, ZM_STAGED, GRP, DROP>), dim3(total), dim3(nt), 0, st,
                       a);
  else
    hipLaunchKernelGGL((fwd_kernel<T, false, ZM_GATHER, GRP, DROP>), dim3(total), dim3(nt), 0, st,
                       a);
  return hipGetLastError();
}

// In-block relation (16-bit inputs, query-side terms only, one wave group).
template <typename T, bool DROP>
static hipError_t launch_fwd_inblock(const AttnArgs& a, hipStream_t st) {
  const int total = a.B * a.H * a.nqb;
  hipLaunchKernelGGL((fwd_kernel<T, false, ZM_INBLOCK, false, DROP>), dim3(total),
                     dim3(fwd_threads<T, false>()), 0, st, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_fwd_t(const AttnArgs& a, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (a.flags & F_ZIB) {
      if (a.flags & F_DROP) return launch_fwd_inblock<T, true>(a, st);
      return launch_fwd_inblock<T, false>(a, st);
    }
    if (a.flags & F_DROP) {
      if (a.split) return launch_fwd_g<T, true, true>(a, st);
      return launch_fwd_g<T, false, true>(a, st);
    }
    if (a.split) return launch_fwd_g<T, true, false>(a, st);
  }
  return launch_fwd_g<T, false, false>(a, st);
}

hipError_t launch_fwd(int dtype, const AttnArgs& a, hipStream_t st) {
  switch (dtype) {
    case 0: return launch_fwd_t<float>(a, st);
    case 1: return launch_fwd_t<_Float16>(a, st);
    default: return launch_fwd_t<__bf16>(a, st);
  }
}

}  // namespace relpos
