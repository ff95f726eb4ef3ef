// attn_bwd_q.hpp -- the query-parallel backward pass (one block of it).
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
// One workgroup = one (batch, head, 128-query block); 4 waves x 32 queries;
// per 64-key tile the K and V rows are loaded straight into LDS (K^T, the
// operand of dQ = dS K, through transpose reads); the key loop runs in three
// segments like the forward.
#pragma once
#include "dropout.hpp"
#include "qside.hpp"

namespace relpos {

__device__ inline int floor_div_q(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
__device__ inline int ceil_div_q(int a, int b) { return -floor_div_q(-a, b); }

constexpr int kStagePitch = 36;  // floats per staged row (16-byte aligned, bank-spread)
// per wave and subtile position: Z^Q rows of the subtile (RowStage), later
// reused for the subtile's band stores ([32][kStagePitch])
constexpr int kStageFloats = 32 * kStagePitch;
static_assert(kStageFloats >= RowStage::kFloats, "stage area holds the Z^Q rows");

// Groups of 4 waves per workgroup: for a causal 16-bit launch whose blocks all
// fit on the device at once (the longest block bounds it) two
// groups take alternate key tiles of the block and sum their dQ and
// saturated-row sums through LDS at the end, which halves the longest
// (last) query blocks; otherwise one.
template <typename T, bool GRP>
constexpr int query_groups() {
  return (GRP && sizeof(T) == 2) ? 2 : 1;
}
template <typename T, bool GRP>
constexpr int query_threads() {
  return kThreads * query_groups<T, GRP>();
}
// blocks per CU for 2 waves per SIMD (fp32: 1 block)
template <typename T, bool GRP>
constexpr int query_blocks_per_cu() {
  return (query_groups<T, GRP>() == 1 && sizeof(T) == 2) ? 2 : 1;
}

// STAGE: band stores go through an LDS staging area (chosen for wide bands);
// GRP: two groups of waves split the key tiles; DROP: attention dropout.
// SCHED: use the compiler's scheduling strategy 0 in the subtile loop.
template <typename T, bool STAGE, bool GRP, bool DROP, bool SCHED>
struct BwdQ {
  static constexpr int kGroups = query_groups<T, GRP>();
  using M = MT<T>;
  using frag = typename M::frag;
  static constexpr bool kHalf = sizeof(T) == 2;
  static constexpr int KS = M::KS, E = M::E, NSD = kHeadDim / KS;
  static constexpr int KPS = 32 / KS;  // MFMA k-steps per 32-key half
  static constexpr int TB = DTile<T>::BYTES;

  // LDS buffers, two of each (separate arrays, so that the compiler can tell
  // the asynchronous loads into one buffer from the reads of the other)
  char* sK[2];     // K rows (group 0's buffers; this group's start goff bytes in)
  char* sV[2];     // V rows
  float* sZK[2];   // saturated Z^K scalars [group][2][kTile]
  int grp, goff;   // this wave's group, byte offset of its K / V buffers

  Geo g;
  QCtx c;
  int w, lane, hl, l32, i0, iw0, nkt, N, kv_lim;
  float cst_lo, cst_hi, sc2, tau, lse2, Dl;
  f32x16 dseed;  // -D in every entry: the starting value of dP (unused under dropout)
  DropCtx dr;    // DROP only
  bool need_dz;
  const T* Kb;
  const T* Vb;
  int64_t sk, sv, Np;
  DLoader<T> ldK, ldV;
  // per-lane LDS byte offsets of the 16-bit operand fragments (buffer 0):
  // K / V row sigma(l32) at k-step ks
  int kofs[kHalf ? NSD : 1];
  // K^T (contracted over the keys in dQ = dS K) comes from the K row tile
  // through transpose reads
  TrReader<std::conditional_t<kHalf, T, _Float16>> tr;
  frag qf[NSD], df[NSD];
  f32x16 dq[2];
  float acc_lo, acc_hi;
  float* dz_row;
  float* dz_w;     // dZ^Q row of this wave's first query (iw0)
  // STAGE: this wave's two LDS areas (subtile positions 0 / 1); each first
  // holds the Z^Q rows of its subtile, then takes its band stores
  RowStage zs;

  // Whether this wave reads staged Z^Q rows on tile t.
  __device__ __forceinline__ bool band_here(int t) const {
    if constexpr (!STAGE) return false;
    const int j0 = t * kTile;
    return c.has_zq && t < nkt && iw0 < N && !(g.causal && j0 > iw0 + 31) &&
           tile_kind_q(g, j0, iw0) == KIND_BAND;
  }
  template <int ST>
  __device__ __forceinline__ void stage_zq(int t) {
    zs.template issue_q<ST>(g, c, iw0, t * kTile + 32 * ST, lane);
  }

  template <int BUF>
  __device__ __forceinline__ void issue(int t) {
    const int j0 = t * kTile;
    ldK.load(sK[BUF] + goff, Kb + (int64_t)j0 * sk, N - j0, lane);
    ldV.load(sV[BUF] + goff, Vb + (int64_t)j0 * sv, N - j0, lane);
    if (c.has_zk && w < 2) {
      const float* p = kside_sat_ptr(g, c.zkb, j0 + lane, w);
      dword_direct((char*)(sZK[BUF] + (2 * grp + w) * kTile), p, p != nullptr, lane);
    }
  }

  // Store tau * ds of the 32 x 32 subtile (keys jb .. jb + 31) into dZ^Q:
  // entry (query iw0 + q, key jb + k) goes to offset o = jb + k - iw0 - q of
  // row iw0 + q when it is live and strictly inside the band.
  __device__ __forceinline__ void band_store(const float (&ds)[16], int jb, float* stage) {
    // registers -> LDS [query][key]: lane (l32, hl) holds keys kappa(hl, e)
    // (16-bit types: runs of 4 consecutive keys)
    if constexpr (kHalf) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int k0 = kappa<T>(hl, 4 * e4);
        *reinterpret_cast<f32x4*>(stage + l32 * kStagePitch + k0) = f32x4{
            tau * ds[4 * e4], tau * ds[4 * e4 + 1], tau * ds[4 * e4 + 2], tau * ds[4 * e4 + 3]};
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) stage[l32 * kStagePitch + kappa<T>(hl, e)] = tau * ds[e];
    }
    // LDS -> HBM: rows q = 2 r + hl, key l32 of each
    const int j = jb + l32;
#pragma unroll 1
    for (int r = 0; r < 16; ++r) {
      const int q = 2 * r + hl;
      const float v = stage[q * kStagePitch + l32];
      const int i = iw0 + q;
      const int o = j - i;
      if (o > g.lo && o < g.hi && i < N && j < N && !(g.causal && j > i))
        dz_w[(int64_t)q * g.Wp + o - g.lo - c.wsq + ((i + g.lo + c.wsq) & g.dsm)] = v;
    }
  }

  // Whether every entry of the 32 x 32 subtile (this wave's queries, keys
  // [jb, jb + 32)) is live and strictly inside the band (wave-uniform).
  __device__ __forceinline__ bool band_interior(int jb) const {
    return jb - iw0 - 31 > g.lo && jb + 31 - iw0 < g.hi && iw0 + 31 < N && jb + 31 < c.kv_end &&
           !(g.causal && jb + 31 > iw0);
  }

  // Band stores of an interior subtile (16-bit operands): a lane's elements
  // e = 0..7 and 8..15 are eight consecutive keys each (kappa), hence eight
  // consecutive offsets of its query's dZ^Q row, written as four 16-byte
  // stores.
  __device__ __forceinline__ void band_store_row(const float (&ds)[16], int jb) {
    float* p = dz_row + (jb + E * hl - c.iq - g.lo - c.wsq);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e0 = 4 * u;
      store_f32x4_a4(p + (u < 2 ? 4 * u : 16 + 4 * (u - 2)),
                     f32x4{tau * ds[e0], tau * ds[e0 + 1], tau * ds[e0 + 2], tau * ds[e0 + 3]});
    }
  }

  // Band stores of an interior subtile through the LDS area `stage`
  // (registers -> [query][key] as in band_store); then each lane takes four
  // consecutive keys of one query row, so that eight lanes write one 128-byte
  // run and one store instruction covers eight rows.
  __device__ __forceinline__ void band_store_runs(const float (&ds)[16], int jb, float* stage) {
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int k0 = kappa<T>(hl, 4 * e4);
      *reinterpret_cast<f32x4*>(stage + l32 * kStagePitch + k0) = f32x4{
          tau * ds[4 * e4], tau * ds[4 * e4 + 1], tau * ds[4 * e4 + 2], tau * ds[4 * e4 + 3]};
    }
    const int qr = lane >> 3, kc = 4 * (lane & 7);
    // row iw0 + q, key jb + kc: offset jb + kc - iw0 - q; rows qr, qr + 8,
    // qr + 16, qr + 24 of the area (8 rows = 8 * kStagePitch floats apart)
    constexpr int RB = 8 * kStagePitch * 4;
    f32x4 v[4];
    lds_read4x16<0, RB, 2 * RB, 3 * RB>(stage + qr * kStagePitch + kc, v[0], v[1], v[2], v[3]);
    // with the row shift (dz_shift, dsm = 31) every run starts on a 128-byte
    // line
    float* base = dz_w + (jb + kc - iw0 - g.lo - c.wsq);
    const int t = iw0 + g.lo + c.wsq;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = 8 * r + qr;
      store_f32x4_a4(base + (int64_t)q * (g.Wp - 1) + ((t + q) & g.dsm), v[r]);
    }
  }

  // One 64-key tile from LDS buffer BUF; BAND: the wave's tile crosses the
  // band, otherwise it is saturated on side `sat`.
  // stage_next: the Z^Q rows of tile t + 1 are staged from this tile's band
  // path, each subtile's once its area is free again.
  template <bool BAND, int BUF>
  __device__ __forceinline__ void tile(int t, int sat, bool stage_next) {
    const int j0 = t * kTile;
    if (iw0 >= N || (g.causal && j0 > iw0 + 31)) return;
    const int kind = BAND ? tile_kind_q(g, j0, iw0) : sat;
    // masks are only applied in the band body (a saturated body is only
    // used for tiles that need no mask anywhere in the block)
    const bool needmask = BAND && ((j0 + kTile > c.kv_end) || (g.causal && j0 + kTile - 1 > iw0));
    const char* tK = sK[BUF];
    const char* tV = sV[BUF];
    const float* zk = sZK[BUF] + 2 * grp * kTile;
    const float cst = kind == KIND_LO ? cst_lo : (kind == KIND_HI ? cst_hi : 0.f);
    const float off = cst * sc2 - lse2;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      // scheduling strategy 0 of the compiler (interleave the LDS operand
      // reads with the MFMAs), as in the key pass
      if constexpr (SCHED) __builtin_amdgcn_iglp_opt(0);
      frag kf[NSD];
#pragma unroll
      for (int ks = 0; ks < NSD; ++ks) kf[ks] = kfrag<T>(tK, kofs, c, st, ks);
      f32x16 s;
      if (BAND && kind == KIND_BAND)
        s = qside_scores<T, STAGE>(g, c, kf, zk, qf, KIND_BAND, j0, st, needmask,
                            STAGE ? zs.row(st, l32) + E * hl : nullptr);
      else
        s = qside_scores<T>(g, c, kf, zk, qf, kind == KIND_HI ? KIND_HI : KIND_LO, j0, st,
                            needmask);
      // dP' = dP - D: the product accumulates onto -D (from zero under
      // dropout, whose kept entries scale dP before D is subtracted)
      f32x16 dp = M::mma(kfrag<T>(tV, kofs, c, st, 0), df[0], DROP ? zero16() : dseed);
#pragma unroll
      for (int ks = 1; ks < NSD; ++ks) dp = M::mma(kfrag<T>(tV, kofs, c, st, ks), df[ks], dp);

      float ds[16];
      if constexpr (DROP) {
        // kept: dS = P (dP / (1 - p) - D); dropped: dS = -P D
        const uint32_t kb = drop_bits<T, true>(dr, c.iq, j0 + 32 * st, hl);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2_fast(fmaf(s[e], sc2, off));
          ds[e] = p * (((kb >> e) & 1u) ? fmaf(dr.scale, dp[e], -Dl) : -Dl);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2_fast(fmaf(s[e], sc2, off));
          ds[e] = p * dp[e];
        }
      }
      if (need_dz) {
        if (!BAND || kind != KIND_BAND) {
          float tsum = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) tsum += ds[e];
          if (kind == KIND_LO) acc_lo += tsum; else acc_hi += tsum;
        } else if (kHalf && band_interior(j0 + 32 * st)) {
          if constexpr (STAGE) band_store_runs(ds, j0 + 32 * st, zs.buf[st]);
          else band_store_row(ds, j0 + 32 * st);
        } else {
          // saturated entries go to the two per-query accumulators (masked
          // entries have ds = 0).  With a wide band (most tiles inside it)
          // the subtile goes through LDS so that each store instruction
          // writes two 128-byte runs of dZ^Q rows (a query row holds its 32
          // keys at consecutive offsets) instead of 64 scattered words; a
          // narrow band has few fully interior subtiles and stores directly.
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int j = j0 + 32 * st + kappa<T>(hl, e);
            const int o = j - c.iq;
            if (o <= g.lo) {
              acc_lo += ds[e];
            } else if (o >= g.hi) {
              acc_hi += ds[e];
            } else if (!STAGE && c.iq < N && j < N && !(g.causal && j > c.iq)) {
              dz_row[o - g.lo - c.wsq] = tau * ds[e];
            }
          }
          if constexpr (STAGE) band_store(ds, j0 + 32 * st, zs.buf[st]);
        }
      }
      if (BAND && STAGE && kind == KIND_BAND && stage_next) {
        if (st == 0) stage_zq<0>(t + kGroups); else stage_zq<1>(t + kGroups);
      }
      frag sf[KPS];
#pragma unroll
      for (int kk = 0; kk < KPS; ++kk) sf[kk] = M::pack(&ds[kk * E]);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int kk = 0; kk < KPS; ++kk) {
          frag kf;
          if constexpr (kHalf) {
            kf = tr.read(tK, dt, KPS * st + kk);
          } else {
            kf = dfrag_t32(tK, 32 * dt + l32, KS * (KPS * st + kk) + E * hl);
          }
          dq[dt] = M::mma(kf, sf[kk], dq[dt]);
        }
    }
  }

  // Key tile t (none once t >= nkt) from buffer BUF with the loads of the
  // group's next tile in flight; tiles [0, t1) are left-saturated, [t2, nkt)
  // right-saturated.
  template <int BUF>
  __device__ __forceinline__ void step(int t, int t1, int t2) {
    const int tn = t + kGroups;
    if (tn < nkt) issue<BUF ^ 1>(tn);
    // (one group: t < nkt always holds)
    // Z^Q rows of the group's next tile: staged now when tile t leaves the
    // areas free, else from tile t's band path
    const bool bn = band_here(tn), bc = band_here(t);
    if (bn && !bc) {
      stage_zq<0>(tn);
      stage_zq<1>(tn);
    }
    if (kGroups == 1 || t < nkt) {
      // tiles with masked entries also take the band body
      const int j0 = t * kTile;
      const bool masked = (j0 + kTile > c.kv_end) || (g.causal && j0 + kTile - 1 > iw0);
      if ((t >= t1 && t < t2) || masked)
        tile<true, BUF>(t, KIND_BAND, bn && bc);
      else
        tile<false, BUF>(t, t < t1 ? KIND_LO : KIND_HI, false);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  }

  // Group grp takes key tiles grp, grp + kGroups, ...; every group runs the
  // same number of steps (one workgroup barrier each), step m in buffer m & 1.
  __device__ __forceinline__ void run(int t1, int t2) {
    const int t0 = grp;
    if (t0 < nkt) issue<0>(t0);
    if (band_here(t0)) {
      stage_zq<0>(t0);
      stage_zq<1>(t0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    const int nsteps = (nkt + kGroups - 1) / kGroups;
    for (int m = 0; m < nsteps; m += 2) {
      step<0>(t0 + kGroups * m, t1, t2);
      if (m + 1 < nsteps) step<1>(t0 + kGroups * (m + 1), t1, t2);
    }
  }
};

// ZQ / ZK: whether the query-side / key-side relation term is present
// (compile-time switches: code for an absent term is not generated, which
// keeps its registers out of the allocation); STAGE: band stores staged
// through LDS; GRP: grouped workgroup.
// One query block of the pass: block number bid of a launch over
// B*H*nblk blocks.  LDS (sizes for G = query_groups groups): sK0..sV1
// G*DTile bytes each, sZK0/sZK1 G*2*kTile floats, sSt0/sSt1 (STAGE only)
// 4*G*kStageFloats floats.
template <typename T, bool ZQ, bool ZK, bool STAGE, bool GRP, bool DROP, bool SCHED>
__device__ __forceinline__ void bwd_q_block(const AttnArgs& a, int bid, char* sK0, char* sK1,
                                            char* sV0, char* sV1, float* sZK0, float* sZK1,
                                            float* sSt0, float* sSt1) {
  using M = MT<T>;
  using B = BwdQ<T, STAGE, GRP, DROP, SCHED>;
  constexpr int TB = DTile<T>::BYTES;
  constexpr int G = B::kGroups;

  const int tid = threadIdx.x, wall = wave_id(), lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int grp = G == 2 ? wall >> 2 : 0, w = wall & 3;
  B q;
  q.grp = grp;
  // the group offset goes into the per-lane fragment offsets, so that the
  // LDS reads keep compile-time buffer bases
  q.goff = grp * TB;
  q.sK[0] = sK0;
  q.sK[1] = sK1;
  q.sV[0] = sV0;
  q.sV[1] = sV1;
  q.sZK[0] = sZK0;
  q.sZK[1] = sZK1;
  q.g = a.geo;
  const Geo& g = q.g;
  const int N = g.N;
  q.N = N;
  q.w = w;
  q.lane = lane;
  q.hl = hl;
  q.l32 = l32;
  // the pass covers the query blocks [qb0, qb0 + nqb) of every (b, h)
  const int total = a.B * a.H * a.nqb;
  int bh, qb;
  block_of(bid, total, a.nqb, g.causal, bh, qb);
  if (g.causal) qb = a.nqb - 1 - qb;  // longest rows first
  qb += a.qb0;
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int i0 = qb * kBlockRows, iw0 = i0 + 32 * w, iq = iw0 + l32;
  q.i0 = i0;
  q.iw0 = iw0;

  int kv_end = N;
  if (a.flags & F_KEYPAD) kv_end = imax(0, imin(N, a.key_len[bb]));
  int kv_blk = kv_end;
  if (g.causal) kv_blk = imin(kv_blk, i0 + kBlockRows);
  const int nkt = kv_blk > 0 ? (kv_blk + kTile - 1) / kTile : 0;
  q.nkt = nkt;
  q.kv_lim = imin(N, nkt * kTile);  // keys written by the band stores

  q.Kb = (const T*)a.k + bb * a.sk.b + hh * a.sk.h;
  q.Vb = (const T*)a.v + bb * a.sv.b + hh * a.sv.h;
  q.sk = a.sk.n;
  q.sv = a.sv.n;
  q.Np = a.Np;
  q.ldK.init(a.sk.n, w, lane);
  q.ldV.init(a.sv.n, w, lane);
  if constexpr (B::kHalf) {
    q.tr.init(lane, q.goff);
    const int sig = sigma<T>(l32);
#pragma unroll
    for (int ks = 0; ks < B::NSD; ++ks)
      q.kofs[ks] = q.goff + dt_off<T>(sig, B::KS * ks + B::E * hl);
  }

  QCtx& c = q.c;
  c.iq = iq;
  c.hl = hl;
  c.sig = sigma<T>(l32);
  c.kv_end = kv_end;
  c.has_zq = ZQ && (a.flags & F_ZQ);
  c.has_zk = ZK;
  // (with a query-side table b is folded into Z^Q: no lookup of its own,
  // and no code for one)
  c.has_b = !ZQ && (a.flags & F_B);
  c.wsq = win_q(g, qb);
  c.zq_row = c.has_zq ? a.zq + zq_off(g, bh, imin(iq, zq_last(g))) : nullptr;
  c.zkb = c.has_zk ? a.zk + (int64_t)bh * N * g.Wp : nullptr;
  c.bun = c.has_b ? a.bunf + hh * a.bunf_hs : nullptr;
  q.need_dz = a.flags & F_ZQ_NEEDED;
  qside_consts(g, c, qb, q.cst_lo, q.cst_hi);
  q.sc2 = a.scale2;
  q.tau = a.tau;
  if constexpr (DROP) q.dr = drop_ctx(a, bh, lane);

  {
    const T* qrow = (const T*)a.q + bb * a.sq.b + hh * a.sq.h + (int64_t)iq * a.sq.n;
    const T* drow = (const T*)a.dO + bb * a.sdo.b + hh * a.sdo.h + (int64_t)iq * a.sdo.n;
#pragma unroll
    for (int ks = 0; ks < B::NSD; ++ks) {
      q.qf[ks] = iq < N ? frag_g<T>(qrow, B::KS * ks + B::E * hl) : M::zero();
      q.df[ks] = iq < N ? frag_g<T>(drow, B::KS * ks + B::E * hl) : M::zero();
    }
    // padded row terms: +inf / 0 beyond N and for rows with every key masked
    q.lse2 = a.L2[(int64_t)bh * a.Np + imin(iq, a.Np - 1)];
    q.Dl = a.D[(int64_t)bh * a.Np + imin(iq, a.Np - 1)];
#pragma unroll
    for (int e = 0; e < 16; ++e) q.dseed[e] = -q.Dl;
  }
  // (dz_row at the row's column shift, dz_shift; dz_w at row iw0, unshifted)
  q.dz_row = q.need_dz ? a.dzq + zq_off(g, bh, iq) + ((iq + g.lo + c.wsq) & g.dsm) : nullptr;
  q.dz_w = q.need_dz ? a.dzq + zq_off(g, bh, iw0) : nullptr;
  q.zs.buf[0] = STAGE ? sSt0 + wall * kStageFloats : sSt0;
  q.zs.buf[1] = STAGE ? sSt1 + wall * kStageFloats : sSt1;
  q.zs.init(g, c.has_zq ? a.zq + zq_off(g, bh, 0) : nullptr, -1, lane);
  q.dq[0] = zero16();
  q.dq[1] = zero16();
  q.acc_lo = 0.f;
  q.acc_hi = 0.f;

  // this wave's segments: key tiles [0, t1) have all offsets <= lo for its
  // 32 queries, [t2, nkt) all offsets >= hi, the band in between (a tile
  // goes through the band body only for the waves that need it)
  const int t1 = imin(nkt, imax(0, floor_div_q(g.lo + iw0 - (kTile - 1), kTile) + 1));
  const int t2 = imin(nkt, imax(t1, ceil_div_q(g.hi + iw0 + 31, kTile)));

  q.run(t1, t2);

  if constexpr (G == 2) {
    // group 1 hands dQ and the two sums to group 0 (lane-contiguous, in the
    // K / V buffers, which every wave is done with after the last barrier)
    const int t = tid & (4 * 64 - 1);
    float* x0 = reinterpret_cast<float*>(sK0);
    float* x1 = reinterpret_cast<float*>(sK1);
    float* x2 = reinterpret_cast<float*>(sV0);
    static_assert(G * TB >= 16 * 256 * 4, "combine buffers");
    if (grp == 1) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        x0[e * 256 + t] = q.dq[0][e];
        x1[e * 256 + t] = q.dq[1][e];
      }
      x2[t] = q.acc_lo;
      x2[256 + t] = q.acc_hi;
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      q.dq[0][e] += x0[e * 256 + t];
      q.dq[1][e] += x1[e * 256 + t];
    }
    q.acc_lo += x2[t];
    q.acc_hi += x2[256 + t];
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
          store4<float>(prow + d, a.tau * q.dq[dt][4 * e4], a.tau * q.dq[dt][4 * e4 + 1],
                        a.tau * q.dq[dt][4 * e4 + 2], a.tau * q.dq[dt][4 * e4 + 3]);
        }
    } else {
      T* orow = (T*)a.dq + bb * a.sdq.b + hh * a.sdq.h + (int64_t)iq * a.sdq.n;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int d = 32 * dt + 8 * e4 + 4 * hl;
          store4<T>(orow + d, a.tau * q.dq[dt][4 * e4], a.tau * q.dq[dt][4 * e4 + 1],
                    a.tau * q.dq[dt][4 * e4 + 2], a.tau * q.dq[dt][4 * e4 + 3]);
        }
    }
  }

  if (q.need_dz) {
    float acc_lo = sum_xor32(q.acc_lo);
    float acc_hi = sum_xor32(q.acc_hi);
    float* dz_row = q.dz_row;
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
      for (int col = imax(ib, q.kv_lim - shift) + hl; col < ie; col += 2) dz_row[col] = 0.f;
    }
  }
}

}  // namespace relpos
