// attn_bwd_k.hpp -- the key-parallel backward pass (one block of it).
//
// Source: "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (nanless.github.io digest), section on the backward pass: the
// key-parallel pass recomputes the scores and accumulates dK, dV and the
// key-side relation gradient dZ^K[j, r] = tau * sum_{i: phi(i,j) = r} dS_ij
// (Eq. 4), stored per offset by the block that owns the key (for a fixed key,
// queries and offsets correspond one to one); the saturated rows collect in
// two on-chip sums per key.
//
// One workgroup = one (batch, head, 128-key block): 4 waves x 32 keys, or,
// for a causal 16-bit launch whose blocks all fit on the device at once, 8
// waves in two groups of 4 x 32 keys that take alternate 64-query tiles (each
// group with its own LDS buffers) and sum their accumulators through LDS at
// the end: the early key blocks of a causal problem hold most of the work, so
// the longest block bounds such a launch, and splitting its query range halves
// it.  (With more blocks the longest-first order balances the CUs, and two
// independent 4-wave blocks per CU overlap MFMA and vector work better than
// one 8-wave block whose groups share every barrier.)  Orientation
// S = Q K^T: lane l owns key l % 32.
#pragma once
#include "dropout.hpp"
#include "qside.hpp"

namespace relpos {

__device__ inline int tile_kind_k(const Geo& g, int qt0, int jw0) {
  int omax = jw0 + 31 - qt0;
  int omin = jw0 - (qt0 + kTile - 1);
  return omax <= g.lo ? KIND_LO : (omin >= g.hi ? KIND_HI : KIND_BAND);
}

__device__ inline int floor_div_k(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
__device__ inline int ceil_div_k(int a, int b) { return -floor_div_k(-a, b); }

constexpr int kStagePitchK = 36;  // floats per staged key row (16-byte aligned, bank-spread)
// Window width from which band dZ^K stores are staged: the band's tiles are
// few but each holds many interior entries.
constexpr int kStageMinWK = 512;

// Groups of 4 waves per workgroup (see the header comment).
template <typename T, bool GRP>
constexpr int key_groups() {
  return (GRP && sizeof(T) == 2) ? 2 : 1;
}

template <typename T, bool GRP>
constexpr int key_threads() {
  return kThreads * key_groups<T, GRP>();
}
// blocks per CU for 2 waves per SIMD (fp32: 1 block)
template <typename T, bool GRP>
constexpr int key_blocks_per_cu() {
  return (key_groups<T, GRP>() == 1 && sizeof(T) == 2) ? 2 : 1;
}

// STAGE: band dZ^K stores go through an LDS staging area; GRP: two groups
// of waves split the query tiles; DROP: attention dropout.
// SCHED: use the compiler's scheduling strategy 0 in the subtile loop.
template <typename T, bool STAGE, bool GRP, bool DROP, bool SCHED>
struct BwdK {
  static constexpr int kGroups = key_groups<T, GRP>();
  using M = MT<T>;
  using frag = typename M::frag;
  static constexpr bool kHalf = sizeof(T) == 2;
  static constexpr int KS = M::KS, E = M::E, NSD = kHeadDim / KS;
  static constexpr int KPS = 32 / KS;  // MFMA k-steps per 32-query half
  static constexpr int TB = DTile<T>::BYTES;
  static constexpr int ROWB = DTile<T>::ROWB;

  // LDS buffers, two of each (separate arrays, so that the compiler can tell
  // the asynchronous loads into one buffer from the reads of the other)
  char* sQ[2];     // Q rows (group 0's buffers; this group's start goff bytes in)
  char* sO[2];     // dO rows
  int goff;        // byte offset of this group's Q / dO buffers
  float* sR[2];    // [4][kTile] per-query seeds of the tile (see RowTermArgs)

  Geo g;
  int w, lane, hl, l32, j0b, jw0, jk, sig, ntq, N, kv_end, wsk;  // w: wave within its group
  int grp;                                                        // this wave's group
  bool has_zq, has_zk, has_b;
  float off_lo, off_hi, sc2, tau;
  // Padded keys (key >= the batch's key length) need no mask: a lane's P and
  // dS only reach its own key's dK, dV and dZ^K, which are written as zeros
  // at the end (and its band dZ^K stores are skipped), so key padding never
  // sends a tile to the band body.
  const T* Qb;
  const T* Ob;
  const float* seeds;   // [4][B*H][Np]: LO seed, HI seed, band seed, -D (-D (1 - p): dropout)
  int64_t seed_stride;  // B*H*Np
  const float* zq_bh;
  const float* zk_row;
  const float* bun;
  float* dz_row;
  float* dz_w;    // dZ^K row of this wave's first key (jw0)
  float* stage;   // STAGE: this wave's [32][kStagePitchK] LDS area
  int64_t sq, so, Np;
  DLoader<T> ldQ, ldO;
  // per-lane LDS byte offsets of the 16-bit row fragments (Q / dO row
  // sigma(l32) at k-step ks); transposed fragments (Q^T, dO^T, contracted
  // over the queries) come from the same row tiles through transpose reads
  int rofs[kHalf ? NSD : 1];
  TrReader<std::conditional_t<kHalf, T, _Float16>> tr;
  frag kf[NSD], vf[NSD];
  f32x16 dk[2], dv[2];
  float acc_lo, acc_hi;
  DropCtx dr;  // DROP only

  template <int BUF>
  __device__ __forceinline__ void issue(int t) {
    const int q0 = t * kTile;
    ldQ.load(sQ[BUF] + goff, Qb + (int64_t)q0 * sq, N - q0, lane);
    ldO.load(sO[BUF] + goff, Ob + (int64_t)q0 * so, N - q0, lane);
    // wave w brings seed vector w of the tile's 64 queries
    dword_direct((char*)(sR[BUF] + w * kTile), seeds + w * seed_stride + q0 + lane, true, lane);
  }

  // Row fragment (tile row 32 st + sigma(l32), k-step ks) of Q or dO.
  __device__ __forceinline__ frag rfrag(const char* tile, int st, int ks) const {
    if constexpr (kHalf) {
      return *reinterpret_cast<const frag*>(tile + rofs[ks] + st * 32 * ROWB);
    } else {
      return dfrag<T>(tile + goff, 32 * st + sig, KS * ks + E * hl);
    }
  }
  // Transposed fragment (d row 32 dt + l32, query chunk column c4) of Q^T or
  // dO^T, read from the row tile.
  __device__ __forceinline__ frag tfrag(const char* rowtile, int dt, int c4) const {
    if constexpr (kHalf) {
      return tr.read(rowtile, dt, c4);
    } else {
      return dfrag_t32(rowtile + goff, 32 * dt + l32, KS * c4 + E * hl);
    }
  }

  // Relation response of this lane's key against the 16 band queries
  // ib + kap0(e) (all in the query group of the tile).  Every load is issued
  // without a branch at an address clamped into its row (rows clamped to
  // N - 1), so the loads of a subtile are in flight together.  Entries that
  // are not live are replaced by -inf afterwards or belong to a discarded
  // key; for a live entry the clamps are the identity.
  __device__ __forceinline__ void band_rel(int ib, int wq, float (&v)[16]) const {
    const int Wm = g.W - 1;
    if (has_zq) {
      const int ilast = zq_last(g);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int i = imin(ib + kap0<T>(e), ilast);
        v[e] += zq_bh[(int64_t)i * g.Wp + imin(imax(jk - i - g.lo - wq, 0), Wm)];
      }
    }
    if (has_zk) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        v[e] += zk_row[imin(imax(jk - ib - kap0<T>(e) - g.lo - wsk, 0), Wm)];
    }
    if (has_b) {
      // (all loads first, then the sums, so that they are in flight together)
      float bv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) bv[e] = bun[imin(imax(jk - ib - kap0<T>(e) - g.lo, 0), g.R - 1)];
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] += bv[e];
    }
  }

  // Store tau * ds of the 32 x 32 subtile (queries ib .. ib + 31) into dZ^K
  // through LDS: entry (key jw0 + q, query ib + k) goes to offset
  // o = jw0 + q - ib - k of key row jw0 + q when it is live and strictly
  // inside the band.  A store instruction then writes two 128-byte runs of
  // key rows (a key's 32 queries sit at consecutive offsets) instead of 64
  // scattered words.
  __device__ __forceinline__ void band_store(const float (&ds)[16], int ib) {
    // registers -> LDS [key][query]: lane (l32, hl) holds queries kappa(hl, e)
    if constexpr (kHalf) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int k0 = kappa<T>(hl, 4 * e4);
        *reinterpret_cast<f32x4*>(stage + l32 * kStagePitchK + k0) = f32x4{
            tau * ds[4 * e4], tau * ds[4 * e4 + 1], tau * ds[4 * e4 + 2], tau * ds[4 * e4 + 3]};
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) stage[l32 * kStagePitchK + kappa<T>(hl, e)] = tau * ds[e];
    }
    // LDS -> HBM: key rows q = 2 r + hl, query l32 of each
    const int i = ib + l32;
#pragma unroll 1
    for (int r = 0; r < 16; ++r) {
      const int q = 2 * r + hl;
      const float v = stage[q * kStagePitchK + l32];
      const int j = jw0 + q;
      const int o = j - i;
      if (o > g.lo && o < g.hi && i < N && j < kv_end && !(g.causal && j > i))
        dz_w[(int64_t)q * g.Wp + o - g.lo - wsk] = v;
    }
  }

  // Whether every entry of the 32 x 32 subtile (this wave's keys, queries
  // [qb, qb + 32)) is live and strictly inside the band (wave-uniform).
  __device__ __forceinline__ bool band_interior(int qb) const {
    return jw0 - qb - 31 > g.lo && jw0 + 31 - qb < g.hi && qb + 31 < N &&
           jw0 + 31 < imin(N, kv_end) && !(g.causal && jw0 + 31 > qb);
  }

  // Band stores of an interior subtile (16-bit operands): a lane's elements
  // e = 0..7 and 8..15 are eight consecutive queries each (kappa), hence
  // eight consecutive offsets of its key's dZ^K row in descending order,
  // written as four 16-byte stores.
  __device__ __forceinline__ void band_store_row(const float (&ds)[16], int qb) {
    float* p = dz_row + (jk - qb - E * hl - g.lo - wsk);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e0 = 4 * u;
      store_f32x4_a4(p - (u < 2 ? 4 * u + 3 : 16 + 4 * (u - 2) + 3),
                     f32x4{tau * ds[e0 + 3], tau * ds[e0 + 2], tau * ds[e0 + 1], tau * ds[e0]});
    }
  }

  // One 64-query tile from LDS buffer BUF.  BAND: the wave's tile crosses
  // the band or holds masked entries (each wave refines the kind for its
  // own keys); otherwise the whole tile is saturated on side `sat`.
  //
  // Per 32-query half: S' = seed + Q K^T, where the seed (per query, from
  // the row-term pass) already holds -LSE/(tau log2 e) and, on saturated
  // tiles, the query-side saturated relation scalar; P = exp2(S' * tau
  // log2 e + key-side constant).  dP' = -D + dO V^T, so dS = P * dP' (the
  // dropout variant below rescales it).
  template <bool BAND, int BUF>
  __device__ __forceinline__ void tile(int t, int sat) {
    const int qt0 = t * kTile;
    // (a wave whose keys are all padded contributes nothing: its band tiles
    // are skipped, and whatever its saturated tiles accumulate is discarded)
    if (BAND && (jw0 >= imin(N, kv_end) || (g.causal && qt0 + kTile - 1 < jw0))) return;
    const int kind = BAND ? tile_kind_k(g, qt0, jw0) : sat;
    // masks are only applied in the band body (a saturated body is only
    // used for tiles that need no mask anywhere in the block)
    const bool needmask =
        BAND && ((qt0 + kTile > N) || (g.causal && jw0 + 31 > qt0));
    const char* tQ = sQ[BUF];
    const char* tO = sO[BUF];
    const float* sr = sR[BUF];
    const float off = kind == KIND_LO ? off_lo : (kind == KIND_HI ? off_hi : 0.f);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      // scheduling strategy 0 of the compiler (interleave the LDS operand
      // reads with the MFMAs): -1% to -2% on the passes, measured
      if constexpr (SCHED) __builtin_amdgcn_iglp_opt(0);
      f32x16 s;
      {
        float v[16];
        if (!BAND || kind != KIND_BAND) {
          lds_rows16<T>(sr + (kind == KIND_LO ? 0 : kTile) + 32 * st, hl, v);
        } else {
          lds_rows16<T>(sr + 2 * kTile + 32 * st, hl, v);
          band_rel(qt0 + 32 * st + E * hl, win_q(g, qt0 / kGroup), v);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = v[e];
      }
#pragma unroll
      for (int ks = 0; ks < NSD; ++ks) s = M::mma(rfrag(tQ, st, ks), kf[ks], s);
      if (needmask) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int i = qt0 + 32 * st + kappa<T>(hl, e);
          if (i >= N || (g.causal && jk > i)) s[e] = -INFINITY;
        }
      }
      f32x16 dp;
      if constexpr (DROP) {
        dp = zero16();  // the seed is added per entry below
      } else {
        float v[16];
        lds_rows16<T>(sr + 3 * kTile + 32 * st, hl, v);
#pragma unroll
        for (int e = 0; e < 16; ++e) dp[e] = v[e];
      }
#pragma unroll
      for (int ks = 0; ks < NSD; ++ks) dp = M::mma(rfrag(tO, st, ks), vf[ks], dp);

      float p[16], ds[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = exp2_fast(fmaf(s[e], sc2, off));
        ds[e] = p[e] * dp[e];
      }
      if constexpr (DROP) {
        // with the seed v = -D (1 - p) of each query: kept, dS = P (dP /
        // (1 - p) - D) = P (dP + v) / (1 - p); dropped, dS = -P D = P v /
        // (1 - p); dV takes the kept P only (its 1 / (1 - p) is applied once,
        // at the end)
        const uint32_t kb = drop_bits<T, false>(dr, jk, qt0 + 32 * st, hl);
        float v[16];
        lds_rows16<T>(sr + 3 * kTile + 32 * st, hl, v);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const bool kp = (kb >> e) & 1u;
          ds[e] = p[e] * dr.scale * (kp ? dp[e] + v[e] : v[e]);
          p[e] = kp ? p[e] : 0.f;
        }
      }
      if (has_zk) {
        if (!BAND || kind != KIND_BAND) {
          float tsum = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) tsum += ds[e];
          if (kind == KIND_LO) acc_lo += tsum; else acc_hi += tsum;
        } else if (kHalf && band_interior(qt0 + 32 * st)) {
          band_store_row(ds, qt0 + 32 * st);
        } else {
          // saturated entries of a band tile go to the two accumulators
          // (masked entries have ds = 0); interior live entries are stored
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int i = qt0 + 32 * st + kappa<T>(hl, e);
            const int o = jk - i;
            // (lo == hi: an offset equal to both counts once, on the low side)
            acc_lo += o <= g.lo ? ds[e] : 0.f;
            acc_hi += (o > g.lo && o >= g.hi) ? ds[e] : 0.f;
            if (!STAGE && o > g.lo && o < g.hi && i < N && jk < kv_end && !(g.causal && jk > i))
              dz_row[o - g.lo - wsk] = tau * ds[e];
          }
          if constexpr (STAGE) band_store(ds, qt0 + 32 * st);
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
          dv[dt] = M::mma(tfrag(tO, dt, KPS * st + kk), pf[kk], dv[dt]);
          dk[dt] = M::mma(tfrag(tQ, dt, KPS * st + kk), sf[kk], dk[dt]);
        }
    }
  }

  // Query tile t from buffer BUF with the loads of tile t + 1 in flight;
  // Query tile t (none once t >= ntq) from buffer BUF with the loads of the
  // group's next tile in flight; tiles before tA have all offsets >= hi,
  // tiles from tB on all <= lo.
  template <int BUF>
  __device__ __forceinline__ void step(int t, int tA, int tB) {
    if (t + kGroups < ntq) issue<BUF ^ 1>(t + kGroups);
    if (t < ntq) {
      // tiles with masked entries also take the band body
      const int qt0 = t * kTile;
      const bool masked = (qt0 + kTile > N) || (g.causal && jw0 + 31 > qt0);
      if ((t >= tA && t < tB) || masked)
        tile<true, BUF>(t, KIND_BAND);
      else
        tile<false, BUF>(t, t < tA ? KIND_HI : KIND_LO);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  }

  // Group grp takes tiles t_begin + grp, t_begin + grp + kGroups, ...; every
  // group runs the same number of steps (one workgroup barrier each), step m
  // in buffer m & 1.
  __device__ __forceinline__ void run(int t_begin, int tA, int tB) {
    const int t0 = t_begin + grp;
    if (t0 < ntq) issue<0>(t0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    const int nsteps = ntq > t_begin ? (ntq - t_begin + kGroups - 1) / kGroups : 0;
    for (int m = 0; m < nsteps; m += 2) {
      step<0>(t0 + kGroups * m, tA, tB);
      if (m + 1 < nsteps) step<1>(t0 + kGroups * (m + 1), tA, tB);
    }
  }
};

// ZQ / ZK: whether the query-side / key-side relation term is present
// (compile-time switches: code for an absent term is not generated, which
// keeps its registers out of the allocation); STAGE: band dZ^K stores staged
// through LDS; GRP: grouped workgroup.
// One key block of the pass: block number bid of a launch over B*H*nblk
// blocks.  LDS (sizes for G = key_groups groups): sQ0..sO1 G*DTile bytes
// each, sR0/sR1 G*4*kTile floats, sSt (STAGE only) 4*G*32*kStagePitchK
// floats.
template <typename T, bool ZQ, bool ZK, bool STAGE, bool GRP, bool DROP, bool SCHED>
__device__ __forceinline__ void bwd_k_block(const AttnArgs& a, int bid, char* sQ0, char* sQ1,
                                            char* sO0, char* sO1, float* sR0, float* sR1,
                                            float* sSt) {
  using M = MT<T>;
  using K = BwdK<T, STAGE, GRP, DROP, SCHED>;
  constexpr int TB = DTile<T>::BYTES;
  constexpr int G = K::kGroups;

  const int tid = threadIdx.x, wall = wave_id(), lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int grp = G == 2 ? wall >> 2 : 0, w = wall & 3;
  K k;
  k.grp = grp;
  // the group offset goes into the per-lane fragment offsets, so that the
  // LDS reads keep compile-time buffer bases
  k.goff = grp * TB;
  k.sQ[0] = sQ0;
  k.sQ[1] = sQ1;
  k.sO[0] = sO0;
  k.sO[1] = sO1;
  k.sR[0] = sR0 + grp * 4 * kTile;
  k.sR[1] = sR1 + grp * 4 * kTile;
  k.g = a.geo;
  const Geo& g = k.g;
  const int N = g.N;
  k.N = N;
  k.w = w;
  k.lane = lane;
  k.hl = hl;
  k.l32 = l32;
  const int total = a.B * a.H * a.nblk;
  int bh, kb;  // causal: early key blocks have the most queries (first)
  block_of(bid, total, a.nblk, g.causal, bh, kb);
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int j0b = kb * kBlockRows, jw0 = j0b + 32 * w, jk = jw0 + l32;
  k.j0b = j0b;
  k.jw0 = jw0;
  k.jk = jk;
  k.sig = sigma<T>(l32);
  k.has_zq = ZQ;
  k.has_zk = ZK && (a.flags & F_ZK);
  // (with a query-side table b is folded into Z^Q: no lookup of its own,
  // and no code for one)
  k.has_b = !ZQ && (a.flags & F_B);

  int kv_end = N;
  if (a.flags & F_KEYPAD) kv_end = imax(0, imin(N, a.key_len[bb]));
  k.kv_end = kv_end;
  // query tiles of this launch: [qt0, qt1), from the causal diagonal on
  const int qt_begin = imax(g.causal ? j0b / kTile : 0, a.qt0);
  const int ntq = imin((N + kTile - 1) / kTile, a.qt1);
  k.ntq = ntq;
  // Whole block padded away: nothing to recompute, every output is zero.
  const int t_begin = (j0b >= kv_end) ? ntq : imin(qt_begin, ntq);

  k.Qb = (const T*)a.q + bb * a.sq.b + hh * a.sq.h;
  k.Ob = (const T*)a.dO + bb * a.sdo.b + hh * a.sdo.h;
  k.sq = a.sq.n;
  k.so = a.sdo.n;
  k.Np = a.Np;
  k.ldQ.init(a.sq.n, w, lane);
  k.ldO.init(a.sdo.n, w, lane);
  if constexpr (K::kHalf) {
    k.tr.init(lane, k.goff);
    const int sg = sigma<T>(l32);
#pragma unroll
    for (int ks = 0; ks < K::NSD; ++ks)
      k.rofs[ks] = k.goff + dt_off<T>(sg, K::KS * ks + K::E * hl);
  }
  k.seed_stride = (int64_t)a.B * a.H * a.Np;
  k.seeds = a.kseed + (int64_t)bh * a.Np;
  k.zq_bh = k.has_zq ? a.zq + zq_off(g, bh, 0) : nullptr;
  k.bun = k.has_b ? a.bunf + hh * a.bunf_hs : nullptr;
  k.wsk = win_k(g, kb);
  k.zk_row = k.has_zk ? a.zk + ((int64_t)bh * N + imin(jk, N - 1)) * g.Wp : nullptr;
  k.dz_row = k.has_zk ? a.dzk + ((int64_t)bh * N + jk) * g.Wp : nullptr;
  k.dz_w = k.has_zk ? a.dzk + ((int64_t)bh * N + jw0) * g.Wp : nullptr;
  k.stage = STAGE ? sSt + wall * 32 * kStagePitchK : sSt;
  k.sc2 = a.scale2;
  k.tau = a.tau;
  if constexpr (DROP) k.dr = drop_ctx(a, bh, lane);

  // Key-side constants of saturated tiles, Z^K[j, first/last row] + b, in
  // the exp2 domain.
  float cst_lo = 0.f, cst_hi = 0.f;
  if (k.has_zk && jk < N) {
    int cb, ce;
    cols_k(g, kb, cb, ce);
    const int c0 = 0 - k.wsk, c1 = g.R - 1 - k.wsk;
    if (c0 >= cb && c0 < ce) cst_lo += k.zk_row[c0];
    if (c1 >= cb && c1 < ce) cst_hi += k.zk_row[c1];
  }
  if (k.has_b) {
    cst_lo += k.bun[0];
    cst_hi += k.bun[g.R - 1];
  }
  k.off_lo = cst_lo * a.scale2;
  k.off_hi = cst_hi * a.scale2;
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

  // this wave's segments over the query tiles [t_begin, ntq): for its 32
  // keys all offsets >= hi first, then the band, then all offsets <= lo (a
  // tile goes through the band body only for the waves that need it)
  const int tA = imin(ntq, imax(t_begin, floor_div_k(jw0 - (kTile - 1) - g.hi, kTile) + 1));
  const int tB = imin(ntq, imax(tA, ceil_div_k(jw0 + 31 - g.lo, kTile)));

  k.run(t_begin, tA, tB);

  if constexpr (G == 2) {
    // group 1 hands dV, dK and the two sums to group 0 (lane-contiguous, in
    // the Q / dO buffers, which every wave is done with after the last
    // barrier); group 0 adds them and writes everything
    const int t = tid & (4 * 64 - 1);
    float* x0 = reinterpret_cast<float*>(sQ0);
    float* x1 = reinterpret_cast<float*>(sQ1);
    float* x2 = reinterpret_cast<float*>(sO0);
    float* x3 = reinterpret_cast<float*>(sO1);
    static_assert(G * TB >= 16 * 256 * 4, "combine buffers");
    if (grp == 1) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        x0[e * 256 + t] = k.dv[0][e];
        x1[e * 256 + t] = k.dv[1][e];
        x2[e * 256 + t] = k.dk[0][e];
        x3[e * 256 + t] = k.dk[1][e];
      }
      sR0[t] = k.acc_lo;
      sR0[256 + t] = k.acc_hi;
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      k.dv[0][e] += x0[e * 256 + t];
      k.dv[1][e] += x1[e * 256 + t];
      k.dk[0][e] += x2[e * 256 + t];
      k.dk[1][e] += x3[e * 256 + t];
    }
    k.acc_lo += sR0[t];
    k.acc_hi += sR0[256 + t];
  }

  if constexpr (DROP) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      k.dv[0][e] *= a.drop_scale;
      k.dv[1][e] *= a.drop_scale;
    }
  }
  if (jk >= kv_end) {
    // a padded key: exact zeros (its unmasked scores were accumulated)
    k.dk[0] = zero16();
    k.dk[1] = zero16();
    k.dv[0] = zero16();
    k.dv[1] = zero16();
    k.acc_lo = 0.f;
    k.acc_hi = 0.f;
  }
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) k.dk[dt][e] *= a.tau;
  if (jk < N && a.kacc) {
    // one of several launches over disjoint query ranges: the fp32 sums of
    // the earlier ones are added in launch order, and all but the last
    // launch hand theirs on instead of writing the outputs
    float* av = a.dv_acc + ((int64_t)bh * N + jk) * kHeadDim;
    float* ak = a.dk_acc + ((int64_t)bh * N + jk) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = 32 * dt + 8 * e4 + 4 * hl;
        if (a.kacc & 1) {
          const f32x4 pv = *reinterpret_cast<const f32x4*>(av + d);
          const f32x4 pk = *reinterpret_cast<const f32x4*>(ak + d);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            k.dv[dt][4 * e4 + t] = pv[t] + k.dv[dt][4 * e4 + t];
            k.dk[dt][4 * e4 + t] = pk[t] + k.dk[dt][4 * e4 + t];
          }
        }
        if (a.kacc & 2) {
          store4<float>(av + d, k.dv[dt][4 * e4], k.dv[dt][4 * e4 + 1], k.dv[dt][4 * e4 + 2],
                        k.dv[dt][4 * e4 + 3]);
          store4<float>(ak + d, k.dk[dt][4 * e4], k.dk[dt][4 * e4 + 1], k.dk[dt][4 * e4 + 2],
                        k.dk[dt][4 * e4 + 3]);
        }
      }
  }
  if (jk < N && !(a.kacc & 2)) {
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
          store4<float>(prow + d, k.dk[dt][4 * e4], k.dk[dt][4 * e4 + 1], k.dk[dt][4 * e4 + 2],
                        k.dk[dt][4 * e4 + 3]);
        }
    } else {
      T* krow = (T*)a.dk + bb * a.sdk.b + hh * a.sdk.h + (int64_t)jk * a.sdk.n;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int d = 32 * dt + 8 * e4 + 4 * hl;
          store4<T>(krow + d, k.dk[dt][4 * e4], k.dk[dt][4 * e4 + 1], k.dk[dt][4 * e4 + 2],
                    k.dk[dt][4 * e4 + 3]);
        }
    }
  }

  if (k.has_zk) {
    const float acc_lo = sum_xor32(k.acc_lo);
    const float acc_hi = sum_xor32(k.acc_hi);
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
      // Queries written by the band stores: [q_lo, q_hi) (none for a padded
      // key).  Interior columns of any other query carry no gradient and are
      // zeroed.
      const bool wave_ran = jw0 < imin(N, kv_end) && t_begin < ntq;
      const int q_lo = t_begin * kTile;
      const int q_hi = (wave_ran && jk < kv_end) ? N : q_lo;
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

}  // namespace relpos
