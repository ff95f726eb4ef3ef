// qside.hpp -- the score tile in "lane = query" orientation, shared by the
// forward kernel and the query-parallel backward kernel.
//
// Source: "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (nanless.github.io digest), sections on the score formula (Eq. 2:
// S_ij = tau (q_i.k_j + Z^Q[i, r] + Z^K[j, r] + b[r]) + M_ij) and on constant
// tiles:
//  * two comparisons of a tile's extreme offsets against the thresholds tell
//    whether the whole tile maps to the first row (LO), the last row (HI) or
//    crosses the band (BAND);
//  * on a constant tile the query term and b are one scalar per query, added
//    outside the tile, and the key term one scalar per key;
//  * only band tiles look up a row per score.
//
// Orientation: S^T = K Q^T is computed with K rows as MFMA operand A (loaded
// with the sigma row permutation) and the wave's 32 queries as operand B, so
// lane l owns query l % 32 and 16 keys per 32-key subtile.  Row statistics of
// the softmax are then lane-local up to one exchange with lane l ^ 32.
// The key-side scalars seed the MFMA accumulator, so adding them costs no
// vector instruction.
#pragma once
#include "tiles.hpp"

namespace relpos {

enum : int { KIND_LO = 0, KIND_BAND = 1, KIND_HI = 2 };

// Kind of the tile of keys [j0, j0 + 64) for the 32 queries [iw0, iw0 + 32).
__device__ inline int tile_kind_q(const Geo& g, int j0, int iw0) {
  int omax = j0 + kTile - 1 - iw0;
  int omin = j0 - (iw0 + 31);
  return omax <= g.lo ? KIND_LO : (omin >= g.hi ? KIND_HI : KIND_BAND);
}

struct QCtx {
  int iq;                // this lane's query
  int hl;                // lane half (l / 32)
  int sig;               // sigma(l % 32)
  int kv_end;            // keys >= kv_end are masked
  int wsq;               // first unfolded row of this group's Z^Q window
  const float* zq_row;   // Z^Q row of min(iq, last row held) (when has_zq)
  const float* zkb;      // Z^K of this (b, h)
  const float* bun;      // unfolded b of this head
  bool has_zq, has_zk, has_b;
};

// Key offset, inside a 32-key subtile, of result element e of lane-half h
// (= kappa(h, e)) split into its lane-independent part.
template <typename T>
__device__ constexpr int kap0(int e) {
  return MT<T>::KS * (e / MT<T>::E) + e % MT<T>::E;
}

// Relation response of the 16 band entries of this lane (keys
// jb + kap0(e), jb = j0 + 32 st + E * hl).  Every load is issued without a
// branch at an address clamped into its row, so the 16 (or 32, 48) loads of
// a subtile are in flight together.  Entries that are not live (key beyond
// the valid keys, causal future, query beyond N) are either replaced by -inf
// afterwards or belong to a discarded row, so what such a clamped load
// returns never reaches a result.  For a live entry the clamp is the
// identity: its unfolded row lies inside the group's window.
// STAGED: zst is this lane's Z^Q row in the LDS stage of the subtile
// (RowStage, offset by E * hl), which then replaces the Z^Q gather from
// global memory (a compile-time switch, so that a staged kernel carries no
// gather path: a load in flight on a path not taken still makes the compiler
// wait for it before registers it shares with the taken path are written).
template <typename T, bool STAGED>
__device__ __forceinline__ void band_seed(const Geo& g, const QCtx& c, int jb, int wk,
                                          const float* zst, f32x16& s) {
  const int Wm = g.W - 1;
  float v[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = 0.f;
  if (c.has_zq) {
    const int base = jb - c.iq - g.lo - c.wsq;
    if constexpr (STAGED) {
      if constexpr (sizeof(T) == 2) {
        // kap0(e): e = 0..7 at floats 0..7, e = 8..15 at floats 16..23
        f32x4 a0, a1, b0, b1;
        lds_read4x16<0, 16, 64, 80>(zst, a0, a1, b0, b1);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[t] = a0[t];
          v[4 + t] = a1[t];
          v[8 + t] = b0[t];
          v[12 + t] = b1[t];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = zst[kap0<T>(e)];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = c.zq_row[imin(imax(base + kap0<T>(e), 0), Wm)];
    }
  } else if (c.has_b) {
    // b is looked up here only without a query-side table (with one it is
    // folded into Z^Q): the loads go straight into v, all in flight at once
    const int base = jb - c.iq - g.lo;
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = c.bun[imin(imax(base + kap0<T>(e), 0), g.R - 1)];
  }
  if (c.has_zk) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int j = imin(jb + kap0<T>(e), g.N - 1);
      const int col = imin(imax(j - c.iq - g.lo - wk, 0), Wm);
      v[e] += c.zkb[(int64_t)j * g.Wp + col];
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) s[e] = v[e];
}

// K fragment of k-step ks for the A operand of S^T = K Q^T: tile row
// 32 st + sigma(l % 32).  16-bit types read at the lane's precomputed byte
// offset kofs[ks] (row sigma, swizzled chunk), shifted by 32 st rows.
template <typename T>
__device__ __forceinline__ typename MT<T>::frag kfrag(const char* sK, const int* kofs,
                                                      const QCtx& c, int st, int ks) {
  constexpr int ROWB = DTile<T>::ROWB;
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const typename MT<T>::frag*>(sK + kofs[ks] + 32 * st * ROWB);
  } else {
    return dfrag<T>(sK, 32 * st + c.sig, MT<T>::KS * ks + MT<T>::E * c.hl);
  }
}

// Raw scores of the 32 keys [j0 + 32 st, j0 + 32 st + 32) for this lane's
// query, masked entries = -inf; element e <-> key j0 + 32 st + kappa(hl, e).
// The per-query constant of a saturated tile (Z^Q of the saturated row plus
// b) is NOT included.
// kf: the NSD K fragments of this subtile (kfrag), already read from LDS.
// STAGED, zst: the lane's staged Z^Q row of a band subtile (see band_seed).
template <typename T, bool STAGED = false>
__device__ __forceinline__ f32x16 qside_scores(const Geo& g, const QCtx& c,
                                               const typename MT<T>::frag* kf, const float* sZK,
                                               const typename MT<T>::frag* qf, int kind,
                                               int j0, int st, bool needmask,
                                               const float* zst = nullptr) {
  using M = MT<T>;
  constexpr int NSD = kHeadDim / M::KS;
  f32x16 s;
  int ks0 = 0;
  if (kind != KIND_BAND && !c.has_zk) {
    // constant tile without a key term: the accumulator starts at literal zero
    s = M::mma(kf[0], qf[0], zero16());
    ks0 = 1;
  } else if (kind != KIND_BAND) {
    // constant tile: one Z^K scalar per key seeds the accumulator
    float v[16];
    lds_rows16<T>(sZK + (kind == KIND_LO ? 0 : kTile) + 32 * st, c.hl, v);
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = v[e];
  } else {
    band_seed<T, STAGED>(g, c, j0 + 32 * st + MT<T>::E * c.hl, win_k(g, j0 / kGroup), zst, s);
  }
#pragma unroll
  for (int ks = 0; ks < NSD; ++ks) {
    if (ks < ks0) continue;
    s = M::mma(kf[ks], qf[ks], s);
  }
  if (needmask) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int j = j0 + 32 * st + kappa<T>(c.hl, e);
      if (j >= c.kv_end || (g.causal && j > c.iq)) s[e] = -INFINITY;
    }
  }
  return s;
}

// Band entries of a relation projection staged in LDS by row DMA instead of
// gathered per score.  For a wave's 32 rows (queries for Z^Q, keys for Z^K)
// and one 32-token subtile of the other side, each row needs a run of 32
// consecutive floats of its own row of Z: row row0 + m from column
// c0 + dc * m (dc = -1 when the subtile's tokens are keys and the rows
// queries, +1 for key rows against queries in reverse order).  One
// global_load_lds_dword moves the runs of two rows (lanes 0-31: row 2p,
// lanes 32-63: row 2p + 1); row pairs sit at a pitch of 68 floats, so that
// 16-byte reads of 16 consecutive rows hit distinct banks.  Each subtile
// position has its own buffer (and LDS array), filled while the other one
// is read.
struct RowStage {
  static constexpr int kPitch = 68;             // floats per row pair
  static constexpr int kFloats = 16 * kPitch;   // one wave, one subtile
  float* buf[2];     // this wave's buffers of subtile 0 / 1
  const float* z;    // Z of this (b, h), row stride Wp, addressed by query row
  int dc;            // column step per row
  int lane_off;      // (lane & 31) + (lane >> 5) * (Wp + dc)
  int rlast;         // last row the buffer holds (rows beyond are clamped to it)

  __device__ __forceinline__ void init(const Geo& g, const float* z_bh, int dc_, int lane) {
    z = z_bh;
    dc = dc_;
    lane_off = (lane & 31) + (lane >> 5) * (g.Wp + dc);
    rlast = zq_last(g);
  }
  // staged row m, position 0 (row pairs at kPitch, odd rows 32 floats in)
  __device__ __forceinline__ const float* row(int st, int m) const {
    return buf[st] + (m >> 1) * kPitch + (m & 1) * 32;
  }
  // Issue the row DMAs of rows [row0, row0 + 32), run k of row row0 + m at
  // column c0 + dc m + k, into buffer ST (asynchronous).  Columns are
  // clamped into [0, W - 1] exactly as the per-score lookup clamps them: for
  // a saturated entry of a band tile the clamp is the truncation of the map
  // (first / last row); rows beyond N read row N - 1 (their results are
  // discarded; rows beyond the buffer's last row read that row).  A subtile
  // that needs no clamp takes the fast path.
  template <int ST>
  __device__ __forceinline__ void issue(const Geo& g, int row0, int c0, int lane) const {
    float* dst = buf[ST];
    const int cmin = c0 + (dc < 0 ? 31 * dc : 0), cmax = c0 + 31 + (dc > 0 ? 31 * dc : 0);
    if (row0 + 31 <= rlast && cmin >= 0 && cmax < g.W) {
      // wave-uniform row-pair address plus a fixed 32-bit lane offset
      const char* base = reinterpret_cast<const char*>(z + (int64_t)row0 * g.Wp + c0);
      const int64_t step = (int64_t)8 * (g.Wp + dc);  // bytes between row pairs
      const uint32_t lb = 4u * (uint32_t)lane_off;
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        __builtin_amdgcn_global_load_lds((glb_void_t*)(base + lb),
                                         (lds_void_t*)(dst + p * kPitch), 4, 0, 0);
        base += step;
      }
    } else {
      // crossing a threshold or the end of the sequence: clamped per lane
      const int h = lane >> 5, k = lane & 31;
#pragma unroll 1
      for (int p = 0; p < 16; ++p) {
        const int m = 2 * p + h;
        const int r = imin(row0 + m, rlast);
        const int col = imin(imax(c0 + dc * m + k, 0), g.W - 1);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(z + (int64_t)r * g.Wp + col),
                                         (lds_void_t*)(dst + p * kPitch), 4, 0, 0);
      }
    }
  }
  // Z^Q rows of queries [iw0, iw0 + 32) against keys [jb, jb + 32) (lane =
  // query kernels)
  template <int ST>
  __device__ __forceinline__ void issue_q(const Geo& g, const QCtx& c, int iw0, int jb,
                                          int lane) const {
    issue<ST>(g, iw0, jb - iw0 - g.lo - c.wsq, lane);
  }
};

// Saturated-row constants of this lane's query: Z^Q[i, first/last row] + b.
// Columns outside the group's live window are never used for a live entry;
// they read as 0 so that no uninitialised value enters the arithmetic.
__device__ inline void qside_consts(const Geo& g, const QCtx& c, int grp, float& lo_c,
                                    float& hi_c) {
  lo_c = 0.f;
  hi_c = 0.f;
  if (c.has_zq && c.iq < g.N) {
    int cb, ce;
    cols_q(g, grp, cb, ce);
    int c0 = 0 - c.wsq, c1 = g.R - 1 - c.wsq;
    if (c0 >= cb && c0 < ce) lo_c += c.zq_row[c0];
    if (c1 >= cb && c1 < ce) hi_c += c.zq_row[c1];
  }
  if (c.has_b) {
    lo_c += c.bun[0];
    hi_c += c.bun[g.R - 1];
  }
}

// Address of the key-side saturated scalar Z^K[j, first (side 0) / last row]
// of key j, or null when j >= N or the column is outside the key group's
// live window (then no live entry uses it).
__device__ __forceinline__ const float* kside_sat_ptr(const Geo& g, const float* zkb, int j,
                                                      int side) {
  if (j >= g.N) return nullptr;
  const int grp = j / kGroup;
  const int wk = win_k(g, grp);
  int cb, ce;
  cols_k(g, grp, cb, ce);
  const int col = (side == 0 ? 0 : g.R - 1) - wk;
  if (col < cb || col >= ce) return nullptr;
  return zkb + (int64_t)j * g.Wp + col;
}
// Same for the query side: Z^Q[i, first / last row] of query i (zqb
// addressed by query row; null for a row the buffer does not hold).
__device__ __forceinline__ const float* qside_sat_ptr(const Geo& g, const float* zqb, int i,
                                                      int side) {
  if (i >= g.N || i < g.z0 || i > zq_last(g)) return nullptr;
  const int grp = i / kGroup;
  const int wq = win_q(g, grp);
  int cb, ce;
  cols_q(g, grp, cb, ce);
  const int col = (side == 0 ? 0 : g.R - 1) - wq;
  if (col < cb || col >= ce) return nullptr;
  return zqb + (int64_t)i * g.Wp + col;
}

}  // namespace relpos
