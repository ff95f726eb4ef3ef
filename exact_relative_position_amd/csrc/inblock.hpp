// inblock.hpp -- the query-side relation term of the forward computed inside
// the attention block, with no stored projection.
//
// Source: "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (nanless.github.io digest): the score formula (Eq. 2, the query
// term Z^Q[i, r] = q_i . aQ[r] plus b[r]) and the limitations and ablation
// sections, where the relation is recomputed inside each block instead of
// being projected and stored, so that the forward needs no memory beyond
// its inputs and outputs (the inference-style variant; short sequences,
// where a stored window is as wide as a dense bias, and the identity map,
// whose stored projection is quadratic).
//
// For a wave's 32 queries [iw0, iw0 + 32) and a 64-key tile [j0, j0 + 64)
// the offsets o = j - i span j0 - iw0 - 31 ... j0 - iw0 + 63: three tiles U
// of 32 offsets, o = j0 - iw0 - 31 + 32 U + u'.  Per tile, one 32 x 32 MFMA
// product T_U[m][u'] = q_(iw0+m) . aQ[r(o)] over the 64 head dims, plus
// b[r(o)] by one more k-step (A = b in k-slot 0, B = 1 in k-slot 0; exact).
// The table row operand comes from an LDS ring: slot o mod 256 holds the
// 16-bit table row of offset o.  A block's tile needs 191 consecutive
// offsets and the next tile 64 more, so 256 slots double buffer it; each
// step DMAs the next tile's 64 new rows with the K and V tiles (row
// addresses looked up per lane: clamped by the truncation, through the fold
// table for bucketed maps), in 16-byte chunks permuted per slot like the K
// and V tiles.
//
// The 32-key subtile st needs T[m][k - m + 31 + 32 st] for key k: a shift
// by the lane's own query.  Lane (m, h) holds T_U[m][kappa(h, e)] in result
// element e, so element e belongs at key column kappa + m + 1 - 32 from tile
// U = st when kappa + m + 1 >= 32, and at kappa + m + 1 from tile st + 1
// otherwise (exactly one of the two).  Each wave writes these 32 x 32 values
// into its own LDS tile (row m rotated left by 4 m, which keeps both the
// 4-byte writes and the 16-byte reads of 8 consecutive rows on distinct
// banks) and reads its 16 seeds back in the score layout.
#pragma once
#include "qside.hpp"

namespace relpos {

constexpr int kRingSlots = 256;
constexpr int kRingBytes = kRingSlots * 128;  // one 64-value 16-bit row per slot
constexpr int kSkewFloats = 32 * 32;          // one wave's tile

// Table row of offset o: the truncated (unfolded) row, through the fold
// table for bucketed maps.
__device__ __forceinline__ int tab_row(const Geo& g, const int32_t* fold, int o) {
  const int r = rrow(g, o);
  return fold ? fold[r] : r;
}

template <typename T>
struct InBlock {
  static_assert(sizeof(T) == 2, "the in-block relation is for 16-bit inputs");
  using M = MT<T>;
  using frag = typename M::frag;

  const T* tab;          // aQ of this head ([R, 64])
  const T* bt;           // b of this head ([R]) or null
  const int32_t* fold;   // unfolded row -> table row, or null
  uint32_t ring;         // LDS byte address of the ring
  uint32_t skw;          // LDS byte address of this wave's skew tile
  int sig;               // sigma(l % 32): the table row this lane feeds as A-row l % 32
  uint32_t ch[4];        // byte offset of the lane's chunk of k-step ks inside a slot
  uint32_t rd[4];        // byte addresses of the four 16-byte seed reads
  uint32_t wrow;         // byte address of row m of the skew tile
  uint32_t p0x4;         // 4 * ((8 h + 5 m + 1) & 31): rotated position of kappa = 8 h
  int lim;               // element e takes tile st iff kap0(e) >= lim
  // DMA plan of one 64-offset block: row (0..63) and source element offset
  // (permuted chunk) of the lane's two chunks
  int dr[2], dc[2];
  int blk0;              // first 1024-byte piece of this wave

  __device__ __forceinline__ void init(uint32_t ring_, uint32_t skw_wave, int w, int lane) {
    const int m = lane & 31, h = lane >> 5;
    ring = ring_;
    skw = skw_wave;
    sig = sigma<T>(m);
    // slot of offset j0 - iw0 - 31 + 32 U + sig is congruent to sig + 1 mod 16
    // (j0 - iw0 a multiple of 32), which fixes its chunk permutation
    const int sw = swz<T>((sig + 1) & 15);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) ch[ks] = (uint32_t)(((2 * ks + h) ^ sw) << 4);
    wrow = skw + 128u * (uint32_t)m;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c0 = 8 * h + (r & 1) * 4 + (r >> 1) * 16;
      rd[r] = wrow + 4u * (uint32_t)((c0 + 4 * m) & 31);
    }
    p0x4 = 4u * (uint32_t)((8 * h + 5 * m + 1) & 31);
    lim = 31 - m - 8 * h;
    blk0 = 2 * w;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int p = (blk0 + u) * 64 + lane;
      const int r = p >> 3, cs = p & 7;
      dr[u] = r;
      dc[u] = (cs ^ swz<T>(r & 15)) * 8;
    }
  }

  // DMA the table rows of offsets [A, A + 64) (A a multiple of 64) into
  // their ring slots (asynchronous; every wave issues two of the eight
  // 1024-byte pieces).
  __device__ __forceinline__ void load_block(const Geo& g, char* ring_ptr, int A) const {
    char* base = ring_ptr + (A & (kRingSlots - 1)) * 128;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const T* src = tab + (int64_t)tab_row(g, fold, A + dr[u]) * kHeadDim + dc[u];
      __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)(base + (blk0 + u) * 1024),
                                       16, 0, 0);
    }
  }

  // b fragment of offset tile U (first offset oU): k-slot 0 of lane half 0
  // holds b of the lane's A-row; everything else is zero.
  __device__ __forceinline__ T b_of(const Geo& g, int oU) const {
    return bt[tab_row(g, fold, oU + sig)];
  }

  // T_U = Q_wave . aQ[rows of offsets oU + 0..31]^T (+ b), lane = query.
  __device__ __forceinline__ f32x16 tmm(int oU, const frag* qf, bool has_b, T bval,
                                        int h) const {
    const uint32_t so = ring + ((uint32_t)((oU + sig) & (kRingSlots - 1)) << 7);
    f32x4 a0, a1, a2, a3;
    // (asm, waiting for its own reads only: the compiler cannot tell the
    // ring from the LDS areas whose direct loads are still in flight)
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3)
        : "v"(so + ch[0]), "v"(so + ch[1]), "v"(so + ch[2]), "v"(so + ch[3])
        : "memory");
    f32x16 t = M::mma(__builtin_bit_cast(frag, a0), qf[0], zero16());
    t = M::mma(__builtin_bit_cast(frag, a1), qf[1], t);
    t = M::mma(__builtin_bit_cast(frag, a2), qf[2], t);
    t = M::mma(__builtin_bit_cast(frag, a3), qf[3], t);
    if (has_b) {
      frag fb = M::zero(), one = M::zero();
      if (h == 0) {
        fb[0] = bval;
        one[0] = M::from_f(1.f);
      }
      t = M::mma(fb, one, t);
    }
    return t;
  }

  // Seeds of subtile st from T_st (ta) and T_(st+1) (tb): written to the
  // wave's skew tile, read back in the score layout (element e <-> key
  // kappa(h, e) of the subtile).
  __device__ __forceinline__ void seeds(const f32x16& ta, const f32x16& tb, float (&v)[16]) const {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int k0 = kap0<T>(e);  // kappa - 8 h
      const float x = k0 >= lim ? ta[e] : tb[e];
      const uint32_t ad = (wrow & ~0x7Cu) | ((p0x4 + 4u * (uint32_t)k0) & 0x7Cu);
      asm volatile("ds_write_b32 %0, %1" : : "v"(ad), "v"(x) : "memory");
    }
    f32x4 r0, r1, r2, r3;
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(rd[0]), "v"(rd[1]), "v"(rd[2]), "v"(rd[3])
        : "memory");
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[t] = r0[t];
      v[4 + t] = r1[t];
      v[8 + t] = r2[t];
      v[12 + t] = r3[t];
    }
  }

  // Saturated constants of this lane's query: q . aQ[first / last row]
  // (+ b), the per-query scalar of the constant tiles.
  __device__ __forceinline__ void consts(const Geo& g, const frag* qf, int h, float& lo_c,
                                         float& hi_c) const {
    const int rl = tab_row(g, fold, g.lo), rh = tab_row(g, fold, g.hi);
    const T* pl = tab + (int64_t)rl * kHeadDim;
    const T* ph = tab + (int64_t)rh * kHeadDim;
    float sl = 0.f, sh = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const frag al = *reinterpret_cast<const frag*>(pl + 16 * ks + 8 * h);
      const frag ah = *reinterpret_cast<const frag*>(ph + 16 * ks + 8 * h);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float q = M::to_f(qf[ks][t]);
        sl = fmaf(q, M::to_f(al[t]), sl);
        sh = fmaf(q, M::to_f(ah[t]), sh);
      }
    }
    lo_c = sum_xor32(sl);
    hi_c = sum_xor32(sh);
    if (bt) {
      lo_c += M::to_f(bt[rl]);
      hi_c += M::to_f(bt[rh]);
    }
  }
};

// Raw scores of a band subtile from in-block seeds (the relation response of
// each entry, see InBlock::seeds): s = seed + K Q^T, masked entries = -inf.
template <typename T>
__device__ __forceinline__ f32x16 seeded_scores(const Geo& g, const QCtx& c,
                                                const typename MT<T>::frag* kf,
                                                const typename MT<T>::frag* qf,
                                                const float (&v)[16], int j0, int st,
                                                bool needmask) {
  using M = MT<T>;
  constexpr int NSD = kHeadDim / M::KS;
  f32x16 s;
#pragma unroll
  for (int e = 0; e < 16; ++e) s[e] = v[e];
#pragma unroll
  for (int ks = 0; ks < NSD; ++ks) s = M::mma(kf[ks], qf[ks], s);
  if (needmask) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int j = j0 + 32 * st + kappa<T>(c.hl, e);
      if (j >= c.kv_end || (g.causal && j > c.iq)) s[e] = -INFINITY;
    }
  }
  return s;
}

}  // namespace relpos
