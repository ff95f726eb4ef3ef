// dropout.hpp -- attention dropout with counter-based random bytes.
//
// The digest page ("Fast and Exact Relative-Position Attention via
// Structure-Aware Kernels", nanless.github.io), in its section on what a
// reproduction has to do first, asks for dropout whose random numbers the
// backward pass recomputes.  Dropout acts on the normalised weights:
// O = (P * K / (1 - p)) V with a keep mask K and drop probability p = t / 256.
//
// Generator: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC 2011).  One call covers a 4 x 4 block of
// scores: counter (j / 4, i / 4, batch * H + head, offset) under the 64-bit
// seed as key; byte j % 4 of output word i % 4 is the random byte u of score
// (i, j), and the score is kept iff u >= t.  The bits therefore do not depend
// on how a kernel tiles the scores.
//
// Sharing one call among a quad.  In the 16-bit MFMA layout a lane holds one
// query (forward and query pass) or one key (key pass) and, per 32 x 32
// subtile, 16 elements in four aligned groups of 4 consecutive keys (or
// queries): element e is in group e / 4.  The 4 lanes of a quad hold 4
// consecutive queries (keys), so the quad's 64 scores of a subtile are
// exactly 4 Philox blocks.  Lane q of the quad computes block q (its
// element group q), turns the 16 bytes into 16 keep bits, and a DPP quad
// broadcast of those bits gives every lane the 4 bits it needs from each
// block: one call per lane per subtile.
#pragma once
#include "device.hpp"

namespace relpos {

// Philox4x32-10 in place on the counter (c0..c3) under key (k0, k1).
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                              uint32_t& c3, uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
  // each 32 x 32 -> 64-bit product as one 64-bit multiply (one v_mad_u64_u32
  // gives both halves)
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)kM0 * c0, p1 = (uint64_t)kM1 * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c0 = n0;
    c1 = (uint32_t)p1;
    c2 = n2;
    c3 = (uint32_t)p0;
    k0 += kW0;
    k1 += kW1;
  }
}

// Keep bits of the 4 bytes of a word (byte b kept iff b >= t), bit b * STRIDE.
// cadd = (256 - t) * 0x00010001: adding it to a byte held in a 16-bit field
// carries into bit 8 of that field exactly when the byte is >= t.
template <int STRIDE>
__device__ __forceinline__ uint32_t keep4(uint32_t x, uint32_t cadd) {
  const uint32_t ev = (x & 0x00FF00FFu) + cadd;         // bytes 0 and 2
  const uint32_t od = ((x >> 8) & 0x00FF00FFu) + cadd;  // bytes 1 and 3
  return ((ev >> 8) & 1u) | (((od >> 8) & 1u) << STRIDE) | (((ev >> 24) & 1u) << (2 * STRIDE)) |
         (((od >> 24) & 1u) << (3 * STRIDE));
}

struct DropCtx {
  uint32_t k0, k1;  // seed
  uint32_t bh;      // batch * H + head
  uint32_t off;     // counter word 3
  uint32_t cadd;    // (256 - t) * 0x00010001
  float scale;      // 1 / (1 - p)
  int q;            // lane within its quad
};

__device__ __forceinline__ DropCtx drop_ctx(const AttnArgs& a, int bh, int lane) {
  DropCtx d;
  d.k0 = a.seed_lo;
  d.k1 = a.seed_hi;
  d.bh = (uint32_t)bh;
  d.off = a.drop_off;
  d.cadd = (256u - a.drop_t) * 0x00010001u;
  d.scale = a.drop_scale;
  d.q = lane & 3;
  return d;
}

// The 16 keep bits of the lane's subtile elements (bit e: element e).
// QLANES: the lane holds query `x` and element group g holds keys
// y0 + kappa(hl, 4g) .. + 3 (forward, query pass); otherwise the lane holds
// key `x` and group g holds queries y0 + kappa(hl, 4g) .. + 3 (key pass).
// Must be reached by all 4 lanes of every quad (uniform control flow).
template <typename T, bool QLANES>
__device__ __forceinline__ uint32_t drop_bits(const DropCtx& d, int x, int y0, int hl) {
  static_assert(sizeof(T) == 2, "dropout uses the 16-bit element layout");
  const uint32_t yb = (uint32_t)(y0 + kappa<T>(hl, 4 * d.q)) >> 2, xb = (uint32_t)x >> 2;
  uint32_t c0 = QLANES ? yb : xb, c1 = QLANES ? xb : yb, c2 = d.bh, c3 = d.off;
  philox4x32_10(c0, c1, c2, c3, d.k0, d.k1);
  // block bits: QLANES, bit 4 w + b (word w = the quad's lane w); else
  // bit 4 b + w (byte b = the quad's lane b)
  uint32_t bits;
  if constexpr (QLANES) {
    bits = keep4<1>(c0, d.cadd) | (keep4<1>(c1, d.cadd) << 4) | (keep4<1>(c2, d.cadd) << 8) |
           (keep4<1>(c3, d.cadd) << 12);
  } else {
    bits = keep4<4>(c0, d.cadd) | (keep4<4>(c1, d.cadd) << 1) | (keep4<4>(c2, d.cadd) << 2) |
           (keep4<4>(c3, d.cadd) << 3);
  }
  // lane q takes bits [4q, 4q + 4) of quad lane g's block as its group g
  const int v = (int)bits;
  const uint32_t b0 = (uint32_t)__builtin_amdgcn_mov_dpp(v, 0x00, 0xF, 0xF, false);
  const uint32_t b1 = (uint32_t)__builtin_amdgcn_mov_dpp(v, 0x55, 0xF, 0xF, false);
  const uint32_t b2 = (uint32_t)__builtin_amdgcn_mov_dpp(v, 0xAA, 0xF, 0xF, false);
  const uint32_t b3 = (uint32_t)__builtin_amdgcn_mov_dpp(v, 0xFF, 0xF, 0xF, false);
  const int sh = 4 * d.q;
  return ((b0 >> sh) & 15u) | (((b1 >> sh) & 15u) << 4) | (((b2 >> sh) & 15u) << 8) |
         (((b3 >> sh) & 15u) << 12);
}

// x where element e is kept, else 0.
__device__ __forceinline__ float keep_or_zero(uint32_t bits, int e, float x) {
  return ((bits >> e) & 1u) ? x : 0.f;
}

}  // namespace relpos
