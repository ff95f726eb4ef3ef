// attn_bwd.hpp -- the two backward passes in one launch.
//
// Source: "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (nanless.github.io digest), section on the backward pass: the
// query-parallel pass (dQ, dZ^Q) and the key-parallel pass (dK, dV, dZ^K)
// both recompute the scores from Q, K, V, dO, the log-sum-exp and D, and
// neither reads what the other writes, so they may run at the same time.
//
// One grid holds the blocks of both passes.  A 12-head 8K problem has 768
// blocks per pass against 512 resident blocks (two per CU), so a pass alone
// ends with a half-empty round; both passes together fill three whole rounds.
// Block order: equal-work problems put the key blocks (the longer ones)
// first, then the query blocks; causal problems deal the two passes rank by
// rank (the key blocks of rank r, then the query blocks of rank r, rank 0
// being the longest block of every head in both passes), which keeps the
// longest-first order over the whole grid.  A launch may also carry one pass
// only (no blocks of the other).
//
// The two passes use the same block shape (4 waves, or 8 in two groups) and
// the same occupancy; their LDS areas are overlaid (each block runs one pass).
#pragma once
#include "attn_bwd_k.hpp"
#include "attn_bwd_q.hpp"

namespace relpos {

static_assert(kStageFloats == 32 * kStagePitchK, "one staging area per wave serves both passes");

// The launch's AttnArgs read through a kernarg pointer that the compiler
// cannot see through: each pass then loads the fields it uses inside its own
// branch.  (Read directly, every field is loaded once at kernel entry and
// kept live into both passes, where the scalar registers overflow into
// vector-register lanes that the passes need.)
__device__ __forceinline__ const AttnArgs& branch_args() {
  auto p = __builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return *(const AttnArgs*)p;
}

// ZQ/ZK: relation tables present; SQ/SK: staged band stores of the query /
// key pass; GRP: two wave groups per block; DROP: attention dropout.  The
// AttnArgs are the kernel's first argument (offset 0 of the kernarg segment).
template <typename T, bool ZQ, bool ZK, bool SQ, bool SK, bool GRP, bool DROP>
__global__ __launch_bounds__((query_threads<T, GRP>()), (query_blocks_per_cu<T, GRP>()))
    void bwd_kernel(AttnArgs a, int kblocks, int weave) {
  static_assert(query_threads<T, GRP>() == key_threads<T, GRP>() &&
                    query_blocks_per_cu<T, GRP>() == key_blocks_per_cu<T, GRP>(),
                "both passes run the same block shape");
  constexpr int TB = DTile<T>::BYTES;
  constexpr int G = query_groups<T, GRP>();
  constexpr int kSmall = G * 4 * kTile;  // key pass: sR; the query pass's sZK is half of it
  constexpr int kSt = (SQ || SK) ? 4 * G * kStageFloats : 4;
  __shared__ __align__(16) char s0[G * TB], s1[G * TB], s2[G * TB], s3[G * TB];
  __shared__ __align__(16) float r0[kSmall], r1[kSmall];
  __shared__ __align__(16) float st0[kSt], st1[SQ ? kSt : 4];

  int bid = blockIdx.x;
  bool key;
  if (weave) {
    const int nbh = a.B * a.H;
    const int r = bid / (2 * nbh), c = bid - r * 2 * nbh;
    key = c < nbh;
    bid = r * nbh + (key ? c : c - nbh);
  } else {
    key = bid < kblocks;
    if (!key) bid -= kblocks;
  }
  // The compiler's scheduling strategy 0 (LDS reads interleaved with the
  // MFMAs) gains 1-2% where it fits the registers; with dropout, or with a
  // key-side term and staged query rows, it doubles the spills (measured),
  // so those kernels keep the default schedule.
  constexpr bool SCHED = !DROP && !(ZK && SQ);
  if (key)
    bwd_k_block<T, ZQ, ZK, SK, GRP, DROP, SCHED>(branch_args(), bid, s0, s1, s2, s3, r0, r1, st0);
  else
    bwd_q_block<T, ZQ, ZK, SQ, GRP, DROP, SCHED>(branch_args(), bid, s0, s1, s2, s3, r0, r1, st0,
                                                 st1);
}

template <typename T, bool GRP, bool DROP, bool ZQ, bool ZK, bool SQ, bool SK>
static void launch_bwd_v(const AttnArgs& a, int grid, int kblocks, int weave, hipStream_t st) {
  hipLaunchKernelGGL((bwd_kernel<T, ZQ, ZK, SQ, SK, GRP, DROP>), dim3(grid),
                     dim3(query_threads<T, GRP>()), 0, st, a, kblocks, weave);
}

template <typename T, bool GRP, bool DROP, bool ZQ>
static void launch_bwd_z(const AttnArgs& a, bool zk, bool sq, bool sk, int grid, int kblocks,
                         int weave, hipStream_t st) {
  // sq (a wide band) implies sk == zk
  if (!zk) {
    if (sq) launch_bwd_v<T, GRP, DROP, ZQ, false, true, false>(a, grid, kblocks, weave, st);
    else launch_bwd_v<T, GRP, DROP, ZQ, false, false, false>(a, grid, kblocks, weave, st);
  } else if (sq) {
    launch_bwd_v<T, GRP, DROP, ZQ, true, true, true>(a, grid, kblocks, weave, st);
  } else if (sk) {
    launch_bwd_v<T, GRP, DROP, ZQ, true, false, true>(a, grid, kblocks, weave, st);
  } else {
    launch_bwd_v<T, GRP, DROP, ZQ, true, false, false>(a, grid, kblocks, weave, st);
  }
}

// Launch the query pass (want_q: the B*H*nqb blocks of its query range),
// the key pass (want_k: B*H*nblk blocks) or both.
template <typename T>
hipError_t launch_bwd_t(const AttnArgs& a, bool want_q, bool want_k, hipStream_t st) {
  const int kblocks = want_k ? a.B * a.H * a.nblk : 0;
  const int grid = kblocks + (want_q ? a.B * a.H * a.nqb : 0);
  if (grid == 0) return hipSuccess;
  const int weave = want_q && want_k && a.geo.causal && a.nqb == a.nblk;
  const bool zq = a.flags & F_ZQ, zk = a.flags & F_ZK;
  // staging of the query pass implies the key pass's
  const bool sq = wide_band(a.geo), sk = zk && (sq || a.geo.W >= kStageMinWK);
  if constexpr (sizeof(T) == 2) {
    if (a.flags & F_DROP) {
      if (a.split) {
        if (zq) launch_bwd_z<T, true, true, true>(a, zk, sq, sk, grid, kblocks, weave, st);
        else launch_bwd_z<T, true, true, false>(a, zk, sq, sk, grid, kblocks, weave, st);
      } else {
        if (zq) launch_bwd_z<T, false, true, true>(a, zk, sq, sk, grid, kblocks, weave, st);
        else launch_bwd_z<T, false, true, false>(a, zk, sq, sk, grid, kblocks, weave, st);
      }
      return hipGetLastError();
    }
    if (a.split) {
      if (zq) launch_bwd_z<T, true, false, true>(a, zk, sq, sk, grid, kblocks, weave, st);
      else launch_bwd_z<T, true, false, false>(a, zk, sq, sk, grid, kblocks, weave, st);
      return hipGetLastError();
    }
  }
  if (zq) launch_bwd_z<T, false, false, true>(a, zk, sq, sk, grid, kblocks, weave, st);
  else launch_bwd_z<T, false, false, false>(a, zk, sq, sk, grid, kblocks, weave, st);
  return hipGetLastError();
}

}  // namespace relpos
