// buckets.hpp -- bucketed offset maps (host and device).
//
// The setup section of "Fast and Exact Relative-Position Attention via
// Structure-Aware Kernels" (nanless.github.io digest) configures T5 with 32
// bidirectional buckets up to distance 128 and DeBERTa with 256 log buckets
// up to distance 512, but prints neither function.
//
// T5: the standard T5 bucket (Raffel et al., 2020): half of the buckets per
// sign when bidirectional (keys after the query take the upper half), exact
// buckets below max_exact, logarithmic buckets up to max_distance, clamped to
// the last bucket.
//
// Log buckets: DeBERTa's log-bucket positions (He et al., 2021) with k
// buckets (mid = k / 2) and maximum distance m: an offset o with |o| <= mid
// keeps bucket o; beyond, bucket = sign(o) * (mid + ceil((mid - 1) *
// ln(|o| / mid) / ln((m - 1) / mid))); the row is bucket + k clamped to
// [0, 2k - 1] (2k rows).
//
// Both logarithms are evaluated in float64.
#pragma once
#include <math.h>

#if defined(__HIPCC__)
#define RP_T5_HD __host__ __device__ inline
#else
#define RP_T5_HD inline
#endif

namespace relpos {

// T5 bucket of offset o (key - query).
RP_T5_HD int t5_bucket_dev(int o, int num_buckets, int max_exact,
                                             int max_distance, int bidirectional) {
  int nb = num_buckets, base = 0, n;
  if (bidirectional) {
    nb = num_buckets / 2;
    base = o > 0 ? nb : 0;
    n = o < 0 ? -o : o;
  } else {
    n = o < 0 ? -o : 0;
  }
  const int me = max_exact > 0 ? max_exact : nb / 2;
  if (n < me) return base + n;
  const double v = log((double)n / (double)me) / log((double)max_distance / (double)me) *
                   (double)(nb - me);
  const int bk = me + (int)v;
  return base + (bk < nb - 1 ? bk : nb - 1);
}

// Log-bucket row of offset o (key - query), in [0, 2 * num_buckets).
RP_T5_HD int log_bucket_dev(int o, int num_buckets, int max_distance) {
  const int mid = num_buckets / 2;
  const int n = o < 0 ? -o : o;
  int b = o;
  if (n > mid) {
    const double v = ceil(log((double)n / (double)mid) /
                          log((double)(max_distance - 1) / (double)mid) * (double)(mid - 1));
    // beyond 2 * num_buckets the row is clamped anyway
    const int t = v < (double)(2 * num_buckets) ? (int)v : 2 * num_buckets;
    b = o < 0 ? -(mid + t) : mid + t;
  }
  const int row = b + num_buckets;
  return row < 0 ? 0 : (row > 2 * num_buckets - 1 ? 2 * num_buckets - 1 : row);
}

}  // namespace relpos
