// t5.hpp -- the T5 relative-position bucket (host and device).
//
// The setup section of "Fast and Exact Relative-Position Attention via
// Structure-Aware Kernels" (nanless.github.io digest) configures T5 with 32
// bidirectional buckets up to distance 128 but does not print the function;
// this is the standard T5 bucket (Raffel et al., 2020): half of the buckets
// per sign when bidirectional (keys after the query take the upper half),
// exact buckets below max_exact, logarithmic buckets up to max_distance,
// clamped to the last bucket; the logarithm is evaluated in float64.
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

}  // namespace relpos
