// attn_bwd_f32.hip -- the backward passes for float operands (one
// translation unit per element type, so that the builds run in parallel).
#include "attn_bwd.hpp"

namespace relpos {

hipError_t launch_bwd_f32(const AttnArgs& a, bool want_q, bool want_k, hipStream_t st) {
  return launch_bwd_t<float>(a, want_q, want_k, st);
}

}  // namespace relpos
