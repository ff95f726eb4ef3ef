// attn_bwd_bf16.hip -- the backward passes for __bf16 operands (one
// translation unit per element type, so that the builds run in parallel).
#include "attn_bwd.hpp"

namespace relpos {

hipError_t launch_bwd_bf16(const AttnArgs& a, bool want_q, bool want_k, hipStream_t st) {
  return launch_bwd_t<__bf16>(a, want_q, want_k, st);
}

}  // namespace relpos
