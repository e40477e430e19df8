// The main pass of gated causal GQA attention (attn_fwd.h) instantiated for head dim 64.
#include "attn_fwd.h"

namespace gqa {

hipError_t launch_fwd_64(const FwdParams& p, int dtype, int mask_kind, int shape, hipStream_t stream) {
  return launch_fwd_d<64>(p, dtype, mask_kind, shape, stream);
}

}  // namespace gqa
