// The main pass of gated causal GQA attention (attn_fwd.h) instantiated for head dim 128.
#include "attn_fwd.h"

namespace gqa {

hipError_t launch_fwd_128(const FwdParams& p, int dtype, int mask_kind, int shape, hipStream_t stream) {
  return launch_fwd_d<128>(p, dtype, mask_kind, shape, stream);
}

}  // namespace gqa
