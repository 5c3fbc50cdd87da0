// Split-KV main kernel: the 16-bit arithmetic mode (bf16 Q x bf16 K, fp16
// P x fp16 V) at head dim 256, and the dispatch over modes and head dims.
#include "splitkv_kernel.h"

namespace pfkv {

hipError_t launch_splitkv_main(const MainParams& p, int group, hipStream_t stream) {
  if (p.kv_split != 1 && !(p.kv_split == 2 && group == 16)) return hipErrorInvalidValue;
  if (p.ws_row_major) {
    // instantiated only where row-major partials are used
    if (p.precision != kMode16 || p.head_dim != 256 || p.token_pages) return hipErrorInvalidValue;
    return launch_splitkv_main_rm(p, group, stream);
  }
  if (p.head_dim == 128) return launch_splitkv_main_hd128(p, group, stream);
  if (p.head_dim != 256) return hipErrorInvalidValue;
  switch (p.precision) {
    case kMode16: return launch_dim<kMode16, 256>(p, group, stream);
    case kModeFp8P: return launch_splitkv_main_fp8p(p, group, stream);
    case kModeFp8QP: return launch_splitkv_main_fp8(p, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pfkv
