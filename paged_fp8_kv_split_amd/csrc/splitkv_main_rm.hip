// Split-KV main kernel: the 16-bit arithmetic mode at head dim 256 writing its
// partials row-major (more than 16 segments), in a translation unit of its own.
#include "splitkv_kernel.h"

namespace pfkv {

hipError_t launch_splitkv_main_rm(const MainParams& p, int group, hipStream_t stream) {
  return launch_shape<kMode16, false, 256, true>(p, group, stream);
}

}  // namespace pfkv
