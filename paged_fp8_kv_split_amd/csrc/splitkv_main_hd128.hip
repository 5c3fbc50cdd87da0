// Split-KV main kernel at head dim 128, all three arithmetic modes.
#include "splitkv_kernel.h"

namespace pfkv {

hipError_t launch_splitkv_main_hd128(const MainParams& p, int group, hipStream_t stream) {
  switch (p.precision) {
    case kMode16: return launch_dim<kMode16, 128>(p, group, stream);
    case kModeFp8P: return launch_dim<kModeFp8P, 128>(p, group, stream);
    case kModeFp8QP: return launch_dim<kModeFp8QP, 128>(p, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pfkv
