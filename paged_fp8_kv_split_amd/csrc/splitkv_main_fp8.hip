// Split-KV main kernel: the e4m3 Q and P arithmetic mode (per-row Q scale;
// both products on the fp8 MFMA) at head dim 256.
#include "splitkv_kernel.h"

namespace pfkv {

hipError_t launch_splitkv_main_fp8(const MainParams& p, int group, hipStream_t stream) {
  return launch_dim<kModeFp8QP, 256>(p, group, stream);
}

}  // namespace pfkv
