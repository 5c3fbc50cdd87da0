// Split-KV main kernel: the e4m3 Q and P arithmetic mode (per-row Q scale;
// both products on the fp8 MFMA).
#include "splitkv_kernel.h"

namespace pfkv {

hipError_t launch_splitkv_main_fp8(const MainParams& p, int group, hipStream_t stream) {
  return launch_mode<kModeFp8QP>(p, group, stream);
}

}  // namespace pfkv
