// Split-KV main kernel: the e4m3-P arithmetic mode (bf16 Q x bf16 K, e4m3 P x
// e4m3 V on the fp8 MFMA).
#include "splitkv_kernel.h"

namespace pfkv {

hipError_t launch_splitkv_main_fp8p(const MainParams& p, int group, hipStream_t stream) {
  return launch_mode<kModeFp8P>(p, group, stream);
}

}  // namespace pfkv
