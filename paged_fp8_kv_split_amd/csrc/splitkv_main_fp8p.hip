// Split-KV main kernel: the e4m3-P arithmetic mode (bf16 Q x bf16 K, e4m3 P x
// e4m3 V on the fp8 MFMA) at head dim 256.
#include "splitkv_kernel.h"

namespace pfkv {

hipError_t launch_splitkv_main_fp8p(const MainParams& p, int group, hipStream_t stream) {
  return launch_dim<kModeFp8P, 256>(p, group, stream);
}

}  // namespace pfkv
