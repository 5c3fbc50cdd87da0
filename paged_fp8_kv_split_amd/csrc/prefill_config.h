// Shape of the fp8 varlen prefill launch shared by the host and the kernel.
#pragma once

namespace pfkv {

constexpr int kPrefillTileRows = 256;   // query rows per prefill work-group (a grid column)

}  // namespace pfkv
