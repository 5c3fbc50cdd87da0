// The allocation-free verify call (include/pfkv.h, pfkv_verify_attn_fwd_noalloc):
// the split-KV partials go to a device array of this library instead of a
// caller-given workspace, for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array, one copy per GPU the library runs on,
// held until the process ends. Its name is only a host-side stand-in for the
// device address: each device's address is looked up once, with that device
// current, by hipGetSymbolAddress, kept per device, and only that address is
// ever handed to the kernels. Every call on a device shares its array, which
// keeps the last call's contents; the kernels rewrite every partial they read
// (empty segments write neutral ones), so nothing has to start at zero, and
// calls that overlap on one device race.
#include <mutex>
#include <string>
#include <vector>

#include "pfkv.h"
#include "pfkv_internal.h"

namespace {

static_assert(PFKV_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[PFKV_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // per device: the device address of `scratch`

// The device address of this device's `scratch`, looked up on its first use
// with the device current.
int scratch_address(int device, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)device >= g_scratch_ptr.size()) g_scratch_ptr.resize(device + 1, nullptr);
  if (g_scratch_ptr[device] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return pfkv::set_error(PFKV_LAUNCH, (std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e)).c_str());
    }
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return PFKV_OK;
}

}  // namespace

extern "C" int pfkv_verify_attn_fwd_noalloc(const pfkv_args* a, void* stream) {
  if (a == nullptr) return pfkv::set_error(PFKV_INVALID, "args is NULL");
  const uint64_t need = pfkv_workspace_bytes(a->num_segments, a->total_q, a->num_q_heads);
  if (need > PFKV_NOALLOC_SCRATCH_BYTES)
    return pfkv::set_error(PFKV_INVALID, ("the call needs " + std::to_string(need) +
                                          " bytes of partials; the allocation-free entry point holds " +
                                          std::to_string((uint64_t)PFKV_NOALLOC_SCRATCH_BYTES) +
                                          " (fewer segments, or pfkv_verify_attn_fwd with a workspace)").c_str());
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return pfkv::set_error(PFKV_LAUNCH, (std::string("hipGetDevice: ") + hipGetErrorString(e)).c_str());
  }
  void* ws = nullptr;
  const int st = scratch_address(device, &ws);
  if (st != PFKV_OK) return st;
  return pfkv::verify_attn_library_workspace(a, ws, PFKV_NOALLOC_SCRATCH_BYTES, stream);
}
