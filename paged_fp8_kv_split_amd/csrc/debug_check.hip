// Debug-mode precondition check (enabled by PFKV_DEBUG=1 or pfkv_set_debug):
// the device-side contract of the verify call that the host cannot see without
// reading device memory (aiter PR #5190, Supported: inputs outside the kernel's
// envelope are rejected rather than served). One work-group per sequence:
//   cu_seqlens_q starts at 0, never decreases and ends at total_q;
//   1 <= n_b <= max_q_len (0 tokens is allowed: the sequence is skipped);
//   n_b <= L_b <= page_size * max_pages_per_seq;
//   the block-table entries of the pages the sequence uses lie in [0, num_pages).
// A violation sets a flag bit and lowers the first-offending-sequence word with
// vector atomics; the host reads the three words after the check.
#include "pfkv_internal.h"

namespace pfkv {
namespace {

typedef __attribute__((address_space(4))) const int32_t const_i32;

__global__ void __launch_bounds__(256) precondition_kernel(CheckParams p, int32_t* status) {
  const int b = blockIdx.x;
  const const_i32* cu = (const const_i32*)p.cu_seqlens_q;
  const const_i32* sl = (const const_i32*)p.seq_lens;
  int flags = 0, detail = 0;
  const int q0 = cu[b], q1 = cu[b + 1];
  const int n = q1 - q0;
  const int L = sl[b];
  if (threadIdx.x == 0) {
    if ((b == 0 && q0 != 0) || n < 0 || (b == p.num_seqs - 1 && q1 != p.total_q)) { flags |= 1; detail = q1; }
    if (n > p.max_q_len) { flags |= 2; detail = n; }
    if (L < n || L < 0 || (int64_t)L > (int64_t)p.page_size * p.max_pages_per_seq) { flags |= 4; detail = L; }
  }
  // table entries of the pages this sequence uses (L clamped so that every read stays in the row)
  const int64_t lc = L < 0 ? 0 : ((int64_t)L > (int64_t)p.page_size * p.max_pages_per_seq
                                      ? (int64_t)p.page_size * p.max_pages_per_seq : L);
  const int pages = (int)((lc + p.page_size - 1) / p.page_size);
  const int32_t* row = p.block_tables + (int64_t)b * p.block_table_stride;
  for (int j = threadIdx.x; j < pages; j += blockDim.x) {
    const int id = row[j];
    if (id < 0 || id >= p.num_pages) { flags |= 8; detail = id; }
  }
  if (flags != 0) {
    __hip_atomic_fetch_or(status + 0, flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int prev = __hip_atomic_fetch_min(status + 1, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (b < prev) __hip_atomic_exchange(status + 2, detail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

hipError_t launch_precondition_check(const CheckParams& p, int32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(precondition_kernel, dim3(p.num_seqs), dim3(256), 0, stream, p, status);
  return hipGetLastError();
}

}  // namespace pfkv
