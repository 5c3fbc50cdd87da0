// Segment reduce: merges the per-segment partials of the split-KV main kernel
// into the bf16 output (aiter PR #5190 "gfx950 assembly MTP-verify attention for
// head_dim 256 fp8 paged KV", section Modifications: a split-KV segment reduce
// after the main kernel). The per-row arithmetic is merge::merge_row
// (segment_merge.h).
// One wave per output row, eight rows per work-group (measured 1 us faster per
// call than four at 16 x 35000: fewer, fuller work-groups): lane s holds
// (m_s, l_s), lane i dims 4i .. 4i + 3 of the fp16 o rows (head dim 128: lanes
// 0-31), whose loads for up to 16 segments are in flight together. Above 16
// segments 2, 4 or (balanced caps above 64) 8 waves share a row; BAL takes each
// row's segment count from the balanced schedule instead of num_segments; RM
// reads row-major partials (ws_slot), which the main kernel writes above 16
// segments in its 16-bit mode at head dim 256.
#include "segment_merge.h"

namespace pfkv {
namespace {

// PARTS waves merge one row (merge::merge_row). With many segments and few
// rows (4 sequences x 64 segments: 256 rows) one wave per row would load its
// segments in several dependent batches on a few CUs.
template <int PARTS, bool BAL, bool RM>
__global__ void __launch_bounds__(512) segment_reduce_kernel(ReduceParams p) {
  constexpr int kRowsPerWg = 8 / PARTS;
  __shared__ merge::f32x4 partial[PARTS > 1 ? 8 : 1][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t rows_total = (int64_t)p.total_q * p.num_q_heads;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWg + wave / PARTS;
  const bool valid = row < rows_total;
  if (PARTS == 1 && !valid) return;
  int S = p.num_segments;
  if (BAL && valid) {
    // the row's sequence and its segment count, as the main kernel scheduled them
    const BalancedSlot sl = balanced_row((int)(row / p.num_q_heads), p.cu_seqlens_q, p.seq_lens, p.num_seqs,
                                         p.max_seq_len, p.window_left, p.num_slots, p.num_segments);
    if (sl.b >= 0) S = __builtin_amdgcn_readfirstlane(sl.count);
  }
  merge::merge_row<PARTS, RM>(p, row, valid, S, wave % PARTS, wave, lane, partial);
}

template <int PARTS>
void launch_rows(const ReduceParams& p, dim3 grid, hipStream_t stream) {
  if (p.balance) {
    if (p.ws_row_major) hipLaunchKernelGGL((segment_reduce_kernel<PARTS, true, true>), grid, dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((segment_reduce_kernel<PARTS, true, false>), grid, dim3(512), 0, stream, p);
  } else {
    if (p.ws_row_major) hipLaunchKernelGGL((segment_reduce_kernel<PARTS, false, true>), grid, dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((segment_reduce_kernel<PARTS, false, false>), grid, dim3(512), 0, stream, p);
  }
}

}  // namespace

hipError_t launch_segment_reduce(const ReduceParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.total_q * p.num_q_heads;
  // waves per row: one up to 16 segments (a single batch of loads), else 2 or 4
  // (balanced segments: a separate instantiation that finds each row's count);
  // row-major partials come only above 16 segments
  if (p.num_segments <= 16) {
    if (p.ws_row_major) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((rows + 7) / 8));
    if (p.balance) hipLaunchKernelGGL((segment_reduce_kernel<1, true, false>), grid, dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((segment_reduce_kernel<1, false, false>), grid, dim3(512), 0, stream, p);
  } else if (p.num_segments <= 32) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    launch_rows<2>(p, grid, stream);
  } else if (p.num_segments <= 64) {
    const dim3 grid((unsigned)((rows + 1) / 2));
    launch_rows<4>(p, grid, stream);
  } else {
    // above 64 segments (balanced caps only): eight waves per row
    if (!p.balance) return hipErrorInvalidValue;
    if (p.ws_row_major) hipLaunchKernelGGL((segment_reduce_kernel<8, true, true>), dim3((unsigned)rows), dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((segment_reduce_kernel<8, true, false>), dim3((unsigned)rows), dim3(512), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pfkv
