// Internal interface between the C ABI (pfkv_host.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct pfkv_args;   // include/pfkv.h

namespace pfkv {

constexpr int kHeadDim = 256;   // largest head_dim served (also 128); the workspace row stride
constexpr int kPageSize = 16;   // tokens per KV page
constexpr int kMaxQLen = 8;     // query tokens per sequence (the pages' 4, or up to 8 with max_q_len)
constexpr int kDefaultMaxQLen = 4;
constexpr int kMaxRows = 64;    // stacked query rows (G x tokens) per work-group
constexpr int kMaxSegments = 64;
constexpr int kMaxBalancedSegments = 128;   // the cap per sequence with balanced segments

// Workspace layout, written by the main kernel and read by the reduce:
//   o  [S][T][Hq][256] fp16  the segment's softmax-weighted mean of V (V without
//                            its descale): sum p V / sum p, 0 when sum p = 0
//                            (head dim 128: the first 128 of each row's 256)
//   ml [S][T][Hq][2]   fp32  (m, l): reference max in log2 units and l = sum p
// so that segment s contributes  2^(m_s - M) l_s o_s / sum_s 2^(m_s - M) l_s.
// Above 16 segments (16-bit arithmetic, head dim 256, pages of 16 or more) the
// two arrays are row-major instead, [T][Hq][S][256] and [T][Hq][S][2]
// (ws_row_major), so that a row's partials are one contiguous run for the merge
// (ws_slot). The layout is a template argument of the kernels: a runtime choice
// costs the segment-major stores their folded address offsets.
constexpr int kPartialBytes = kHeadDim * 2 + 2 * 4;   // workspace bytes per (segment, token, head)
constexpr int kRowMajorAbove = 16;                   // segments above which the partials are row-major

// Slot of (row, segment s) in the o and ml arrays, in units of one row's
// partial (256 fp16, or one (m, l) pair); RM: row-major.
template <bool RM>
__host__ __device__ __forceinline__ int64_t ws_slot(int64_t row, int s, int64_t rows_total, int S) {
  if constexpr (RM) return row * S + s;
  else return (int64_t)s * rows_total + row;
}
// The same for the row of query token q0 + i and query head h0 + g (of T and
// Hq), each sum taken in 64 bits.
template <bool RM>
__host__ __device__ __forceinline__ int64_t ws_slot_tq(int q0, int i, int h0, int g, int seg, int T, int Hq, int S) {
  if constexpr (RM) return (((int64_t)q0 + i) * Hq + h0 + g) * S + seg;
  else return ((int64_t)seg * T + q0 + i) * Hq + h0 + g;
}

// In-launch merge (opt-in): 32-bit sync words per merge group, a (sequence,
// blockIdx.z) pair of the main grid: [0] arrivals (bits 0-7) and generation
// (bits 8-31), [64..65] the 64-bit mask of shares handed to the last arrival,
// on separate 128-byte lines. Zero before the first call; every call leaves
// arrivals and mask at zero and the generation one higher.
constexpr int kMergeSyncWords = 128;
constexpr unsigned kMergeWaitTicksDefault = 5000;   // 50 us of the 100 MHz constant clock

struct MainParams {
  const uint16_t* q;           // bf16 bits
  int64_t q_stride_token, q_stride_head;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;
  int64_t block_table_stride;
  const int32_t* seq_lens;
  const int32_t* cu_seqlens_q;
  const float* k_descale;
  uint16_t* ws_o;              // fp16 bits
  float* ws_ml;
  // with a single segment the main kernel writes the bf16 output itself
  uint16_t* out;               // bf16 bits
  int64_t out_stride_token, out_stride_head;
  const float* v_descale;
  float* lse;                  // optional [Hq][T] fp32, written here when direct
  const float* sinks;          // optional [Hq] fp32 sink logits (used here when direct)
  int32_t window_left;         // < 0: no window
  float softcap;               // > 0: scores soft-capped
  int32_t direct;              // num_segments == 1
  // 2 when 32 query heads share a KV head: each KV head is served by two
  // work-groups of 16 query heads (blockIdx.z = 2 kv_head + half), else 1
  int32_t kv_split;
  // query-token blocks per (sequence, head group): a work-group holds at most
  // q_per_wg tokens (kMaxRows / G); q_split = 2 when a sequence may have more
  // (blockIdx.z = head_group * q_split + block)
  int32_t q_split, q_per_wg;
  // cache pages of 16 << page_ratio_log2 tokens, or of one token when
  // token_pages (page_ratio_log2 = 0 then); num_pages counts cache pages
  int32_t page_ratio_log2;
  int32_t token_pages;
  int32_t max_seq_len;         // max_pages_per_seq * page_size: bound on seq_lens
  int32_t precision;           // 0: 16-bit Q/P, 1: e4m3 P, 2: e4m3 Q (per-row scale) and P
  int32_t head_dim;            // 256 or 128
  int32_t num_seqs, total_q, num_q_heads, num_kv_heads, num_pages, num_segments;
  float score_scale_log2;      // softmax_scale * log2(e); multiplied by *k_descale on the device
  // balanced segments: blockIdx.x is a slot of gridDim.x (>= num_seqs); each
  // sequence gets segment_count() of them (num_segments is the cap), the slots
  // in sequence order; blockIdx.y is 0 and slots past the last one stay idle
  int32_t balance, num_slots;
  // in-launch merge (launched only with the merge instantiation, else NULL):
  // kMergeSyncWords words per merge group, group (b, z) at
  // merge_sync[(b * gridDim.z + z) * kMergeSyncWords]; a work-group waits at
  // most merge_wait_ticks ticks of the 100 MHz clock for the rest of its group
  uint32_t* merge_sync;
  uint32_t merge_wait_ticks;
  int32_t ws_row_major;        // partials row-major (selects the RM instantiations), see ws_slot
};

struct ReduceParams {
  const uint16_t* ws_o;        // fp16 bits
  const float* ws_ml;
  const float* v_descale;
  uint16_t* out;               // bf16 bits
  int64_t out_stride_token, out_stride_head;
  float* lse;                  // optional [Hq][T] fp32
  const float* sinks;          // optional [Hq] fp32 sink logits
  int32_t total_q, num_q_heads, num_segments;
  int32_t head_dim;            // 256 or 128 (o rows keep the kHeadDim stride)
  // balanced segments (see MainParams): a row of sequence b merges
  // segment_count(b) partials; these are the main kernel's inputs to it
  int32_t balance, num_slots, num_seqs, window_left, max_seq_len;
  const int32_t* seq_lens;
  const int32_t* cu_seqlens_q;
  int32_t ws_row_major;        // as MainParams
};

// Pages (16-token blocks) that the segments of a sequence of L keys split:
// with a left window of W positions, only those from the first page some query
// can see (bounded with the largest q_len, so independent of the call's q_len).
__device__ __forceinline__ int segment_span(int L, int window_left) {
  const int pages = (L + kPageSize - 1) / kPageSize;
  const int win = window_left < 0 ? -1 : min(window_left, L);
  const int first = win < 0 ? 0 : min(max(L - kMaxQLen - win, 0) / kPageSize, pages);
  return pages - first;
}

// Balanced segments: of `slots` work-group slots, a sequence whose span is
// `span` pages out of `total` gets 1 + floor((slots - num_seqs) span / total),
// at most `cap`; the counts add up to at most `slots`. Every input comes from
// device data and call arguments, so the schedule is the same on every replay.
__device__ __forceinline__ int segment_count(int span, int64_t total, int slots, int num_seqs, int cap) {
  const int64_t extra = total > 0 ? (int64_t)(slots - num_seqs) * span / total : 0;
  return (int)min((int64_t)cap, 1 + extra);
}

// The clamped KV length of sequence b, as the main kernel reads it.
__device__ __forceinline__ int clamped_len(const int32_t* seq_lens, int b, int max_seq_len) {
  return min(max(((__attribute__((address_space(4))) const int32_t*)seq_lens)[b], 0), max_seq_len);
}

// The balanced schedule, computed by each wave that needs it, every lane
// getting the same result: lane l takes sequences c + l of chunks c = 0, 64, ...
// with one vector load each, where a loop over the sequences would wait on one
// scalar load after another (up to 3 us of the reduce at 8 sequences). Same
// integer formulas, so the same schedule.
__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) v += __shfl_xor(v, k, 64);
  return v;
}
__device__ __forceinline__ int lane_span(const int32_t* seq_lens, int i, int num_seqs, int max_seq_len, int window_left) {
  return i < num_seqs ? segment_span(min(max(seq_lens[i], 0), max_seq_len), window_left) : 0;
}
// sum over the sequences of segment_span
__device__ __forceinline__ int64_t total_span(const int32_t* seq_lens, int num_seqs, int max_seq_len, int window_left) {
  const int lane = threadIdx.x & 63;
  int64_t acc = 0;
  for (int c = 0; c < num_seqs; c += 64) acc += lane_span(seq_lens, c + lane, num_seqs, max_seq_len, window_left);
  return wave_sum_i64(acc);
}
struct BalancedSlot {
  int b, seg, count;   // b = -1: the slot is past the last sequence's segments
};
// Slot x: the first sequence b whose running sum of segment counts passes x,
// its segment x - (slots of sequences before b) and its segment count.
__device__ __forceinline__ BalancedSlot balanced_slot(int x, const int32_t* seq_lens, int num_seqs, int max_seq_len,
                                                      int window_left, int slots, int cap) {
  const int lane = threadIdx.x & 63;
  const int64_t total = total_span(seq_lens, num_seqs, max_seq_len, window_left);
  int carry = 0;   // slots of the sequences of earlier chunks
  for (int c = 0; c < num_seqs; c += 64) {
    const int i = c + lane;
    const int n = i < num_seqs ? segment_count(lane_span(seq_lens, i, num_seqs, max_seq_len, window_left), total, slots,
                                               num_seqs, cap)
                               : 0;
    int pre = n;   // inclusive prefix over the chunk's lanes
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
      const int y = __shfl_up(pre, k, 64);
      if (lane >= k) pre += y;
    }
    const uint64_t hit = __ballot(i < num_seqs && x < carry + pre);
    if (hit != 0) {
      const int j = __builtin_ctzll(hit);
      const int pj = __shfl(pre, j, 64), nj = __shfl(n, j, 64);
      return BalancedSlot{c + j, x - (carry + pj - nj), nj};
    }
    carry += __shfl(pre, 63, 64);
  }
  return BalancedSlot{-1, 0, 0};
}
// Query token t: its sequence b (the first with cu[b] <= t < cu[b + 1], -1 if
// none) and b's segment count.
__device__ __forceinline__ BalancedSlot balanced_row(int t, const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                                                     int num_seqs, int max_seq_len, int window_left, int slots, int cap) {
  const int lane = threadIdx.x & 63;
  const int64_t total = total_span(seq_lens, num_seqs, max_seq_len, window_left);
  for (int c = 0; c < num_seqs; c += 64) {
    const int i = c + lane;
    const bool in = i < num_seqs && t >= cu_seqlens_q[i] && t < cu_seqlens_q[i + 1];
    const uint64_t hit = __ballot(in);
    if (hit != 0) {
      const int j = __builtin_ctzll(hit);
      const int span = __shfl(lane_span(seq_lens, i, num_seqs, max_seq_len, window_left), j, 64);
      return BalancedSlot{c + j, 0, segment_count(span, total, slots, num_seqs, cap)};
    }
  }
  return BalancedSlot{-1, 0, 0};
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN)
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// fp8 varlen prefill (the second workload): e4m3 Q/K/V rows in packed THD
// layout, qk head dim 192, v head dim 128.
struct PrefillParams {
  const uint8_t* q;            // [total_q, Hq, 192] e4m3 bytes
  int64_t q_stride_token, q_stride_head;   // bytes, multiples of 16
  const uint8_t* k;            // [total_k, Hkv, 192]
  int64_t k_stride_token, k_stride_head;
  const uint8_t* v;            // [total_k, Hkv, 128]
  int64_t v_stride_token, v_stride_head;
  uint16_t* out;               // bf16 bits [total_q, Hq, 128]
  int64_t out_stride_token, out_stride_head;   // elements, multiples of 4
  float* lse;                  // optional [Hq][total_q]
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  const float* q_descale;
  const float* k_descale;
  const float* v_descale;
  int32_t num_seqs, total_q, total_k, num_q_heads, num_kv_heads, max_seqlen_q;
  float scale_log2;            // softmax_scale * log2(e); times q and k descales on the device
  int32_t causal;
};

// Debug-mode precondition check of the device-side inputs.
struct CheckParams {
  const int32_t* cu_seqlens_q;
  const int32_t* seq_lens;
  const int32_t* block_tables;
  int64_t block_table_stride;
  int32_t num_seqs, total_q, max_q_len, page_size, max_pages_per_seq, num_pages;
};

hipError_t launch_splitkv_main(const MainParams& p, int group, hipStream_t stream);
// The verify call of pfkv.h on a workspace the library owns (pfkv_host.cpp),
// and the setter of the thread's last-error text.
int verify_attn_library_workspace(const ::pfkv_args* a, void* ws, uint64_t ws_bytes, void* stream);
int set_error(int status, const char* msg);
// the e4m3-P and e4m3-Q/P modes at head dim 256, and every mode at head dim
// 128, one translation unit each
hipError_t launch_splitkv_main_fp8p(const MainParams& p, int group, hipStream_t stream);
hipError_t launch_splitkv_main_fp8(const MainParams& p, int group, hipStream_t stream);
hipError_t launch_splitkv_main_hd128(const MainParams& p, int group, hipStream_t stream);
// the 16-bit mode at head dim 256 with row-major partials (pages of 16 or more)
hipError_t launch_splitkv_main_rm(const MainParams& p, int group, hipStream_t stream);
hipError_t launch_precondition_check(const CheckParams& p, int32_t* status, hipStream_t stream);
hipError_t launch_segment_reduce(const ReduceParams& p, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, uint64_t bytes, int variant, const int32_t* page_order,
                              int64_t num_pages, uint32_t* sink, hipStream_t stream);

}  // namespace pfkv
