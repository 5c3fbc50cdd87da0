// Segment reduce: merges the per-segment partials of the split-KV main kernel
// into the bf16 output (aiter PR #5190 "gfx950 assembly MTP-verify attention for
// head_dim 256 fp8 paged KV", section Modifications: a split-KV segment reduce
// after the main kernel).
//
// For output row (t, hq) with segments s = 0 .. S-1 holding (m_s, l_s, o_s):
//   M = max_s m_s,  c_s = 2^(m_s - M) l_s (0 for an empty segment, m_s = -inf),
//   out = v_descale * sum_s c_s o_s / sum_s c_s   (0 when the sum is 0),
// then rounded to bf16 to nearest even. The numerator is summed in the order
// s = 0, 1, ...; the denominator by a fixed reduction over the wave's lanes.
// With an lse buffer the row's log-sum-exp ln 2 (M + log2 sum_s c_s) goes to
// lse[hq][t] (-inf when the sum is 0), the merge rule of split softmax
// statistics (aiter PR #7375, Behavior and intent). A sink logit of the row's
// head adds e^sink to the denominator (and to the lse sum) and nothing to the
// numerator.
// One wave per output row, eight rows per work-group (measured 1 us faster per
// call than four at 16 x 35000: fewer, fuller work-groups): lane s holds
// (m_s, l_s), lane i dims 4i .. 4i + 3 of the fp16 o rows (head dim 128: lanes
// 0-31), whose loads for up to 16 segments are in flight together. Above 16
// segments 2, 4 or (balanced caps above 64) 8 waves share a row; BAL takes each
// row's segment count from the balanced schedule instead of num_segments.
#include "pfkv_internal.h"

namespace pfkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(4))) const float const_f32;

__device__ __forceinline__ float lane_value(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

constexpr int kBatch = 16;   // segments whose o loads fly together

// Wave-wide max and sum: within each 16-lane row by DPP (swap neighbours,
// swap pairs, mirror halves of 8, mirror the row), then the four row results
// by readlane, combined in a fixed order; every lane gets the same value.
// (0.45 us per call faster at 16 x 35000 than a butterfly of LDS permutes,
// whose 12 round trips sat on the reduce's critical path.)
__device__ __forceinline__ float dpp_f(float x, int ctrl_sel) {
  const int v = __float_as_int(x);
  int r;
  switch (ctrl_sel) {
    case 0: r = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); break;    // quad_perm(1,0,3,2)
    case 1: r = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false); break;    // quad_perm(2,3,0,1)
    case 2: r = __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false); break;   // row_half_mirror
    default: r = __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false); break;  // row_mirror
  }
  return __int_as_float(r);
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int k = 0; k < 4; ++k) x = fmaxf(x, dpp_f(x, k));
  const float r0 = lane_value(x, 0), r1 = lane_value(x, 16), r2 = lane_value(x, 32), r3 = lane_value(x, 48);
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int k = 0; k < 4; ++k) x = x + dpp_f(x, k);
  const float r0 = lane_value(x, 0), r1 = lane_value(x, 16), r2 = lane_value(x, 32), r3 = lane_value(x, 48);
  return (r0 + r1) + (r2 + r3);
}

// PARTS waves merge one row: wave part q sums the numerator over its share
// of the segments (at most kBatch, so its o loads go out together), every part
// computes the same M and denominator from all (m, l), and part 0 adds the
// parts in order q = 0, 1, ... through LDS and writes the row. With many
// segments and few rows (4 sequences x 64 segments: 256 rows) one wave per
// row would load its segments in several dependent batches on a few CUs.
// PARTS = 1 is one wave per row, the segments summed in order s = 0, 1, ...
// PARTS = 8 serves up to 128 segments: each lane then holds two (m, l) pairs.
template <int PARTS, bool BAL>
__global__ void __launch_bounds__(512) segment_reduce_kernel(ReduceParams p) {
  constexpr int kRowsPerWg = 8 / PARTS;
  constexpr bool kWide = PARTS == 8;   // up to 128 segments: two (m, l) per lane
  __shared__ f32x4 partial[PARTS > 1 ? 8 : 1][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t rows_total = (int64_t)p.total_q * p.num_q_heads;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWg + wave / PARTS;
  const int part = wave % PARTS;
  const bool valid = row < rows_total;
  if (PARTS == 1 && !valid) return;
  int S = p.num_segments;
  if (BAL && valid) {
    // the row's sequence and its segment count, as the main kernel scheduled them
    const int t = (int)(row / p.num_q_heads);
    const __attribute__((address_space(4))) int32_t* cu = (const __attribute__((address_space(4))) int32_t*)p.cu_seqlens_q;
    int b = -1;
    for (int i = 0; i < p.num_seqs; ++i)
      if (t >= cu[i] && t < cu[i + 1]) {
        b = i;
        break;
      }
    if (b >= 0) {
      int64_t total = 0;
      for (int i = 0; i < p.num_seqs; ++i) total += segment_span(clamped_len(p.seq_lens, i, p.max_seq_len), p.window_left);
      S = segment_count(segment_span(clamped_len(p.seq_lens, b, p.max_seq_len), p.window_left), total, p.num_slots,
                        p.num_seqs, p.num_segments);
    }
  }
  const int per = (S + PARTS - 1) / PARTS;
  const int sb = min(part * per, S), se = min(sb + per, S);   // this wave's segments

  const bool dims = 4 * lane < p.head_dim;   // this lane's dims exist
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float M = -__builtin_inff(), den = 0.f;
  if (valid) {
    // the o loads of the first segments go out before (m, l) is known
    const _Float16* o = (const _Float16*)p.ws_o + row * kHeadDim + 4 * lane;
    const int64_t seg_stride = rows_total * kHeadDim;
    f16x4 a[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      a[k] = (sb + k < se && dims) ? __builtin_nontemporal_load((const f16x4*)(o + (sb + k) * seg_stride)) : f16x4{};

    float m = -__builtin_inff(), l = 0.f;
    if (lane < S) {
      const f32x2 v = __builtin_nontemporal_load((const f32x2*)(p.ws_ml + (lane * rows_total + row) * 2));
      m = v[0];
      l = v[1];
    }
    // more than 64 segments (balanced caps up to 128): lane s also holds
    // segment s + 64
    float m2 = -__builtin_inff(), l2 = 0.f;
    if constexpr (kWide) {
      if (lane + 64 < S) {
        const f32x2 v = __builtin_nontemporal_load((const f32x2*)(p.ws_ml + ((lane + 64) * rows_total + row) * 2));
        m2 = v[0];
        l2 = v[1];
      }
    }
    M = wave_max(kWide ? fmaxf(m, m2) : m);
    const float coef = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - M) * l;
    const float coef2 = m2 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m2 - M) * l2;
    den = wave_sum(kWide ? coef + coef2 : coef);

    for (int s0 = sb; s0 < se; s0 += kBatch) {
      if (s0 > sb) {
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
          if (s0 + k < se && dims) a[k] = __builtin_nontemporal_load((const f16x4*)(o + (s0 + k) * seg_stride));
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        if (s0 + k < se) {
          const int s = s0 + k;   // wave-uniform
          const float c = kWide && s >= 64 ? lane_value(coef2, s - 64) : lane_value(coef, s & 63);
          num += c * __builtin_convertvector(a[k], f32x4);
        }
    }
  }
  if constexpr (PARTS > 1) {
    partial[wave][lane] = num;
    __syncthreads();
    if (!valid || part != 0) return;
#pragma unroll
    for (int q = 1; q < PARTS; ++q) num += partial[wave + q][lane];
  }
  const int64_t t = row / p.num_q_heads, hq = row - t * p.num_q_heads;
  // a sink logit (log2 units here) joins the denominator: with Mx = max(M, sink),
  // out = num 2^(M - Mx) / (den 2^(M - Mx) + 2^(sink - Mx))
  float scale = 1.f, Mx = M;
  if (p.sinks != nullptr) {
    const float sink2 = ((const const_f32*)p.sinks)[hq] * 1.44269504088896341f;
    Mx = fmaxf(M, sink2);
    scale = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(M - Mx);
    den = den * scale + __builtin_amdgcn_exp2f(sink2 - Mx);
  }
  const float vd = *(const const_f32*)p.v_descale;
  const float inv = den > 0.f ? vd * scale / den : 0.f;
  uint16_t* dst = p.out + t * p.out_stride_token + hq * p.out_stride_head + 4 * lane;
  const uint32_t lo = bf16_rne(num[0] * inv) | (bf16_rne(num[1] * inv) << 16);
  const uint32_t hi = bf16_rne(num[2] * inv) | (bf16_rne(num[3] * inv) << 16);
  if (dims) *(uint2*)dst = make_uint2(lo, hi);
  if (p.lse != nullptr && lane == 0)
    p.lse[hq * p.total_q + t] = den > 0.f ? (Mx + __builtin_amdgcn_logf(den)) * 0.69314718055994531f : -__builtin_inff();
}

}  // namespace

hipError_t launch_segment_reduce(const ReduceParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.total_q * p.num_q_heads;
  // waves per row: one up to 16 segments (a single batch of loads), else 2 or 4
  // (balanced segments: a separate instantiation that finds each row's count)
  if (p.num_segments <= 16) {
    const dim3 grid((unsigned)((rows + 7) / 8));
    if (p.balance) hipLaunchKernelGGL((segment_reduce_kernel<1, true>), grid, dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((segment_reduce_kernel<1, false>), grid, dim3(512), 0, stream, p);
  } else if (p.num_segments <= 32) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (p.balance) hipLaunchKernelGGL((segment_reduce_kernel<2, true>), grid, dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((segment_reduce_kernel<2, false>), grid, dim3(512), 0, stream, p);
  } else if (p.num_segments <= 64) {
    const dim3 grid((unsigned)((rows + 1) / 2));
    if (p.balance) hipLaunchKernelGGL((segment_reduce_kernel<4, true>), grid, dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((segment_reduce_kernel<4, false>), grid, dim3(512), 0, stream, p);
  } else {
    // above 64 segments (balanced caps only): eight waves per row
    hipLaunchKernelGGL((segment_reduce_kernel<8, true>), dim3((unsigned)rows), dim3(512), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pfkv
