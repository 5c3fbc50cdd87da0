// Merge of split-KV partials into the bf16 output: the per-row arithmetic of
// the segment reduce (segment_reduce.hip), and the opt-in merge inside the main
// launch (splitkv_kernel.h), which runs the same per-row code so that both give
// the same bits.
//
// For output row (t, hq) with segments s = 0 .. S-1 holding (m_s, l_s, o_s):
//   M = max_s m_s,  c_s = 2^(m_s - M) l_s (0 for an empty segment, m_s = -inf),
//   out = v_descale * sum_s c_s o_s / sum_s c_s   (0 when the sum is 0),
// then rounded to bf16 to nearest even (aiter PR #5190, Modifications: the
// split-KV segment reduce after the main kernel). The numerator is summed in
// the order s = 0, 1, ...; the denominator by a fixed reduction over the
// wave's lanes. With an lse buffer the row's log-sum-exp ln 2 (M + log2 sum_s
// c_s) goes to lse[hq][t] (-inf when the sum is 0), the merge rule of split
// softmax statistics (aiter PR #7375, Behavior and intent). A sink logit of the
// row's head adds e^sink to the denominator (and to the lse sum) and nothing to
// the numerator.
#pragma once

#include "pfkv_internal.h"

namespace pfkv {
namespace {
namespace merge {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
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

// One output row, merged by PARTS waves of the work-group: wave part q sums
// the numerator over its share of the S segments (at most kBatch, so that its
// o loads go out together), every part computes the same M and denominator
// from all (m, l), and part 0 adds the parts in order q = 0, 1, ... through
// LDS (`partial`, 8 x 64 f32x4) and writes the row. PARTS = 1 is one wave per
// row, the segments summed in order s = 0, 1, ...; PARTS = 8 serves up to 128
// segments, each lane then holding two (m, l) pairs. Lane i holds dims
// 4i .. 4i + 3 (head dim 128: lanes 0-31). With PARTS > 1 every wave of the
// work-group must call this together (it holds a work-group barrier); `valid`
// is false for a wave without a row in this pass.
// (M, den) of a row from its segments' (m, l), lane s holding segment s (and,
// when kWide, segment s + 64 in m2, l2), and each lane's weight c_s
// (coef, coef2) = 2^(m_s - M) l_s.
struct RowWeights {
  float M, den, coef, coef2;
};
template <bool kWide>
__device__ __forceinline__ RowWeights row_weights(float m, float l, float m2, float l2) {
  RowWeights w;
  w.M = wave_max(kWide ? fmaxf(m, m2) : m);
  w.coef = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - w.M) * l;
  w.coef2 = m2 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m2 - w.M) * l2;
  w.den = wave_sum(kWide ? w.coef + w.coef2 : w.coef);
  return w;
}

// The row's output from the weighted sum num = sum_s c_s o_s: sinks, v
// descale (vd = *p.v_descale), bf16 rounding, and the lse.
__device__ __forceinline__ void finish_row(const ReduceParams& p, int64_t row, f32x4 num, float M, float den, int lane,
                                           bool dims, float vd) {
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
  const float inv = den > 0.f ? vd * scale / den : 0.f;
  uint16_t* dst = p.out + t * p.out_stride_token + hq * p.out_stride_head + 4 * lane;
  const uint32_t lo = bf16_rne(num[0] * inv) | (bf16_rne(num[1] * inv) << 16);
  const uint32_t hi = bf16_rne(num[2] * inv) | (bf16_rne(num[3] * inv) << 16);
  if (dims) *(uint2*)dst = make_uint2(lo, hi);
  if (p.lse != nullptr && lane == 0)
    p.lse[hq * p.total_q + t] = den > 0.f ? (Mx + __builtin_amdgcn_logf(den)) * 0.69314718055994531f : -__builtin_inff();
}

template <int PARTS, bool RM>
__device__ __forceinline__ void merge_row(const ReduceParams& p, int64_t row, bool valid, int S, int part, int wave,
                                          int lane, f32x4 (*partial)[64]) {
  constexpr bool kWide = PARTS == 8;   // up to 128 segments: two (m, l) per lane
  if (PARTS == 1 && !valid) return;
  const int64_t rows_total = (int64_t)p.total_q * p.num_q_heads;
  const int per = (S + PARTS - 1) / PARTS;
  const int sb = min(part * per, S), se = min(sb + per, S);   // this wave's segments

  const bool dims = 4 * lane < p.head_dim;   // this lane's dims exist
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  RowWeights w = {-__builtin_inff(), 0.f, 0.f, 0.f};
  if (valid) {
    // the o loads of the first segments go out before (m, l) is known
    const _Float16* o =
        (const _Float16*)p.ws_o + ws_slot<RM>(row, 0, rows_total, p.num_segments) * kHeadDim + 4 * lane;
    const int64_t seg_stride = (RM ? 1 : rows_total) * kHeadDim;
    f16x4 a[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      a[k] = (sb + k < se && dims) ? __builtin_nontemporal_load((const f16x4*)(o + (sb + k) * seg_stride)) : f16x4{};

    float m = -__builtin_inff(), l = 0.f;
    if (lane < S) {
      const f32x2 v = __builtin_nontemporal_load((const f32x2*)(p.ws_ml + ws_slot<RM>(row, lane, rows_total, p.num_segments) * 2));
      m = v[0];
      l = v[1];
    }
    // more than 64 segments (balanced caps up to 128): lane s also holds
    // segment s + 64
    float m2 = -__builtin_inff(), l2 = 0.f;
    if constexpr (kWide) {
      if (lane + 64 < S) {
        const f32x2 v = __builtin_nontemporal_load((const f32x2*)(p.ws_ml + ws_slot<RM>(row, lane + 64, rows_total, p.num_segments) * 2));
        m2 = v[0];
        l2 = v[1];
      }
    }
    w = row_weights<kWide>(m, l, m2, l2);

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
          const float c = kWide && s >= 64 ? lane_value(w.coef2, s - 64) : lane_value(w.coef, s & 63);
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
  finish_row(p, row, num, w.M, w.den, lane, dims, *(const const_f32*)p.v_descale);
}

// ---------------------------------------------------------------- in-launch merge

// A device-scope 8-byte load: it reads the device's coherence point, where
// the main kernel's device-scope partial stores complete, not a cached copy.
template <typename T>
__device__ __forceinline__ T coherent_load(const T* src) {
  static_assert(sizeof(T) == 8, "8-byte partial loads");
  return __builtin_bit_cast(T, __hip_atomic_load((const uint64_t*)src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

constexpr int kMergeTasks = 128;   // (row, segment) o vectors of one share, at most R + S - 1 <= 127
// LDS of the in-launch merge: the gathered o vectors, then 8 x 64 f32x4 part sums
constexpr int kMergeLdsPartial = kMergeTasks * 64 * 8;
constexpr int kMergeLdsBcast = kMergeLdsPartial + 8 * 64 * 16;

// The rows of one share of a merge group: the group's R rows (row r is token
// q0 + r / G, query head hbase + r % G) split into S shares of ceil(R / S)
// rows. All eight waves load the share's (row, segment) o vectors into LDS,
// two vectors per 16-byte load (lanes 0-31 and 32-63), a few loads each: a
// wave's loads of partials written moments before complete one after another
// (about 0.45 us each, measured), so they are spread as thin as possible.
// Then PARTS waves per row sum the row's segments exactly as the segment
// reduce does for S (each part's segments in order, then the parts in order),
// so that the bits equal the reduce's.
template <int PARTS, int G, bool RM>
__device__ __forceinline__ void merge_share(const ReduceParams& p, int share, int S, int R, int q0, int hbase,
                                            int wave, int lane, uint8_t* lds, float vd) {
  const int per = (R + S - 1) / S;
  const int r0 = min(share * per, R), n = min(r0 + per, R) - r0;   // this share's rows
  if (n <= 0) return;   // uniform over the work-group
  const int64_t rows_total = (int64_t)p.total_q * p.num_q_heads;
  const bool dims = 4 * lane < p.head_dim;
  f16x4 (*buf)[64] = (f16x4 (*)[64])lds;   // [i * S + s][lane]
  f32x4 (*partial)[64] = (f32x4 (*)[64])(lds + kMergeLdsPartial);
  auto row_of = [&](int i) -> int64_t {
    const int r = r0 + i;
    return (int64_t)(q0 + r / G) * p.num_q_heads + hbase + r % G;
  };
  // task pair j (tasks 2j, 2j + 1, task t = i S + s) of this wave: j = wave,
  // wave + 8, ...; half h = lane / 32 takes task 2j + h, dims 8 (lane % 32) ..
  const int tasks = n * S;
  const int half = lane >> 5, hl = lane & 31;
  // device-scope (sc1) 16-byte buffer loads; the resource spans the o
  // partials (under 2^31 bytes wherever the merge runs), so that a load
  // outside it returns zeros instead of reading memory
  const __amdgpu_buffer_rsrc_t o_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.ws_o, (short)0, (int)(p.num_segments * rows_total * kHeadDim * 2), 0x00020000);
  constexpr int kSc1 = 16;   // cache policy: device scope
  f16x8 a[kMergeTasks / 16];
#pragma unroll
  for (int k = 0; k < kMergeTasks / 16; ++k) {
    const int t = 2 * (wave + 8 * k) + half;
    const int i = t / S, s = t - i * S;
    a[k] = f16x8{};
    if (2 * (wave + 8 * k) < tasks && t < tasks && 8 * hl < p.head_dim)
      a[k] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                           o_rsrc, (int)((ws_slot<RM>(row_of(i), s, rows_total, p.num_segments) * kHeadDim + 8 * hl) * 2), 0,
                                           kSc1));
  }
  // (m, l) of this wave's row in the first pass go out with them
  const int prow = wave / PARTS, part = wave % PARTS;
  float m = -__builtin_inff(), l = 0.f;
  if (prow < n && lane < S) {
    const f32x2 v = coherent_load((const f32x2*)(p.ws_ml + ws_slot<RM>(row_of(prow), lane, rows_total, p.num_segments) * 2));
    m = v[0];
    l = v[1];
  }
#pragma unroll
  for (int k = 0; k < kMergeTasks / 16; ++k) {
    const int t = 2 * (wave + 8 * k) + half;
    if (2 * (wave + 8 * k) < tasks && t < tasks) *(f16x8*)&buf[t][2 * hl] = a[k];
  }
  __syncthreads();
  const int per_part = (S + PARTS - 1) / PARTS;
  const int sb = min(part * per_part, S), se = min(sb + per_part, S);   // this wave's segments
  for (int base = 0; base < n; base += 8 / PARTS) {   // uniform
    const int i = base + prow;
    const bool valid = i < n;
    const int64_t row = valid ? row_of(i) : 0;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    RowWeights w = {-__builtin_inff(), 0.f, 0.f, 0.f};
    if (valid) {
      if (base > 0) {
        m = -__builtin_inff();
        l = 0.f;
        if (lane < S) {
          const f32x2 v = coherent_load((const f32x2*)(p.ws_ml + ws_slot<RM>(row, lane, rows_total, p.num_segments) * 2));
          m = v[0];
          l = v[1];
        }
      }
      w = row_weights<false>(m, l, -__builtin_inff(), 0.f);
      // at most kBatch segments per part (S <= 64): their LDS reads go out together
      f16x4 v[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        if (sb + k < se) v[k] = buf[i * S + sb + k][lane];
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        if (sb + k < se) acc += lane_value(w.coef, sb + k) * __builtin_convertvector(v[k], f32x4);
    }
    if constexpr (PARTS > 1) {
      partial[wave][lane] = acc;
      __syncthreads();
#pragma unroll
      for (int q = 1; q < PARTS; ++q) acc += partial[wave + q][lane];
    }
    if (valid && part == 0) finish_row(p, row, acc, w.M, w.den, lane, dims, vd);
    if constexpr (PARTS > 1) __syncthreads();   // partial[] is written again by the next pass
  }
  __syncthreads();   // buf is written again by the next share
}

// In-launch merge (opt-in): the S work-groups of a merge group (the segments
// of one sequence and head group) merge the group's rows themselves once all
// of them have written their partials, instead of a second launch. Called by
// every thread of the work-group after its partials are written; share is the
// work-group's segment. sync: the group's kMergeSyncWords words, zero before
// first use: word 0 holds the arrivals in bits 0-7 and a generation above
// them; words 64-65 the 64-bit mask of shares handed to the last arrival.
//
// Ordering without cache maintenance: the partials are written with
// device-scope stores (partial_store), each wave waits for all of its
// stores to complete (at the device's coherence point) before the work-group
// counts its arrival, and the merge reads them with device-scope loads issued
// only after the arrivals are seen. An agent-scope release or acquire fence
// would write back or invalidate this XCD's whole L2, which costs several
// microseconds per work-group when all of them do it at once.
//
// A work-group counts its arrival; the last to arrive returns the count to
// zero and moves the generation on in one addition, and every other one,
// waiting for the generation to move, then merges its own share. The wait is
// bounded by wait_ticks of the 100 MHz constant clock, so that no work-group
// waits for one that cannot start (a grid larger than the device, another
// kernel holding the CUs): one that gives up sets its share's bit in the mask
// and exits, and the last arrival merges the shares it finds there after its
// own. A work-group that gives up sets the bit, then reads the word; the last
// arrival moves the generation, then takes the mask; each side's second
// atomic goes out only once its first is performed at the coherence point, so
// at least one side sees the other: a work-group that gives up and then finds
// the generation moved merges its share itself (a second merge of a share
// writes the same bits).
enum : int { kMergeOwn = 0, kMergeLast = 1, kMergeLeave = 2 };

template <int PARTS, int G, bool RM>
__device__ __forceinline__ void merge_in_launch(const ReduceParams& p, uint32_t* sync, uint32_t wait_ticks, int share,
                                                int S, int R, int q0, int hbase, uint8_t* smem) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // read now, not after the wait
  const float vd = *(const const_f32*)p.v_descale;
  // every wave's partial stores are complete before the arrival is counted
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t* bcast = (uint32_t*)(smem + kMergeLdsBcast);
  uint32_t* word = sync;
  uint64_t* handed = (uint64_t*)(sync + 64);
  if (threadIdx.x == 0) {
    int role;
    const uint32_t old = __hip_atomic_fetch_add(word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t g0 = old >> 8;
    if ((old & 0xffu) == (uint32_t)(S - 1)) {
      // count S + (256 - S) carries into the generation: count 0, generation + 1
      __hip_atomic_fetch_add(word, 256u - (uint32_t)S, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      role = kMergeLast;
    } else {
      role = kMergeLeave;
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      for (;;) {
        if ((__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 8) != g0) {
          role = kMergeOwn;
          break;
        }
        if (__builtin_amdgcn_s_memrealtime() - t0 >= wait_ticks) break;
        __builtin_amdgcn_s_sleep(2);
      }
      if (role == kMergeLeave) {
        const uint64_t bit = (uint64_t)1 << share;
        __hip_atomic_fetch_or(handed, bit, __ATOMIC_SEQ_CST, __HIP_MEMORY_SCOPE_AGENT);
        if ((__hip_atomic_fetch_add(word, 0u, __ATOMIC_SEQ_CST, __HIP_MEMORY_SCOPE_AGENT) >> 8) != g0) {
          // the last arrival came meanwhile and may not have seen the bit
          __hip_atomic_fetch_and(handed, ~bit, __ATOMIC_SEQ_CST, __HIP_MEMORY_SCOPE_AGENT);
          role = kMergeOwn;
        }
      }
    }
    bcast[0] = (uint32_t)role;
  }
  __syncthreads();
  const int role = (int)bcast[0];
  if (role == kMergeLeave) return;
  merge_share<PARTS, G, RM>(p, share, S, R, q0, hbase, wave, lane, smem, vd);
  if (role != kMergeLast) return;
  // the last arrival: the shares handed to it, taken once its addition to the
  // word has been performed (it was issued before the merge above; the wait
  // makes sure)
  if (threadIdx.x == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint64_t rescue = __hip_atomic_exchange(handed, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bcast[1] = (uint32_t)rescue;
    bcast[2] = (uint32_t)(rescue >> 32);
  }
  __syncthreads();
  uint64_t rescue = (uint64_t)bcast[1] | ((uint64_t)bcast[2] << 32);
  while (rescue != 0) {
    const int s = __builtin_ctzll(rescue);
    rescue &= rescue - 1;
    merge_share<PARTS, G, RM>(p, s, S, R, q0, hbase, wave, lane, smem, vd);
  }
}

}  // namespace merge
}  // namespace
}  // namespace pfkv
