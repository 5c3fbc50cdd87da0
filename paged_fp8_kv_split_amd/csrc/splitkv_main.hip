// Split-KV main kernel for verify attention over a paged fp8 KV cache (gfx950).
//
// What it computes follows aiter PR #5190 ("gfx950 assembly MTP-verify attention
// for head_dim 256 fp8 paged KV"), sections Modifications and Kernel notes: one
// work-group per (KV segment, sequence, KV head), partial softmax statistics per
// segment to a workspace, empty segments written neutrally, descales read from
// device pointers. In-kernel q_len 1..4 follows SGLang PR #37465, Modifications.
// The decomposition is this library's own:
//
// * 8 waves per work-group, two per SIMD. A step covers 4 pages (64 keys).
//   Page slot j of the step belongs to the wave pair (j, j + 4): the pair streams
//   it HBM -> LDS (one wave K, the other V) and computes its 16 keys' scores,
//   each wave for half of the G * q_len (<= 64) stacked query rows. For P V every
//   wave covers all 64 keys but only 32 of the 256 output dims, so the fp32
//   accumulator is 32 registers per lane and P V is never duplicated.
// * Q is loaded once into registers in the MFMA operand layout.
// * K/V pages move with global_load_lds_dwordx4 (1 KiB contiguous per
//   instruction) issued from inline asm, so the compiler does not serialise LDS
//   reads behind every outstanding transfer. K and V have rings of their own:
//   K of a step is consumed one step before its V, so K is fetched one step
//   later and both rings (4 stages each) keep three steps ahead in flight,
//   with explicit vmcnt waits.
// * One work-group barrier per step. Between barriers t and t+1 each wave does
//   P V of step t and the scores of step t+1 (independent MFMA chains), then the
//   softmax of step t+1.
// * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: K converts exactly from e4m3fn to
//   bf16 (v_cvt_scalef32_pk_bf16_fp8, scale 1), Q stays bf16. The score layout
//   puts one query row per lane column: row maxima need one in-lane reduction and
//   two cross-lane steps.
// * Online softmax in the log2 domain with a lazy reference max m per row: m
//   moves only when a row's running max exceeds it by more than 8, so
//   P = 2^(s - m) <= 2^8 fits fp16 and the accumulator is rescaled rarely. Each
//   wave computes P against the current m and publishes it with its row maxima.
//   If any wave saw a row exceed m + 8, all waves take the (rare) slow path: new
//   m from the step's maxima, rescale, recompute P, one more barrier. Rows that
//   did not need it keep m and get bit-identical P, so each row's arithmetic
//   depends only on that row.
// * P is rounded to fp16 once; the same values feed the row sum l and P V.
// * O += P V on v_mfma_f32_16x16x32_f16. V's transposed operand comes from
//   ds_read_b64_tr_b8 and converts exactly to fp16.
#include <type_traits>

#include "pfkv_internal.h"

namespace pfkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(4))) const int32_t const_i32;
typedef __attribute__((address_space(4))) const float const_f32;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kPagesPerStep = 4;                       // one page per wave pair
constexpr int kStages = 4;                             // depth of the K ring and of the V ring (steps)
constexpr int kPageBytes = kPageSize * kHeadDim;       // one (page, head) block of K or V: 4 KiB
constexpr int kStageBytes = kPagesPerStep * kPageBytes;       // K (or V) of one step: 16 KiB
constexpr int kDmaPerWave = kPageBytes / 1024;         // 4 x 1 KiB per wave per step
constexpr int kDimsPerWave = kHeadDim / kWaves;        // 32
constexpr float kLazySlack = 8.0f;                     // log2 units

template <int G>
struct Cfg {
  static constexpr int kRowBlocks = G * kMaxQLen / 16;            // 16-row MFMA blocks (all rows)
  static constexpr int kHalfBlocks = kRowBlocks / 2;               // row blocks scored by one wave
  static constexpr int kRows = kRowBlocks * 16;
  static constexpr int kPBytes = kRowBlocks * kPagesPerStep * 64 * 8;   // fp16 P of one step: [rb][slot][lane]
  static constexpr int kMxBytes = kPagesPerStep * 4 * kRows * 4;   // per-lane row maxima (slow path)
  static constexpr int kOffP = 0;                                  // two P buffers
  static constexpr int kOffMx = kOffP + 2 * kPBytes;               // maxima buffer (slow path only)
  static constexpr int kOffFlag = kOffMx + kMxBytes;               // slow-path flag words (4 steps)
  static constexpr int kOffIds = kOffFlag + 64;                    // page-id windows [wave][2][64]
  static constexpr int kOffStage = kOffIds + kWaves * 2 * 64 * 4;  // K ring, then V ring
  static constexpr int kLdsBytes = kOffStage + 2 * kStages * kStageBytes;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
  static_assert(kPagesPerStep * kRows * 4 + kRows * 4 <= kLdsBytes, "epilogue scratch");
};

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One 1 KiB HBM -> LDS transfer: lane i moves 16 bytes from sbase + voff to
// LDS address lds + 16 i. M0 carries the LDS base; it is saved and restored.
__device__ __forceinline__ void dma_1k(const uint8_t* sbase, unsigned voff, unsigned lds) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

// As dma_1k with 4 bytes per lane: lane i moves sbase + voff to lds + 4 i.
__device__ __forceinline__ void dma_4b(const void* sbase, unsigned voff, unsigned lds) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

// Wait until at most `pending` of this wave's vector-memory operations are in
// flight (0, 4 or 8). Inside the main loop the only such operations are the
// page transfers, four 1 KiB transfers per wave and step.
__device__ __forceinline__ void wait_vm(int pending) {
  if (pending >= 8)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (pending >= 4)
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Work-group barrier that orders LDS traffic but does not wait for the page
// transfers still in flight (a __syncthreads() fence would drain vmcnt).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ bf16x8 fp8x8_to_bf16(unsigned lo, unsigned hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ f16x8 fp8x8_to_f16(unsigned lo, unsigned hi) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Geometry of one work-group's (segment, sequence, KV head), uniform.
struct Geo {
  int seg, b, h;
  int q0, q_len, L, pb, pe, rows, n_steps;
  float c2;          // k_descale * softmax_scale * log2(e): raw score -> log2 units
};

// The work of one wave, specialised on the number NRB of 16-row blocks that
// hold real query rows (G * q_len of them) and on the wave's half HF: it
// scores row blocks HF and HF + 2 (those below NRB) of its page slot, and
// accumulates P V for all NRB row blocks over its own 32 dims. With both known
// at compile time the steady-state loop is straight-line code.
template <int G, int NRB, int HF>
__device__ __forceinline__ void wave_main(const MainParams& p, const Geo& geo, uint8_t* smem) {
  using C = Cfg<G>;
  constexpr int NJ = (HF < NRB ? 1 : 0) + (HF + 2 < NRB ? 1 : 0);   // row blocks scored
  constexpr int NJA = NJ > 0 ? NJ : 1;                                // array extent
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pw = w & 3;          // page slot of the step this wave streams and scores
  const int lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int h = geo.h, q0 = geo.q0, q_len = geo.q_len, L = geo.L, pb = geo.pb, pe = geo.pe;
  const int rows = geo.rows, n_steps = geo.n_steps;
  const float c2 = geo.c2;

  const const_i32* bt = (const const_i32*)p.block_tables;
  const int64_t bt_row = (int64_t)geo.b * p.block_table_stride;
  const uint64_t page_stride = (uint64_t)kPageSize * p.num_kv_heads * kHeadDim;

  // ---- per-lane DMA offsets inside one (page, head) block. In LDS, the
  // 16-byte chunk at position pos of key row k (page slot j) holds dim chunk
  // pos ^ sw(k, j), sw(k, j) = (k ^ 12 (j & 1)) & 15: K row reads and V
  // transposed reads are then free of bank conflicts.
  const int jpar = pw & 1;
  unsigned goff[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int k = 4 * jj + g;
    goff[jj] = (unsigned)((k * p.num_kv_heads + h) * kHeadDim + 16 * (n ^ ((k ^ (12 * jpar)) & 15)));
  }
  uint8_t* const k_ring = smem + C::kOffStage;
  uint8_t* const v_ring = k_ring + kStages * kStageBytes;
  // half 0 moves K of page slot pw, half 1 moves V
  const unsigned ring_lds = lds_addr(HF == 0 ? k_ring : v_ring) + pw * kPageBytes;
  const uint8_t* const cache = HF == 0 ? p.k_cache : p.v_cache;

  auto has_page = [&](int t) -> bool { return t < n_steps && pb + kPagesPerStep * t + pw < pe; };

  // Page ids of this wave's steps, cached in LDS: entry k of window w (of
  // this wave, w even / odd in two slots) is the block-table entry of step
  // 64 w + k. The windows are filled with page transfers of their own (4 bytes
  // per lane), window w + 1 while window w is half used, so the vmcnt waits
  // of the page stream cover them and no scalar-load latency is exposed. The id
  // of a wave's next transfer is read from LDS one transfer ahead.
  const unsigned ids_lds = lds_addr(smem + C::kOffIds) + w * (2 * 64 * 4);
  const int* const ids_ptr = (const int*)(smem + C::kOffIds) + w * (2 * 64);
  auto fetch_window = [&](int win) {
    int pidx = pb + kPagesPerStep * (64 * win + lane) + pw;
    pidx = pidx < pe ? pidx : pb;                      // lanes past the segment read a valid entry
    dma_4b(p.block_tables + bt_row, (unsigned)(4 * pidx), ids_lds + (win & 1) * 256);
  };
  auto read_id = [&](int t) -> int { return ids_ptr[((t >> 6) & 1) * 64 + (t & 63)]; };
  int next_id = 0;   // block-table entry of this wave's next transfer (as read from LDS)

  // this wave's transfer of step t (K or V, by its half)
  auto issue = [&](int t) {
    if (has_page(t)) {
      if ((t & 63) == 32 && t + 32 < n_steps) fetch_window((t >> 6) + 1);
      const int id = min(max(__builtin_amdgcn_readfirstlane(next_id), 0), p.num_pages - 1);
      const uint8_t* base = cache + (uint64_t)id * page_stride;
      const unsigned dst = ring_lds + (t % kStages) * kStageBytes;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dma_1k(base, goff[jj], dst + 1024 * jj);
      next_id = read_id(t + 1);
    }
  };
  auto dma_count = [&](int t) -> int { return has_page(t) ? kDmaPerWave : 0; };
  // K runs one step ahead of V: in the iteration of step t the K waves fetch
  // step t+4 and the V waves step t+3; before its barrier a K wave needs step
  // t+1 and a V wave step t, with the two later steps allowed in flight.
  constexpr int kLead = HF == 0 ? 1 : 0;

  // ---- prologue: step 0's pages, the first page-id window and Q fly
  // together; the rest follow.
  if (n_steps > 0) {
    int id = bt[bt_row + pb + pw];
    id = min(max(id, 0), p.num_pages - 1);
    const uint8_t* base = cache + (uint64_t)id * page_stride;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) dma_1k(base, goff[jj], ring_lds + 1024 * jj);
    fetch_window(0);
  }

  // Q^T operand of the score MFMA for rows 16 (HF + 2 j) + n: k-slots 8g..8g+7
  // of k-step 2u + hh hold dims 16 (4u + g) + 8 hh .. + 8.
  bf16x8 qop[NJA][4][2];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int r = 16 * (HF + 2 * j) + n;
    const int rr = r < rows ? r : 0;                 // padding rows read row 0, zeroed below
    const int i = rr / G, gg = rr - (rr / G) * G;
    const uint16_t* src = p.q + (int64_t)(q0 + i) * p.q_stride_token + (int64_t)(h * G + gg) * p.q_stride_head;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) qop[j][u][hh] = *(const bf16x8*)(src + 16 * (4 * u + g) + 8 * hh);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const bool pad = 16 * (HF + 2 * j) + n >= rows;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) qop[j][u][hh] = pad ? bf16x8{} : qop[j][u][hh];
  }
  // The compiler waits for the Q loads before these statements (they read
  // qop); step 0's transfers and the page-id window, issued earlier, have then
  // landed as well. Issuing the later steps only afterwards keeps the
  // compiler's own waits on Q from draining them.
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) asm volatile("" : "+v"(qop[j][u][hh]) :: "memory");
  // Waves without rows to score loaded no Q, so nothing above waited for the
  // page-id window: wait for it (and step 0's pages) explicitly before use.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  next_id = read_id(1);
  issue(1);
  issue(2);
  if (HF == 0) issue(3);

  // ---- per-lane LDS read addresses (a stage adds a constant offset)
  const unsigned kcol = 16u * ((g ^ n ^ (12 * jpar)) & 15);
  unsigned k_addr[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) k_addr[u] = lds_addr(k_ring) + pw * kPageBytes + 256 * n + (kcol ^ (64u * u));
  // V^T operand: source lane n of group g supplies the 8 dims at +8 (n & 1) of
  // key 4g + ((n >> 1) & 3) in page slot 2 ks + (n >> 3), the k-slot (n >> 1)
  // of group g; ds_read_b64_tr_b8 hands lane n byte k of source lane 2k + n/8.
  const int vpar = (n >> 3) & 1;
  const int vkey = 4 * g + ((n >> 1) & 3);
  const unsigned vsw = 16u * ((vkey ^ (12 * vpar)) & 15);
  unsigned v_addr[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
    v_addr[db] = lds_addr(v_ring) + vpar * kPageBytes + 256 * vkey + 8 * (n & 1) +
                 ((unsigned)(kDimsPerWave * w + 16 * db) ^ vsw);
  const unsigned p_lane = lds_addr(smem + C::kOffP) + 8 * lane;   // + ((buf * RB + rb) * 4 + slot) * 512

  // Raw scores of this wave's page of step t for its scored row blocks: lane
  // (g, n) holds key 4g + r of the page against row 16 (HF + 2 j) + n. In tail
  // steps the page may be missing and keys past a row's causal limit (or the
  // sequence end) are masked to -inf; steady-state steps need neither.
  auto score_step = [&](int t, int kst, f32x4 (&sv)[NJA], auto tail) {
    constexpr bool kTail = decltype(tail)::value;
    if constexpr (NJ > 0) {
      const int pidx = pb + kPagesPerStep * t + pw;
      if (!kTail || has_page(t)) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) sv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const u32x4 raw = *(const u32x4*)(smem + (k_addr[u] - lds_addr(smem)) + kst * kStageBytes);
          const bf16x8 k0 = fp8x8_to_bf16(raw[0], raw[1]);
          const bf16x8 k1 = fp8x8_to_bf16(raw[2], raw[3]);
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            sv[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qop[j][u][0], sv[j], 0, 0, 0);
            sv[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qop[j][u][1], sv[j], 0, 0, 0);
          }
        }
        if (kTail && kPageSize * (pidx + 1) > L - q_len + 1) {
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int i = (16 * (HF + 2 * j) + n) / G;
            const int lim = min(L - 1, L - q_len + i);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = kPageSize * pidx + 4 * g + r;
              sv[j][r] = key <= lim ? sv[j][r] : -__builtin_inff();
            }
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) sv[j] = f32x4{-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
      }
    }
  };

  f32x4 acc[NRB][2];
  float m_ref[NRB];         // reference max (log2 units) of row 16 rb + n, identical in every wave
  float thr[NJA];           // raw-score threshold of scored row block j: (m + slack) / c2
  float l_lane[NJA];        // this lane's share of the row sums of its scored rows
  const float inv_c2 = 1.0f / c2;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    m_ref[rb] = -__builtin_inff();
    acc[rb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[rb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int j = 0; j < NJA; ++j) {
    thr[j] = -__builtin_inff();
    l_lane[j] = 0.f;
  }
  int* const flag = (int*)(smem + C::kOffFlag);   // one word per step, 4 in rotation
  if (tid < 4) flag[tid] = 0;

  // softmax of a step whose raw scores are in sv (stage st): slow-path flag (a
  // raw score above its row's threshold) and P = 2^(s c2 - m) against the
  // current reference max, published to LDS and kept in pv for the row sums.
  f32x4 sv[NJA];
  f16x4 pv[NJA];
  auto softmax = [&](int st) {
    if constexpr (NJ > 0) {
      bool over = false;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) over |= sv[j][r] > thr[j];
      if (__any(over) && lane == 0) flag[st] = 1;
      uint8_t* const pb_ = smem + C::kOffP + (st & 1) * C::kPBytes + 8 * lane;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float mref = m_ref[HF + 2 * j] == -__builtin_inff() ? 0.f : m_ref[HF + 2 * j];
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[j][r] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sv[j][r], c2, -mref));
        *(f16x4*)(pb_ + ((HF + 2 * j) * 4 + pw) * 512) = pv[j];
      }
    }
  };

  // step 0 has landed in every wave (later steps may still fly): score it.
  // The two halves of the work-group order their work differently so that a
  // SIMD's two waves overlap VALU with MFMA work: half 0 does softmax(t),
  // barrier, P V(t), scores(t+1); half 1 does barrier, scores(t+1),
  // softmax(t+1), P V(t) -- so half 1 computes softmax(0) here.
  lds_barrier();
  if (n_steps > 4)
    score_step(0, 0, sv, std::false_type{});
  else
    score_step(0, 0, sv, std::true_type{});
  if (HF == 1) softmax(0);

  // One step: softmax of step t, barrier, P V of step t and the scores of step
  // t+1. Steady-state steps (t + 4 < n_steps) have every page of steps t to
  // t+3 present and need no masking; there the stage index ST = t % 4 is a
  // compile-time constant, so every LDS address is a fixed offset.
  auto step = [&](int t, auto tail, auto stage) {
    constexpr bool kTail = decltype(tail)::value;
    constexpr int kSt = decltype(stage)::value;
    const int st = kSt >= 0 ? kSt : (t % kStages);
    const int buf = st & 1;
    const unsigned p_buf = p_lane + buf * C::kPBytes;

    if (HF == 0) softmax(st);
    if (w == 0 && lane == 0) flag[(st + 2) & 3] = 0;   // last read two steps ago

    // K of step t+1 and V of step t must have landed (two later steps may fly)
    if constexpr (kTail)
      wait_vm(dma_count(t + kLead + 1) + dma_count(t + kLead + 2));
    else
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    lds_barrier();

    const int slow = flag[st];

    // every wave is past step t-1: the K stage of step t and the V stage of
    // step t-1 are free
    issue(t + 3 + kLead);

    // ---- O[:, own dims] += P V over step t's 64 keys (two k-steps of 32).
    // k-slot 8g + e of k-step ks is key 4g + (e & 3) of page slot 2 ks + (e >> 2).
    // The V operands do not depend on the slow path: read them first, so that
    // their latency and the flag's overlap.
    f16x8 vf[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const unsigned a = v_addr[db] + st * kStageBytes + ks * 2 * kPageBytes;
        const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(smem + (a - lds_addr(smem))));
        vf[ks][db] = fp8x8_to_f16((unsigned)raw[0], (unsigned)raw[1]);
      }
      if constexpr (kTail) {
        // keys of pages past the segment (never loaded: stale or uninitialised
        // LDS) and past the sequence end get V = 0, so P = 0 never meets a NaN
        if (t == n_steps - 1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int page = pb + kPagesPerStep * t + 2 * ks + (e >> 2);
            const int key = kPageSize * page + 4 * g + (e & 3);
            const bool keep = page < pe && key < L;
            vf[ks][0][e] = keep ? vf[ks][0][e] : (_Float16)0.f;
            vf[ks][1][e] = keep ? vf[ks][1][e] : (_Float16)0.f;
          }
        }
      }
    }

    if (slow) {
      // slow path (uniform over the work-group): publish per-lane maxima of the
      // raw scores, move m where a row's step maximum passes its threshold,
      // rescale, recompute and republish P
      float* mx_buf = (float*)(smem + C::kOffMx);        // [page slot][group][row]
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        mx_buf[(pw * 4 + g) * C::kRows + 16 * (HF + 2 * j) + n] =
            fmaxf(fmaxf(sv[j][0], sv[j][1]), fmaxf(sv[j][2], sv[j][3]));
      lds_barrier();
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        float M = mx_buf[16 * rb + n];
#pragma unroll
        for (int v = 1; v < kPagesPerStep * 4; ++v) M = fmaxf(M, mx_buf[v * C::kRows + 16 * rb + n]);
        const float th = (m_ref[rb] + kLazySlack) * inv_c2;
        float alpha = 1.f;
        if (M > th) {
          const float m_new = M * c2;
          alpha = __builtin_amdgcn_exp2f(m_ref[rb] - m_new);   // 0 when m was -inf
          m_ref[rb] = m_new;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = __shfl(alpha, 4 * g + r, 64);     // lane 4g+r holds row 4g+r
          acc[rb][0][r] *= a;
          acc[rb][1][r] *= a;
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if (rb == HF + 2 * j) {
            l_lane[j] *= alpha;
            thr[j] = (m_ref[rb] + kLazySlack) * inv_c2;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float mref = m_ref[HF + 2 * j] == -__builtin_inff() ? 0.f : m_ref[HF + 2 * j];
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[j][r] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sv[j][r], c2, -mref));
        *(f16x4*)(smem + (p_buf - lds_addr(smem)) + ((HF + 2 * j) * 4 + pw) * 512) = pv[j];
      }
      lds_barrier();   // new P visible; every wave is done reading the maxima
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const f16x2 lo = {pv[j][0], pv[j][1]}, hi = {pv[j][2], pv[j][3]};
      const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
      l_lane[j] = __builtin_amdgcn_fdot2(hi, one, __builtin_amdgcn_fdot2(lo, one, l_lane[j], false), false);
    }

    auto pv_mfma = [&]() {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const uint8_t* pr = smem + (p_buf - lds_addr(smem)) + (rb * 4 + 2 * ks) * 512;
          const f16x4 lo = *(const f16x4*)pr;
          const f16x4 hi = *(const f16x4*)(pr + 512);
          const f16x8 pa = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc[rb][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vf[ks][0], acc[rb][0], 0, 0, 0);
          acc[rb][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vf[ks][1], acc[rb][1], 0, 0, 0);
        }
      }
    };
    // ---- scores of step t+1 (its K landed before the barrier above)
    auto scores_next = [&]() {
      const int kst = (st + 1) & 3;
      if (kTail || t + 5 >= n_steps)
        score_step(t + 1, kst, sv, std::true_type{});
      else
        score_step(t + 1, kst, sv, std::false_type{});
    };
    if constexpr (HF == 0) {
      pv_mfma();
      scores_next();
    } else {
      scores_next();
      if (!kTail || t + 1 < n_steps) softmax((st + 1) & 3);
      pv_mfma();
    }
  };

  int t = 0;
  for (; t + 7 < n_steps; t += 4) {
    step(t, std::false_type{}, std::integral_constant<int, 0>{});
    step(t + 1, std::false_type{}, std::integral_constant<int, 1>{});
    step(t + 2, std::false_type{}, std::integral_constant<int, 2>{});
    step(t + 3, std::false_type{}, std::integral_constant<int, 3>{});
  }
  for (; t < n_steps; ++t) step(t, std::true_type{}, std::integral_constant<int, -1>{});

  // ---- partials of this segment: m is identical in every wave; l sums the
  // page slots' key subsets in a fixed order; each wave writes its own dims.
  __syncthreads();   // all transfers have landed (last wait was vmcnt(0)); LDS is free
  float* lsum = (float*)smem;                     // [page slot][row]
  float* mrow = lsum + kPagesPerStep * C::kRows;  // [row]
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    float l = l_lane[j];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (g == 0) lsum[pw * C::kRows + 16 * (HF + 2 * j) + n] = l;
  }
  if (w == 0 && g == 0) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) mrow[16 * rb + n] = m_ref[rb];
  }
  __syncthreads();

  const int T = p.total_q, Hq = p.num_q_heads;
  if (tid < rows) {
    const int row = tid;
    float l = lsum[row];
#pragma unroll
    for (int v = 1; v < kPagesPerStep; ++v) l += lsum[v * C::kRows + row];
    const int i = row / G, gg = row - (row / G) * G;
    float* dst = p.ws_ml + (((int64_t)geo.seg * T + q0 + i) * Hq + h * G + gg) * 2;
    dst[0] = mrow[row];
    dst[1] = l;
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * rb + 4 * g + r;
      if (row < rows) {
        const int i = row / G, gg = row - (row / G) * G;
        float* dst = p.ws_acc + (((int64_t)geo.seg * T + q0 + i) * Hq + h * G + gg) * kHeadDim +
                     kDimsPerWave * w + n;
        dst[0] = acc[rb][0][r];
        dst[16] = acc[rb][1][r];
      }
    }
}

template <int G, int NRB>
__device__ __forceinline__ void verify_segment(const MainParams& p, const Geo& geo, uint8_t* smem) {
  if (threadIdx.x < 256)
    wave_main<G, NRB, 0>(p, geo, smem);
  else
    wave_main<G, NRB, 1>(p, geo, smem);
}

template <int G>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
splitkv_main_kernel(MainParams p) {
  using C = Cfg<G>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kLdsBytes];

  const const_i32* cu = (const const_i32*)p.cu_seqlens_q;
  const const_i32* sl = (const const_i32*)p.seq_lens;
  Geo geo;
  geo.seg = blockIdx.x;
  geo.b = blockIdx.y;
  geo.h = blockIdx.z;
  // out-of-contract values are clamped so that every access stays in its buffer
  geo.q0 = cu[geo.b];
  int q_len = cu[geo.b + 1] - geo.q0;
  if (geo.q0 < 0 || geo.q0 >= p.total_q) q_len = 0;
  q_len = min(max(q_len, 0), min(kMaxQLen, p.total_q - max(geo.q0, 0)));
  if (q_len <= 0) return;
  geo.q_len = q_len;
  geo.L = min(max(sl[geo.b], 0), p.max_pages_per_seq * kPageSize);
  const int pages = (geo.L + kPageSize - 1) / kPageSize;
  const int chunk = (pages + p.num_segments - 1) / p.num_segments;
  geo.pb = min(geo.seg * chunk, pages);
  geo.pe = min(geo.pb + chunk, pages);
  geo.rows = G * q_len;
  geo.n_steps = (geo.pe - geo.pb + kPagesPerStep - 1) / kPagesPerStep;
  geo.c2 = *(const const_f32*)p.k_descale * p.score_scale_log2;

  const int nrb = (geo.rows + 15) >> 4;
  if constexpr (G == 16) {
    switch (nrb) {
      case 1: verify_segment<16, 1>(p, geo, smem); break;
      case 2: verify_segment<16, 2>(p, geo, smem); break;
      case 3: verify_segment<16, 3>(p, geo, smem); break;
      default: verify_segment<16, 4>(p, geo, smem); break;
    }
  } else {
    if (nrb == 1)
      verify_segment<8, 1>(p, geo, smem);
    else
      verify_segment<8, 2>(p, geo, smem);
  }
}

}  // namespace

hipError_t launch_splitkv_main(const MainParams& p, int group, hipStream_t stream) {
  const dim3 grid(p.num_segments, p.num_seqs, p.num_kv_heads);
  if (group == 16) {
    hipLaunchKernelGGL(splitkv_main_kernel<16>, grid, dim3(kThreads), 0, stream, p);
  } else if (group == 8) {
    hipLaunchKernelGGL(splitkv_main_kernel<8>, grid, dim3(kThreads), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pfkv
