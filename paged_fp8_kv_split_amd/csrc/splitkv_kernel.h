// Split-KV main kernel for verify attention over a paged fp8 KV cache (gfx950):
// the kernel templates, instantiated per arithmetic mode by splitkv_main.hip,
// splitkv_main_fp8p.hip and splitkv_main_fp8.hip (compiled in parallel).
//
// What it computes follows aiter PR #5190 ("gfx950 assembly MTP-verify attention
// for head_dim 256 fp8 paged KV"), sections Modifications and Kernel notes: one
// work-group per (KV segment, sequence, KV head), partial softmax statistics per
// segment to a workspace, empty segments written neutrally, descales read from
// device pointers. In-kernel q_len 1..4 follows SGLang PR #37465, Modifications.
// The decomposition is this library's own:
//
// * 8 waves per work-group (one work-group per CU), in two roles. A step covers
//   4 pages (64 keys); page slot j of a step belongs to waves j and j + 4, which
//   share a SIMD.
//   - Score wave j (waves 0-3) streams the K block of its page HBM -> LDS,
//     converts it once and scores its 16 keys against all G * q_len (<= 64)
//     stacked query rows, with Q held in registers; it then forms the softmax
//     numerators P of those keys.
//   - P.V wave j (waves 4-7) streams the V block of its page and accumulates
//     O[:, 64 j .. 64 j + 63] += P V over all 64 keys of a step.
//   The two waves of a SIMD are in different phases of their work, so one
//   feeds the matrix core while the other converts or exponentiates.
// * One work-group barrier per phase. In phase t (between barriers t and t + 1)
//   the score waves form P of step t - 1 and compute the scores of step t; the
//   P.V waves accumulate step t - 2. A step's scores stay in registers across
//   one barrier, so every score wave knows, before forming P, whether any of
//   them saw a row pass its threshold (below).
// * K and V take different paths to their LDS rings (4 stages each), so that
//   the two kinds of read share the memory system: K pages move with
//   global_load_lds_dwordx4 (1 KiB contiguous per instruction, HBM -> LDS with
//   no registers) issued by the score waves from inline asm, three steps ahead
//   of their use, with explicit vmcnt waits; V pages are read by the P.V waves
//   with 16-byte vector loads into registers one phase before they go to LDS.
//   On random 4 KiB pages vector loads alone stream about 6.9 TB/s, LDS DMA
//   alone about 6.1 TB/s (and unevenly across the XCDs), a half-and-half mix
//   about 6.8 TB/s; the mix also keeps the P.V waves' registers within budget.
//   Page ids are staged in LDS windows by 4-byte LDS transfers.
// * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: K converts exactly from e4m3fn to
//   bf16 (v_cvt_scalef32_pk_bf16_fp8, scale 1), Q stays bf16. The score layout
//   puts one query row per lane column.
// * Online softmax in the log2 domain with a lazy reference max m per row: m
//   moves only when a row's running max exceeds it by more than 8, so
//   P = 2^(s - m) <= 2^8 fits fp16 and the accumulator is rescaled rarely. A
//   score wave that sees a row pass m + 8 raises its flag; in the next phase, if
//   any flag is up, all waves take one extra barrier while the score waves
//   exchange the step's row maxima, move m where a row's maximum passed its
//   threshold and publish the rescale factors for the P.V waves. Rows that did
//   not pass keep m and get bit-identical P, so each row's arithmetic depends
//   only on that row.
// * P is rounded to fp16 once; the same values feed the row sum l and P V.
// * O += P V on v_mfma_f32_16x16x32_f16. V's transposed operand comes from
//   ds_read_b64_tr_b8 and converts exactly to fp16.
// * Epilogue (16-bit arithmetic): o = O / l leaves the P.V waves' registers
//   through a transpose inside groups of lanes (DPP swaps) and goes straight
//   to memory, each row as runs of contiguous 8-byte device-scope stores
//   (written through, see partial_store).
// * The opt-in fp8 modes (splitkv_main_fp8p.hip, splitkv_main_fp8.hip) round P
//   to e4m3 under a power-of-two scale per (row, 32-key block), which the
//   scaled fp8 MFMA takes in its A-scale operand, and follow each row's
//   running maximum exactly (no slack), so that a row's largest weight is
//   exact in e4m3. With e4m3 Q as well, Q is quantised per 32 dims and its
//   scales ride in the score MFMA's B-scale operand.
// * Work-group ids are renumbered so that each XCD runs a contiguous run of
//   them (a whole sequence's segments where the grid allows), with the
//   work-groups that read the same pages (the two halves of 32 query heads per
//   KV head, the two query blocks of an 8-token draft) next to each other, so
//   that the second read of a page comes from that XCD's L2.
#pragma once

#include <type_traits>

#include "pfkv_internal.h"
#include "segment_merge.h"

namespace pfkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(4))) const int32_t const_i32;
typedef __attribute__((address_space(4))) const float const_f32;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kPagesPerStep = 4;                       // one page slot per score wave
constexpr int kStages = 4;                             // depth of the K ring and of the V ring (steps)
constexpr float kLazySlack = 8.0f;                     // log2 units
// arithmetic modes (the C ABI's precision values)
constexpr int kMode16 = 0;      // bf16 Q x bf16 K, fp16 P x fp16 V
constexpr int kModeFp8P = 1;    // bf16 Q x bf16 K, e4m3 P x e4m3 V
constexpr int kModeFp8QP = 2;   // e4m3 Q x e4m3 K, e4m3 P x e4m3 V

// Sizes that follow from the head dim D (256, or 128)
template <int D>
struct Dim {
  static_assert(D == 256 || D == 128, "head dims 256 and 128");
  static constexpr int kPageBytes = kPageSize * D;          // one (16-token block, head) of K or V: 4 / 2 KiB
  static constexpr int kStageBytes = kPagesPerStep * kPageBytes;   // K (or V) of one step: 16 / 8 KiB
  static constexpr int kDmaPerWave = kPageBytes / 1024;     // 1 KiB transfers per wave and step: 4 / 2
  static constexpr int kVDims = D / kPagesPerStep;          // output dims per P.V wave: 64 / 32
  static constexpr int kChunks = D / 16;                    // 16-byte chunks of an fp8 K/V row
  static constexpr int kRowsPerKiB = 1024 / D;              // K/V rows per 1 KiB transfer
  static constexpr int kKU = D / 64;                        // 16-byte K chunks a score lane reads per step
  static constexpr int kQRowBytes = 2 * D;                  // a bf16 Q row
  static constexpr int kQRowsPerKiB = 1024 / kQRowBytes;
  // LDS chunk swizzle of key row k in a page slot of parity j: within 16 lanes
  // that read one chunk of 16 rows (K rows) or 8 bytes of 8 rows in two slots
  // (V transposed), every 16-byte (8-byte) slot of a 256-byte bank line is hit once
  static __device__ __forceinline__ int sw(int k, int j) {
    return D == 256 ? ((k ^ (12 * j)) & 15) : (((k >> 1) ^ (4 * j)) & 7);
  }
};

template <int G, int D>
struct Cfg {
  // 16-row MFMA blocks (all rows); at least two, so that the 32-row tiles of
  // the fp8 P.V path stay inside the P, maximum and rescale buffers
  static constexpr int kRowBlocks = G * kMaxQLen / 16 < 2 ? 2 : (G * kMaxQLen / 16 > kMaxRows / 16 ? kMaxRows / 16 : G * kMaxQLen / 16);
  static constexpr int kRows = kRowBlocks * 16;
  static constexpr int kPBytes = kRowBlocks * 2 * 64 * 16;         // fp16 P of a step: [rb][k-step][lane] x 16 B
  static constexpr int kOffP = 0;                                  // two P buffers
  // fp8 P uses the first kRows * 64 bytes of a P buffer; behind them, in the
  // same buffer, each page slot's row maxima of the step ([row][slot] fp32)
  // and the E8M0 scales of P's two 32-key blocks ([row][block] bytes)
  static constexpr int kP8Xmax = kRows * 64;
  static constexpr int kP8Scale = kP8Xmax + kRows * kPagesPerStep * 4;
  static_assert(kP8Scale + kRows * 2 <= kPBytes, "fp8 P buffer");
  static constexpr int kOffMx = kOffP + 2 * kPBytes;               // step row maxima [row][slot] (slow path)
  static constexpr int kOffAlpha = kOffMx + kRows * kPagesPerStep * 4;   // two [row] rescale-factor buffers
  static constexpr int kOffFlag = kOffAlpha + 2 * kRows * 4;       // two flag words, byte j from score wave j
  static constexpr int kOffIds = kOffFlag + 64;                    // page-id windows [wave][2][64]
  static constexpr int kOffStage = (kOffIds + kWaves * 2 * 64 * 4 + 1023) & ~1023;   // K ring, then V ring
  static constexpr int kLdsBytes = kOffStage + 2 * kStages * Dim<D>::kStageBytes;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
  static constexpr int kOffObuf = 2048;                             // epilogue: fp16 o rows [row][D]
  static_assert((kPagesPerStep + 1) * kRows * 4 <= kOffObuf, "epilogue row sums and sink terms");
  static_assert(kOffObuf + kRows * D * 2 <= kLdsBytes, "epilogue o staging");
  // Q is staged in V ring stages 2-3 (unused before the first barrier)
  static_assert(kRows * Dim<D>::kQRowBytes <= 2 * Dim<D>::kStageBytes, "Q staging");
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

// As dma_1k with a 64-bit source address per lane (lane i moves addr_i).
__device__ __forceinline__ void dma_1k_addr(const uint8_t* addr, unsigned lds) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(addr), "s"(lds)
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
// flight (rounded down to an even count, at most 16). Inside the main loop the
// only such operations are the page transfers (kDmaPerWave 1 KiB transfers per
// stream and step) and the page-id window refills, which are older than the
// transfers they precede, so extra refills only make a wait stricter.
__device__ __forceinline__ void wait_vm(int pending) {
  if (pending >= 16)
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (pending >= 14)
    asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
  else if (pending >= 12)
    asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else if (pending >= 10)
    asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
  else if (pending >= 8)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (pending >= 6)
    asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else if (pending >= 4)
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if (pending >= 2)
    asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
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
// A store of the segment partials: a device-scope store, which completes only
// once the value has reached the device's coherence point. The partials are
// read once, by the reduce or by the in-launch merge (on other XCDs, with no
// cache maintenance); written through as they are produced, they leave no
// dirty L2 lines for the end of the launch to write back (0.5-0.7 us per call
// faster than streaming stores at 16 x 35000, GQA 16 and 8, decode and 4 x
// 35000, measured interleaved; the same bits).
template <typename T>
__device__ __forceinline__ void partial_store(T v, T* dst) {
  if constexpr (sizeof(T) == 8)
    __hip_atomic_store((uint64_t*)dst, __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Geo {
  int seg, b, h;     // h: this work-group's group of G query heads (query heads h G .. h G + G - 1)
  int hkv;           // the KV head those query heads read
  int q0, q_len, L, pb, pe, rows, n_steps;   // q0, q_len: this work-group's query tokens
  int qoff;          // KV position of the work-group's first query token
  int win;           // left window (clamped to L), -1 when none
  float c2;          // k_descale * softmax_scale * log2(e): raw score -> log2 units
};

// Table entries behind one transfer: with cache pages of 16 or more tokens, one
// entry, uniform over the wave; with one-token pages, this lane's entries for
// the rows it moves (token R jj + r of the 16-token block in part jj, R rows per
// 1 KiB part, r = lane / (D / 16)).
template <bool TOK, int D>
struct PageIds {
  using type = int;
};
template <>
struct PageIds<true, 256> {
  using type = i32x4;
};
template <>
struct PageIds<true, 128> {
  using type = i32x2;
};

// One wave's stream of one page slot (K or V blocks) into its LDS ring: the
// 16-token block of page slot `slot` of step t goes to ring stage t % 4.
// TOK: the cache has one-token pages, so each key row of a block is gathered
// from its own page (a 1 KiB transfer then covers 1024 / D rows).
template <bool TOK, int D>
struct PageStream {
  using Dm = Dim<D>;
  using Ids = typename PageIds<TOK, D>::type;
  static constexpr int kParts = Dm::kDmaPerWave;
  const uint8_t* cache;
  const int32_t* bt_row;      // this sequence's block-table row
  uint64_t page_stride;       // bytes between 16-token blocks (TOK: between tokens) of the cache
  int pshift;                 // log2(page_stride) when it is a power of two, else -1
  unsigned goff[kParts];      // per-lane source offsets inside a block (TOK: inside a token's page)
  unsigned lane_lds;          // vector transport: slot * block bytes + 16 lane (the LDS-DMA lane layout)
  u32x4 buf[kParts];          // vector transport: the block in flight between load() and store()
  unsigned ring;              // LDS address of this slot in stage 0
  unsigned ids_lds;           // this wave's two page-id windows
  const int* ids;
  int pb, pe, slot, n_steps, num_pages, L, lane_ids;
  int rlog;                   // log2(cache page size / 16)
  Ids next_id;                // table entries of the next transfer (read from LDS)

  // In part jj of a block, lane (r, c) = (lane / (D / 16), lane % (D / 16))
  // moves 16 bytes of key row k = R jj + r. In LDS, the 16-byte chunk at
  // position c of key row k (page slot parity j) holds dim chunk c ^ sw(k, j)
  // (Dim::sw): K row reads and V transposed reads are then free of bank conflicts.
  __device__ void init(const MainParams& p, const Geo& geo, uint8_t* smem, int wave, int slot_, int lane,
                       const uint8_t* cache_, unsigned ring_stage0, int off_ids) {
    cache = cache_;
    bt_row = p.block_tables + (int64_t)geo.b * p.block_table_stride;
    page_stride = (uint64_t)(TOK ? 1 : kPageSize) * p.num_kv_heads * D;
    pshift = (page_stride & (page_stride - 1)) == 0 ? __builtin_ctzll(page_stride) : -1;
    slot = slot_;
    pb = geo.pb;
    pe = geo.pe;
    n_steps = geo.n_steps;
    num_pages = p.num_pages;
    L = geo.L;
    rlog = p.page_ratio_log2;
    const int r = lane / Dm::kChunks, c = lane % Dm::kChunks, jpar = slot & 1;
    lane_ids = r * kParts;
#pragma unroll
    for (int jj = 0; jj < kParts; ++jj) {
      const int k = Dm::kRowsPerKiB * jj + r;
      goff[jj] = (unsigned)(((TOK ? 0 : k * p.num_kv_heads) + geo.hkv) * D + 16 * (c ^ Dm::sw(k, jpar)));
      buf[jj] = u32x4{0u, 0u, 0u, 0u};
    }
    ring = ring_stage0 + slot * Dm::kPageBytes;
    lane_lds = (unsigned)(slot * Dm::kPageBytes + 16 * lane);
    ids_lds = lds_addr(smem + off_ids) + wave * (2 * 64 * 4);
    ids = (const int*)(smem + off_ids) + wave * (2 * 64);
    next_id = Ids{};
  }
  __device__ bool has(int t) const { return t < n_steps && pb + kPagesPerStep * t + slot < pe; }
  __device__ int count(int t) const { return has(t) ? kParts : 0; }
  // Pages here are 16-token blocks. A cache page of 16 R tokens (R = 2^rlog)
  // holds R of them back to back in NHD order, so 16-token block pidx is part
  // pidx mod R of cache page block_tables[pidx / R], at 16-token index
  // block_tables[pidx / R] R + pidx mod R.
  // Windows (two slots, w even / odd): with 16 R-token pages entry k of window
  // w is the table entry of step 64 w + k; with one-token pages, window w
  // covers steps 4 w .. 4 w + 3 and entry 16 s + kParts r + jj holds token
  // R jj + r of step 4 w + s (a lane's entries are adjacent). Tokens past the
  // sequence end read the last token's entry, so no unused entry is read.
  __device__ void fetch_window(int win, int lane) {
    if constexpr (TOK) {
      const int s = lane >> 4, r = (lane & 15) / kParts, jj = lane % kParts;
      int pidx = pb + kPagesPerStep * (4 * win + s) + slot;
      pidx = pidx < pe ? pidx : pb;
      const int tok = min(kPageSize * pidx + Dm::kRowsPerKiB * jj + r, L - 1);
      dma_4b(bt_row, (unsigned)(4 * tok), ids_lds + (win & 1) * 256);
    } else {
      int pidx = pb + kPagesPerStep * (64 * win + lane) + slot;
      pidx = pidx < pe ? pidx : pb;                    // lanes past the segment read a valid entry
      dma_4b(bt_row, (unsigned)(4 * (pidx >> rlog)), ids_lds + (win & 1) * 256);
    }
  }
  // the next window is fetched at the step that starts (TOK) or half uses the
  // current one; it lands at least three phases before its first use
  __device__ void refill(int t, int lane) {
    if constexpr (TOK) {
      if ((t & 3) == 0 && t + 4 < n_steps) fetch_window((t >> 2) + 1, lane);
    } else {
      if ((t & 63) == 32 && t + 32 < n_steps) fetch_window((t >> 6) + 1, lane);
    }
  }
  // 16-token block of step t from its table entry (clamped into the cache first)
  __device__ int resolve(int t, int entry) const {
    const int id = min(max(entry, 0), num_pages - 1);
    return (id << rlog) + ((pb + kPagesPerStep * t + slot) & ((1 << rlog) - 1));
  }
  __device__ Ids read_id(int t) const {
    if constexpr (TOK)
      return *(const Ids*)(ids + ((t >> 2) & 1) * 64 + (t & 3) * 16 + lane_ids);
    else
      return ids[((t >> 6) & 1) * 64 + (t & 63)];
  }
  __device__ int first_id(int t) const {            // scalar load, before the windows land
    return ((const const_i32*)bt_row)[(has(t) ? pb + kPagesPerStep * t + slot : pb) >> rlog];
  }
  // first byte of 16-token block (TOK: token) blk >= 0: a shift where the stride
  // is a power of two (one KV head: 4 KiB), a 64-bit product otherwise
  __device__ const uint8_t* block_base(int blk) const {
    return pshift >= 0 ? cache + ((uint64_t)(unsigned)blk << pshift) : cache + (uint64_t)(unsigned)blk * page_stride;
  }
  // TOK: source of part jj (this lane's token R jj + r), its page clamped into the cache
  __device__ const uint8_t* token_src(const Ids& e, int jj) const {
    const int id = min(max((int)e[jj], 0), num_pages - 1);
    return cache + (uint64_t)id * page_stride + goff[jj];
  }
  __device__ void put(int t, const Ids& entry) {
    const unsigned dst = ring + (t % kStages) * Dm::kStageBytes;
    if constexpr (TOK) {
#pragma unroll
      for (int jj = 0; jj < kParts; ++jj) dma_1k_addr(token_src(entry, jj), dst + 1024 * jj);
    } else {
      const uint8_t* base = block_base(resolve(t, entry));
#pragma unroll
      for (int jj = 0; jj < kParts; ++jj) dma_1k(base, goff[jj], dst + 1024 * jj);
    }
  }
  // The transfer of step t in kParts parts that the caller spreads over its
  // work: begin() resolves the page (and refills the window when due),
  // part(q, jj) moves the jj-th KiB. FULL: the caller knows that step t
  // exists and has this page slot (steady-state phases), so nothing is tested.
  struct Pending {
    const uint8_t* base;
    unsigned dst;
    bool on;
    Ids e;
  };
  template <bool FULL = false>
  __device__ Pending begin(int t, int lane) {
    Pending q{nullptr, 0u, FULL || has(t), Ids{}};
    if (q.on) {
      refill(t, lane);
      // one-token pages: the entries (four per lane) are read from their
      // window here rather than a step ahead, to keep registers free
      if constexpr (TOK)
        q.e = read_id(t);
      else
        q.base = block_base(resolve(t, __builtin_amdgcn_readfirstlane(next_id)));
      q.dst = ring + (t % kStages) * Dm::kStageBytes;
      if constexpr (!TOK) next_id = read_id(t + 1);
    }
    return q;
  }
  __device__ void part(const Pending& q, int jj) const {
    if (q.on) {
      if constexpr (TOK)
        dma_1k_addr(token_src(q.e, jj), q.dst + 1024 * jj);
      else
        dma_1k(q.base, goff[jj], q.dst + 1024 * jj);
    }
  }
  // Vector transport: load() brings the block of step t (begin()'s pending
  // transfer) into registers with 16-byte loads, lane i taking the 16 bytes
  // that an LDS-DMA transfer would place at 16 i (the swizzle lives in the
  // source offsets); store() writes them to the ring stage of step t. Between
  // the two the block is in flight while the wave computes.
  __device__ void load(const Pending& q, u32x4 (&dst)[kParts]) const {
    if (q.on) {
#pragma unroll
      for (int jj = 0; jj < kParts; ++jj) {
        if constexpr (TOK)
          dst[jj] = __builtin_nontemporal_load((const u32x4*)token_src(q.e, jj));
        else
          dst[jj] = __builtin_nontemporal_load((const u32x4*)(q.base + goff[jj]));
      }
    }
  }
  __device__ void load(const Pending& q) { load(q, buf); }
  __device__ void store(int t, uint8_t* ring_base, const u32x4 (&src)[kParts]) const {
    uint8_t* dst = ring_base + lane_lds + (t % kStages) * Dm::kStageBytes;
#pragma unroll
    for (int jj = 0; jj < kParts; ++jj) *(u32x4*)(dst + 1024 * jj) = src[jj];
  }
  __device__ void store(int t, uint8_t* ring_base) const { store(t, ring_base, buf); }
};

// Stores the staged 16-bit rows ([row][D] in LDS) of the work-group, all
// 512 threads: fp16 o rows to the workspace (row stride kHeadDim) with 16-byte
// streaming stores, or, with a single segment, the final bf16 rows to out with
// 8-byte stores (out rows are 8-byte aligned).
template <int G, int D, bool RM>
__device__ __forceinline__ void store_rows(const MainParams& p, const Geo& geo, const uint8_t* obuf) {
  constexpr int kQuads = D / 4, kOcts = D / 8;   // 8-byte and 16-byte pieces of a row
  if (p.direct) {
    for (int idx = threadIdx.x; idx < geo.rows * kQuads; idx += kThreads) {
      const int row = idx / kQuads, c = idx % kQuads;
      const int i = row / G, gg = row - (row / G) * G;
      uint16_t* dst = p.out + (int64_t)(geo.q0 + i) * p.out_stride_token + (int64_t)(geo.h * G + gg) * p.out_stride_head + 4 * c;
      *(uint2*)dst = *(const uint2*)(obuf + row * (2 * D) + 8 * c);
    }
    return;
  }
  const int T = p.total_q, Hq = p.num_q_heads;
  for (int idx = threadIdx.x; idx < geo.rows * kOcts; idx += kThreads) {
    const int row = idx / kOcts, c = idx % kOcts;
    const int i = row / G, gg = row - (row / G) * G;
    uint16_t* dst = p.ws_o + ws_slot_tq<RM>(geo.q0, i, geo.h * G, gg, geo.seg, T, Hq, p.num_segments) * kHeadDim + 8 * c;
    __builtin_nontemporal_store(*(const u32x4*)(obuf + row * (2 * D) + 16 * c), (u32x4*)dst);
  }
}

// fp8 (e4m3fn) MFMAs with E8M0 block scales (127 = 2^0), one per 32 k-elements.
// Which lane's scale covers which bytes (measured on gfx950): on 16x16x128 the
// scale of lane n + 16 j covers bytes 16 (j >> 1) .. + 15 of lanes n + 16 g,
// g in {2 (j & 1), 2 (j & 1) + 1}; on 32x32x64 the scale of lane c + 32 j
// covers bytes 16 j .. + 15 of lanes c and c + 32. A operand (K) unscaled,
// B operand (Q) scaled:
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(const i32x8& a, const i32x8& b, const f32x4& c, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, scale_b);
}
// A operand (P) scaled, B operand (V) unscaled:
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(const i32x8& a, const i32x8& b, const f32x16& c, int scale_a) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, 127);
}
// max of v over lanes l, l ^ 16, l ^ 32 and l ^ 48 (one position in each of
// the four 16-lane rows) by the row-swap permutes: each swap hands a lane its
// partner row's value in one of its two results and keeps its own in the
// other, with no LDS round trip
__device__ __forceinline__ float rows_max(float v) {
  const u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(v, fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1])));
  const u32x2 b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(v, fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1])));
}

__device__ __forceinline__ i32x8 cat8(const u32x4& lo, const u32x4& hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Score wave w (page slot w): K stream, S^T = K Q^T for all NRB row blocks,
// lazy softmax, P to LDS, row sums; writes m and l of the segment. With F8,
// Q is quantised to e4m3 with a power-of-two scale per 32 dims and S^T runs on
// the scaled fp8 MFMA; with F8P, P is rounded to e4m3 with a power-of-two
// scale per (row, 32 keys).
template <int G, int NRB, int MODE, bool TOK, int D, bool RM>
__device__ __forceinline__ void score_wave(const MainParams& p, const Geo& geo, uint8_t* smem) {
  using C = Cfg<G, D>;
  using Dm = Dim<D>;
  constexpr int kPageBytes = Dm::kPageBytes, kStageBytes = Dm::kStageBytes, kKU = Dm::kKU;
  constexpr bool F8 = MODE == kModeFp8QP;    // e4m3 Q, S^T on the fp8 MFMA
  constexpr bool F8P = MODE != kMode16;      // e4m3 P
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int h = geo.h, q0 = geo.q0, q_len = geo.q_len, L = geo.L, pb = geo.pb;
  const int rows = geo.rows, n_steps = geo.n_steps;
  const float c2 = geo.c2;
  // left window: the first step of a segment that starts below the largest
  // lower key bound (that of the last query row) masks keys from below
  const int win = geo.win;
  const int qoff = geo.qoff;
  const bool win_head = win >= 0 && kPageSize * pb < qoff + q_len - 1 - win;
  const bool capped = p.softcap > 0.f;
  uint8_t* const k_ring = smem + C::kOffStage;

  PageStream<TOK, D> ks;   // K of page slot w: streamed by LDS DMA and read here
  ks.init(p, geo, smem, w, w, lane, p.k_cache, lds_addr(k_ring), C::kOffIds);

  // ---- prologue. Q goes HBM -> LDS (V ring stages 2-3, not used before
  // phase 1) by page-style transfers, 16-byte chunk c of row r at position
  // c ^ (r & 15), score wave w moving rows 16w..16w+15; then the K stream's
  // first three steps, while the P.V waves start the V stream. Q moves to
  // registers after the first barrier.
  constexpr int kQRow = Dm::kQRowBytes, kQRpk = Dm::kQRowsPerKiB, kQLanes = 64 / kQRpk;
  uint8_t* const q_stage = smem + C::kOffStage + (kStages + 2) * kStageBytes;
  if (n_steps > 0) {
    if (w < NRB) {
      const uint8_t* q_base = (const uint8_t*)(p.q + (int64_t)q0 * p.q_stride_token + (int64_t)h * G * p.q_stride_head);
#pragma unroll
      for (int k = 0; k < 16 / kQRpk; ++k) {
        const int r = 16 * w + kQRpk * k + lane / kQLanes;
        const int rr = r < rows ? r : 0;            // padding rows read row 0, zeroed in registers
        const int i = rr / G, gg = rr - (rr / G) * G;
        const unsigned voff = (unsigned)((i * p.q_stride_token + gg * p.q_stride_head) * 2) + 16u * ((lane % kQLanes) ^ (r & 15));
        dma_1k(q_base, voff, lds_addr(q_stage) + (16 * w + kQRpk * k) * kQRow);
      }
    }
    ks.fetch_window(0, lane);
    if constexpr (TOK) {
      if (4 < n_steps) ks.fetch_window(1, lane);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      // one step's entries at a time (four per lane), to keep registers free
      if (ks.has(0)) ks.put(0, ks.read_id(0));
      if (ks.has(1)) ks.put(1, ks.read_id(1));
      if (ks.has(2)) ks.put(2, ks.read_id(2));
    } else {
      const int id0 = ks.first_id(0), id1 = ks.first_id(1), id2 = ks.first_id(2);
      if (ks.has(0)) ks.put(0, id0);
      if (ks.has(1)) ks.put(1, id1);
      if (ks.has(2)) ks.put(2, id2);
    }
    wait_vm(ks.count(1) + ks.count(2));   // Q, the windows and K of step 0
    ks.next_id = ks.read_id(3);
  }
  // Q^T operand of the score MFMA for row 16 rb + n: k-slots 8g..8g+7 of
  // k-step 2u + hh hold dims 16 (4u + g) + 8 hh .. + 8 (chunk 8u + 2g + hh).
  // With F8 (q8): byte b of k-step ks holds dim 128 ks + 64 (b >> 4) + 16 g +
  // (b & 15), so that the MFMA's scale block j (bytes 16 (j >> 1) .. + 15 of
  // lanes 2 (j & 1) and 2 (j & 1) + 1) is the 32 consecutive dims
  // 128 ks + 32 j .. + 31. Each block is in e4m3 under its own power-of-two
  // scale, which lane group j supplies in q8sc. The scales ride in the MFMA, so
  // the scores come out in the same units as the 16-bit path's.
  constexpr int kKS8 = D / 128;   // k-steps of the fp8 score MFMA
  bf16x8 qop[F8 ? 1 : NRB][kKU][2];
  i32x8 q8[F8 ? NRB : 1][kKS8];
  int q8sc[F8 ? NRB : 1][kKS8];
  const float inv_c2 = 1.0f / c2;
  float cap_a = 0.f, cap_b = 0.f;   // soft-cap in raw-score units: s -> cap_b tanh(cap_a s)
  auto load_q = [&]() {
    if constexpr (F8) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int r = 16 * rb + n;
        const bool pad = r >= rows;
#pragma unroll
        for (int ks = 0; ks < kKS8; ++ks) {
          bf16x8 x[4];
          float amax[2] = {0.f, 0.f};   // bytes 0..15 and 16..31 of this lane
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            const int pos = (16 * ks + 8 * (c4 >> 1) + 2 * g + (c4 & 1)) ^ n;   // dims 8 pos .. + 7
            const bf16x8 v = *(const bf16x8*)(q_stage + r * kQRow + 16 * pos);
            x[c4] = pad ? bf16x8{} : v;
#pragma unroll
            for (int e = 0; e < 8; ++e) amax[c4 >> 1] = fmaxf(amax[c4 >> 1], fabsf((float)x[c4][e]));
          }
          // block 2 hb + (g >> 1) (dims 128 ks + 64 hb + 32 (g >> 1) .. + 31): lanes
          // g and g ^ 1 hold its two halves; 2^e puts its largest |q| in [128, 256)
          int eb[2];
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            const float a = fmaxf(amax[hb], __shfl_xor(amax[hb], 16, 64));
            eb[hb] = a > 0.f ? max(__builtin_amdgcn_frexp_expf(a) - 8, -127) : 0;
          }
#pragma unroll
          for (int d = 0; d < 8; ++d) {
            const bf16x8& xv = x[d >> 1];
            const int e = 4 * (d & 1);
            const float qs = __builtin_amdgcn_ldexpf(1.0f, -eb[d >> 2]);
            int word = __builtin_amdgcn_cvt_pk_fp8_f32((float)xv[e] * qs, (float)xv[e + 1] * qs, 0, false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32((float)xv[e + 2] * qs, (float)xv[e + 3] * qs, word, true);
            q8[rb][ks][d] = word;
          }
          // block g (half g >> 1 of lane pair g & 1) is held by lane groups 2 (g & 1), 2 (g & 1) + 1
          const int src = n + 32 * (g & 1);
          const int e0 = __shfl(eb[0], src, 64), e1 = __shfl(eb[1], src, 64);
          q8sc[rb][ks] = 127 + ((g >> 1) ? e1 : e0);
        }
      }
      return;
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = 16 * rb + n;
      const bool pad = r >= rows;
#pragma unroll
      for (int u = 0; u < kKU; ++u)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int pos = (8 * u + 2 * g + hh) ^ n;
          const bf16x8 v = *(const bf16x8*)(q_stage + r * kQRow + 16 * pos);
          qop[rb][u][hh] = pad ? bf16x8{} : v;
        }
    }
  };

  // ---- per-lane LDS addresses
  // K of key n: bf16 path chunks 4u + g (u < D / 64); fp8 path chunks g and
  // g + 4 of k-step u / 2 (8 chunks per k-step); a chunk c sits at c ^ sw
  const unsigned ksw = (unsigned)Dm::sw(n, w & 1);
  unsigned k_off[kKU];
#pragma unroll
  for (int u = 0; u < kKU; ++u) {
    const unsigned c = F8 ? (unsigned)(g + 4 * (u & 1) + 8 * (u >> 1)) : (unsigned)(4 * u + g);
    k_off[u] = C::kOffStage + w * kPageBytes + D * n + 16u * (c ^ ksw);
  }
  // P of row 16 rb + n, keys 4g..4g+3 of slot w: half (w & 1) of the 16-byte
  // A operand of lane (g, n) in k-step w >> 1
  const int p_off = C::kOffP + ((w >> 1) * 64 + lane) * 16 + (w & 1) * 8;
  // fp8 P: row-major [row][64 keys], 16-key chunk (page slot) w of row r at
  // position w ^ ((r >> 2) & 3); this lane writes keys 4g..4g+3
  auto p8_off = [&](int rb) { const int r = 16 * rb + n; return C::kOffP + r * 64 + 16 * (w ^ ((r >> 2) & 3)) + 4 * g; };
  float* const mx = (float*)(smem + C::kOffMx);
  float* const alpha_buf = (float*)(smem + C::kOffAlpha);

  f32x4 sv[NRB];            // raw scores of the current step: lane (g, n) key 4g + r, row 16 rb + n
  float m_ref[NRB];         // reference max (log2 units) of row 16 rb + n, identical in every score wave
  float m_off[NRB];         // m_ref, or 0 while it is -inf: P = 2^(s c2 - m_off)
  float thr[NRB];           // raw-score threshold (m + slack) / c2
  float l_lane[NRB];        // this lane's share of the row sums
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    m_ref[rb] = -__builtin_inff();
    m_off[rb] = 0.f;
    thr[rb] = -__builtin_inff();
    l_lane[rb] = 0.f;
  }

  // raw scores of this wave's page of step t from its K block (kraw, read
  // from LDS by the caller). In tail steps the page may be missing and keys
  // past a row's causal limit (or the sequence end) are masked to -inf;
  // steady-state steps need neither.
  auto score_step = [&](int t, const u32x4 (&kraw)[kKU], auto tail) {
    constexpr bool kTail = decltype(tail)::value;
    const int pidx = pb + kPagesPerStep * t + w;
    if (!kTail || ks.has(t)) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) sv[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (F8) {
#pragma unroll
        for (int ks = 0; ks < kKS8; ++ks) {
          const i32x8 ka = cat8(kraw[2 * ks], kraw[2 * ks + 1]);
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) sv[rb] = mfma_fp8_16x16x128(ka, q8[rb][ks], sv[rb], q8sc[rb][ks]);
        }
      } else {
#pragma unroll
        for (int u = 0; u < kKU; ++u) {
          const bf16x8 k0 = fp8x8_to_bf16(kraw[u][0], kraw[u][1]);
          const bf16x8 k1 = fp8x8_to_bf16(kraw[u][2], kraw[u][3]);
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) {
            sv[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qop[rb][u][0], sv[rb], 0, 0, 0);
            sv[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qop[rb][u][1], sv[rb], 0, 0, 0);
          }
        }
      }
      if (capped) {
        // s -> cap tanh(s / cap) in the row's raw-score units; tanh y =
        // 1 - 2 / (1 + e^(2y)), which saturates to +-1 without overflow
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = __builtin_amdgcn_exp2f(2.88539008177792681f * cap_a * sv[rb][r]);
            sv[rb][r] = cap_b * (1.f - 2.f * __builtin_amdgcn_rcpf(1.f + e));
          }
      }
      if (kTail && (kPageSize * (pidx + 1) > qoff + 1 || (win >= 0 && kPageSize * pidx < qoff + q_len - 1 - win))) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const int i = (16 * rb + n) / G;
          const int lim = min(L - 1, qoff + i);
          const int lo = win < 0 ? 0 : qoff + i - win;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kPageSize * pidx + 4 * g + r;
            sv[rb][r] = (key <= lim && key >= lo) ? sv[rb][r] : -__builtin_inff();
          }
        }
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) sv[rb] = f32x4{-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
    }
  };

  // P of step u (scores in sv). 16-bit P: P is first formed against the
  // current m, while the flag word (any score wave saw a row pass its
  // threshold in step u) is still in flight; in the rare slow path it is
  // formed again.
  //
  // F8P: m follows the row's running maximum exactly (no slack), so a new
  // maximum is P = 2^0, which e4m3 holds exactly: the largest weight of a row
  // is not rounded. The page slots' row maxima of step u are already in LDS
  // (exchanged in the phase that computed the scores for the block scales), so
  // the flagged update reads them there, without the slow path's extra
  // barrier. Page slots w and w ^ 2 form the 32-key block (w & 1) of P in the
  // P.V MFMA: the block's largest P, 2^(top c2 - m) <= 1, sets a power of two
  // 2^e that puts it in [128, 256) before rounding to e4m3 (e <= -7); a block
  // below 2^-100 contributes nothing (shift +inf: every P of it is 0, e = 0),
  // so e >= -107. 2^-e is folded into the exponent; the scale rides in the
  // MFMA's A-scale operand.
  auto form_p = [&](int u, int pbuf, unsigned flag_word) {
    f32x4 pv[NRB];
    float top[F8P ? NRB : 1], shift[F8P ? NRB : 1];
    int eb[F8P ? NRB : 1];
    if constexpr (F8P) {
      if (__builtin_amdgcn_readfirstlane(flag_word) != 0) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const f32x4 xm = *(const f32x4*)(smem + C::kOffP + pbuf * C::kPBytes + C::kP8Xmax + (16 * rb + n) * 16);
          const float M = fmaxf(fmaxf(xm[0], xm[1]), fmaxf(xm[2], xm[3]));
          const float m_new = fmaxf(m_ref[rb], M * c2);
          const float alpha = m_new == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(m_ref[rb] - m_new);
          m_ref[rb] = m_new;
          m_off[rb] = m_new == -__builtin_inff() ? 0.f : m_new;
          thr[rb] = m_new * inv_c2;
          l_lane[rb] *= alpha;
          if (w == 0 && g == 0) alpha_buf[(u & 1) * C::kRows + 16 * rb + n] = alpha;
        }
      }
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const float* xm = (const float*)(smem + C::kOffP + pbuf * C::kPBytes + C::kP8Xmax + (16 * rb + n) * 16);
        top[rb] = fmaxf(xm[w & 1], xm[(w & 1) + 2]);
      }
    }
    auto exps = [&]() {
      if constexpr (F8P) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const float x = __builtin_fmaf(top[rb], c2, -m_off[rb]);
          const bool live = x >= -100.f;
          eb[rb] = live ? (int)__builtin_floorf(x) - 7 : 0;
          shift[rb] = live ? m_off[rb] + (float)eb[rb] : __builtin_inff();
        }
      }
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          pv[rb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[rb][r], c2, -(F8P ? shift[rb] : m_off[rb])));
    };
    exps();
    if (!F8P && __builtin_amdgcn_readfirstlane(flag_word) != 0) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const float v = rows_max(fmaxf(fmaxf(sv[rb][0], sv[rb][1]), fmaxf(sv[rb][2], sv[rb][3])));
        if (g == 0) mx[(16 * rb + n) * kPagesPerStep + w] = v;
      }
      lds_barrier();   // the P.V waves take this barrier too
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const f32x4 m4 = *(const f32x4*)(mx + (16 * rb + n) * kPagesPerStep);
        const float M = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
        float alpha = 1.f;
        if (M > thr[rb]) {
          const float m_new = M * c2;
          alpha = __builtin_amdgcn_exp2f(m_ref[rb] - m_new);   // 0 when m was -inf
          m_ref[rb] = m_new;
          m_off[rb] = m_new == -__builtin_inff() ? 0.f : m_new;
          thr[rb] = (m_new + kLazySlack) * inv_c2;
        }
        l_lane[rb] *= alpha;
        if (w == 0 && g == 0) alpha_buf[(u & 1) * C::kRows + 16 * rb + n] = alpha;
      }
      exps();
    }
    if constexpr (F8P) {
      // e4m3 P (round to nearest even) under the block's scale; l sums the
      // rounded values times 2^e, the weights the MFMA applies
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(pv[rb][0], pv[rb][1], 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(pv[rb][2], pv[rb][3], word, true);
        *(int*)(smem + p8_off(rb) + pbuf * C::kPBytes) = word;
        if (w < 2 && g == 0)
          smem[C::kOffP + pbuf * C::kPBytes + C::kP8Scale + 2 * (16 * rb + n) + w] = (uint8_t)(127 + eb[rb]);
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
        l_lane[rb] += __builtin_amdgcn_ldexpf((lo[0] + lo[1]) + (hi[0] + hi[1]), eb[rb]);
      }
    } else {
      const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        // the packed halves pass through an empty asm so that the compiler keeps
        // them for the row sum instead of converting every value a second time
        f16x2 lo = {(_Float16)pv[rb][0], (_Float16)pv[rb][1]}, hi = {(_Float16)pv[rb][2], (_Float16)pv[rb][3]};
        asm volatile("" : "+v"(lo), "+v"(hi));
        *(f16x4*)(smem + p_off + pbuf * C::kPBytes + rb * (2 * 64 * 16)) = f16x4{lo[0], lo[1], hi[0], hi[1]};
        l_lane[rb] = __builtin_amdgcn_fdot2(hi, one, __builtin_amdgcn_fdot2(lo, one, l_lane[rb], false), false);
      }
    }
  };

  // Phase t: P of step t-1, scores and flag of step t, barrier. The LDS reads of the phase (flag word,
  // K block) are issued first. Steady-state phases (4 <= t, t + 4 < n_steps)
  // have full steps t..t+3, no masking, and the ring stage ST = t % 4 as a
  // compile-time constant.
  auto phase = [&](int t, auto tail, auto stage) {
    constexpr bool kTail = decltype(tail)::value;
    constexpr int kSt = decltype(stage)::value;
    const int kst = kSt >= 0 ? kSt : (t & 3);
    const bool have_p = !kTail || (t >= 1 && t <= n_steps);
    const bool have_s = !kTail || t < n_steps;
    unsigned flag_word = 0;
    if (have_p) flag_word = *(const unsigned*)(smem + C::kOffFlag + 4 * ((kst + 3) & 1));
    u32x4 kraw[kKU];
    if (!kTail || ks.has(t)) {
#pragma unroll
      for (int u = 0; u < kKU; ++u) kraw[u] = *(const u32x4*)(smem + k_off[u] + kst * kStageBytes);
    }
    {
      const typename PageStream<TOK, D>::Pending kq = ks.template begin<!kTail>(t + 3, lane);
#pragma unroll
      for (int jj = 0; jj < PageStream<TOK, D>::kParts; ++jj) ks.part(kq, jj);
    }
    if (have_p) form_p(t - 1, (kst + 3) & 1, flag_word);
    if (have_s) {
      if (kTail && (t + 2 >= n_steps || (t == 0 && win_head)))
        score_step(t, kraw, std::true_type{});
      else
        score_step(t, kraw, std::false_type{});
      bool over = false;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const float v = fmaxf(fmaxf(sv[rb][0], sv[rb][1]), fmaxf(sv[rb][2], sv[rb][3]));
        over |= v > thr[rb];
        if constexpr (F8P) {
          // this page slot's row maximum, for the block scales of P (formed next phase)
          const float r = rows_max(v);
          if (g == 0) *(float*)(smem + C::kOffP + (kst & 1) * C::kPBytes + C::kP8Xmax + (16 * rb + n) * 16 + 4 * w) = r;
        }
      }
      const bool any = __any(over);
      if (lane == 0) smem[C::kOffFlag + 4 * (kst & 1) + w] = any ? 1 : 0;
    }
    // K of step t+1 must have landed; steps t+2 and t+3 may fly
    if constexpr (kTail)
      wait_vm(ks.count(t + 2) + ks.count(t + 3));
    else
      wait_vm(2 * PageStream<TOK, D>::kParts);
    lds_barrier();
  };

  if (n_steps > 0) {
    lds_barrier();   // Q and step 0's K are in LDS
    load_q();
    if (capped) {
      cap_a = c2 * 0.69314718055994531f / p.softcap;
      cap_b = 1.f / cap_a;
    }
    int t = 0;
    for (; t < 4 && t < n_steps + 2; ++t) phase(t, std::true_type{}, std::integral_constant<int, -1>{});
    for (; t + 7 < n_steps; t += 4) {
      phase(t, std::false_type{}, std::integral_constant<int, 0>{});
      phase(t + 1, std::false_type{}, std::integral_constant<int, 1>{});
      phase(t + 2, std::false_type{}, std::integral_constant<int, 2>{});
      phase(t + 3, std::false_type{}, std::integral_constant<int, 3>{});
    }
    for (; t < n_steps + 2; ++t) phase(t, std::true_type{}, std::integral_constant<int, -1>{});
  }

  // ---- segment partials. The loop's last barrier has retired every LDS
  // access and transfer. l of a row sums the page slots' key subsets in a
  // fixed order (score and P.V waves alike); m is identical in every score
  // wave. The P.V waves divide their accumulators by l and stage fp16 o in LDS
  // for full-row stores.
  float* const lsum = (float*)smem;   // [slot][row]
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    float l = l_lane[rb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (g == 0) lsum[w * C::kRows + 16 * rb + n] = l;
    // one segment with sink logits: the sink's share of the denominator,
    // 2^(sink - m), joins the row sums as a fifth slot for the P.V waves
    if (g == 0 && w == 0 && p.direct && p.sinks != nullptr) {
      const int row = 16 * rb + n;
      const int gg = (row < rows ? row : 0) % G;
      const float sink2 = ((const const_f32*)p.sinks)[h * G + gg] * 1.44269504088896341f;
      lsum[kPagesPerStep * C::kRows + row] = __builtin_amdgcn_exp2f(sink2 - m_ref[rb]);
    }
  }
  lds_barrier();   // row sums of every page slot
  if (w == 0 && g == 0 && (!p.direct || p.lse != nullptr)) {
    const int T = p.total_q, Hq = p.num_q_heads;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int row = 16 * rb + n;
      if (row < rows) {
        float l = lsum[row];
#pragma unroll
        for (int v = 1; v < kPagesPerStep; ++v) l += lsum[v * C::kRows + row];
        const int i = row / G, gg = row - (row / G) * G;
        if (p.direct) {
          // one segment: the row's log-sum-exp goes straight to lse (natural
          // log), a sink logit joining the sum as 2^(sink - mx), mx = max(m, sink)
          float mx = m_ref[rb], den = l;
          if (p.sinks != nullptr) {
            const float sink2 = ((const const_f32*)p.sinks)[h * G + gg] * 1.44269504088896341f;
            mx = fmaxf(m_ref[rb], sink2);
            den = (m_ref[rb] == -__builtin_inff() ? 0.f : l * __builtin_amdgcn_exp2f(m_ref[rb] - mx)) +
                  __builtin_amdgcn_exp2f(sink2 - mx);
          }
          p.lse[(int64_t)(h * G + gg) * T + q0 + i] =
              den > 0.f ? (mx + __builtin_amdgcn_logf(den)) * 0.69314718055994531f : -__builtin_inff();
        } else {
          float* dst = p.ws_ml + ws_slot_tq<RM>(q0, i, h * G, gg, geo.seg, T, Hq, p.num_segments) * 2;
          partial_store(m_ref[rb], dst);
          partial_store(l, dst + 1);
        }
      }
    }
  }
  if constexpr (F8P) {
    lds_barrier();   // o staged
    store_rows<G, D, RM>(p, geo, smem + C::kOffObuf);
  }
}

// P.V wave v = w - 4: V stream of page slot v, O[:, 64 v .. 64 v + 63] for all
// NRB row blocks; stages its slice of the segment's normalised output o. With
// F8, O += P V runs on the 32x32x64 fp8 MFMA over 32-row tiles, P and V as
// e4m3 bytes.
template <int G, int NRB, int MODE, bool TOK, int D, bool RM>
__device__ __forceinline__ void pv_wave(const MainParams& p, const Geo& geo, uint8_t* smem) {
  using C = Cfg<G, D>;
  using Dm = Dim<D>;
  constexpr int kPageBytes = Dm::kPageBytes, kStageBytes = Dm::kStageBytes, kVDims = Dm::kVDims;
  constexpr int kParts = Dm::kDmaPerWave;   // 1 KiB parts per stream and step
  constexpr int NDB = kVDims / 16;          // 16-dim output blocks of this wave
  constexpr bool F8 = MODE != kMode16;       // e4m3 P and V on the fp8 MFMA
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int v = w - 4;
  const int lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int h = geo.h, q0 = geo.q0, L = geo.L, pb = geo.pb, pe = geo.pe;
  const int rows = geo.rows, n_steps = geo.n_steps;
  uint8_t* const k_ring = smem + C::kOffStage;
  uint8_t* const v_ring = k_ring + kStages * kStageBytes;

  // The V block of page slot v streams through this wave by vector loads into
  // registers, one phase before it goes to its ring stage and two before its
  // use here.
  PageStream<TOK, D> vs;
  vs.init(p, geo, smem, w, v, lane, p.v_cache, lds_addr(v_ring), C::kOffIds);
  if (n_steps > 0) {
    using Pend = typename PageStream<TOK, D>::Pending;
    vs.fetch_window(0, lane);
    Pend v0;
    if constexpr (TOK) {
      if (4 < n_steps) vs.fetch_window(1, lane);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      v0 = Pend{nullptr, 0u, vs.has(0), vs.read_id(0)};
    } else {
      v0 = Pend{vs.block_base(vs.resolve(0, vs.first_id(0))), 0u, vs.has(0), {}};
    }
    vs.load(v0);
    wait_vm(vs.count(0));
    vs.next_id = vs.read_id(1);
  }

  // V^T operand: source lane n of group g supplies the 8 dims at +8 (n & 1) of
  // key 4g + ((n >> 1) & 3) in page slot 2 ks + (n >> 3), the k-slot (n >> 1)
  // of group g; ds_read_b64_tr_b8 hands lane n byte k of source lane 2k + n/8.
  const int vpar = (n >> 3) & 1;
  const int vkey = 4 * g + ((n >> 1) & 3);
  const unsigned vsw = 16u * (unsigned)Dm::sw(vkey, vpar);
  unsigned v_off[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    v_off[db] = C::kOffStage + kStages * kStageBytes + vpar * kPageBytes + D * vkey + 8 * (n & 1) +
                ((unsigned)(kVDims * v + 16 * db) ^ vsw);
  const int p_off = C::kOffP + lane * 16;
  const float* const alpha_buf = (const float*)(smem + C::kOffAlpha);

  // fp8 path. Lane l of a 32x32x64 tile: A (P) row 32 rt + (l & 31) with keys
  // 32 q .. 32 q + 31 (q = l >> 5) of the step as bytes 0..31; B (V) dim
  // 32 dt + (l & 31) of this wave's 64 with the same keys, gathered by four
  // ds_read_b64_tr_b8 of 8 keys each: in its 16-lane group, source lane
  // 2k + hb supplies the 8 dims at +8 hb of key 32 q + 8 j + k. Bytes 0..15
  // are page slot 2q, bytes 16..31 slot 2q + 1, so the MFMA's scale block j
  // (bytes 16 j .. + 15 of both lane halves, scale from lane c + 32 j) is slots
  // j and j + 2, whose E8M0 scale the score waves store per row.
  constexpr int NRT = (NRB + 1) / 2;    // 32-row tiles
  constexpr int NDT = kVDims / 32;      // 32-dim tiles of this wave
  unsigned v8_off[F8 ? NDT : 1][4];
  int p8_rd[F8 ? NRT : 1];
  int p8_sc[F8 ? NRT : 1];   // this lane's P block scale: row 32 rt + (l & 31), block l >> 5 (-1: padding row)
  if constexpr (F8) {
    const int q = lane >> 5, sub = (lane >> 4) & 1, src = lane & 15, kk8 = src >> 1, hb = src & 1;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int slot = 2 * q + (j >> 1), kin = 8 * (j & 1) + kk8;
        const unsigned chunk = (unsigned)((kVDims / 16) * v + 2 * dt + sub);
        const unsigned sw = (unsigned)Dm::sw(kin, slot & 1);
        v8_off[dt][j] = C::kOffStage + kStages * kStageBytes + slot * kPageBytes + D * kin + 16u * (chunk ^ sw) + 8 * hb;
      }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int r = 32 * rt + (lane & 31);
      p8_rd[rt] = C::kOffP + r * 64 + 16 * ((2 * q) ^ ((r >> 2) & 3));   // chunk 2q; chunk 2q+1 at ^1
      // rows past the score waves' NRB blocks (an odd NRB) have no scale written
      p8_sc[rt] = r < 16 * NRB ? C::kOffP + C::kP8Scale + 2 * r + q : -1;
    }
  }

  f32x4 acc[F8 ? 1 : NRB][NDB];
  f32x16 acc8[F8 ? NRT : 1][F8 ? NDT : 1];
  if constexpr (F8) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc8[rt][dt] = f32x16{};
  } else {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  bool slow1 = false;   // flag of step t-1 in phase t
  bool slow2 = false;   // flag of step t-2 in phase t

  // Phase t: V of step t to its ring stage and the loads of V of step t+1;
  // the LDS reads of step t-2 (V block, P) and of the flag word of step t-1;
  // an extra barrier if step t-1 takes the slow path; O += P V of step t-2
  // (rescaled first if step t-2 moved m); barrier.
  auto phase = [&](int t, auto tail, auto stage) {
    constexpr bool kTail = decltype(tail)::value;
    constexpr int kSt = decltype(stage)::value;
    const bool have_f = !kTail || (t >= 1 && t <= n_steps);
    const bool have_pv = !kTail || (t >= 2 && t - 2 < n_steps);
    const int u = t - 2;
    const int vst = kSt >= 0 ? ((kSt + 2) & 3) : (u & 3);
    const int pbuf = kSt >= 0 ? (kSt & 1) : (u & 1);
    // V of step t (loaded in the previous phase) to its ring stage, then the
    // loads of V of step t+1 go out; they land while this phase computes.
    // Steady-state phases (t + 7 < n_steps) have every page slot of steps t
    // and t + 1.
    if (!kTail || vs.has(t)) vs.store(t, v_ring);
    {
      const typename PageStream<TOK, D>::Pending vq = vs.template begin<!kTail>(t + 1, lane);
      vs.load(vq);
    }
    unsigned flag_word = 0;
    if (have_f) flag_word = *(const unsigned*)(smem + C::kOffFlag + 4 * ((t - 1) & 1));
    // k-slot 8g + e of k-step kk is key 4g + (e & 3) of page slot 2 kk + (e >> 2)
    i32x2 vraw[2][NDB > 4 ? NDB : 4];
    f16x8 pa[F8 ? 1 : NRB][2];
    i32x8 pa8[F8 ? NRT : 1];
    int sa8[F8 ? NRT : 1];
    if (F8 && have_pv) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vraw[dt][j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(smem + v8_off[dt][j] + vst * kStageBytes));
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const uint8_t* pr = smem + p8_rd[rt] + pbuf * C::kPBytes;
        pa8[rt] = cat8(*(const u32x4*)pr, *(const u32x4*)(smem + ((p8_rd[rt] + pbuf * C::kPBytes) ^ 16)));
        sa8[rt] = p8_sc[rt] >= 0 ? (int)smem[p8_sc[rt] + pbuf * C::kPBytes] : 127;
      }
    }
    if (!F8 && have_pv) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          vraw[kk][db] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (lds_i32x2*)(smem + v_off[db] + vst * kStageBytes + kk * 2 * kPageBytes));
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          pa[rb][kk] = *(const f16x8*)(smem + p_off + pbuf * C::kPBytes + (rb * 2 + kk) * (64 * 16));
    }
    slow2 = slow1;
    slow1 = have_f && __builtin_amdgcn_readfirstlane(flag_word) != 0;
    if (!F8 && slow1) lds_barrier();   // matches the score waves' maxima exchange (F8: none)
    if (F8 && have_pv) {
      if constexpr (kTail) {
        // keys past the segment or the sequence end: V bytes 0
        if (u == n_steps - 1) {
          const int q = lane >> 5;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int page = pb + kPagesPerStep * u + 2 * q + (j >> 1);
            unsigned lo = 0, hi = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const int key = kPageSize * page + 8 * (j & 1) + k;
              const unsigned m8 = (page < pe && key < L) ? 0xffu : 0u;
              if (k < 4) lo |= m8 << (8 * k); else hi |= m8 << (8 * (k - 4));
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
              vraw[dt][j][0] &= (int)lo;
              vraw[dt][j][1] &= (int)hi;
            }
          }
        }
      }
      i32x8 vb[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        vb[dt] = i32x8{vraw[dt][0][0], vraw[dt][0][1], vraw[dt][1][0], vraw[dt][1][1],
                       vraw[dt][2][0], vraw[dt][2][1], vraw[dt][3][0], vraw[dt][3][1]};
      auto accumulate = [&]() {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) acc8[rt][dt] = mfma_fp8_32x32x64(pa8[rt], vb[dt], acc8[rt][dt], sa8[rt]);
      };
      if (slow2) {
        // rows 32 rt + 8 c + 4 (lane >> 5) + e hold acc8[rt][dt][4 c + e]; rows
        // past the score waves' NRB blocks (an odd NRB) have no alpha and are
        // never stored
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (32 * rt + 8 * c >= 16 * NRB) continue;
            const f32x4 a = *(const f32x4*)(alpha_buf + (u & 1) * C::kRows + 32 * rt + 8 * c + 4 * (lane >> 5));
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
              for (int e = 0; e < 4; ++e) acc8[rt][dt][4 * c + e] *= a[e];
          }
      }
      accumulate();
    } else if (!F8 && have_pv) {
      // V^T of k-step kk, converted exactly to fp16; keys of pages past the
      // segment (never loaded: stale or uninitialised LDS) and past the
      // sequence end get V = 0, so P = 0 never meets a NaN. Converted one
      // k-step at a time, so that only half of the operands are live.
      auto v_operands = [&](int kk, f16x8 (&vf)[NDB]) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) vf[db] = fp8x8_to_f16((unsigned)vraw[kk][db][0], (unsigned)vraw[kk][db][1]);
        if constexpr (kTail) {
          if (u == n_steps - 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int page = pb + kPagesPerStep * u + 2 * kk + (e >> 2);
              const int key = kPageSize * page + 4 * g + (e & 3);
              const bool keep = page < pe && key < L;
#pragma unroll
              for (int db = 0; db < NDB; ++db) vf[db][e] = keep ? vf[db][e] : (_Float16)0.f;
            }
          }
        }
      };
      auto accumulate = [&]() {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          f16x8 vf[NDB];
          v_operands(kk, vf);
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
              acc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[rb][kk], vf[db], acc[rb][db], 0, 0, 0);
          }
        }
      };
      if (slow2) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const f32x4 a = *(const f32x4*)(alpha_buf + (u & 1) * C::kRows + 16 * rb + 4 * g);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[rb][db][r] *= a[r];
        }
      }
      accumulate();
    }
    lds_barrier();
  };

  if (n_steps > 0) {
    lds_barrier();
    int t = 0;
    for (; t < 4 && t < n_steps + 2; ++t) phase(t, std::true_type{}, std::integral_constant<int, -1>{});
    for (; t + 7 < n_steps; t += 4) {
      phase(t, std::false_type{}, std::integral_constant<int, 0>{});
      phase(t + 1, std::false_type{}, std::integral_constant<int, 1>{});
      phase(t + 2, std::false_type{}, std::integral_constant<int, 2>{});
      phase(t + 3, std::false_type{}, std::integral_constant<int, 3>{});
    }
    for (; t < n_steps + 2; ++t) phase(t, std::true_type{}, std::integral_constant<int, -1>{});
  }

  lds_barrier();   // the score waves' row sums of every page slot
  const float* const lsum = (const float*)smem;
  _Float16* const obuf = (_Float16*)(smem + C::kOffObuf);   // [row][D]
  uint16_t* const obuf_bits = (uint16_t*)obuf;
  const float vd = p.direct ? *(const const_f32*)p.v_descale : 1.f;
  if constexpr (F8) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * rt + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < rows) {
          float l = lsum[row];
#pragma unroll
          for (int s2 = 1; s2 < kPagesPerStep; ++s2) l += lsum[s2 * C::kRows + row];
          if (p.direct && p.sinks != nullptr) l += lsum[kPagesPerStep * C::kRows + row];
          const float inv = l > 0.f ? vd / l : 0.f;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const int at = row * D + kVDims * v + 32 * dt + (lane & 31);
            if (p.direct)
              obuf_bits[at] = (uint16_t)bf16_rne(acc8[rt][dt][r] * inv);
            else
              obuf[at] = (_Float16)(acc8[rt][dt][r] * inv);
          }
        }
      }
    lds_barrier();
    store_rows<G, D, RM>(p, geo, smem + C::kOffObuf);
  } else {
    // o = acc / l (0 with no visible key); a single segment writes out = vd o.
    // Lane (g, n) holds dims kVDims v + 16 db + n of rows 16 rb + 4 g + r. A
    // transpose inside each group of NDB lanes (butterflies over the lane
    // index on packed 16-bit pairs) leaves lane n = NDB q + j with the NDB
    // consecutive dims kVDims v + 16 j + NDB q + e, which it stores with one
    // write: no staging through LDS, and the 16 lanes of a row write one
    // contiguous run.
    const int j = n & (NDB - 1), q = n / NDB;
    const int dim0 = kVDims * v + 16 * j + NDB * q;
    const bool odd = (n & 1) != 0, half = ((n >> 1) & 1) != 0;
    const unsigned sel = odd ? 0x03020706u : 0x05040100u;   // (partner.hi, own.hi) : (own.lo, partner.lo)
    auto epilogue = [&](auto direct_tag) {
      constexpr bool kDirect = decltype(direct_tag)::value;
      const int T = p.total_q, Hq = p.num_q_heads;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * rb + 4 * g + r;
          float l = lsum[row];
#pragma unroll
          for (int s2 = 1; s2 < kPagesPerStep; ++s2) l += lsum[s2 * C::kRows + row];
          if (kDirect && p.sinks != nullptr) l += lsum[kPagesPerStep * C::kRows + row];
          const float inv = l > 0.f ? vd * __builtin_amdgcn_rcpf(l) : 0.f;
          unsigned wd[NDB / 2];
#pragma unroll
          for (int k = 0; k < NDB / 2; ++k) {
            const float a = acc[rb][2 * k][r] * inv, b = acc[rb][2 * k + 1][r] * inv;
            if constexpr (kDirect) {
              wd[k] = bf16_rne(a) | (bf16_rne(b) << 16);
            } else {
              const f16x2 hv = {(_Float16)a, (_Float16)b};
              wd[k] = __builtin_bit_cast(unsigned, hv);
            }
          }
          if constexpr (NDB == 4) {
            // lanes n and n ^ 2 trade the pair whose bit 1 differs from theirs
            const unsigned t0 = (unsigned)__builtin_amdgcn_mov_dpp((int)wd[0], 0x4E, 0xF, 0xF, false);
            const unsigned t1 = (unsigned)__builtin_amdgcn_mov_dpp((int)wd[1], 0x4E, 0xF, 0xF, false);
            const unsigned w0 = half ? t1 : wd[0], w1 = half ? wd[1] : t0;
            wd[0] = w0;
            wd[1] = w1;
          }
          // lanes n and n ^ 1 trade the 16-bit half whose bit differs from theirs
#pragma unroll
          for (int k = 0; k < NDB / 2; ++k)
            wd[k] = __builtin_amdgcn_perm((unsigned)__builtin_amdgcn_mov_dpp((int)wd[k], 0xB1, 0xF, 0xF, false), wd[k], sel);
          if (row < rows) {
            const int i = row / G, gg = row - (row / G) * G;
            if constexpr (kDirect) {
              uint16_t* dst = p.out + (int64_t)(q0 + i) * p.out_stride_token + (int64_t)(h * G + gg) * p.out_stride_head + dim0;
              if constexpr (NDB == 4)
                *(uint2*)dst = make_uint2(wd[0], wd[1]);
              else
                *(unsigned*)dst = wd[0];
            } else {
              uint16_t* dst = p.ws_o + ws_slot_tq<RM>(q0, i, h * G, gg, geo.seg, T, Hq, p.num_segments) * kHeadDim + dim0;
              if constexpr (NDB == 4)
                partial_store(u32x2{wd[0], wd[1]}, (u32x2*)dst);
              else
                partial_store(wd[0], (unsigned*)dst);
            }
          }
        }
    };
    if (p.direct)
      epilogue(std::true_type{});
    else
      epilogue(std::false_type{});
  }
}

template <int G, int NRB, int MODE, bool TOK, int D, bool RM>
__device__ __forceinline__ void verify_segment(const MainParams& p, const Geo& geo, uint8_t* smem) {
  if (threadIdx.x < 64 * kPagesPerStep)
    score_wave<G, NRB, MODE, TOK, D, RM>(p, geo, smem);
  else
    pv_wave<G, NRB, MODE, TOK, D, RM>(p, geo, smem);
}

// TOK: the cache has one-token pages; D: head dim; MERGE: the in-launch merge
// (merge::merge_in_launch) follows the segment; RM: row-major partials
template <int G, int MODE, bool TOK, int D, bool BAL, bool MERGE = false, bool RM = false>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
splitkv_main_kernel(MainParams p) {
  using C = Cfg<G, D>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kLdsBytes];

  const const_i32* cu = (const const_i32*)p.cu_seqlens_q;
  const const_i32* sl = (const const_i32*)p.seq_lens;
  Geo geo;
  geo.seg = blockIdx.x;
  geo.b = blockIdx.y;
  int wg_z = blockIdx.z;
  if constexpr (!BAL) {
    // Consecutive work-group ids are dispatched to the eight XCDs in turn.
    // Renumber them so that each XCD runs a contiguous run of ids (a whole
    // sequence's segments, when the grid allows): the sequence's queries and
    // block-table row are then fetched into one XCD's L2, not into all eight.
    // The work-groups that read the same pages (the kv_split halves of a
    // 32-head group and the q_split query blocks, z = hkv * nsplit + sub) are
    // made neighbours in the new order, so that they run on one XCD at the
    // same time and the second reader of each page finds it in that XCD's L2.
    // The renumbering is a bijection of [0, total) only while its 32-bit
    // arithmetic is exact: grids of 2^32 work-groups or more keep their ids.
    const uint64_t total64 = (uint64_t)gridDim.x * gridDim.y * gridDim.z;
    if ((total64 & 7u) == 0 && total64 <= 0xffffffffull) {
      const unsigned gx = gridDim.x, gxy = gx * gridDim.y, total = (unsigned)total64;
      const unsigned nsplit = (unsigned)(p.kv_split * p.q_split);
      const unsigned id = blockIdx.x + gx * (blockIdx.y + gridDim.y * blockIdx.z);
      const unsigned r = (id & 7u) * (total >> 3) + (id >> 3);
      const unsigned rr = r / nsplit;
      geo.seg = (int)(rr % gx);
      geo.b = (int)((rr / gx) % gridDim.y);
      wg_z = (int)((rr / gxy) * nsplit + r % nsplit);
    }
  }
  // BAL: balanced segments (a separate instantiation, so that the default
  // kernel's code does not carry the schedule)
  int seg_count = p.num_segments;
  if constexpr (BAL) {
    // slot blockIdx.x -> (sequence, segment) by the balanced schedule; idle
    // slots past the last sequence's segments return before any barrier
    const BalancedSlot sl = balanced_slot((int)blockIdx.x, p.seq_lens, p.num_seqs, p.max_seq_len, p.window_left,
                                          (int)gridDim.x, p.num_segments);
    geo.b = __builtin_amdgcn_readfirstlane(sl.b);
    geo.seg = __builtin_amdgcn_readfirstlane(sl.seg);
    seg_count = __builtin_amdgcn_readfirstlane(sl.count);
    if (geo.b < 0) return;
  }
  geo.h = wg_z / p.q_split;
  geo.hkv = geo.h / p.kv_split;
  // out-of-contract values are clamped so that every access stays in its buffer
  const int seq_q0 = cu[geo.b];
  int seq_qlen = cu[geo.b + 1] - seq_q0;
  if (seq_q0 < 0 || seq_q0 >= p.total_q) seq_qlen = 0;
  seq_qlen = min(max(seq_qlen, 0), min(kMaxQLen, p.total_q - max(seq_q0, 0)));
  // this work-group's block of the sequence's query tokens
  const int i0 = (wg_z % p.q_split) * p.q_per_wg;
  const int q_len = min(seq_qlen - i0, p.q_per_wg);
  if (q_len <= 0) return;
  geo.q0 = seq_q0 + i0;
  geo.q_len = q_len;
  geo.L = min(max(sl[geo.b], 0), p.max_seq_len);
  geo.qoff = geo.L - seq_qlen + i0;
  const int pages = (geo.L + kPageSize - 1) / kPageSize;
  // with a left window the segments split only the pages some query can see;
  // the first page is bounded with the largest q_len, so that the partition,
  // and with it every row's bits, does not depend on the call's q_len
  geo.win = p.window_left < 0 ? -1 : min(p.window_left, geo.L);
  const int span = segment_span(geo.L, p.window_left);
  const int first = pages - span;
  const int chunk = (span + seg_count - 1) / seg_count;
  geo.pb = first + min(geo.seg * chunk, span);
  geo.pe = first + min(geo.seg * chunk + chunk, span);
  geo.rows = G * q_len;
  geo.n_steps = (geo.pe - geo.pb + kPagesPerStep - 1) / kPagesPerStep;
  geo.c2 = *(const const_f32*)p.k_descale * p.score_scale_log2;

  const int nrb = (geo.rows + 15) >> 4;
  const int merge_group = geo.b * (int)gridDim.z + wg_z;
  if constexpr (G == 16) {
    switch (nrb) {
      case 1: verify_segment<16, 1, MODE, TOK, D, RM>(p, geo, smem); break;
      case 2: verify_segment<16, 2, MODE, TOK, D, RM>(p, geo, smem); break;
      case 3: verify_segment<16, 3, MODE, TOK, D, RM>(p, geo, smem); break;
      default: verify_segment<16, 4, MODE, TOK, D, RM>(p, geo, smem); break;
    }
  } else if constexpr (G == 8) {
    switch (nrb) {
      case 1: verify_segment<8, 1, MODE, TOK, D, RM>(p, geo, smem); break;
      case 2: verify_segment<8, 2, MODE, TOK, D, RM>(p, geo, smem); break;
      case 3: verify_segment<8, 3, MODE, TOK, D, RM>(p, geo, smem); break;
      default: verify_segment<8, 4, MODE, TOK, D, RM>(p, geo, smem); break;
    }
  } else {
    if (nrb == 1)
      verify_segment<4, 1, MODE, TOK, D, RM>(p, geo, smem);
    else
      verify_segment<4, 2, MODE, TOK, D, RM>(p, geo, smem);
  }
  if constexpr (MERGE) {
    // the segment reduce's per-row arithmetic, on this group's rows
    ReduceParams rp = {};
    rp.ws_o = p.ws_o;
    rp.ws_ml = p.ws_ml;
    rp.v_descale = p.v_descale;
    rp.out = p.out;
    rp.out_stride_token = p.out_stride_token;
    rp.out_stride_head = p.out_stride_head;
    rp.lse = p.lse;
    rp.sinks = p.sinks;
    rp.total_q = p.total_q;
    rp.num_q_heads = p.num_q_heads;
    rp.num_segments = p.num_segments;
    rp.head_dim = p.head_dim;
    rp.ws_row_major = RM;
    static_assert(merge::kMergeLdsBcast + 16 <= C::kLdsBytes, "the merge's LDS fits the kernel's allocation");
    uint32_t* sync = p.merge_sync + (int64_t)merge_group * kMergeSyncWords;
    const int S = p.num_segments;
    // the summation order of the segment reduce for S (waves per row there; S <= 64 here)
    if (!RM && S <= 16)
      merge::merge_in_launch<1, G, RM>(rp, sync, p.merge_wait_ticks, geo.seg, S, geo.rows, geo.q0, geo.h * G, smem);
    else if (S <= 32)
      merge::merge_in_launch<2, G, RM>(rp, sync, p.merge_wait_ticks, geo.seg, S, geo.rows, geo.q0, geo.h * G, smem);
    else
      merge::merge_in_launch<4, G, RM>(rp, sync, p.merge_wait_ticks, geo.seg, S, geo.rows, geo.q0, geo.h * G, smem);
  }
}

// TOK: one-token cache pages; D: head dim; RM: row-major partials
template <int MODE, bool TOK, int D, bool RM = false>
hipError_t launch_shape(const MainParams& p, int group, hipStream_t stream) {
  // balanced: p.num_slots slots along x (see MainParams), else segments x sequences
  const dim3 grid(p.balance ? p.num_slots : p.num_segments, p.balance ? 1 : p.num_seqs,
                  p.num_kv_heads * p.kv_split * p.q_split);
  if (p.balance) {
    if (group == 16)
      hipLaunchKernelGGL((splitkv_main_kernel<16, MODE, TOK, D, true, false, RM>), grid, dim3(kThreads), 0, stream, p);
    else if (group == 8)
      hipLaunchKernelGGL((splitkv_main_kernel<8, MODE, TOK, D, true, false, RM>), grid, dim3(kThreads), 0, stream, p);
    else if (group == 4)
      hipLaunchKernelGGL((splitkv_main_kernel<4, MODE, TOK, D, true, false, RM>), grid, dim3(kThreads), 0, stream, p);
    else
      return hipErrorInvalidValue;
  } else if (p.merge_sync != nullptr) {
    // the in-launch merge: 16-bit arithmetic, head dim 256, pages of 16 or more
    if constexpr (MODE == kMode16 && !TOK && D == 256) {
      if (group == 16)
        hipLaunchKernelGGL((splitkv_main_kernel<16, MODE, TOK, D, false, true, RM>), grid, dim3(kThreads), 0, stream, p);
      else if (group == 8)
        hipLaunchKernelGGL((splitkv_main_kernel<8, MODE, TOK, D, false, true, RM>), grid, dim3(kThreads), 0, stream, p);
      else if (group == 4)
        hipLaunchKernelGGL((splitkv_main_kernel<4, MODE, TOK, D, false, true, RM>), grid, dim3(kThreads), 0, stream, p);
      else
        return hipErrorInvalidValue;
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    if (group == 16)
      hipLaunchKernelGGL((splitkv_main_kernel<16, MODE, TOK, D, false, false, RM>), grid, dim3(kThreads), 0, stream, p);
    else if (group == 8)
      hipLaunchKernelGGL((splitkv_main_kernel<8, MODE, TOK, D, false, false, RM>), grid, dim3(kThreads), 0, stream, p);
    else if (group == 4)
      hipLaunchKernelGGL((splitkv_main_kernel<4, MODE, TOK, D, false, false, RM>), grid, dim3(kThreads), 0, stream, p);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// group: query heads per work-group (16, 8 or 4; 32 query heads per KV head run
// as two 16-head work-groups, p.kv_split = 2)
template <int MODE, int D>
hipError_t launch_dim(const MainParams& p, int group, hipStream_t stream) {
  return p.token_pages ? launch_shape<MODE, true, D>(p, group, stream) : launch_shape<MODE, false, D>(p, group, stream);
}

}  // namespace
}  // namespace pfkv
