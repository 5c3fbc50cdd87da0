// fp8 varlen prefill attention (gfx950): e4m3 Q/K/V with per-tensor descales,
// packed THD rows, qk head dim 192, v head dim 128, bf16 output, optional LSE,
// causal aligned to the bottom right or not. What it computes follows aiter PR
// #7375 ("gfx1250 fp8 varlen FMHA"), section Summary; the kernel there is
// gfx1250 assembly, this one is written for gfx950:
//
// * A work-group of 8 waves serves 256 query rows of one (sequence, query
//   head); wave w owns rows 32 w .. 32 w + 31 whole (no cross-wave softmax).
// * Key stages of 128 rows (two 64-key sub-tiles) stream HBM/L2 -> LDS through
//   a 3-stage ring with global_load_lds_dwordx4 (one barrier per stage, two
//   stages in flight, five 1 KiB transfers per wave and stage). K rows (192
//   bytes) sit at rotated 16-byte positions and V rows (128 bytes) at
//   XOR-swizzled ones, so the MFMA operand reads below are free of bank
//   conflicts.
// * The MFMA groups run at raised wave priority, so the two waves of a SIMD
//   drift apart: one feeds the matrix core while the other does its softmax.
// * S^T = K Q^T on v_mfma_scale_f32_32x32x64_f8f6f4 (three k-steps over the
//   192 dims), Q held in registers. A lane then holds 32 scores of one query row.
// * Online softmax in the log2 domain with a lazy reference max (moved only
//   when a row's max passes it by more than 8), so rescaling is rare.
// * P in e4m3 with an E8M0 block scale per 32 keys of a row: each block's
//   probabilities are scaled by a power of two that puts their maximum in
//   [128, 256) before rounding, and the scale rides in the MFMA's B-scale
//   operand. Small probabilities then keep their 3-bit mantissa instead of
//   flushing to zero (the underflow the same page's review works through).
//   The row sum l is the same MFMA with an all-ones operand in place of V^T, so
//   it adds the rounded, rescaled values, and O and the LSE use the
//   same weights. On this MFMA the scale in lane c + 32 kb covers bytes
//   16 kb .. 16 kb + 15 of both lane halves of column c (measured), which here
//   are keys 32 kb .. 32 kb + 31 of the row: both lanes of a row share each
//   block's exponent, and lane half kb supplies block kb's.
// * O^T = V^T P^T on the same scaled MFMA (four 32-dim tiles), V^T from LDS by
//   ds_read_b64_tr_b8, so each lane's accumulators belong to its own row.
#include "pfkv_internal.h"
#include "prefill_config.h"

namespace pfkv {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(4))) const int32_t const_i32;
typedef __attribute__((address_space(4))) const float const_f32;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kTileRows = kWaves * kRowsPerWave;      // 256 query rows per work-group
static_assert(kTileRows == kPrefillTileRows, "the host sizes the grid with kPrefillTileRows");
constexpr int kKeys = 64;                             // keys per sub-tile
constexpr int kSubs = 2;                              // sub-tiles per stage
constexpr int kStageKeys = kSubs * kKeys;             // 128 keys per stage
constexpr int kDqk = 192, kDv = 128;
constexpr int kKBytes = kKeys * kDqk;                 // 12 KiB
constexpr int kVBytes = kKeys * kDv;                  // 8 KiB
constexpr int kSubBytes = kKBytes + kVBytes;          // one sub-tile: K then V
constexpr int kStageBytes = kSubs * kSubBytes;        // 40 KiB
constexpr int kStages = 3;
constexpr int kKParts = kKBytes / 1024;               // 12 transfers of 1 KiB
constexpr int kSubParts = kKParts + kVBytes / 1024;   // 20 per sub-tile
constexpr int kPartsPerWave = kSubs * kSubParts / kWaves;   // 5
static_assert(kSubs * kSubParts == kWaves * kPartsPerWave, "transfers split evenly over the waves");
constexpr float kLazySlack = 8.0f;
constexpr int kCausalBands = 4;

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One 1 KiB HBM -> LDS transfer, 16 bytes per lane from its own 64-bit address
// to LDS address lds + 16 i. M0 carries the LDS base; it is saved and restored.
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

// max(x of lane i, x of lane i ^ 32) in every lane, by one VALU swap of the
// wave's 32-lane halves (a general shuffle is an LDS round trip). With both
// operands x, the swap returns (x[i mod 32], x[i mod 32 + 32]) in lane i.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// K row `key` keeps its 16-byte chunk c at position (c + rot(key)) mod 12.
__device__ __forceinline__ int k_rot(int key) { return (key >> 2) & 3; }
// V row `key` keeps its 16-byte chunk c at position c ^ vsw(key).
__device__ __forceinline__ int v_sw(int key) { return 2 * ((key >> 1) & 1) + 4 * ((key >> 3) & 1); }

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c, int scale_a, int scale_b) {
  // e4m3 A and B with E8M0 block scales (one per lane's 32 k-elements)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

template <bool CAUSAL>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 31, h = lane >> 5;
  const int b = blockIdx.z;
  // Consecutive work-group ids go to the eight XCDs in turn, so a head's tiles
  // in consecutive ids would run on every XCD and each XCD's L2 would fetch
  // that head's K and V. xcd_order maps position j of a run of n ids (n a
  // multiple of 8, the run starting at a multiple of 8) to the order in which
  // the work is laid out, so that each XCD takes a contiguous eighth of it: a
  // few heads at a time, their K and V fetched once for that XCD. Otherwise j
  // itself.
  auto xcd_order = [](int j, int n) { return (n & 7) == 0 ? (j & 7) * (n >> 3) + (j >> 3) : j; };
  const int nt = gridDim.x, nh = gridDim.y;
  // the slice of sequence b starts at a multiple of 8 exactly when nt nh is one
  const bool aligned = ((nt * nh) & 7) == 0;
  const int lin = blockIdx.x + nt * blockIdx.y;
  int hq, qt;
  if (!CAUSAL) {
    // head-major: the tiles of one head, then the next
    const int r = aligned ? xcd_order(lin, nt * nh) : lin;
    hq = r / nt;
    qt = r - hq * nt;
  } else {
    // Causal tiles differ in length (the last query tile sees every key). In
    // dispatch order, the tiles go in kCausalBands bands of decreasing length,
    // each band head-major: long work first and short work last across all
    // heads (no long tile starts near the end). The XCD order applies within a
    // band, so that every XCD gets the same mix of lengths.
    const int tpb = (nt + kCausalBands - 1) / kCausalBands;   // tiles per band
    const int band = lin / (nh * tpb);
    const int j = lin - nh * tpb * band;
    const int sz = min(tpb, nt - band * tpb);                 // tiles in this band
    const int r = aligned && ((nh * tpb) & 7) == 0 ? xcd_order(j, nh * sz) : j;
    hq = r / sz;
    qt = nt - 1 - (band * tpb + r % sz);                      // rank 0: the longest tile
  }

  // sequence geometry, clamped so that every access stays inside the buffers
  const const_i32* cq = (const const_i32*)p.cu_seqlens_q;
  const const_i32* ck = (const const_i32*)p.cu_seqlens_k;
  const int q0 = min(max(cq[b], 0), p.total_q);
  const int lq = min(max(cq[b + 1] - q0, 0), min(p.max_seqlen_q, p.total_q - q0));
  const int k0 = min(max(ck[b], 0), p.total_k);
  const int lk = min(max(ck[b + 1] - k0, 0), p.total_k - k0);
  const int i0 = qt * kTileRows;
  if (i0 >= lq) return;
  const int hkv = hq / (p.num_q_heads / p.num_kv_heads);
  const int rows_end = min(i0 + kTileRows, lq);
  // keys some row of the work-group (the wave) can see
  const int kv_end = CAUSAL ? min(max(lk - lq + rows_end, 0), lk) : lk;
  const int n_tiles = (kv_end + kStageKeys - 1) / kStageKeys;   // stages
  const int r0 = i0 + kRowsPerWave * w;              // this wave's first row
  const bool wave_rows = r0 < lq;
  const int kv_end_w = !wave_rows ? 0 : (CAUSAL ? min(max(lk - lq + min(r0 + kRowsPerWave, lq), 0), lk) : lk);
  const int row = r0 + col;                          // this lane's query row
  const bool row_ok = row < lq;

  const float c2 = *(const const_f32*)p.q_descale * *(const const_f32*)p.k_descale * p.scale_log2;

  // ---- Q^T operand: lane (col, h) holds dims 64 kc + 32 h .. + 31 of its row
  i32x8 qop[3];
  {
    const uint8_t* qrow = p.q + (int64_t)(q0 + (row_ok ? row : 0)) * p.q_stride_token + (int64_t)hq * p.q_stride_head;
#pragma unroll
    for (int kc = 0; kc < 3; ++kc) {
      const i32x4 lo = *(const i32x4*)(qrow + 64 * kc + 32 * h);
      const i32x4 hi = *(const i32x4*)(qrow + 64 * kc + 32 * h + 16);
      qop[kc] = row_ok ? i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]} : i32x8{};
    }
    // Consume Q here, so the compiler waits for these loads now. Left pending,
    // its wait would sit in the key loop as a full vmcnt(0), which also counts
    // the LDS transfers of the stages in flight and would drain the ring there.
    asm volatile("" ::"v"(qop[0]), "v"(qop[1]), "v"(qop[2]));
  }

  // ---- stage transfers: wave w moves parts w + 8 j (j < 5) of every stage;
  // part m is part m mod 20 of sub-tile m / 20 (K parts 0-11, V parts 12-19)
  const uint8_t* kbase = p.k + (int64_t)k0 * p.k_stride_token + (int64_t)hkv * p.k_stride_head;
  const uint8_t* vbase = p.v + (int64_t)k0 * p.v_stride_token + (int64_t)hkv * p.v_stride_head;
  const unsigned ring = lds_addr(smem);
  int x_key[kPartsPerWave];        // key of this lane's 16 bytes in the stage (0..127)
  int x_off[kPartsPerWave];        // byte offset inside that key's row
  bool x_isk[kPartsPerWave];
#pragma unroll
  for (int j = 0; j < kPartsPerWave; ++j) {
    const int m = w + kWaves * j, sub = m / kSubParts, mm = m - kSubParts * sub;
    if (mm < kKParts) {
      const int u = 64 * mm + lane;                   // 16-byte unit of the K sub-tile
      const int key = u / 12, pos = u - 12 * key;
      x_key[j] = kKeys * sub + key;
      x_off[j] = 16 * ((pos + 12 - k_rot(key)) % 12);
      x_isk[j] = true;
    } else {
      const int key = 8 * (mm - kKParts) + (lane >> 3), pos = lane & 7;
      x_key[j] = kKeys * sub + key;
      x_off[j] = 16 * (pos ^ v_sw(key));
      x_isk[j] = false;
    }
  }
  auto issue = [&](int t) {
    const int kt = kStageKeys * t;
    const unsigned stage = ring + (t % kStages) * kStageBytes;
#pragma unroll
    for (int j = 0; j < kPartsPerWave; ++j) {
      const int kg = min(kt + x_key[j], lk - 1);       // keys past the end read the last (masked)
      const uint8_t* src = x_isk[j] ? kbase + (int64_t)kg * p.k_stride_token : vbase + (int64_t)kg * p.v_stride_token;
      dma_1k_addr(src + x_off[j], stage + 1024 * (w + kWaves * j));
    }
  };
  if (n_tiles > 0) issue(0);
  if (n_tiles > 1) issue(1);

  // ---- per-lane LDS read offsets
  // K operand (S^T = K Q^T): key 32 kb + col, chunks 4 kc + 2 h and + 1
  // V^T operand (O^T = V^T P^T): source lane (gq, s = 2 k + hb) of instruction
  // mm reads the 8 bytes at +8 hb of dim block 2 dt + gq of key
  // 32 (mm >> 1) + 16 (mm & 1) + 8 (k >> 2) + 4 h + (k & 3); ds_read_b64_tr_b8
  // hands lane n of the group byte k of source lane 2 k + n / 8, so lane
  // (col, h) receives dim 32 dt + col of the keys of k-slots 32 h + 8 mm .. + 7.
  // The swizzle of a V row depends only on key bits 1 and 3, which the 16-key
  // steps of mm leave alone, so instruction mm reads at a per-lane base for
  // tile dt plus the constant (32 (mm >> 1) + 16 (mm & 1)) kDv, which the
  // instruction's immediate offset carries; likewise a K row's rotation
  // depends on key bits 2-3 only, so the second 32-key block is the first's
  // addresses plus 32 kDqk.
  int v_base[4];
  {
    const int gq = (lane >> 4) & 1, s = lane & 15, k = s >> 1, hb = s & 1;
    const int key = 8 * (k >> 2) + 4 * h + (k & 3);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) v_base[dt] = kKBytes + key * kDv + 16 * ((2 * dt + gq) ^ v_sw(key)) + 8 * hb;
  }
  int k_off[3][2];   // [kc][half]: chunk 4 kc + 2 h + half of key col, rotated
  {
    const int rot = k_rot(col);
#pragma unroll
    for (int kc = 0; kc < 3; ++kc)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) k_off[kc][hf] = 16 * (12 * col + (4 * kc + 2 * h + hf + rot) % 12);
  }

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m_ref = -__builtin_inff();     // reference max of this lane's row (log2 units)
  float thr = -__builtin_inff();       // raw-score threshold (m_ref + slack) / c2
  // row sum l = sum of the rounded, block-scaled P, from the matrix core: the
  // same MFMA as O^T with an all-ones A operand (every element of ol is l)
  f32x16 ol = f32x16{};
  i32x8 pb = {};   // P^T operand of the current sub-tile: e4m3 bytes of this lane's row
  i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};   // e4m3 1.0

  for (int t = 0; t < n_tiles; ++t) {
    // this wave's transfers of stage t have landed (stage t + 1 may fly), then
    // everyone's have, and everyone is done with the stage t + 2 reuses
    if (t + 1 < n_tiles)
      asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (t + 2 < n_tiles) issue(t + 2);
#pragma unroll 1
    for (int sub = 0; sub < kSubs; ++sub) {
      const int kt = kStageKeys * t + kKeys * sub;
      if (kt >= kv_end_w) break;                      // every key from here on is masked for this wave
      const uint8_t* stage = smem + (t % kStages) * kStageBytes + sub * kSubBytes;

      // scores: s[kb][r] = S^T[key 32 kb + 8 (r >> 2) + 4 h + (r & 3)][row]
      f32x16 sc[2];
      __builtin_amdgcn_s_setprio(1);
      const uint8_t* kp[3][2];
#pragma unroll
      for (int kc = 0; kc < 3; ++kc)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) kp[kc][hf] = stage + k_off[kc][hf];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sc[kb] = f32x16{};
#pragma unroll
        for (int kc = 0; kc < 3; ++kc) {
          const i32x4 lo = *(const i32x4*)(kp[kc][0] + 32 * kDqk * kb);
          const i32x4 hi = *(const i32x4*)(kp[kc][1] + 32 * kDqk * kb);
          const i32x8 ka = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          sc[kb] = mfma8(ka, qop[kc], sc[kb], 127, 127);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // masks: keys past the sequence, and (causal) past the row's diagonal
      const bool edge = kt + kKeys > lk || (CAUSAL && kt + kKeys - 1 > lk - lq + r0);
      if (edge) {
        // (the empty volatile asm keeps this a branch: the compiler would
        // otherwise turn it into per-score selects on every sub-tile)
        asm volatile("");
        const int lim = CAUSAL ? min(lk - 1, lk - lq + row) : lk - 1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
            sc[kb][r] = key <= lim ? sc[kb][r] : -__builtin_inff();
          }
      }
      // raw-score maxima of the two 32-key blocks and of the row (both lanes of
      // the row agree on all three)
      float bmx[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float x = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 16; ++r) x = fmaxf(x, sc[kb][r]);
        bmx[kb] = pair_max(x);
      }
      const float mx = fmaxf(bmx[0], bmx[1]);
      const bool move = mx > thr;
      if (__any(move)) {
        float alpha = 1.f;
        if (move) {
          const float m_new = mx * c2;
          alpha = __builtin_amdgcn_exp2f(m_ref - m_new);   // 0 when m_ref was -inf
          m_ref = m_new;
          thr = (m_new + kLazySlack) / c2;
        }
        ol *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
      // P = 2^(s c2 - m) (0 for a masked key) in e4m3 with a power-of-two scale
      // 2^e per block of 32 keys (block kb: this lane's bytes 16 kb .. + 15 and
      // its partner lane's): the block's largest P, 2^(bmx c2 - m), sets e so
      // that it lands in [128, 256), and 2^-e is folded into the exponent.
      // P never exceeds 2^8 (lazy max), so e <= 1; a block whose largest P is
      // below 2^-100 contributes nothing: its shift is +inf, so every P of it
      // is 2^-inf = 0, and e = 0, so e >= -107. A masked score (-inf) gives
      // 2^-inf = 0 as well; edge sub-tiles still zero masked keys explicitly,
      // which keeps them 0 even for a zero descale.
      const float mref = m_ref == -__builtin_inff() ? 0.f : m_ref;
      int eb[2];
      float shift[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // log2 of the block's largest P; e = floor of it - 7 puts that P in [128, 256)
        const float top2 = __builtin_fmaf(bmx[kb], c2, -mref);
        const bool live = top2 >= -100.f;
        eb[kb] = live ? (int)__builtin_floorf(top2) - 7 : 0;
        shift[kb] = live ? mref + (float)eb[kb] : __builtin_inff();
      }
      float pv[32];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pv[16 * kb + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r], c2, -shift[kb]));
      if (edge) {
        asm volatile("");   // a branch, as above
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            pv[16 * kb + r] = sc[kb][r] == -__builtin_inff() ? 0.f : pv[16 * kb + r];
      }
      // packed in place into the MFMA operand (loop-carried, so its registers
      // stay one tuple); both 16-bit halves of each word are written, so the
      // word's prior value is free
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pb[j] = __builtin_amdgcn_cvt_pk_fp8_f32(pv[4 * j], pv[4 * j + 1], pb[j], false);
        pb[j] = __builtin_amdgcn_cvt_pk_fp8_f32(pv[4 * j + 2], pv[4 * j + 3], pb[j], true);
      }
      const int e = h == 0 ? eb[0] : eb[1];   // the scale this lane supplies
      // O^T += V^T P^T over the sub-tile's 64 keys, four 32-dim tiles
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint8_t* vp = stage + v_base[dt];
        i32x2 vr[4];
#pragma unroll
        for (int mm = 0; mm < 4; ++mm)
          vr[mm] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vp + (32 * (mm >> 1) + 16 * (mm & 1)) * kDv));
        const i32x4 v01 = __builtin_shufflevector(vr[0], vr[1], 0, 1, 2, 3);
        const i32x4 v23 = __builtin_shufflevector(vr[2], vr[3], 0, 1, 2, 3);
        const i32x8 va = __builtin_shufflevector(v01, v23, 0, 1, 2, 3, 4, 5, 6, 7);
        o[dt] = mfma8(va, pb, o[dt], 127, 127 + e);
      }
      // (the empty asm makes ones opaque, so it stays resident in registers
      // across sub-tiles instead of being rebuilt by moves every time)
      asm volatile("" : "+v"(ones));
      ol = mfma8(ones, pb, ol, 127, 127 + e);
      __builtin_amdgcn_s_setprio(0);
    }
  }

  // ---- epilogue: o = O / l (0 without a visible key), bf16 out, optional lse
  if (!wave_rows) return;
  const float l = ol[0];
  if (!row_ok) return;
  const float inv = l > 0.f ? *(const const_f32*)p.v_descale / l : 0.f;
  uint16_t* dst = p.out + (int64_t)(q0 + row) * p.out_stride_token + (int64_t)hq * p.out_stride_head;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d = 32 * dt + 8 * c + 4 * h;
      const uint32_t lo = bf16_rne(o[dt][4 * c] * inv) | (bf16_rne(o[dt][4 * c + 1] * inv) << 16);
      const uint32_t hi = bf16_rne(o[dt][4 * c + 2] * inv) | (bf16_rne(o[dt][4 * c + 3] * inv) << 16);
      *(uint2*)(dst + d) = make_uint2(lo, hi);
    }
  if (p.lse != nullptr && h == 0)
    p.lse[(int64_t)hq * p.total_q + q0 + row] =
        l > 0.f ? (m_ref + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -__builtin_inff();
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.max_seqlen_q + kTileRows - 1) / kTileRows), (unsigned)p.num_q_heads,
                  (unsigned)p.num_seqs);
  if (p.causal)
    hipLaunchKernelGGL(prefill_kernel<true>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_kernel<false>, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pfkv
