// Split-KV main kernel for verify attention over a paged fp8 KV cache (gfx950).
//
// What it computes follows aiter PR #5190 ("gfx950 assembly MTP-verify attention
// for head_dim 256 fp8 paged KV"), sections Modifications and Kernel notes: one
// work-group per (KV segment, sequence, KV head), partial softmax statistics per
// segment to a workspace, empty segments written neutrally, descales read from
// device pointers. In-kernel q_len 1..4 follows SGLang PR #37465, Modifications.
// The decomposition is this library's own:
//
// * 4 waves per work-group, one per SIMD. A step covers 4 pages (64 keys): wave
//   w streams page w of the step HBM -> LDS and computes its 16 keys' scores
//   against all G * q_len (<= 64) stacked query rows; for P V every wave covers
//   all 64 keys but only its own 64 of the 256 output dims, so the fp32
//   accumulator is 64 registers per lane and no work is duplicated.
// * K/V pages move with global_load_lds_dwordx4 (1 KiB contiguous per
//   instruction) issued from inline asm, so the compiler does not serialise LDS
//   reads behind every outstanding transfer; a 3-stage ring keeps two steps
//   (64 KiB per work-group) in flight, with explicit vmcnt waits.
// * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: K converts exactly from e4m3fn to
//   bf16 (v_cvt_scalef32_pk_bf16_fp8, scale 1), Q stays bf16. The score layout
//   puts one query row per lane column: row maxima need one in-lane reduction and
//   two cross-lane steps.
// * Online softmax in the log2 domain with a lazy reference max m per row: m
//   moves only when a row's running max exceeds it by more than 8, so
//   P = 2^(s - m) <= 2^8 fits fp16 and the accumulator is rescaled rarely. Each
//   wave computes P against the current m and publishes it with its local row
//   maxima; one barrier per step. If any wave saw a row exceed m + 8, all waves
//   take the (rare) slow path: new m from the step's maxima, rescale, recompute
//   P, second barrier. Rows that did not need it keep m and get bit-identical P,
//   so each row's arithmetic depends only on that row.
// * P is rounded to fp16 once; the same values feed the row sum l and P V.
// * O += P V on v_mfma_f32_16x16x32_f16. V's transposed operand comes from
//   ds_read_b64_tr_b8 and converts exactly to fp16.
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
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(4))) const int32_t const_i32;
typedef __attribute__((address_space(4))) const float const_f32;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPagesPerStep = kWaves;                  // one page per wave per step
constexpr int kStages = 3;                             // LDS ring depth
constexpr int kPageBytes = kPageSize * kHeadDim;       // one (page, head) block of K or V: 4 KiB
constexpr int kStageBytes = 2 * kPagesPerStep * kPageBytes;   // K and V of the step: 32 KiB
constexpr int kDmaPerPage = 2 * kPageBytes / 1024;     // 8 x 1 KiB (K and V)
constexpr int kDimsPerWave = kHeadDim / kWaves;        // 64
constexpr float kLazySlack = 8.0f;                     // log2 units

template <int G>
struct Cfg {
  static constexpr int kRowBlocks = G * kMaxQLen / 16;            // 16-row MFMA blocks
  static constexpr int kRows = kRowBlocks * 16;
  static constexpr int kQBytes = kRows * kHeadDim * 2;             // bf16 Q rows
  static constexpr int kPBytes = kRowBlocks * kWaves * 64 * 8;     // fp16 P of one step
  static constexpr int kMxBytes = kWaves * kRows * 4;              // per-wave row maxima of one step
  static constexpr int kOffP = kQBytes;                            // two P buffers
  static constexpr int kOffMx = kOffP + 2 * kPBytes;               // two maxima buffers
  static constexpr int kOffFlag = kOffMx + 2 * kMxBytes;           // two flag words per wave
  static constexpr int kOffStage = kOffFlag + 64;
  static constexpr int kLdsBytes = kOffStage + kStages * kStageBytes;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
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

// Wait until at most `pending` of this wave's vector-memory operations are in
// flight. Inside the main loop the only such operations are the page transfers.
__device__ __forceinline__ void wait_vm(int pending) {
  if (pending >= 8)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
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

template <int G>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
splitkv_main_kernel(MainParams p) {
  using C = Cfg<G>;
  constexpr int RB = C::kRowBlocks;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kLdsBytes];

  const int seg = blockIdx.x, b = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, n = lane & 15;

  const const_i32* cu = (const const_i32*)p.cu_seqlens_q;
  const const_i32* sl = (const const_i32*)p.seq_lens;
  const const_i32* bt = (const const_i32*)p.block_tables;

  // ---- sequence geometry (uniform); out-of-contract values are clamped so that
  // every access stays inside its buffer.
  const int q0 = cu[b];
  int q_len = cu[b + 1] - q0;
  if (q0 < 0 || q0 >= p.total_q) q_len = 0;
  q_len = min(max(q_len, 0), min(kMaxQLen, p.total_q - max(q0, 0)));
  if (q_len <= 0) return;
  const int L = min(max(sl[b], 0), p.max_pages_per_seq * kPageSize);
  const int pages = (L + kPageSize - 1) / kPageSize;
  const int chunk = (pages + p.num_segments - 1) / p.num_segments;
  const int pb = min(seg * chunk, pages);
  const int pe = min(pb + chunk, pages);
  const int rows = G * q_len;
  const int n_steps = (pe - pb + kPagesPerStep - 1) / kPagesPerStep;
  const float c2 = *(const const_f32*)p.k_descale * p.score_scale_log2;

  const int64_t bt_row = (int64_t)b * p.block_table_stride;
  const uint64_t page_stride = (uint64_t)kPageSize * p.num_kv_heads * kHeadDim;

  // ---- per-lane DMA offsets inside one (page, head) block. In LDS, the
  // 16-byte chunk at position pos of key row k (page slot j) holds dim chunk
  // pos ^ sw(k, j), sw(k, j) = (k ^ 12 (j & 1)) & 15: K row reads and V
  // transposed reads are then free of bank conflicts.
  const int jpar = w & 1;
  unsigned goff[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int k = 4 * jj + g;
    goff[jj] = (unsigned)((k * p.num_kv_heads + h) * kHeadDim + 16 * (n ^ ((k ^ (12 * jpar)) & 15)));
  }
  uint8_t* const stage0 = smem + C::kOffStage;
  const unsigned stage0_lds = lds_addr(stage0);

  auto issue_step = [&](int t) {
    const int pidx = pb + kPagesPerStep * t + w;
    if (pidx < pe) {
      int id = bt[bt_row + pidx];
      id = min(max(id, 0), p.num_pages - 1);
      const uint8_t* kbase = p.k_cache + (uint64_t)id * page_stride;
      const uint8_t* vbase = p.v_cache + (uint64_t)id * page_stride;
      const unsigned dst = stage0_lds + (t % kStages) * kStageBytes + w * kPageBytes;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        dma_1k(kbase, goff[jj], dst + 1024 * jj);
        dma_1k(vbase, goff[jj], dst + kPagesPerStep * kPageBytes + 1024 * jj);
      }
    }
  };
  auto has_page = [&](int t) -> bool { return t < n_steps && pb + kPagesPerStep * t + w < pe; };

  // ---- prologue: two steps in flight, then stage Q while they land.
  issue_step(0);
  if (n_steps > 1) issue_step(1);

  // Q rows r = i * G + gg (query i of the sequence, head h * G + gg); row r's
  // 16-byte chunk c16 sits at position c16 ^ (r & 15).
  // All loads are issued before any LDS write so their latencies overlap.
  constexpr int kQChunks = C::kRows * 32 / kThreads;
  u32x4 qv[kQChunks];
#pragma unroll
  for (int c = 0; c < kQChunks; ++c) {
    const int idx = tid + c * kThreads;
    const int r = idx >> 5, c16 = idx & 31;
    // padding rows load row 0 (always valid) and are zeroed below: no branch
    const int rr = r < rows ? r : 0;
    const int i = rr / G, gg = rr - (rr / G) * G;
    const uint16_t* src = p.q + (int64_t)(q0 + i) * p.q_stride_token + (int64_t)(h * G + gg) * p.q_stride_head;
    qv[c] = *(const u32x4*)(src + 8 * c16);
  }
#pragma unroll
  for (int c = 0; c < kQChunks; ++c) {
    const int r = (tid + c * kThreads) >> 5;
    if (r >= rows) qv[c] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int c = 0; c < kQChunks; ++c) {
    const int idx = tid + c * kThreads;
    const int r = idx >> 5, c16 = idx & 31;
    *(u32x4*)(smem + r * 512 + 16 * (c16 ^ (r & 15))) = qv[c];
  }
  __syncthreads();

  // ---- per-lane LDS read offsets
  const unsigned kcol = 16u * ((g ^ n ^ (12 * jpar)) & 15);
  unsigned qcol[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) qcol[hh] = 16u * ((2 * g + hh) ^ n);
  // V^T operand: source lane n of group g supplies the 8 dims at +8 (n & 1) of
  // key 4g + ((n >> 1) & 3) in page slot 2 ks + (n >> 3), the k-slot (n >> 1)
  // of group g; ds_read_b64_tr_b8 hands lane n byte k of source lane 2k + n/8.
  const int vpar = (n >> 3) & 1;
  const int vkey = 4 * g + ((n >> 1) & 3);
  const unsigned vrow = (unsigned)(kPagesPerStep * kPageBytes + vpar * kPageBytes + 256 * vkey + 8 * (n & 1));
  const unsigned vsw = 16u * ((vkey ^ (12 * vpar)) & 15);

  f32x4 acc[RB][4];
  float m_ref[RB], l_lane[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_ref[rb] = -__builtin_inff();
    l_lane[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int t = 0; t < n_steps; ++t) {
    const int st = t % kStages, buf = t & 1;
    const uint8_t* sp = stage0 + st * kStageBytes;
    const int pidx = pb + kPagesPerStep * t + w;        // this wave's page
    const bool mine = pidx < pe;
    wait_vm(has_page(t + 1) ? kDmaPerPage : 0);

    // ---- S^T[key][row] = K Q^T for this wave's page (k-slots permuted consistently)
    float sv[RB][4];
    if (mine) {
      f32x4 sacc[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x4 raw = *(const u32x4*)(sp + w * kPageBytes + 256 * n + (kcol ^ (64u * u)));
        const bf16x8 k0 = fp8x8_to_bf16(raw[0], raw[1]);
        const bf16x8 k1 = fp8x8_to_bf16(raw[2], raw[3]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const uint8_t* qrow = smem + 8192 * rb + 512 * n;
          const bf16x8 qa = *(const bf16x8*)(qrow + (qcol[0] ^ (128u * u)));
          const bf16x8 qb = *(const bf16x8*)(qrow + (qcol[1] ^ (128u * u)));
          sacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qa, sacc[rb], 0, 0, 0);
          sacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qb, sacc[rb], 0, 0, 0);
        }
      }
      // scale to log2 units; mask keys past the row's causal limit or the sequence
      const bool need_mask = kPageSize * (pidx + 1) > L - q_len + 1;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int i = (16 * rb + n) / G;
        const int lim = min(L - 1, L - q_len + i);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float s = sacc[rb][r] * c2;
          const int key = kPageSize * pidx + 4 * g + r;
          sv[rb][r] = (!need_mask || key <= lim) ? s : -__builtin_inff();
        }
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[rb][r] = -__builtin_inff();
    }

    // ---- local row maxima, slow-path flag, P against the current reference
    float* mx_buf = (float*)(smem + C::kOffMx + buf * C::kMxBytes);
    int* flags = (int*)(smem + C::kOffFlag) + buf * kWaves;
    uint8_t* p_buf = smem + C::kOffP + buf * C::kPBytes;
    bool over = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = fmaxf(fmaxf(sv[rb][0], sv[rb][1]), fmaxf(sv[rb][2], sv[rb][3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      over |= mx > m_ref[rb] + kLazySlack;
      if (g == 0) mx_buf[w * C::kRows + 16 * rb + n] = mx;
    }
    const bool wave_over = __any(over);
    if (lane == 0) flags[w] = wave_over ? 1 : 0;

    f16x4 pv[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float mref = m_ref[rb] == -__builtin_inff() ? 0.f : m_ref[rb];
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[rb][r] = (_Float16)__builtin_amdgcn_exp2f(sv[rb][r] - mref);
      *(f16x4*)(p_buf + ((rb * kWaves + w) * 64 + lane) * 8) = pv[rb];
    }
    lds_barrier();

    if (flags[0] | flags[1] | flags[2] | flags[3]) {
      // slow path (uniform over the work-group): move m where a row's step max
      // exceeds it by more than the slack, rescale, recompute and republish P
      float alpha[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float M = mx_buf[0 * C::kRows + 16 * rb + n];
#pragma unroll
        for (int v = 1; v < kWaves; ++v) M = fmaxf(M, mx_buf[v * C::kRows + 16 * rb + n]);
        alpha[rb] = 1.f;
        if (M > m_ref[rb] + kLazySlack) {
          alpha[rb] = __builtin_amdgcn_exp2f(m_ref[rb] - M);   // 0 when m was -inf
          m_ref[rb] = M;
        }
        l_lane[rb] *= alpha[rb];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = __shfl(alpha[rb], 4 * g + r, 64);   // lane 4g+r holds row 4g+r
#pragma unroll
          for (int db = 0; db < 4; ++db) acc[rb][db][r] *= a;
        }
        const float mref = m_ref[rb] == -__builtin_inff() ? 0.f : m_ref[rb];
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[rb][r] = (_Float16)__builtin_amdgcn_exp2f(sv[rb][r] - mref);
      }
      // nobody reads this step's P before the barrier below
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) *(f16x4*)(p_buf + ((rb * kWaves + w) * 64 + lane) * 8) = pv[rb];
      lds_barrier();
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      l_lane[rb] += ((float)pv[rb][0] + (float)pv[rb][1]) + ((float)pv[rb][2] + (float)pv[rb][3]);

    // every wave is past step t-1: its stage can take step t+2
    if (t + 2 < n_steps) issue_step(t + 2);

    // ---- O[:, own dims] += P V over the step's 64 keys (two k-steps of 32).
    // k-slot 8g + e of k-step ks is key 4g + (e & 3) of page slot 2 ks + (e >> 2).
    // keys of pages past the segment (never loaded: stale or uninitialised LDS)
    // and past the sequence end get V = 0, so that P = 0 never meets a NaN
    const int step_end = pb + kPagesPerStep * (t + 1);
    const bool mask_v = step_end > pe || kPageSize * step_end > L;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f16x8 pa[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const f16x4 lo = *(const f16x4*)(p_buf + ((rb * kWaves + 2 * ks) * 64 + lane) * 8);
        const f16x4 hi = *(const f16x4*)(p_buf + ((rb * kWaves + 2 * ks + 1) * 64 + lane) * 8);
        pa[rb] = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      bool keep[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int page = pb + kPagesPerStep * t + 2 * ks + (e >> 2);
        const int key = kPageSize * page + 4 * g + (e & 3);
        keep[e] = !mask_v || (page < pe && key < L);
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const unsigned off = vrow + 2u * ks * kPageBytes + ((unsigned)(kDimsPerWave * w + 16 * db) ^ vsw);
        const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(sp + off));
        f16x8 vf = fp8x8_to_f16((unsigned)raw[0], (unsigned)raw[1]);
        if (mask_v) {
#pragma unroll
          for (int e = 0; e < 8; ++e) vf[e] = keep[e] ? vf[e] : (_Float16)0.f;
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[rb], vf, acc[rb][db], 0, 0, 0);
      }
    }
  }

  // ---- partials of this segment: m is identical in every wave; l sums the
  // waves' key subsets in a fixed order; each wave writes its own dims of acc.
  __syncthreads();   // all transfers have landed (last step waited vmcnt(0)); LDS is free
  float* lsum = (float*)smem;                 // [wave][row]
  float* mrow = lsum + kWaves * C::kRows;     // [row]
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float l = l_lane[rb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (g == 0) {
      lsum[w * C::kRows + 16 * rb + n] = l;
      if (w == 0) mrow[16 * rb + n] = m_ref[rb];
    }
  }
  __syncthreads();

  const int T = p.total_q, Hq = p.num_q_heads;
  if (tid < rows) {
    const int row = tid;
    float l = lsum[row];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) l += lsum[v * C::kRows + row];
    const int i = row / G, gg = row - (row / G) * G;
    float* dst = p.ws_ml + (((int64_t)seg * T + q0 + i) * Hq + h * G + gg) * 2;
    dst[0] = mrow[row];
    dst[1] = l;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * rb + 4 * g + r;
      if (row < rows) {
        const int i = row / G, gg = row - (row / G) * G;
        float* dst = p.ws_acc + (((int64_t)seg * T + q0 + i) * Hq + h * G + gg) * kHeadDim + kDimsPerWave * w + n;
#pragma unroll
        for (int db = 0; db < 4; ++db) dst[16 * db] = acc[rb][db][r];
      }
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
