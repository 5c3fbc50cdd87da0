// Streaming-read microbenchmark kernels: the practical HBM read ceiling that the
// verify-attention bandwidth is measured against (aiter PR #5190, Microbenchmark:
// a streaming-read microbenchmark sets the device's practical read ceiling).
//
// Every variant reads the buffer as 4 KiB blocks, each wave of 8 per work-group
// taking blocks gw, gw + nw, ... (gw its global wave index, nw the waves of the
// grid), one work-group per CU:
//   variant 0: blocks in address order, 16-byte vector loads into registers;
//   variant 1: blocks in address order through LDS with global_load_lds_dwordx4
//              (a 3-block ring per wave; each block is read back from LDS);
//   variant 2: as 1, blocks in a caller-given order (e.g. a random permutation);
//   variant 3: as 0, blocks in a caller-given order.
// Each variant XORs every 32-bit word it reads and folds the result into
// *sink with one atomic XOR per wave, so a caller who zeroes the sink can check
// that every byte was read once (the XOR of the whole buffer, whatever the order
// when the order is a permutation of all blocks).
#include "pfkv_internal.h"

namespace pfkv {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kRing = 3;   // LDS blocks per wave in flight (variants 1, 2)

__device__ __forceinline__ uint32_t xor4(const u32x4& v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

// wave-wide XOR, then one atomic per wave
__device__ __forceinline__ void fold_into_sink(uint32_t x, uint32_t* sink) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, x);
}

// block index i of the read order, clamped into the buffer
template <bool kOrdered>
__device__ __forceinline__ int64_t block_id(const int32_t* order, int64_t i, int64_t buf_blocks) {
  int64_t id = kOrdered ? (int64_t)__builtin_amdgcn_readfirstlane(((const __attribute__((address_space(4))) int32_t*)order)[i]) : i;
  return id < 0 ? 0 : (id >= buf_blocks ? buf_blocks - 1 : id);
}

template <bool kOrdered>
__global__ void __launch_bounds__(64 * kWaves) stream_vec_kernel(const uint8_t* __restrict__ buf,
                                                                 const int32_t* __restrict__ order,
                                                                 int64_t num_blocks, int64_t buf_blocks,
                                                                 uint32_t* sink) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * kWaves + w, nw = (int64_t)gridDim.x * kWaves;
  uint32_t x = 0;
  for (int64_t i = gw; i < num_blocks; i += nw) {
    const u32x4* src = (const u32x4*)(buf + block_id<kOrdered>(order, i, buf_blocks) * 4096);
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = __builtin_nontemporal_load(src + 64 * j + lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) x ^= xor4(v[j]);
  }
  fold_into_sink(x, sink);
}

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

template <bool kOrdered>
__global__ void __launch_bounds__(64 * kWaves) stream_dma_kernel(const uint8_t* __restrict__ buf,
                                                                 const int32_t* __restrict__ order,
                                                                 int64_t num_blocks, int64_t buf_blocks,
                                                                 uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kWaves][kRing][4096];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const unsigned base = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)&ring[w][0][0];
  const int64_t gw = (int64_t)blockIdx.x * kWaves + w, nw = (int64_t)gridDim.x * kWaves;
  uint32_t x = 0;
  auto consume = [&](int slot) {
#pragma unroll
    for (int j = 0; j < 4; ++j) x ^= xor4(*(const u32x4*)&ring[w][slot][1024 * j + 16 * lane]);
  };
  int it = 0;
  for (int64_t i = gw; i < num_blocks; i += nw, ++it) {
    const uint8_t* src = buf + block_id<kOrdered>(order, i, buf_blocks) * 4096;
    const unsigned dst = base + (it % kRing) * 4096;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma_1k(src, (unsigned)(1024 * j + 16 * lane), dst + 1024 * j);
    if (it >= kRing - 1) {
      // the block issued kRing - 1 iterations ago has landed; the later ones may fly
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      consume((it - (kRing - 1)) % kRing);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  for (int k = it - (kRing - 1) < 0 ? 0 : it - (kRing - 1); k < it; ++k) consume(k % kRing);
  fold_into_sink(x, sink);
}

}  // namespace

hipError_t launch_stream_read(const void* buf, uint64_t bytes, int variant, const int32_t* page_order,
                              int64_t num_pages, uint32_t* sink, hipStream_t stream) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t blocks = (int64_t)(bytes / 4096);
  const uint8_t* b = (const uint8_t*)buf;
  const dim3 grid(cus), block(64 * kWaves);
  switch (variant) {
    case 0: hipLaunchKernelGGL(stream_vec_kernel<false>, grid, block, 0, stream, b, nullptr, blocks, blocks, sink); break;
    case 1: hipLaunchKernelGGL(stream_dma_kernel<false>, grid, block, 0, stream, b, nullptr, blocks, blocks, sink); break;
    case 2: hipLaunchKernelGGL(stream_dma_kernel<true>, grid, block, 0, stream, b, page_order, num_pages, blocks, sink); break;
    case 3: hipLaunchKernelGGL(stream_vec_kernel<true>, grid, block, 0, stream, b, page_order, num_pages, blocks, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pfkv
