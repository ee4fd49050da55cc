// Paged KV append (slot-mapping scatter) and copy-on-write block copy.
//
// Both are byte copies in 16-byte vectors; bits are preserved exactly.
//  - append: the newest token of a sequence is written into the slot of the
//    block its sequence is filling (vLLM/PagedAttention paged-KV analysis page,
//    section 3.2; vLLM entity page, "what it is": blocks are taken on demand).
//  - block copy: a block shared by several sequences is duplicated before one
//    of them writes into it (same page, sections 2.3 and 3.2).  All pairs go in
//    one launch: many small per-block copies are what makes KV movement slow
//    (vLLM entity page, key observations).
//  - swap out / swap in: every block of a preempted request moves between the
//    pools and pinned host memory (Cross-Paper Synthesis page, section 3, the
//    preemption item), again in one launch per block list, into a block-first
//    host layout (entry i = K tile then V tile of block ids[i]) so one
//    request's KV is one contiguous host run (vLLM entity page, key
//    observations).  The GPU's own loads and stores cross the host link; the
//    scattered pool side is read or written in whole tiles.
#include "pa_common.hpp"
#include "pa_launch.hpp"

namespace pa {

// One thread moves one 16-byte chunk of one (token, head) row of K and of V.
// grid-stride over num_tokens * num_kv_heads * chunks_per_row.  The new rows
// are read once and the pool is streamed through by the next decode call, so
// loads and stores carry the non-temporal hint.
#ifndef PA_APPEND_NT
#define PA_APPEND_NT 1
#endif
constexpr int kAppendAux = PA_APPEND_NT ? kStreamAux : kAuxDefault;
__global__ __launch_bounds__(256) void kv_append_kernel(
    const u32x4* __restrict__ key, const u32x4* __restrict__ value, u32x4* __restrict__ k_pool,
    u32x4* __restrict__ v_pool, const int64_t* __restrict__ slot_mapping, int64_t total_chunks,
    int32_t num_kv_heads, int32_t chunks_per_row, int32_t block_size, int64_t num_slots) {
  const int64_t per_token = (int64_t)num_kv_heads * chunks_per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_chunks;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / per_token;
    const int32_t r = (int32_t)(i - t * per_token);
    const int64_t slot = slot_mapping[t];
    PA_FLAG_IF(slot >= num_slots, kViolationSlot);
    if (slot < 0 || slot >= num_slots) continue;
    const int32_t h = r / chunks_per_row;
    const int32_t c = r - h * chunks_per_row;
    const int64_t b = slot / block_size;
    const int32_t o = (int32_t)(slot - b * block_size);
    const int64_t dst = ((b * num_kv_heads + h) * block_size + o) * chunks_per_row + c;
    const u32x4 kv = ld16_aux<kAppendAux>(key + i);
    const u32x4 vv = ld16_aux<kAppendAux>(value + i);
    st16_aux<kAppendAux>(k_pool + dst, kv);
    st16_aux<kAppendAux>(v_pool + dst, vv);
  }
}

// One workgroup per (pair, K-or-V); each thread moves kChunksPerThread 16-byte
// chunks per iteration, loads first then stores, to keep several in flight.
constexpr int kCopyThreads = 256;
constexpr int kChunksPerThread = 4;

__global__ __launch_bounds__(kCopyThreads) void block_copy_kernel(
    u32x4* __restrict__ k_pool, u32x4* __restrict__ v_pool, const int32_t* __restrict__ block_mapping,
    int32_t chunks_per_block, int32_t num_blocks) {
  const int32_t pair = blockIdx.x >> 1;
  u32x4* pool = (blockIdx.x & 1) ? v_pool : k_pool;
  const int32_t src = block_mapping[2 * pair];
  const int32_t dst = block_mapping[2 * pair + 1];
  PA_FLAG_IF(src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks, kViolationBlockId);
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const u32x4* s = pool + (int64_t)src * chunks_per_block;
  u32x4* d = pool + (int64_t)dst * chunks_per_block;
  constexpr int step = kCopyThreads * kChunksPerThread;
  for (int32_t base = 0; base < chunks_per_block; base += step) {
    u32x4 tmp[kChunksPerThread];
#pragma unroll
    for (int j = 0; j < kChunksPerThread; ++j) {
      const int32_t c = base + j * kCopyThreads + threadIdx.x;
      if (c < chunks_per_block) tmp[j] = s[c];
    }
#pragma unroll
    for (int j = 0; j < kChunksPerThread; ++j) {
      const int32_t c = base + j * kCopyThreads + threadIdx.x;
      if (c < chunks_per_block) d[c] = tmp[j];
    }
  }
}

// One workgroup per (list entry, K-or-V): moves one (block, all heads) tile
// between its pool and its place in the block-first host buffer.  Eight
// 16-byte chunks per thread in flight (32 KiB per workgroup) to cover the
// host link's latency.  OUT: pool -> host; otherwise host -> pool.
constexpr int kSwapChunksPerThread = 8;

template <bool OUT>
__global__ __launch_bounds__(kCopyThreads) void swap_kernel(u32x4* __restrict__ k_pool,
                                                            u32x4* __restrict__ v_pool,
                                                            u32x4* __restrict__ host,
                                                            const int32_t* __restrict__ block_ids,
                                                            int32_t chunks_per_block, int32_t num_blocks) {
  const int32_t entry = blockIdx.x >> 1;
  const int32_t kv = blockIdx.x & 1;
  const int32_t id = block_ids[entry];
  PA_FLAG_IF(id < 0 || id >= num_blocks, kViolationBlockId);
  if (id < 0 || id >= num_blocks) return;
  u32x4* pool = (kv ? v_pool : k_pool) + (int64_t)id * chunks_per_block;
  u32x4* h = host + ((int64_t)entry * 2 + kv) * chunks_per_block;
  const u32x4* s = OUT ? pool : h;
  u32x4* d = OUT ? h : pool;
  constexpr int step = kCopyThreads * kSwapChunksPerThread;
  for (int32_t base = 0; base < chunks_per_block; base += step) {
    u32x4 tmp[kSwapChunksPerThread];
#pragma unroll
    for (int j = 0; j < kSwapChunksPerThread; ++j) {
      const int32_t c = base + j * kCopyThreads + threadIdx.x;
      if (c < chunks_per_block) tmp[j] = s[c];
    }
#pragma unroll
    for (int j = 0; j < kSwapChunksPerThread; ++j) {
      const int32_t c = base + j * kCopyThreads + threadIdx.x;
      if (c < chunks_per_block) d[c] = tmp[j];
    }
  }
}

hipError_t launch_swap(bool out, void* k_pool, void* v_pool, void* host, const int32_t* block_ids,
                       int32_t num_ids, int64_t block_bytes, int32_t num_blocks, hipStream_t stream) {
  const int32_t chunks = (int32_t)(block_bytes / 16);
  auto kern = out ? swap_kernel<true> : swap_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(2 * num_ids), dim3(kCopyThreads), 0, stream,
                     reinterpret_cast<u32x4*>(k_pool), reinterpret_cast<u32x4*>(v_pool),
                     reinterpret_cast<u32x4*>(host), block_ids, chunks, num_blocks);
  return hipGetLastError();
}

// Streaming read of a buffer (the measurement's achievable-bandwidth line):
// workgroup b sweeps its own contiguous range of 16-byte chunks, eight loads
// in flight per thread, folding every 32-bit word into an XOR so no load can
// be dropped; one partial per workgroup.  Contiguous ranges streamed 4-10 %
// faster than a grid-stride sweep, and 16384 workgroups of eight loads were
// the fastest of the shapes tried; the non-temporal hint lifts the sweep from
// about 6.3 to 7.1 TB/s.
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* __restrict__ p, uint64_t n16,
                                                                     uint32_t* __restrict__ partials) {
  uint32_t acc = 0;
  const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const uint64_t lo = (uint64_t)blockIdx.x * per;
  const uint64_t hi = lo + per < n16 ? lo + per : n16;
  uint64_t i = lo + threadIdx.x;
  for (; i + (kStreamUnroll - 1) * kStreamThreads < hi; i += kStreamUnroll * kStreamThreads) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = ld16_stream(p + i + u * kStreamThreads);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += kStreamThreads) {
    const u32x4 v = ld16_stream(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, kWave);
  __shared__ uint32_t wave_acc[kStreamThreads / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) wave_acc[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w = 0; w < kStreamThreads / kWave; ++w) x ^= wave_acc[w];
    partials[blockIdx.x] = x;
  }
}

hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* partials, int32_t num_partials,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(num_partials), dim3(kStreamThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(buf), bytes / 16, partials);
  return hipGetLastError();
}

hipError_t launch_kv_append(const void* key, const void* value, void* k_pool, void* v_pool,
                            const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                            int32_t row_bytes, int32_t block_size, int32_t num_blocks,
                            hipStream_t stream) {
  const int32_t chunks_per_row = row_bytes / 16;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * chunks_per_row;
  const int64_t want = (total + 255) / 256;
  const int32_t grid = (int32_t)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(kv_append_kernel, dim3(grid), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(key), reinterpret_cast<const u32x4*>(value),
                     reinterpret_cast<u32x4*>(k_pool), reinterpret_cast<u32x4*>(v_pool), slot_mapping,
                     total, num_kv_heads, chunks_per_row, block_size,
                     (int64_t)num_blocks * block_size);
  return hipGetLastError();
}

hipError_t launch_block_copy(void* k_pool, void* v_pool, const int32_t* block_mapping,
                             int32_t num_pairs, int64_t block_bytes, int32_t num_blocks,
                             hipStream_t stream) {
  const int32_t chunks = (int32_t)(block_bytes / 16);
  hipLaunchKernelGGL(block_copy_kernel, dim3(2 * num_pairs), dim3(kCopyThreads), 0, stream,
                     reinterpret_cast<u32x4*>(k_pool), reinterpret_cast<u32x4*>(v_pool),
                     block_mapping, chunks, num_blocks);
  return hipGetLastError();
}

PA_VIOLATIONS_GETTER(debug_violations_copy)

}  // namespace pa
