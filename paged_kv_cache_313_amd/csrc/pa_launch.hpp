// Host-side launch entry points of the libpagedkv kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct DecodeArgs;
struct GroupArgs;

enum class Elem { F32 = 0, F16 = 1, BF16 = 2 };

hipError_t launch_kv_append(const void* key, const void* value, void* k_pool, void* v_pool,
                            const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                            int32_t row_bytes, int32_t block_size, int32_t num_blocks,
                            hipStream_t stream);

// Swap: out = pool tiles of block_ids -> block-first host buffer; else back.
// `host` is the device-side address of pinned host memory.
hipError_t launch_swap(bool out, void* k_pool, void* v_pool, void* host, const int32_t* block_ids,
                       int32_t num_ids, int64_t block_bytes, int32_t num_blocks, hipStream_t stream);

hipError_t launch_block_copy(void* k_pool, void* v_pool, const int32_t* block_mapping,
                             int32_t num_pairs, int64_t block_bytes, int32_t num_blocks,
                             hipStream_t stream);

// Workgroups of `kernel` (block of `block_threads`) that the current device
// keeps resident at once, at most max_per_cu per compute unit (0: no cap) and
// max_wg in all; cached per kernel/device.
hipError_t balanced_grid(const void* kernel, int block_threads, int max_per_cu, int max_wg, int* nwg);

// Streaming read of bytes (a multiple of 16) at buf, one XOR partial per
// workgroup into partials[0 .. num_partials).
hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* partials, int32_t num_partials,
                              hipStream_t stream);

// Decode: the segment kernel of the chosen mode plus, when results are split,
// its merge kernel.  f16/bf16 with group size 2..16 run the MFMA core, all
// other cases the VALU core.  With prefix groups (fixed partitions) the
// matrix-core P.V path runs the grouped kernel instead.
hipError_t launch_decode(const DecodeArgs& args, Elem elem, int head_dim, int block_size,
                         int group, hipStream_t stream, const GroupArgs* groups = nullptr);
// the same, one per storage type (separate translation units)
hipError_t launch_decode_f32(const DecodeArgs& args, int head_dim, int block_size, int group, hipStream_t stream,
                             const GroupArgs* groups);
hipError_t launch_decode_f16(const DecodeArgs& args, int head_dim, int block_size, int group, hipStream_t stream,
                             const GroupArgs* groups);
hipError_t launch_decode_bf16(const DecodeArgs& args, int head_dim, int block_size, int group, hipStream_t stream,
                              const GroupArgs* groups);

// Contract-violation flags of each translation unit (zero unless built with
// PA_DEBUG_CHECKS=1); read, and cleared when asked, synchronously.
hipError_t debug_violations_decode_f32(uint32_t* flags, bool clear);
hipError_t debug_violations_decode_f16(uint32_t* flags, bool clear);
hipError_t debug_violations_decode_bf16(uint32_t* flags, bool clear);
hipError_t debug_violations_prefill(uint32_t* flags, bool clear);
hipError_t debug_violations_copy(uint32_t* flags, bool clear);

// Device scratch of the no-allocation decode entry point: a file-scope
// __device__ array of kDecodeScratchBytes, one per GPU, whose device address
// is looked up once per device (with that device current) and cached.
constexpr size_t kDecodeScratchBytes = (size_t)64 << 20;
hipError_t decode_scratch(void** ptr);

// Prefill over a cached prefix (f16/bf16, group size 1..16): one launch.
hipError_t launch_prefill(const PrefillArgs& args, Elem elem, int head_dim, int block_size, int group,
                          hipStream_t stream);

}  // namespace pa
