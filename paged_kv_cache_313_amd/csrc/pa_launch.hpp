// Host-side launch entry points of the libpagedkv kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct DecodeArgs;

enum class Elem { F32 = 0, F16 = 1, BF16 = 2 };

hipError_t launch_kv_append(const void* key, const void* value, void* k_pool, void* v_pool,
                            const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                            int32_t row_bytes, int32_t block_size, int32_t num_blocks,
                            hipStream_t stream);

hipError_t launch_block_copy(void* k_pool, void* v_pool, const int32_t* block_mapping,
                             int32_t num_pairs, int64_t block_bytes, int32_t num_blocks,
                             hipStream_t stream);

// Decode: partition pass (direct output for single-partition sequences) plus,
// when split, the merge kernel.  `use_mfma` selects the grouped-query MFMA
// kernel (f16/bf16, group size 2..16); otherwise the VALU kernel.
hipError_t launch_decode(const DecodeArgs& args, Elem elem, int head_dim, int block_size,
                         int group, hipStream_t stream);

}  // namespace pa
