// Decode kernels over bf16 pools (one instantiation unit per storage type,
// compiled in parallel).
#include "pa_decode_core.hpp"

namespace pa {

hipError_t launch_decode_bf16(const DecodeArgs& a, int head_dim, int block_size, int group, hipStream_t st,
                           const GroupArgs* groups) {
  return dispatch_t<BF16>(a, head_dim, block_size, group, st, groups);
}

PA_VIOLATIONS_GETTER(debug_violations_decode_bf16)

}  // namespace pa
