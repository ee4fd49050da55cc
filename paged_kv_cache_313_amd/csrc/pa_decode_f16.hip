// Decode kernels over f16 pools (one instantiation unit per storage type,
// compiled in parallel).
#include "pa_decode_core.hpp"

namespace pa {

hipError_t launch_decode_f16(const DecodeArgs& a, int head_dim, int block_size, int group, hipStream_t st,
                           const GroupArgs* groups) {
  return dispatch_t<F16>(a, head_dim, block_size, group, st, groups);
}

PA_VIOLATIONS_GETTER(debug_violations_decode_f16)

}  // namespace pa
