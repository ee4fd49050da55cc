// Decode attention over a paged KV cache: the entry into the kernels of
// pa_decode_core.hpp (instantiated per storage type in pa_decode_f32.hip,
// pa_decode_f16.hip and pa_decode_bf16.hip), and the device scratch of the
// no-allocation entry point.
#include <mutex>

#include "pa_common.hpp"
#include "pa_launch.hpp"

namespace pa {

// Workspace of pa_decode_attention_noalloc, for callers that cannot allocate:
// each GPU the library runs on holds its own copy until the process ends.
// Host code never uses this name as an address (on the host it is only a
// stand-in); decode_scratch() returns the device address.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, Elem elem, int head_dim, int block_size, int group,
                         hipStream_t st, const GroupArgs* groups) {
  switch (elem) {
    case Elem::F32: return launch_decode_f32(a, head_dim, block_size, group, st, groups);
    case Elem::F16: return launch_decode_f16(a, head_dim, block_size, group, st, groups);
    case Elem::BF16: return launch_decode_bf16(a, head_dim, block_size, group, st, groups);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
