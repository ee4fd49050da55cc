// libpagedkv C ABI: host-side argument checks, launch geometry and status codes.
// Every check happens before the first HIP call, so a rejected call has no
// side effect and the checks work without a GPU.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <map>
#include <mutex>
#include <utility>

#include "../../include/pa.h"
#include "pa_common.hpp"
#include "pa_launch.hpp"

#define PA_EXPORT extern "C" __attribute__((visibility("default")))

static_assert(pa::kDecodeScratchBytes == (size_t)PA_DECODE_SCRATCH_BYTES, "scratch size in pa.h");

namespace {

thread_local int g_last_hip_error = 0;

bool dtype_ok(pa_dtype d) { return d == PA_F32 || d == PA_F16 || d == PA_BF16; }
int elt_bytes(pa_dtype d) { return d == PA_F32 ? 4 : 2; }
bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }
bool block_size_ok(int32_t b) { return b == 8 || b == 16 || b == 32; }
bool group_ok(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pa::Elem elem_of(pa_dtype d) {
  return d == PA_F32 ? pa::Elem::F32 : (d == PA_F16 ? pa::Elem::F16 : pa::Elem::BF16);
}

pa_status hip_status(hipError_t e) {
  if (e == hipSuccess) return PA_OK;
  g_last_hip_error = (int)e;
  return PA_ERR_HIP;
}

int64_t num_partitions(int32_t max_context_len, int32_t partition_size) {
  if (partition_size <= 0 || max_context_len <= 0) return 1;
  return ((int64_t)max_context_len + partition_size - 1) / partition_size;
}

size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Balanced-mode workspace: one 32-byte merge descriptor per wave boundary,
// then 2 partial slots per wave of group-size rows (head_dim partial outputs,
// m, l).
constexpr size_t kDescBytes = 4 * sizeof(int64_t);
size_t balanced_ws_bytes(int32_t group, int32_t head_dim) {
  const size_t rows = 2 * (size_t)pa::kBalancedMaxWaves * (size_t)group;
  return (size_t)pa::kBalancedMaxWaves * kDescBytes + rows * ((size_t)head_dim + 2) * sizeof(float);
}

}  // namespace

namespace pa {

hipError_t balanced_grid(const void* kernel, int block_threads, int max_per_cu, int max_wg, int* nwg) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find({kernel, dev});
  if (it != cache.end()) {
    *nwg = it->second;
    return hipSuccess;
  }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block_threads, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  if (max_per_cu > 0 && per_cu > max_per_cu) per_cu = max_per_cu;
  int n = cus * per_cu;
  if (n > max_wg) n = max_wg;
  cache[{kernel, dev}] = n;
  *nwg = n;
  return hipSuccess;
}

}  // namespace pa

PA_EXPORT const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: a size is out of range or inconsistent";
    case PA_ERR_BLOCK_SIZE: return "PA_ERR_BLOCK_SIZE: block_size must be 8, 16 or 32";
    case PA_ERR_DTYPE: return "PA_ERR_DTYPE: dtype must be PA_F32, PA_F16 or PA_BF16";
    case PA_ERR_PARTITION:
      return "PA_ERR_PARTITION: partition_size must be 0, PA_PARTITION_BALANCED (at most 4096 "
             "sequences) or a positive multiple of 16 and of block_size";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: a HIP launch failed (see pa_last_hip_error)";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN: data pointers must be 16-byte aligned";
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS: not enough free blocks for the batch";
    case PA_ERR_SEQUENCE: return "PA_ERR_SEQUENCE: no live sequence has this id";
    case PA_ERR_CAPACITY: return "PA_ERR_CAPACITY: an output buffer is too small";
    case PA_ERR_HOST_MEMORY:
      return "PA_ERR_HOST_MEMORY: the host buffer is not pinned memory mapped for the GPU";
    case PA_ERR_UNSUPPORTED:
      return "PA_ERR_UNSUPPORTED: the library was compiled without this call (PA_DEBUG_CHECKS)";
  }
  return "unknown pa_status";
}

PA_EXPORT int pa_last_hip_error(void) { return g_last_hip_error; }

PA_EXPORT pa_status pa_kv_append(const void* key, const void* value, void* k_pool, void* v_pool,
                                 const int64_t* slot_mapping, int32_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, pa_dtype dtype, void* stream) {
  if (!dtype_ok(dtype)) return PA_ERR_DTYPE;
  if (!block_size_ok(block_size)) return PA_ERR_BLOCK_SIZE;
  if (num_tokens < 0 || num_kv_heads < 1 || !head_dim_ok(head_dim) || num_blocks < 1)
    return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_pool || !v_pool || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_pool) || !aligned16(v_pool))
    return PA_ERR_ALIGN;
  return hip_status(pa::launch_kv_append(key, value, k_pool, v_pool, slot_mapping, num_tokens,
                                         num_kv_heads, head_dim * elt_bytes(dtype), block_size,
                                         num_blocks, reinterpret_cast<hipStream_t>(stream)));
}

PA_EXPORT pa_status pa_block_copy(void* k_pool, void* v_pool, const int32_t* block_mapping,
                                  int32_t num_pairs, int32_t num_kv_heads, int32_t block_size,
                                  int32_t head_dim, int32_t num_blocks, pa_dtype dtype,
                                  void* stream) {
  if (!dtype_ok(dtype)) return PA_ERR_DTYPE;
  if (!block_size_ok(block_size)) return PA_ERR_BLOCK_SIZE;
  if (num_pairs < 0 || num_kv_heads < 1 || !head_dim_ok(head_dim) || num_blocks < 1)
    return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > INT32_MAX / 2) return PA_ERR_SHAPE;
  if (!k_pool || !v_pool || !block_mapping) return PA_ERR_NULL;
  if (!aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_ALIGN;
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * elt_bytes(dtype);
  if (block_bytes / 16 > INT32_MAX) return PA_ERR_SHAPE;
  return hip_status(pa::launch_block_copy(k_pool, v_pool, block_mapping, num_pairs, block_bytes,
                                          num_blocks, reinterpret_cast<hipStream_t>(stream)));
}

static pa_status swap_call(bool out, void* k_pool, void* v_pool, void* host, const int32_t* block_ids,
                           int32_t num_ids, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                           int32_t num_blocks, pa_dtype dtype, void* stream) {
  if (!dtype_ok(dtype)) return PA_ERR_DTYPE;
  if (!block_size_ok(block_size)) return PA_ERR_BLOCK_SIZE;
  if (num_ids < 0 || num_kv_heads < 1 || !head_dim_ok(head_dim) || num_blocks < 1) return PA_ERR_SHAPE;
  if (num_ids == 0) return PA_OK;
  if (num_ids > INT32_MAX / 2) return PA_ERR_SHAPE;
  if (!k_pool || !v_pool || !block_ids || !host) return PA_ERR_NULL;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(host)) return PA_ERR_ALIGN;
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * elt_bytes(dtype);
  if (block_bytes / 16 > INT32_MAX) return PA_ERR_SHAPE;
  // the host buffer must be pinned host memory the GPU can address
  // (hipHostMalloc): HIP must classify it as host memory and map it at the
  // same address (as ROCm maps pinned memory); anything else is refused
  hipPointerAttribute_t attr;
  void* dev_host = nullptr;
  if (hipPointerGetAttributes(&attr, host) != hipSuccess || attr.type != hipMemoryTypeHost ||
      hipHostGetDevicePointer(&dev_host, host, 0) != hipSuccess || dev_host != host) {
    (void)hipGetLastError();   // do not leave the lookup's error for the caller's next call
    return PA_ERR_HOST_MEMORY;
  }
  return hip_status(pa::launch_swap(out, k_pool, v_pool, dev_host, block_ids, num_ids, block_bytes,
                                    num_blocks, reinterpret_cast<hipStream_t>(stream)));
}

PA_EXPORT pa_status pa_swap_out(const void* k_pool, const void* v_pool, const int32_t* block_ids,
                                int32_t num_ids, void* host_dst, int32_t num_kv_heads, int32_t block_size,
                                int32_t head_dim, int32_t num_blocks, pa_dtype dtype, void* stream) {
  return swap_call(true, const_cast<void*>(k_pool), const_cast<void*>(v_pool), host_dst, block_ids, num_ids,
                   num_kv_heads, block_size, head_dim, num_blocks, dtype, stream);
}

PA_EXPORT pa_status pa_swap_in(const void* host_src, void* k_pool, void* v_pool, const int32_t* block_ids,
                               int32_t num_ids, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                               int32_t num_blocks, pa_dtype dtype, void* stream) {
  return swap_call(false, k_pool, v_pool, const_cast<void*>(host_src), block_ids, num_ids, num_kv_heads,
                   block_size, head_dim, num_blocks, dtype, stream);
}

PA_EXPORT pa_status pa_stream_read(const void* buf, uint64_t bytes, uint32_t* partials, void* stream) {
  if (bytes == 0) return PA_OK;
  if (!buf || !partials) return PA_ERR_NULL;
  if (bytes % 16 != 0) return PA_ERR_SHAPE;
  if (!aligned16(buf)) return PA_ERR_ALIGN;
  return hip_status(pa::launch_stream_read(buf, bytes, partials, PA_STREAM_READ_PARTIALS,
                                           reinterpret_cast<hipStream_t>(stream)));
}

// Two-level tables: the large-page arguments of the *_hier entry points.
struct HierTables {
  const int32_t* large_tables = nullptr;
  const int32_t* num_large = nullptr;
  int32_t max_large_per_seq = 0;
  int32_t shift = 0;
};

// Host checks of the large-page arguments; fills h.shift.
static pa_status check_hier(HierTables& h, int32_t pages_per_large, int32_t max_blocks_per_seq,
                            int32_t block_size) {
  if (!h.large_tables || !h.num_large) return PA_ERR_NULL;
  if (h.max_large_per_seq < 1 || pages_per_large < 1 || pages_per_large > 1024 ||
      (pages_per_large & (pages_per_large - 1)) != 0)
    return PA_ERR_SHAPE;
  while ((1 << h.shift) < pages_per_large) ++h.shift;
  const int64_t tokens = ((int64_t)h.max_large_per_seq * pages_per_large + max_blocks_per_seq) * block_size;
  if (tokens > INT32_MAX) return PA_ERR_SHAPE;
  return PA_OK;
}

static pa_status prefill_impl(void* out, const void* query, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* context_lens,
                              const int32_t* query_start, int32_t num_seqs, int32_t num_tokens,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                              int32_t max_query_len, float scale, pa_dtype dtype, void* stream,
                              const HierTables& hier) {
  if (!dtype_ok(dtype) || dtype == PA_F32) return PA_ERR_DTYPE;
  if (!block_size_ok(block_size)) return PA_ERR_BLOCK_SIZE;
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads < 1 || num_kv_heads < 1 || !head_dim_ok(head_dim) ||
      max_blocks_per_seq < 1 || num_blocks < 1 || max_query_len < 0)
    return PA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0 || !group_ok(num_q_heads / num_kv_heads)) return PA_ERR_SHAPE;
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PA_OK;
  if (!out || !query || !k_pool || !v_pool || !block_tables || !context_lens || !query_start)
    return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(query) || !aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_ALIGN;
  const int32_t group = num_q_heads / num_kv_heads;
  const int64_t qblocks = ((int64_t)max_query_len + 64 / group - 1) / (64 / group);
  if ((int64_t)num_seqs * num_kv_heads * qblocks > INT32_MAX) return PA_ERR_SHAPE;
  pa::PrefillArgs a{};
  a.out = out;
  a.query = query;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.num_tokens = num_tokens;
  a.max_query_len = max_query_len;
  a.scale_log2 = scale * pa::kLog2e;
  a.large_tables = hier.large_tables;
  a.num_large = hier.num_large;
  a.max_large_per_seq = hier.max_large_per_seq;
  a.large_shift = hier.shift;
  return hip_status(pa::launch_prefill(a, elem_of(dtype), head_dim, block_size, group,
                                       reinterpret_cast<hipStream_t>(stream)));
}

PA_EXPORT pa_status pa_prefill_attention(void* out, const void* query, const void* k_pool,
                                         const void* v_pool, const int32_t* block_tables,
                                         const int32_t* context_lens, const int32_t* query_start,
                                         int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                         int32_t max_blocks_per_seq, int32_t num_blocks,
                                         int32_t max_query_len, float scale, pa_dtype dtype,
                                         void* stream) {
  return prefill_impl(out, query, k_pool, v_pool, block_tables, context_lens, query_start, num_seqs,
                      num_tokens, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                      num_blocks, max_query_len, scale, dtype, stream, HierTables{});
}

PA_EXPORT pa_status pa_prefill_attention_hier(void* out, const void* query, const void* k_pool,
                                              const void* v_pool, const int32_t* small_tables,
                                              const int32_t* large_tables, const int32_t* num_large,
                                              const int32_t* context_lens, const int32_t* query_start,
                                              int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                              int32_t max_small_per_seq, int32_t max_large_per_seq,
                                              int32_t pages_per_large, int32_t num_blocks,
                                              int32_t max_query_len, float scale, pa_dtype dtype,
                                              void* stream) {
  if (!dtype_ok(dtype) || dtype == PA_F32) return PA_ERR_DTYPE;
  if (!block_size_ok(block_size)) return PA_ERR_BLOCK_SIZE;
  if (max_small_per_seq < 1) return PA_ERR_SHAPE;
  HierTables h{large_tables, num_large, max_large_per_seq, 0};
  if (num_seqs > 0 && num_tokens > 0 && max_query_len > 0) {
    const pa_status st = check_hier(h, pages_per_large, max_small_per_seq, block_size);
    if (st != PA_OK) return st;
  }
  return prefill_impl(out, query, k_pool, v_pool, small_tables, context_lens, query_start, num_seqs,
                      num_tokens, num_q_heads, num_kv_heads, head_dim, block_size, max_small_per_seq,
                      num_blocks, max_query_len, scale, dtype, stream, h);
}

PA_EXPORT size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t max_context_len,
                                           int32_t partition_size) {
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 ||
      head_dim < 1 || max_context_len < 0 || partition_size < PA_PARTITION_BALANCED)
    return (size_t)-1;
  if (partition_size == PA_PARTITION_BALANCED)
    return balanced_ws_bytes(num_q_heads / num_kv_heads, head_dim);
  const int64_t np = num_partitions(max_context_len, partition_size);
  if (partition_size == 0 || np <= 1) return 0;
  return (size_t)num_seqs * (size_t)num_q_heads * (size_t)np * ((size_t)head_dim + 2) * sizeof(float);
}

PA_EXPORT int32_t pa_decode_choose_partition(int32_t num_seqs, int32_t num_kv_heads,
                                             int32_t max_context_len, int32_t block_size) {
  (void)num_kv_heads;
  (void)block_size;
  // The balanced split gives every resident workgroup the same number of
  // tiles, so ragged batches and a few very long sequences finish together;
  // tiny batches (one table window or less) are not worth a second launch.
  if (max_context_len <= 64 || num_seqs > pa::kBalancedMaxSeqs) return 0;
  return PA_PARTITION_BALANCED;
}

// Prefix groups of pa_decode_attention_grouped.
struct PrefixGroups {
  const int32_t* group_start;
  const int32_t* group_shared;
  int32_t num_groups, max_group_size, max_shared_len;
};

static pa_status decode_impl(void* out, const void* query, const void* k_pool, const void* v_pool,
                             const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                             int32_t max_context_len, float scale, int32_t partition_size, pa_dtype dtype,
                             void* workspace, size_t workspace_bytes, void* stream,
                             const HierTables& hier, bool use_scratch = false,
                             const PrefixGroups* groups = nullptr) {
  if (!dtype_ok(dtype)) return PA_ERR_DTYPE;
  if (!block_size_ok(block_size)) return PA_ERR_BLOCK_SIZE;
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || !head_dim_ok(head_dim) ||
      max_blocks_per_seq < 1 || num_blocks < 1 || max_context_len < 0)
    return PA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0 || !group_ok(num_q_heads / num_kv_heads)) return PA_ERR_SHAPE;
  const bool balanced = partition_size == PA_PARTITION_BALANCED;
  if (partition_size < PA_PARTITION_BALANCED ||
      (partition_size > 0 && (partition_size % 16 != 0 || partition_size % block_size != 0)))
    return PA_ERR_PARTITION;
  if (balanced && num_seqs > pa::kBalancedMaxSeqs) return PA_ERR_PARTITION;
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !k_pool || !v_pool || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(query) || !aligned16(k_pool) || !aligned16(v_pool))
    return PA_ERR_ALIGN;

  const int32_t group = num_q_heads / num_kv_heads;
  const int64_t np = balanced ? 1 : num_partitions(max_context_len, partition_size);
  const bool split = balanced || np > 1;
  const bool mfma = dtype != PA_F32 && group >= 2;
  const int32_t heads_per_unit = mfma ? group : (group < 4 ? group : 4);
  const int64_t chunks = mfma ? num_kv_heads : num_q_heads / heads_per_unit;
  const int64_t units = (int64_t)num_seqs * chunks * np;
  if (units > INT32_MAX) return PA_ERR_SHAPE;

  pa::DecodeArgs a{};
  a.out = out;
  a.query = query;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.partition_size = (partition_size > 0 && np > 1) ? partition_size
                                                    : (max_context_len > 16 ? max_context_len : 16);
  a.num_parts = (int32_t)np;
  a.split = split ? 1 : 0;
  a.head_chunks = (int32_t)chunks;
  a.mode = balanced ? pa::kModeBalanced : pa::kModeUnit;
  a.scale_log2 = scale * pa::kLog2e;
  if (split) {
    const size_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                  max_context_len, partition_size);
    if (use_scratch) {   // the library's static device scratch instead of a caller's workspace
      if (need > pa::kDecodeScratchBytes) return PA_ERR_WORKSPACE;
      void* p = nullptr;
      const hipError_t e = pa::decode_scratch(&p);
      if (e != hipSuccess) return hip_status(e);
      workspace = p;
      workspace_bytes = pa::kDecodeScratchBytes;
    }
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return PA_ERR_ALIGN;
    char* ws = static_cast<char*>(workspace);
    size_t rows;
    if (balanced) {
      a.ws_desc = reinterpret_cast<int64_t*>(ws);
      ws += (size_t)pa::kBalancedMaxWaves * kDescBytes;
      rows = 2 * (size_t)pa::kBalancedMaxWaves * (size_t)heads_per_unit;
    } else {
      rows = (size_t)num_seqs * num_q_heads * (size_t)np;
    }
    // partial outputs first: each row of head_dim floats starts 16-byte aligned
    a.ws_o = reinterpret_cast<float*>(ws);
    a.ws_m = a.ws_o + rows * (size_t)head_dim;
    a.ws_l = a.ws_m + rows;
  }
  a.large_tables = hier.large_tables;
  a.num_large = hier.num_large;
  a.max_large_per_seq = hier.max_large_per_seq;
  a.large_shift = hier.shift;
  pa::GroupArgs ga{};
  const bool grouped = groups && groups->num_groups > 0 && np > 1;
  if (grouped) {
    ga.group_start = groups->group_start;
    ga.group_shared = groups->group_shared;
    ga.num_groups = groups->num_groups;
    ga.max_group_size = groups->max_group_size;
    const int64_t sp = ((int64_t)groups->max_shared_len + partition_size - 1) / partition_size;
    ga.shared_parts = (int32_t)(sp < np ? sp : np);
    // shared units (at most max_group_size member chunks) plus the partition units
    if ((int64_t)groups->max_group_size * groups->num_groups * chunks * ga.shared_parts + units > INT32_MAX)
      return PA_ERR_SHAPE;
  }
  return hip_status(pa::launch_decode(a, elem_of(dtype), head_dim, block_size, group,
                                      reinterpret_cast<hipStream_t>(stream), grouped ? &ga : nullptr));
}

PA_EXPORT pa_status pa_decode_attention(void* out, const void* query, const void* k_pool,
                                        const void* v_pool, const int32_t* block_tables,
                                        const int32_t* context_lens, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size,
                                        int32_t max_blocks_per_seq, int32_t num_blocks,
                                        int32_t max_context_len, float scale,
                                        int32_t partition_size, pa_dtype dtype, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return decode_impl(out, query, k_pool, v_pool, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, max_context_len,
                     scale, partition_size, dtype, workspace, workspace_bytes, stream, HierTables{});
}

PA_EXPORT pa_status pa_decode_attention_grouped(void* out, const void* query, const void* k_pool,
                                                const void* v_pool, const int32_t* block_tables,
                                                const int32_t* context_lens, const int32_t* group_start,
                                                const int32_t* group_shared, int32_t num_groups,
                                                int32_t max_group_size, int32_t max_shared_len, int32_t num_seqs,
                                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                                int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                                int32_t max_context_len, float scale, int32_t partition_size,
                                                pa_dtype dtype, void* workspace, size_t workspace_bytes,
                                                void* stream) {
  if (!dtype_ok(dtype)) return PA_ERR_DTYPE;
  if (!block_size_ok(block_size)) return PA_ERR_BLOCK_SIZE;
  if (partition_size <= 0 || partition_size % 16 != 0 || partition_size % block_size != 0)
    return PA_ERR_PARTITION;
  if (num_groups < 0 || max_shared_len < 0 || (num_groups > 0 && max_group_size < 1)) return PA_ERR_SHAPE;
  if (num_groups > 0 && num_seqs > 0 && (!group_start || !group_shared)) return PA_ERR_NULL;
  const PrefixGroups g{group_start, group_shared, num_groups, max_group_size, max_shared_len};
  return decode_impl(out, query, k_pool, v_pool, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, max_context_len,
                     scale, partition_size, dtype, workspace, workspace_bytes, stream, HierTables{}, false, &g);
}

PA_EXPORT pa_status pa_decode_attention_hier(void* out, const void* query, const void* k_pool,
                                             const void* v_pool, const int32_t* small_tables,
                                             const int32_t* large_tables, const int32_t* num_large,
                                             const int32_t* context_lens, int32_t num_seqs,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t max_small_per_seq,
                                             int32_t max_large_per_seq, int32_t pages_per_large,
                                             int32_t num_blocks, int32_t max_context_len, float scale,
                                             int32_t partition_size, pa_dtype dtype, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return PA_ERR_DTYPE;
  if (!block_size_ok(block_size)) return PA_ERR_BLOCK_SIZE;
  if (max_small_per_seq < 1) return PA_ERR_SHAPE;
  HierTables h{large_tables, num_large, max_large_per_seq, 0};
  if (num_seqs > 0) {
    const pa_status st = check_hier(h, pages_per_large, max_small_per_seq, block_size);
    if (st != PA_OK) return st;
  }
  return decode_impl(out, query, k_pool, v_pool, small_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, max_small_per_seq, num_blocks, max_context_len,
                     scale, partition_size, dtype, workspace, workspace_bytes, stream, h);
}

PA_EXPORT pa_status pa_decode_attention_noalloc(void* out, const void* query, const void* k_pool,
                                                const void* v_pool, const int32_t* block_tables,
                                                const int32_t* context_lens, int32_t num_seqs,
                                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                                int32_t block_size, int32_t max_blocks_per_seq,
                                                int32_t num_blocks, int32_t max_context_len, float scale,
                                                int32_t partition_size, pa_dtype dtype, void* stream) {
  return decode_impl(out, query, k_pool, v_pool, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, max_context_len,
                     scale, partition_size, dtype, nullptr, 0, stream, HierTables{}, true);
}

PA_EXPORT pa_status pa_debug_violations(uint32_t* flags, int32_t clear) {
  if (!flags) return PA_ERR_NULL;
#if PA_DEBUG_CHECKS
  hipError_t (*const units[])(uint32_t*, bool) = {pa::debug_violations_decode_f32, pa::debug_violations_decode_f16,
                                                  pa::debug_violations_decode_bf16, pa::debug_violations_prefill,
                                                  pa::debug_violations_copy};
  uint32_t all = 0;
  for (auto unit : units) {
    uint32_t f = 0;
    const hipError_t e = unit(&f, clear != 0);
    if (e != hipSuccess) return hip_status(e);
    all |= f;
  }
  *flags = all;
  return PA_OK;
#else
  (void)clear;
  return PA_ERR_UNSUPPORTED;
#endif
}
