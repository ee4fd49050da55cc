/*
 * pa.h -- C ABI of libpagedkv: the data-parallel hot path of PagedAttention on
 * AMD Instinct MI355X (gfx950).
 *
 * The KV cache of every sequence is cut into fixed-size blocks of
 * `block_size` tokens that live anywhere in a shared physical pool; each
 * sequence reaches its blocks through its own block table (vLLM/PagedAttention
 * paged-KV analysis page, sections 2.2 and 2.3; vLLM entity page, "what it
 * is").  Operations on the device:
 *
 *   pa_kv_append         write the newest tokens' K/V into their slots
 *   pa_block_copy        copy-on-write duplication of shared blocks
 *   pa_decode_attention  one query token per sequence attends over its paged
 *                        context
 *   pa_prefill_attention the new tokens of each sequence attend causally over
 *                        its paged context (prefill over a cached prefix)
 *   pa_swap_out/_in      move whole blocks between the pools and pinned host
 *                        memory (preemption)
 *
 * The host-side block manager that decides where tokens live is declared in
 * pa_block_manager.h.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked DEVICE are device (HBM) addresses; HOST means host memory.
 *   The caller owns every buffer.  The library never allocates, frees or
 *   synchronises; every call is enqueued on `stream` (a hipStream_t; NULL is
 *   the null stream) and returns as soon as the launches are queued.  Inputs
 *   must stay alive until the stream has passed the call.
 * - Pools `k_pool` and `v_pool` are each laid out
 *   [num_blocks][num_kv_heads][block_size][head_dim] (row-major, head_dim
 *   fastest), so one (block, KV head) tile of block_size * head_dim elements is
 *   contiguous.
 * - Supported: dtype f32 / f16 / bf16 (the same for query, pools and output;
 *   bf16 is the upper half of an IEEE float32), head_dim 64 or 128,
 *   block_size 8, 16 or 32, num_q_heads a multiple of num_kv_heads with group
 *   size Hq/Hkv in {1, 2, 4, 8, 16}.  Pool pointers and the key/value/query/out
 *   pointers must be 16-byte aligned.
 * - Argument checks are pure host checks made before any HIP call (the swap
 *   calls also ask HIP whether their host buffer is pinned), so a rejected
 *   call has no side effect.  A failed launch returns PA_ERR_HIP and
 *   pa_last_hip_error() gives the hipError_t value.
 * - Device-side contents are the caller's contract: table entries and slot
 *   ids in range, slots unique within a call, CoW destinations distinct and
 *   disjoint from all sources.  The kernels never access memory outside the
 *   buffers described by the size arguments: out-of-range physical ids, slots
 *   and lengths are clamped or skipped (results for such inputs are
 *   unspecified, but memory stays safe).
 * - All entry points are reentrant; the library holds no state other than the
 *   thread-local last HIP error, the cached launch geometry and the device
 *   scratch of pa_decode_attention_noalloc (whose calls on one GPU must not
 *   overlap).
 */
#ifndef PAGEDKV_PA_H
#define PAGEDKV_PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  PA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent            */
  PA_ERR_BLOCK_SIZE = 3,  /* block_size not in {8, 16, 32}                     */
  PA_ERR_DTYPE = 4,       /* dtype not one of pa_dtype                         */
  PA_ERR_PARTITION = 5,   /* partition_size invalid (see pa_decode_attention)       */
  PA_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required        */
  PA_ERR_HIP = 7,         /* a kernel launch failed; see pa_last_hip_error()   */
  PA_ERR_ALIGN = 8,       /* a data pointer is not 16-byte aligned             */
  PA_ERR_NO_BLOCKS = 9,   /* block manager: the free blocks do not cover a batch */
  PA_ERR_SEQUENCE = 10,   /* block manager: a sequence id that is not live     */
  PA_ERR_CAPACITY = 11,   /* block manager: a caller's output buffer is too small */
  PA_ERR_HOST_MEMORY = 12, /* swap: the host buffer is not pinned, GPU-mapped memory */
  PA_ERR_UNSUPPORTED = 13 /* the library was compiled without the call (pa_debug_violations needs PA_DEBUG_CHECKS) */
} pa_status;

/* In C++ the enum has a fixed 32-bit underlying type, so that any int32 a C
 * caller passes is a value of the type (and is rejected with PA_ERR_DTYPE
 * unless it names a dtype); the ABI is that of a C enum, a 32-bit int. */
#ifdef __cplusplus
typedef enum : int32_t { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;
#else
typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;
#endif

/* partition_size value selecting the balanced split of pa_decode_attention */
#define PA_PARTITION_BALANCED (-1)

/*
 * pa_kv_append -- paged KV append (slot-mapping scatter).
 *
 * Defined by the pages as the write of a newly generated token into the block
 * that its sequence is filling (paged-KV analysis page, section 3.2, the
 * copy-on-write paragraph; blocks are taken on demand, vLLM entity page,
 * "what it is").  For every token i with slot = slot_mapping[i] >= 0:
 *     b = slot / block_size, o = slot % block_size,
 *     k_pool[b][h][o][:] = key[i][h][:]   and   v_pool[b][h][o][:] = value[i][h][:]
 * for every KV head h.  Tokens with a negative slot are skipped, and so are
 * slots >= num_blocks * block_size.  Byte copy: bits are preserved exactly.
 *
 *   key, value     DEVICE [num_tokens][num_kv_heads][head_dim] of dtype
 *   k_pool, v_pool DEVICE pools (see above), written in place
 *   slot_mapping   DEVICE int64 [num_tokens]
 * num_tokens == 0 is a no-op returning PA_OK.
 */
pa_status pa_kv_append(const void* key, const void* value, void* k_pool, void* v_pool,
                       const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                       void* stream);

/*
 * pa_decode_workspace_bytes -- size of the workspace that pa_decode_attention
 * needs for this shape and partition_size (see there); 0 when none is needed
 * (no split, or a single partition), (size_t)-1 for invalid arguments.  The
 * balanced split's size depends only on the group size Hq/Hkv and head_dim.
 * HOST only; makes no HIP call.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len, int32_t partition_size);

/*
 * pa_decode_choose_partition -- the partition_size the library prefers for a
 * batch of this shape: PA_PARTITION_BALANCED for most batches, 0 (no split)
 * for tiny contexts or more sequences than a balanced launch takes.  HOST
 * only; never fails.
 */
int32_t pa_decode_choose_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                                   int32_t block_size);

/*
 * pa_decode_attention -- single-query decode attention over a paged KV cache.
 *
 * The pages give the operation per sequence: the query of every head reads the
 * sequence's K/V block by block through its block table, the blocks being
 * non-contiguous (paged-KV analysis page, section 3.1, simplified attention
 * sketch).  The sketch is marked as simplified; the operation computed here is
 * one softmax over the whole context, scaled, with the unfilled tail of the last
 * block excluded:
 *     for sequence s, q head h, KV head g = h / (num_q_heads / num_kv_heads),
 *     L = context_lens[s], token t in [0, L) at block block_tables[s][t / bs],
 *     slot t % bs:
 *         s_t = scale * <query[s][h], k_t>,
 *         out[s][h] = sum_t exp(s_t - max) v_t / sum_t exp(s_t - max).
 * L == 0 gives a zero row.  Accumulation is fp32; the output is rounded once
 * (round to nearest even) to dtype.
 *
 *   out            DEVICE [num_seqs][num_q_heads][head_dim] of dtype, written
 *   query          DEVICE [num_seqs][num_q_heads][head_dim] of dtype
 *   k_pool, v_pool DEVICE pools (see above), read only
 *   block_tables   DEVICE int32 [num_seqs][max_blocks_per_seq]; entries past a
 *                  sequence's last block never affect the result (the
 *                  balanced split may read any entry of the array when it
 *                  compares a row with its neighbours', see below)
 *   context_lens   DEVICE int32 [num_seqs]; counts every token attended to,
 *                  including one appended in the same step (append first)
 *   max_context_len HOST upper bound of context_lens (sizes the grid);
 *                  lengths above it, or above max_blocks_per_seq * block_size,
 *                  are clamped
 *   partition_size how the context is cut into work units:
 *                  0: one unit per (sequence, head group), no workspace;
 *                  P > 0 (a multiple of 16 and of block_size): units of P
 *                  tokens; each writes partial results (running max, running
 *                  sum, un-normalised output) to `workspace` and a second
 *                  kernel merges them with the log-sum-exp rescale (a
 *                  sequence that fits one partition is written directly);
 *                  PA_PARTITION_BALANCED: the grid holds the workgroups the
 *                  GPU keeps resident and each takes an equal share of all
 *                  tiles of the batch, so ragged batches finish together;
 *                  pieces of a (sequence, head group) that several units
 *                  share are merged the same way (num_seqs <= 4096).
 *   workspace      DEVICE, 16-byte aligned, >= pa_decode_workspace_bytes(...)
 *                  bytes when that is non-zero (may be NULL otherwise);
 *                  scratch only, overwritten.  Calls that share a workspace
 *                  must be ordered on one stream.
 *
 * Cache policy (performance only, never the result): the balanced split
 * loads K/V tiles with the non-temporal hint, except the leading blocks of a
 * table that sequence s-1 or s+1 maps to the same physical blocks at the same
 * logical positions (a shared prompt).  Those keep the default policy, so
 * that neighbouring sequences hit in the caches.  Place the sequences that
 * share blocks (the samples or beams of one request) next to each other in
 * the batch.  The other modes use the default policy throughout.
 */
pa_status pa_decode_attention(void* out, const void* query, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                              int32_t num_blocks, int32_t max_context_len, float scale,
                              int32_t partition_size, pa_dtype dtype, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * pa_decode_attention_grouped -- pa_decode_attention for a batch in which
 * consecutive sequences share the physical blocks of a common prefix: the
 * samples of parallel sampling or the beams of beam search, which the
 * pages give refcounted shared blocks (vLLM entity page, "what it is";
 * paged-KV analysis page, section 3.2).  The same operation and results as
 * pa_decode_attention with the same fixed partition_size; only the reads of
 * the shared blocks change.
 *
 *   group_start    DEVICE int32 [num_groups + 1], non-decreasing from 0:
 *                  group i is sequences group_start[i] .. group_start[i+1]-1
 *                  (sequences outside every group run alone).
 *   group_shared   DEVICE int32 [num_groups]: the first group_shared[i]
 *                  tokens of every member of group i map to the same
 *                  physical blocks (the caller's contract, like the table
 *                  entries themselves).  The call uses the largest multiple
 *                  of partition_size that is at most this, at most
 *                  max_shared_len rounded up to a partition, and shorter than
 *                  every member's context (a group with an empty member
 *                  shares nothing).
 *   num_groups     >= 0;  max_group_size >= 1 when num_groups > 0: a host
 *                  bound of the group sizes (members past it read their
 *                  shared blocks alone);  max_shared_len >= 0: a host bound
 *                  of group_shared.
 *   partition_size > 0, a multiple of 16 and of block_size (else
 *                  PA_ERR_PARTITION); workspace as for pa_decode_attention
 *                  with this partition_size.
 *
 * Each shared partition is computed once per group of 16 / G members
 * (G = Hq / Hkv): their query rows fill the 16 columns of the matrix-core
 * products that one sequence's G rows pad, so each shared K/V tile is read
 * and multiplied once for all of them.  Their partial results (max, sum,
 * un-normalised output per partition) are the ones the plain partition pass
 * writes, bit for bit, and the same merge combines them.  On the other cores
 * (group size below 4, head_dim 64, f32) the call runs the plain partition
 * pass.
 */
pa_status pa_decode_attention_grouped(void* out, const void* query, const void* k_pool, const void* v_pool,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      const int32_t* group_start, const int32_t* group_shared, int32_t num_groups,
                                      int32_t max_group_size, int32_t max_shared_len, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                      int32_t max_context_len, float scale, int32_t partition_size,
                                      pa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_attention_noalloc -- pa_decode_attention without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same operation, arguments, kernels, results and errors as
 * pa_decode_attention, except that the partial results of a split go to a
 * static device scratch buffer of PA_DECODE_SCRATCH_BYTES that the library
 * holds on every GPU it runs on, until the process ends.  The call allocates
 * nothing.  Its first call on a device (with that device current) looks up
 * the buffer's device address; make that first call outside graph capture.
 *   - A call whose split needs more than PA_DECODE_SCRATCH_BYTES
 *     (pa_decode_workspace_bytes) returns PA_ERR_WORKSPACE with no side
 *     effect.  The balanced split (PA_PARTITION_BALANCED, the library's
 *     choice) always fits; fixed partitions fit while
 *     num_seqs * num_q_heads * ceil(max_context_len / P) * (head_dim + 2) * 4
 *     <= PA_DECODE_SCRATCH_BYTES.
 *   - Every call on one GPU shares that GPU's buffer, and a call leaves its
 *     partial results there.  Nothing in it needs to start at zero: a call
 *     reads only what it wrote itself.  Calls that may overlap on one GPU
 *     (different streams, or different threads without ordering) race on the
 *     buffer and give undefined results: order them on one stream.
 */
#define PA_DECODE_SCRATCH_BYTES (64u << 20)
pa_status pa_decode_attention_noalloc(void* out, const void* query, const void* k_pool, const void* v_pool,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                      int32_t num_blocks, int32_t max_context_len, float scale,
                                      int32_t partition_size, pa_dtype dtype, void* stream);

/*
 * pa_prefill_attention -- causal multi-token attention over a paged, partly
 * cached context (chunked prefill, prefix reuse).
 *
 * When a prompt shares a cached prefix, only its new tokens run through
 * prefill and read the prefix's KV pages instead of recomputing them
 * (paged-KV analysis page, section 3.2 and the TTFT row of section 4.1).
 * Sequence s holds L = context_lens[s] tokens in its pages, the last
 * n = query_start[s+1] - query_start[s] of which are its new tokens, already
 * written with pa_kv_append.  Query row query_start[s] + j is the token at
 * position p = L - n + j; for q head h (KV head h / (Hq / Hkv)):
 *     out[row][h] = sum_{t <= p} exp(s_t - max) v_t / sum_{t <= p} exp(s_t - max),
 *     s_t = scale * <query[row][h], k_t>.
 * n = 1 is decode attention.  Probabilities are rounded to dtype for the
 * matrix-core product with V; accumulation is fp32; the output is rounded
 * once (nearest even) to dtype.
 *
 *   out            DEVICE [num_tokens][num_q_heads][head_dim] of dtype
 *   query          DEVICE [num_tokens][num_q_heads][head_dim] of dtype
 *   k_pool, v_pool DEVICE pools (see above), read only
 *   block_tables   DEVICE int32 [num_seqs][max_blocks_per_seq]
 *   context_lens   DEVICE int32 [num_seqs]
 *   query_start    DEVICE int32 [num_seqs + 1], non-decreasing, from 0 to
 *                  num_tokens (packed new tokens of every sequence)
 *   max_query_len  HOST upper bound of the per-sequence n (sizes the grid;
 *                  up to 2048 it also selects workgroups of 256 query rows,
 *                  above it of 128 -- a tuning choice, the results are equal
 *                  up to rounding order)
 * dtype must be PA_F16 or PA_BF16 (PA_ERR_DTYPE otherwise).  Rows of a
 * sequence with n > L, or past max_query_len, are not written; ranges outside
 * [0, num_tokens) are skipped.  No workspace.
 */
pa_status pa_prefill_attention(void* out, const void* query, const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, const int32_t* context_lens,
                               const int32_t* query_start, int32_t num_seqs, int32_t num_tokens,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                               int32_t max_query_len, float scale, pa_dtype dtype, void* stream);

/*
 * pa_decode_attention_hier / pa_prefill_attention_hier -- the same operations
 * as pa_decode_attention / pa_prefill_attention over two-level tables.
 *
 * Two page granularities at once, like an OS's huge and small pages: large
 * pages where a prompt is written in one go (fewer table entries), small
 * blocks where a sequence grows token by token (less fragmentation)
 * (Cross-Paper Synthesis page, section 5, the adaptive block size item).  A
 * large page is an aligned run of H = pages_per_large consecutive blocks of
 * the same pools, large page P covering blocks [P H, P H + H).  Sequence s's
 * logical block j (tokens [j bs, (j + 1) bs)) is
 *     large_tables[s][j / H] * H + j % H    for j < num_large[s] * H,
 *     small_tables[s][j - num_large[s] * H] otherwise.
 *
 *   small_tables   DEVICE int32 [num_seqs][max_small_per_seq]
 *   large_tables   DEVICE int32 [num_seqs][max_large_per_seq] (large-page ids)
 *   num_large      DEVICE int32 [num_seqs], clamped to [0, max_large_per_seq]
 *   pages_per_large H, a power of two in [1, 1024]
 * Lengths are clamped to (num_large[s] * H + max_small_per_seq) * block_size.
 * All other arguments, the workspace and the errors are those of the flat
 * calls.
 */
pa_status pa_decode_attention_hier(void* out, const void* query, const void* k_pool, const void* v_pool,
                                   const int32_t* small_tables, const int32_t* large_tables,
                                   const int32_t* num_large, const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_small_per_seq, int32_t max_large_per_seq,
                                   int32_t pages_per_large, int32_t num_blocks, int32_t max_context_len,
                                   float scale, int32_t partition_size, pa_dtype dtype, void* workspace,
                                   size_t workspace_bytes, void* stream);

pa_status pa_prefill_attention_hier(void* out, const void* query, const void* k_pool, const void* v_pool,
                                    const int32_t* small_tables, const int32_t* large_tables,
                                    const int32_t* num_large, const int32_t* context_lens,
                                    const int32_t* query_start, int32_t num_seqs, int32_t num_tokens,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t max_small_per_seq, int32_t max_large_per_seq,
                                    int32_t pages_per_large, int32_t num_blocks, int32_t max_query_len,
                                    float scale, pa_dtype dtype, void* stream);

/*
 * pa_block_copy -- copy-on-write block duplication, all pairs in one launch.
 *
 * Shared blocks (parallel samples, beams, common prompts) are reference
 * counted; a sequence about to write into a block that others still use gets
 * a private copy first (vLLM entity page, "what it is"; paged-KV analysis
 * page, sections 2.3 and 3.2).  For every pair p:
 *     src = block_mapping[2p], dst = block_mapping[2p + 1],
 *     k_pool[dst] = k_pool[src], v_pool[dst] = v_pool[src]   (all heads, all slots)
 * Bits are preserved.  Pairs with an id outside [0, num_blocks) are skipped.
 * Destinations must be distinct and must not be sources of the same call.
 *
 *   k_pool, v_pool DEVICE pools, written in place
 *   block_mapping  DEVICE int32 [num_pairs][2]
 * num_pairs == 0 is a no-op returning PA_OK.
 */
pa_status pa_block_copy(void* k_pool, void* v_pool, const int32_t* block_mapping, int32_t num_pairs,
                        int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                        int32_t num_blocks, pa_dtype dtype, void* stream);

/*
 * pa_swap_out / pa_swap_in -- move whole blocks between the pools and pinned
 * host memory, one launch per block list.
 *
 * Preemption evicts every block of a request at once and brings them back
 * when it resumes (Cross-Paper Synthesis page, section 3, the preemption
 * item); the pages blame slow KV movement on many small copies and credit a
 * block-first layout (vLLM entity page, key observations).  The host buffer is
 * block-first: entry i is block block_ids[i]'s K tile followed by its V tile,
 *     host[i][0][h][o][:] = k_pool[block_ids[i]][h][o][:]
 *     host[i][1][h][o][:] = v_pool[block_ids[i]][h][o][:]
 * (shape [num_ids][2][num_kv_heads][block_size][head_dim] of dtype).
 * pa_swap_out writes the host buffer from the pools; pa_swap_in writes the
 * listed pool blocks from the host buffer.  Byte copies; ids outside
 * [0, num_blocks) are skipped (their host entries are not touched).  For
 * pa_swap_in the ids must be distinct.
 *
 *   k_pool, v_pool DEVICE pools (read by swap_out, written by swap_in)
 *   block_ids      DEVICE int32 [num_ids]
 *   host_dst/src   HOST pinned memory from hipHostMalloc (torch: pin_memory),
 *                  16-byte aligned, >= num_ids * 2 * Hkv * bs * D * elt bytes;
 *                  the GPU reads or writes it directly over the host link.
 *                  PA_ERR_HOST_MEMORY unless HIP knows it as pinned host
 *                  memory mapped for the GPU at the same address (checked
 *                  with hipPointerGetAttributes and hipHostGetDevicePointer,
 *                  which have no other effect).  The host sees swap_out's data, and may
 *                  reuse swap_in's buffer, once the stream has passed the call.
 * num_ids == 0 is a no-op returning PA_OK.  Blocks that a block manager frees
 * on swap-out may be handed out again at once: enqueue pa_swap_out before any
 * work that writes them, on the same stream.
 */
pa_status pa_swap_out(const void* k_pool, const void* v_pool, const int32_t* block_ids, int32_t num_ids,
                      void* host_dst, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                      int32_t num_blocks, pa_dtype dtype, void* stream);

pa_status pa_swap_in(const void* host_src, void* k_pool, void* v_pool, const int32_t* block_ids,
                     int32_t num_ids, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                     int32_t num_blocks, pa_dtype dtype, void* stream);

/*
 * pa_stream_read -- measurement aid, not a step of the method: the
 * achievable HBM read bandwidth that the decode kernel's streaming is judged
 * against (a plain sweep has no table, softmax or output).
 *   buf       DEVICE, 16-byte aligned (PA_ERR_ALIGN), read once
 *   bytes     a multiple of 16 (PA_ERR_SHAPE); 0 is a no-op returning PA_OK
 *   partials  DEVICE uint32 [PA_STREAM_READ_PARTIALS], caller-owned; receives
 *             one XOR of 32-bit words per workgroup, and the XOR of all
 *             partials is the XOR of every 32-bit word of the buffer (so the
 *             result can be checked and no load can be skipped)
 * Asynchronous on `stream`; allocates nothing.
 */
#define PA_STREAM_READ_PARTIALS 16384
pa_status pa_stream_read(const void* buf, uint64_t bytes, uint32_t* partials, void* stream);

/*
 * pa_debug_violations -- what the caller's contract checks of a checked build
 * found.
 *
 * The normal build does not check device-side contents: kernels clamp or skip
 * whatever breaks the contract stated above (memory stays safe, results for
 * such inputs are unspecified).  A build with PA_DEBUG_CHECKS=1
 * (paged_kv_cache_313_amd/_build.py build_checked(): libpagedkv_checked.so,
 * same ABI) also records, in device flag words, each kind of violation a
 * kernel met.  This call stores the bits met since the last clear, OR-ed over
 * all kernels, in *flags, and resets them when clear != 0.
 *   flags   HOST uint32, written (PA_VIOLATION_* bits)
 * HOST; unlike every other entry point it synchronises with the device (it
 * copies the flag words).  The normal build returns PA_ERR_UNSUPPORTED and
 * makes no HIP call; a NULL flags gives PA_ERR_NULL.
 */
#define PA_VIOLATION_TABLE_ID 1u  /* a block-table entry in use was outside [0, num_blocks)         */
#define PA_VIOLATION_LENGTH 2u    /* a length was negative or above its bound (max_context_len, the
                                     table's capacity; prefill: query_start ranges, max_query_len)  */
#define PA_VIOLATION_SLOT 4u      /* an append slot >= num_blocks * block_size                       */
#define PA_VIOLATION_BLOCK_ID 8u  /* a copy-on-write or swap block id outside [0, num_blocks)        */
pa_status pa_debug_violations(uint32_t* flags, int32_t clear);

/* Static, human-readable name of a status code.  HOST only. */
const char* pa_status_string(pa_status status);

/* hipError_t (as int) of the last call on this thread that returned PA_ERR_HIP;
 * 0 if none.  HOST only. */
int pa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_PA_H */
