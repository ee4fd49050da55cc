// Device-side helpers shared by the libpagedkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Contract checks (builds with PA_DEBUG_CHECKS=1 only).  Every kernel clamps
// or skips what breaks the caller's contract (a table entry outside the pool,
// a length above its bound, a slot or block id out of range); a checked build
// also records each kind in this translation unit's flag word, which
// pa_debug_violations() reads and clears.  Bits as in include/pa.h.
#ifndef PA_DEBUG_CHECKS
#define PA_DEBUG_CHECKS 0
#endif
constexpr uint32_t kViolationTableId = 1u;   // PA_VIOLATION_TABLE_ID
constexpr uint32_t kViolationLength = 2u;    // PA_VIOLATION_LENGTH
constexpr uint32_t kViolationSlot = 4u;      // PA_VIOLATION_SLOT
constexpr uint32_t kViolationBlockId = 8u;   // PA_VIOLATION_BLOCK_ID
#if PA_DEBUG_CHECKS
static __device__ uint32_t violations;
#define PA_FLAG_IF(cond, bit)                           \
  do {                                                  \
    if (cond) atomicOr(&::pa::violations, (bit));       \
  } while (0)
// host side of one translation unit: read (and optionally clear) its flags
#define PA_VIOLATIONS_GETTER(name)                                                  \
  hipError_t name(uint32_t* flags, bool clear) {                                    \
    hipError_t e = hipMemcpyFromSymbol(flags, HIP_SYMBOL(violations), sizeof(uint32_t)); \
    if (e != hipSuccess || !clear) return e;                                        \
    const uint32_t zero = 0;                                                        \
    return hipMemcpyToSymbol(HIP_SYMBOL(violations), &zero, sizeof(uint32_t));      \
  }
#else
#define PA_FLAG_IF(cond, bit) ((void)0)
#define PA_VIOLATIONS_GETTER(name)                     \
  hipError_t name(uint32_t* flags, bool) {             \
    *flags = 0;                                        \
    return hipSuccess;                                 \
  }
#endif

constexpr int kWave = 64;
constexpr int kNumXcd = 8;          // MI355X: 8 XCDs of 32 CUs, workgroups dealt round-robin
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// storage tags: the element type as stored in HBM
struct F32 { using elem = float;    static constexpr int bytes = 4; };
struct F16 { using elem = uint16_t; static constexpr int bytes = 2; };
struct BF16 { using elem = uint16_t; static constexpr int bytes = 2; };

// Buffer resource over [base, base + bytes): loads through it are range
// checked by the hardware (an offset past the end reads zeros), and the
// base lives in SGPRs, so a lane only supplies a 32-bit offset.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit data, gfx9-family buffer descriptor
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ u32x4 buf_ld16(rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// Loads of data a kernel reads once (the K/V stream of a decode call, a
// bandwidth sweep) carry the non-temporal hint (`nt`).  Measured on MI355X
// over 4 GiB: 6.8-7.0 TB/s with it against 6.0-6.2 TB/s without, for
// contiguous ranges and for randomly placed 4 KiB blocks alike.
// Data that other waves of the same call read too keeps the default policy,
// so that they hit in L2 and the MALL.
#ifndef PA_STREAM_AUX
#define PA_STREAM_AUX 2
#endif
constexpr int kAuxDefault = 0;
constexpr int kStreamAux = PA_STREAM_AUX;   // buffer-load cache-policy bits (2 = nt)
template <int AUX>
__device__ __forceinline__ u32x4 buf_ld16_aux(rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, AUX);
}
template <int AUX>
__device__ __forceinline__ u32x4 ld16_aux(const void* p) {
  if constexpr (AUX == 2) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return ld16(p);
}
__device__ __forceinline__ u32x4 ld16_stream(const void* p) { return ld16_aux<kStreamAux>(p); }
template <int AUX>
__device__ __forceinline__ void st16_aux(void* p, u32x4 v) {
  if constexpr (AUX == 2) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  else st16(p, v);
}

// ---- unpack 16 loaded bytes to fp32 (exact) --------------------------------
template <class T> struct Unpack;
template <> struct Unpack<F32> {
  static constexpr int n = 4;
  __device__ __forceinline__ static void run(u32x4 v, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v[i]);
  }
};
template <> struct Unpack<BF16> {
  static constexpr int n = 8;
  __device__ __forceinline__ static void run(u32x4 v, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(v[i] << 16);
      o[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
};
template <> struct Unpack<F16> {
  static constexpr int n = 8;
  __device__ __forceinline__ static void run(u32x4 v, float* o) {
    // element by element from a scalar copy: clang mis-lowers a bit_cast
    // whose operand is an element of an ext_vector (it reads element 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = v[i];
      o[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
      o[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
    }
  }
};

// ---- dot products of one 16-byte chunk pair, into 4 independent partials ----
// (16-bit types: v_dot2c_f32_{f16,bf16}, products exact in fp32)
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <class T> struct Dot16;
template <> struct Dot16<F32> {
  __device__ __forceinline__ static void run(u32x4 q, u32x4 k, float* d) {
#pragma unroll
    for (int e = 0; e < 4; ++e) d[e] = fmaf(__uint_as_float(q[e]), __uint_as_float(k[e]), d[e]);
  }
};
template <> struct Dot16<F16> {
  __device__ __forceinline__ static void run(u32x4 q, u32x4 k, float* d) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t qe = q[e], ke = k[e];
      d[e] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, qe), __builtin_bit_cast(f16x2, ke), d[e], false);
    }
  }
};
template <> struct Dot16<BF16> {
  __device__ __forceinline__ static void run(u32x4 q, u32x4 k, float* d) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t qe = q[e], ke = k[e];
      d[e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qe), __builtin_bit_cast(bf16x2, ke),
                                             d[e], false);
    }
  }
};

// acc[0..NE) += p * (16-byte chunk v), fp32 accumulate (fp16: v_fma_mix_f32)
template <class T> struct Axpy16;
template <> struct Axpy16<F32> {
  __device__ __forceinline__ static void run(float p, u32x4 v, float* acc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(p, __uint_as_float(v[e]), acc[e]);
  }
};
template <> struct Axpy16<F16> {
  __device__ __forceinline__ static void run(float p, u32x4 v, float* acc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x = v[e];
      acc[2 * e] = fmaf(p, (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu)), acc[2 * e]);
      acc[2 * e + 1] = fmaf(p, (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16)), acc[2 * e + 1]);
    }
  }
};
template <> struct Axpy16<BF16> {
  __device__ __forceinline__ static void run(float p, u32x4 v, float* acc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x = v[e];
      acc[2 * e] = fmaf(p, __uint_as_float(x << 16), acc[2 * e]);
      acc[2 * e + 1] = fmaf(p, __uint_as_float(x & 0xffff0000u), acc[2 * e + 1]);
    }
  }
};

// ---- fp32 -> storage, round to nearest even --------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32 rounds to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
template <class T> __device__ __forceinline__ void store_elem(void* base, size_t idx, float v);
template <> __device__ __forceinline__ void store_elem<F32>(void* base, size_t idx, float v) {
  reinterpret_cast<float*>(base)[idx] = v;
}
template <> __device__ __forceinline__ void store_elem<BF16>(void* base, size_t idx, float v) {
  reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16_rne(v);
}
template <> __device__ __forceinline__ void store_elem<F16>(void* base, size_t idx, float v) {
  reinterpret_cast<uint16_t*>(base)[idx] = f32_to_f16_rne(v);
}

// ---- matrix cores -----------------------------------------------------------
// D[16x16] += A[16x32] B[32x16] in fp32.  Lane l supplies A row l % 16 and B
// column l % 16, each as the 8 k-values 8 (l / 16) .. 8 (l / 16) + 7 packed in
// 16 bytes; it receives D rows 4 (l / 16) .. 4 (l / 16) + 3 of column l % 16.
template <class T>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma_16x16x32<BF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma_16x16x32<F16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// D[16x16] += A[16x16] B[16x16] in fp32.  Lane l supplies A row l % 16 and B
// column l % 16, each as the 4 k-values 4 (l / 16) .. 4 (l / 16) + 3 packed in
// 8 bytes (the lower half of the first dword is the first); it receives D
// rows 4 (l / 16) .. 4 (l / 16) + 3 of column l % 16.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
template <class T>
__device__ __forceinline__ f32x4 mfma_16x16x16(u32x2 a, u32x2 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma_16x16x16<BF16>(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b),
                                                   c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma_16x16x16<F16>(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c,
                                               0, 0, 0);
}

// two fp32 values rounded (to nearest even) into one packed 16-bit pair
template <class T> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <> __device__ __forceinline__ uint32_t pack2<BF16>(float lo, float hi) {
  // one v_cvt_pk_bf16_f32 on gfx950 (round to nearest even)
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
template <> __device__ __forceinline__ uint32_t pack2<F16>(float lo, float hi) {
  return (uint32_t)f32_to_f16_rne(lo) | ((uint32_t)f32_to_f16_rne(hi) << 16);
}

// the two values of a packed 16-bit pair, exactly in fp32
template <class T> __device__ __forceinline__ void unpack2(uint32_t x, float& lo, float& hi);
template <> __device__ __forceinline__ void unpack2<BF16>(uint32_t x, float& lo, float& hi) {
  lo = __uint_as_float(x << 16);
  hi = __uint_as_float(x & 0xffff0000u);
}
template <> __device__ __forceinline__ void unpack2<F16>(uint32_t x, float& lo, float& hi) {
  lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
  hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
}

// ---- cross-lane moves -------------------------------------------------------
// butterfly exchange with lane ^ mask (ds_swizzle / bpermute through the LDS crossbar
// for masks >= 16, DPP for the in-row masks)
template <int MASK>
__device__ __forceinline__ float xor_lane(float x) {
  if constexpr (MASK == 1) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false));  // quad_perm [1,0,3,2]
  } else if constexpr (MASK == 2) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false));  // quad_perm [2,3,0,1]
  } else {
    return __shfl_xor(x, MASK, kWave);
  }
}

// x combined with the value of lane ^ 16 or lane ^ 32 by the VALU lane swaps
// of gfx950 (v_permlane16_swap / v_permlane32_swap, no LDS crossbar): the
// swap leaves the lane's own value in one result and its partner's in the
// other, and both operations below are exact in either operand order, so
// the results equal those of a butterfly through the crossbar bit for bit.
template <int MASK>
__device__ __forceinline__ float swap_pair_sum(float x) {
  static_assert(MASK == 16 || MASK == 32, "lane swaps");
  const uint32_t u = __float_as_uint(x);
  if constexpr (MASK == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}
template <int MASK>
__device__ __forceinline__ float swap_pair_max(float x) {
  static_assert(MASK == 16 || MASK == 32, "lane swaps");
  const uint32_t u = __float_as_uint(x);
  if constexpr (MASK == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
}

// the value of lane (i + N) mod 16 within each 16-lane row (DPP row_ror:N)
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  static_assert(N >= 1 && N <= 15, "row rotate");
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}

// broadcast lane `src` of each quad (DPP quad_perm) -- src in 0..3
template <int SRC>
__device__ __forceinline__ float quad_bcast(float x) {
  constexpr int ctrl = SRC * 0x55;
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xf, 0xf, false));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- work-unit mapping -----------------------------------------------------
// Workgroup b runs on XCD b % 8 (dealt round-robin).  Map b to a logical unit
// so that each XCD receives runs of 8 consecutive logical units, the runs
// dealt round-robin: neighbouring units (e.g. samples that share a prompt's
// blocks) meet in one XCD's L2 at about the same time, and every XCD still
// gets an even mix of the whole grid.  Bijective on [0, n); the last n % 64
// units map to themselves.
__device__ __forceinline__ uint32_t xcd_unit(uint32_t b, uint32_t n) {
  const uint32_t full = n & ~63u;
  if (b >= full) return b;
  const uint32_t x = b & 7u, k = b >> 3;
  return ((k >> 3) << 6) | (x << 3) | (k & 7u);
}

constexpr int kModeUnit = 0;       // one workgroup per (sequence, head group[, partition])
constexpr int kModeBalanced = 1;   // resident grid, equal share of the flattened tiles each
constexpr int kBalancedMaxSeqs = 4096;   // sequences a balanced launch can take (LDS prefix)
// Waves a balanced workspace is sized for.  MI355X keeps 256 CUs x one 4-wave
// workgroup resident in the balanced grid (1,024 waves); the grid is capped
// here, so a device with more CUs gets fewer workgroups per CU, never more
// partial slots than the workspace holds.
constexpr int kBalancedMaxWaves = 2048;

// Arguments of the decode kernels (by value, in the kernarg segment).
struct DecodeArgs {
  void* out;                  // [S, Hq, D] dtype
  const void* query;          // [S, Hq, D] dtype
  const void* k_pool;         // [NB, Hkv, BS, D]
  const void* v_pool;
  const int32_t* block_tables;  // [S, MB]
  const int32_t* context_lens;  // [S]
  float* ws_o;                // [S, Hq, NP, D] un-normalised partial outputs, 16-byte aligned
                              // (balanced mode: 2 slots per wave of H rows each)
  float* ws_m;                // [S, Hq, NP] running max (log2 domain)
  float* ws_l;                // [S, Hq, NP] running sum
  int64_t* ws_desc;           // balanced mode: [kBalancedMaxWaves][4] merge descriptors, one per
                              // wave boundary: {A0 (< 0: nothing to merge), ntot, output row, pieces}
  int32_t num_seqs, num_q_heads, num_kv_heads;
  int32_t max_blocks_per_seq, num_blocks, max_context_len;
  int32_t partition_size;     // tokens per unit (>= max_context_len when not split)
  int32_t num_parts;          // partitions in the grid (1 when not split)
  int32_t split;              // 1 when partial results go through the workspace
  int32_t head_chunks;        // head groups per sequence (Hkv on the MFMA path)
  int32_t mode;               // kModeUnit or kModeBalanced
  float scale_log2;           // scale * log2(e)
  // two-level tables (nullptr: block_tables is the whole table)
  const int32_t* large_tables;  // [S, max_large_per_seq] large-page ids
  const int32_t* num_large;     // [S] large pages in use
  int32_t max_large_per_seq;
  int32_t large_shift;          // log2(blocks per large page)
};

// Prefix groups of the grouped decode: sequences group_start[i] ..
// group_start[i+1] - 1 hold the same blocks for their first group_shared[i]
// tokens.  A kernel argument of its own, so that DecodeArgs (and with it
// every other decode kernel) stays as it is.
struct GroupArgs {
  const int32_t* group_start;   // [num_groups + 1]
  const int32_t* group_shared;  // [num_groups]
  int32_t num_groups;
  int32_t max_group_size;       // host bound of group_start[i+1] - group_start[i]
  int32_t shared_parts;         // partitions of the longest shared prefix in the grid
};

// Arguments of the prefill kernel.
struct PrefillArgs {
  void* out;                    // [T, Hq, D] dtype
  const void* query;            // [T, Hq, D] dtype
  const void* k_pool;           // [NB, Hkv, BS, D]
  const void* v_pool;
  const int32_t* block_tables;  // [S, MB]
  const int32_t* context_lens;  // [S]
  const int32_t* query_start;   // [S + 1]
  int32_t num_seqs, num_q_heads, num_kv_heads;
  int32_t max_blocks_per_seq, num_blocks;
  int32_t num_tokens;           // rows of query and out
  int32_t max_query_len;        // host bound of query_start[s+1] - query_start[s]
  int32_t qblocks;              // query blocks per (sequence, KV head) in the grid
  float scale_log2;             // scale * log2(e)
  const int32_t* large_tables;  // two-level tables, as in DecodeArgs (nullptr: flat)
  const int32_t* num_large;
  int32_t max_large_per_seq;
  int32_t large_shift;
};

// One sequence's block table, flat or two-level.  In the two-level form a
// large page P is the aligned run of blocks [P << shift, (P + 1) << shift);
// logical blocks [0, nl_blocks) sit in the sequence's large pages, the rest in
// its small-block row.  entry() is unchecked: callers clamp ids into the pool.
struct TableView {
  const int32_t* small;
  const int32_t* large;
  int32_t nl_blocks;
  int32_t shift;
  int32_t capacity;    // logical blocks the tables can describe
  __device__ __forceinline__ int entry(int j) const {
    if (j < nl_blocks) return (large[j >> shift] << shift) + (j & ((1 << shift) - 1));
    return small[j - nl_blocks];
  }
  // The same value from one load of whichever level holds entry j, with no
  // branch around it, so that the loads of several entries can all be in
  // flight at once.
  __device__ __forceinline__ int entry_sel(int j) const {
    const bool in_large = j < nl_blocks;
    const int32_t* base = in_large ? large : small;
    const int x = base[in_large ? (j >> shift) : (j - nl_blocks)];
    return in_large ? (x << shift) + (j & ((1 << shift) - 1)) : x;
  }
};

template <class Args>
__device__ __forceinline__ TableView table_view(const Args& a, int s) {
  TableView v;
  v.small = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  v.large = nullptr;
  v.nl_blocks = 0;
  v.shift = 0;
  if (a.large_tables) {
    int nl = a.num_large[s];
    nl = nl < 0 ? 0 : (nl > a.max_large_per_seq ? a.max_large_per_seq : nl);
    v.large = a.large_tables + (size_t)s * a.max_large_per_seq;
    v.shift = a.large_shift;
    v.nl_blocks = nl << a.large_shift;
  }
  v.capacity = v.nl_blocks + a.max_blocks_per_seq;
  return v;
}

__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int s, int block_size) {
  int L = a.context_lens[s];
  const int cap_tbl = table_view(a, s).capacity * block_size;
  PA_FLAG_IF(L < 0 || L > cap_tbl || L > a.max_context_len, kViolationLength);
  L = L < 0 ? 0 : L;
  L = L > cap_tbl ? cap_tbl : L;
  L = L > a.max_context_len ? a.max_context_len : L;
  return L;
}

}  // namespace pa
