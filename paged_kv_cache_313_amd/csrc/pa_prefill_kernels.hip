// Multi-token (prefill) attention over a paged, partly cached context
// (gfx950, wave64, MFMA).
//
// When a prompt reuses a cached prefix, only its new tokens run through
// prefill, reading the prefix's KV pages instead of recomputing them
// (vLLM/PagedAttention paged-KV analysis page, sections 3.2 and 4.1).  New
// token j of sequence s sits at position p = L - n + j and attends causally
// to the tokens t <= p of the sequence's paged context.  This is a dense
// contraction on both sides of the softmax, so both run on the matrix cores.
//
// Work unit: one workgroup of 8 waves per (sequence, KV head, block of
// query tokens).  The 256 query rows of a workgroup are (token, head)
// pairs of the G heads sharing the KV head, heads fastest: each wave owns two
// groups of 16.  Keys advance 64 at a time through double-buffered LDS tiles:
// K and V row-major (V's operand comes from gfx950's transposing LDS read),
// both gathered through the block table by all threads, the next tile's
// loads in flight while the current one is used.
//
// Per tile, each wave computes, for each of its row groups and 16-key slices,
//   S^T[key][row] = K Q^T          (A = K from LDS, B = its query rows, kept
//                                   in registers for the whole unit)
// so that lane l holds the scores of query row l % 16 for keys
// 4 (l / 16) + {0..3} and 16 + 4 (l / 16) + {0..3}: exactly the 8 k-values
// that lane supplies as the B operand of
//   O^T[d][row] += V^T P^T          (A = V^T from LDS)
// once k-slot 8 (l / 16) + j is taken to mean those keys (the contraction
// order is free as long as A and B agree).  The probabilities never leave the
// lane; a query row's running max is shared by the 4 lanes l % 16 = row (two
// row swaps form it when it has to move) and its sum comes from the matrix
// cores.  Online softmax in the log2 domain
// with a lazy rescale (a row's reference max moves only when a score exceeds
// it by more than 2^8), P rounded to the input type for the MFMA, fp32
// accumulation.
#include <type_traits>

#include "pa_common.hpp"
#include "pa_launch.hpp"

namespace pa {

// Workgroups of 8 waves (256 query rows) stage each K/V tile once for twice
// the rows of a 4-wave one.  With the query blocks handed out longest band
// first (below) they were faster on every workload measured: 8-14 % on
// chunked prefill, and on fresh prompts 578 against 606 us (4 x 4K), 1,046
// against 1,114 us (2 x 8K), 2,029 against 2,187 us (16K), 7,977 against
// 8,656 us (32K), 3,550 against 4,034 us for 4 x 4K new tokens on 16K
// contexts (bit-identical results).  Before that order, fresh 4K-8K prompts
// had run 5-11 % faster in 4-wave workgroups.  PA_PREFILL_WAVES=4 builds the
// 4-wave form.
#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 8
#endif
constexpr int kPfWaves = PA_PREFILL_WAVES;
static_assert(kPfWaves == 4 || kPfWaves == 8, "prefill workgroup");
#ifndef PA_PREFILL_KEYS
#define PA_PREFILL_KEYS 64
#endif
constexpr int kPfKeys = PA_PREFILL_KEYS;  // keys per tile (32 or 64)
constexpr int kPfSub = kPfKeys / 16;     // 16-key score tiles per key tile
static_assert(kPfKeys == 32 || kPfKeys == 64, "key tile");
constexpr float kPfLazy = 8.f;
// Row groups of 16 per wave: every K or V^T operand a wave reads from LDS
// feeds NG matrix-core products, which keeps LDS traffic per product below
// what the matrix cores consume (one 16x16x32 product needs a 1 KiB operand).
#ifndef PA_PREFILL_GROUPS
#define PA_PREFILL_GROUPS 2
#endif
// LDS operand reads issued this many reads ahead of the products that use
// them (the compiler otherwise waits on each read right before its product)
#ifndef PA_PREFILL_SCHED
#define PA_PREFILL_SCHED 3
#endif
constexpr int kPfGroups = PA_PREFILL_GROUPS;

// K is staged row-major.  V is staged transposed: row d of a tile holds its
// key pairs as dwords (the d-th elements of keys 2p and 2p + 1).  The pairs
// sit in the order the matrix-core operand takes them: dword 4 (4 h + gq) +
// slot holds pair 16 h + 2 gq + (slot & 1) + 8 (slot >> 1), i.e. keys
// 4 gq .. 4 gq + 3 and 16 + 4 gq .. 16 + 4 gq + 3 of half h, so lane (c, gq)
// reads its 8 keys of a row as one aligned 16-byte load.  A thread owns one
// such pair position of one 16-byte d-chunk and writes the pair to each of
// its 8 d rows as one dword.  The 64 lanes of a write instruction cover 16
// d-chunks (rows 8 apart, which the 144-byte row pitch maps onto 2 bank
// groups) and 4 consecutive positions, so row r keeps position x at
// x ^ vt_swizzle(r), which spreads those lanes over all 64 banks.  The swizzle
// is a multiple of 4, so each lane's 16-byte group stays whole.
__device__ __forceinline__ int vt_swizzle(int row) { return 4 * ((row >> 4) & (kPfKeys / 8 - 1)); }
// pair (within the tile) stored at position x
__device__ __forceinline__ int vt_pair(int x) {
  return 16 * (x >> 4) + 2 * ((x >> 2) & 3) + (x & 1) + 8 * ((x >> 1) & 1);
}
// V staging: 1 (the default) keeps V row-major in LDS (two 16-byte stores
// per key pair, like K) and forms the P.V operand with gfx950's transposing
// LDS read, two 8-byte reads per operand; 0 stores V transposed (8 dword
// stores per key pair, one 16-byte operand read).  Both give bit-identical
// results.  Timed after 30 warm-up calls each, in alternating order: equal
// on the 16 x 512-token chunked prefill (medians 502-514 us for both and the
// later changes), 1-2 % faster on 4 fresh 4096-token prompts.  Filling the
// tiles with gfx950's global-to-LDS loads instead of registers (1 KiB runs,
// padded or swizzled images) was slower.
#ifndef PA_PREFILL_VTR
#define PA_PREFILL_VTR 1
#endif
template <int D, int NW>
struct PfLayout {
  static constexpr int kThreads = NW * kWave;
  // K row pitch: D + 16 elements.  With 8 elements of padding rocprofv3
  // counted 31.7 M LDS bank-conflict cycles per chunked-prefill call (D 128;
  // 15.9 M at D 64), none of them from V (changing V's pitch or its read
  // left that count alone); with 16 it counts none, and the call is about
  // 1 % faster.  24 or 32 elements gave the same conflicts as 8; 80 gave
  // none but ran slower at D 64.
  static constexpr int kRowB = D * 2 + 32;
  static constexpr int kVtB = kPfKeys * 2 + 16;      // V^T row pitch in LDS (bytes), padded, 16-byte aligned
  // V row pitch: D + 16 elements, so that the 4 rows one transposing read
  // touches (32 bytes each) start 8 dwords apart in the 64 banks
  static constexpr int kVrB = D * 2 + 32;
  static constexpr int kKBytes = kPfKeys * kRowB;
  static constexpr int kVBytes = PA_PREFILL_VTR ? kPfKeys * kVrB : D * kVtB;
  static constexpr int kBufBytes = kKBytes + kVBytes;
  static constexpr int CPR = D / 8;                  // 16-byte chunks per token row
  static constexpr int kPairs = kPfKeys / 2 * CPR;   // (key pair, d-chunk) units per tile
  static constexpr bool kPartial = kPairs < kThreads;   // then threads >= kPairs load nothing
  static constexpr int NPAIR = kPartial ? 1 : kPairs / kThreads;   // key pairs per thread per tile
  static constexpr int NCH = 2 * NPAIR;              // chunks per thread per tile
  static_assert(kPartial || NPAIR * kThreads == kPairs, "tile split");
  static_assert(kRowB % 16 == 0 && kVtB % 16 == 0 && kVrB % 16 == 0 && kBufBytes % 16 == 0, "16-byte LDS rows");
};

// max over the 4 lanes of a query row (c, c + 16, c + 32, c + 48): the row
// swaps exchange 16-lane rows and 32-lane halves without the LDS crossbar
__device__ __forceinline__ float row_max4(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const uint32_t v = __float_as_uint(x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

template <class T, int D, int G, int NW>
__global__ __launch_bounds__(NW * kWave) void prefill_kernel(PrefillArgs a, int block_size, int bs_shift) {
  using Lay = PfLayout<D, NW>;
  constexpr int kPfThreads = Lay::kThreads;
  constexpr int NG = kPfGroups;
  constexpr int QB = NW * 16 * NG / G;     // query tokens per workgroup
  constexpr int TPW = 16 * NG / G;         // query tokens per wave
  constexpr int NKC = D / 32;              // k-chunks of the score MFMA
  constexpr int NDT = D / 16;              // 16-row d tiles of the output
  __shared__ __align__(16) char lds[2 * Lay::kBufBytes];

  // unit: (sequence, KV head, query block).  Query blocks go in bands of 8
  // counted from each sequence's last block (the most keys under the causal
  // mask), the first band first for every (sequence, KV head), so that the
  // longest units start first over the whole grid, also when sequences bring
  // different numbers of new tokens; within a band a (sequence, KV head)'s
  // blocks are consecutive, last first, and the 8 of a band form one of
  // xcd_unit's runs, so they share an L2.  A unit with no block of its
  // sequence left exits.  Against the order with each (sequence, KV head)'s blocks
  // all together, whose last pairs' long blocks started near the end: fresh
  // 4K prompts 797 -> 590 us, fresh 8K 1,328 -> 1,100 us, 16 x 2,048 new
  // tokens on 8K contexts 3,979 -> 3,573 us (bit-identical; the same order
  // when a sequence has at most 8 blocks).  Bands of 4 or no bands at all
  // (longest first, (sequence, KV head) fastest) were slower on the 2,048-
  // token chunks: their blocks meet less often in an L2.  Counting the bands
  // from each sequence's own last block rather than from the batch's longest
  // took a mixed batch (16 sequences, 8 to 2,048 new tokens on 2K-8K
  // contexts) from 1,115 to 1,095 us.
  constexpr uint32_t kBand = 8;
  const uint32_t u = xcd_unit(blockIdx.x, gridDim.x);
  const uint32_t SG = (uint32_t)a.num_seqs * (uint32_t)a.num_kv_heads;
  const uint32_t band = (uint32_t)(u / ((uint64_t)SG * kBand));
  const uint32_t bw = min(kBand, (uint32_t)a.qblocks - band * kBand);   // blocks in this band
  const uint32_t rest = (uint32_t)(u - (uint64_t)band * SG * kBand);
  const int r = (int)(band * kBand + rest % bw);   // blocks after this one in its sequence
  const int sg = (int)(rest / bw);
  const int g = sg % a.num_kv_heads;
  const int s = sg / a.num_kv_heads;
  if (s >= a.num_seqs) return;
  // memory safety on inconsistent inputs: rows outside [0, num_tokens), more
  // new tokens than the context holds, or a query block past the sequence's
  // new tokens leave the unit idle (and those rows unwritten)
  const int q0 = a.query_start[s];
  const int n = a.query_start[s + 1] - q0;
  const TableView trow = table_view(a, s);
  const int L = min(a.context_lens[s], trow.capacity * block_size);
  PA_FLAG_IF(threadIdx.x == 0 && r == 0 &&
                 (a.context_lens[s] > trow.capacity * block_size || q0 < 0 || n < 0 || n > a.num_tokens - q0 ||
                  n > L || n > a.max_query_len),
             kViolationLength);
  if (q0 < 0 || n <= 0 || n > a.num_tokens - q0 || n > L) return;
  // blocks of this sequence (never more than the grid's: past max_query_len
  // its later tokens stay unwritten), this unit's block counted from its start
  const int qb = min((n + QB - 1) / QB, a.qblocks) - 1 - r;
  if (qb < 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int c = lane & 15, gq = lane >> 4;

  // this lane's query rows: column c of each of the wave's NG row groups;
  // row r = 16 (NG wave + grp) + c of the workgroup is token r / G, head r % G
  // A negative scale goes into Q (flipping the sign bits is exact), so the
  // kernel scales by sp > 0; a zero scale becomes the smallest normal float,
  // which keeps -inf * sp = -inf for masked scores and changes no weight.
  const uint32_t qneg = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  const float sp = fmaxf(fabsf(a.scale_log2), 1.17549435e-38f);
  int tq[NG], pos[NG];
  bool row_ok[NG];
  u32x4 qop[NG][NKC];
  const int hh = c % G;                  // the same head in every group (16 % G == 0)
#pragma unroll
  for (int grp = 0; grp < NG; ++grp) {
    tq[grp] = qb * QB + (16 * (NG * wave + grp) + c) / G;
    row_ok[grp] = tq[grp] < n;
    pos[grp] = L - n + (row_ok[grp] ? tq[grp] : n - 1);
    const u32x4 z = {0u, 0u, 0u, 0u};
    const char* qrow = reinterpret_cast<const char*>(a.query) +
                       (((size_t)(q0 + (row_ok[grp] ? tq[grp] : 0)) * a.num_q_heads + (size_t)g * G + hh) * D) * 2;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      qop[grp][kc] = row_ok[grp] ? ld16(qrow + (32 * kc + 8 * gq) * 2) : z;
#pragma unroll
      for (int e = 0; e < 4; ++e) qop[grp][kc][e] ^= qneg;
    }
  }
  const int wave_last = L - n + min(qb * QB + (wave + 1) * TPW, n) - 1;   // wave's largest position
  const int kend = L - n + min(qb * QB + QB, n);                          // keys the unit needs

  const char* kpool = reinterpret_cast<const char*>(a.k_pool);
  const char* vpool = reinterpret_cast<const char*>(a.v_pool);
  const int bmask = block_size - 1;

  // A key pair (t, t + 1) with t even lies in one block (block sizes are
  // even), so a thread looks up one table entry and computes one address per
  // pair.  Pairs at or past the context's end are read from its last pair:
  // in bounds, and masked below.  The entries a tile needs are loaded one
  // tile before its K/V, so the two dependent loads of a tile (entry, then
  // data) overlap two tiles of compute.
  const int last_pair = (L - 1) & ~1;
  int ids[Lay::NPAIR];
  u32x4 kreg[Lay::NCH], vreg[Lay::NCH];
  // unit jp of this thread: V^T pair position x (d-chunk fastest, so 16
  // lanes cover a token row) holding the key pair vt_pair(x)
  auto pair_pos = [&](int jp) { return (jp * kPfThreads + tid) / Lay::CPR; };
  auto pair_key = [&](int jp) { return 2 * vt_pair(pair_pos(jp)); };
  auto pair_dch = [&](int jp) { return (jp * kPfThreads + tid) % Lay::CPR; };
  const bool loader = !Lay::kPartial || tid < Lay::kPairs;
  auto load_ids = [&](int t0) {
    if (!loader) return;
#pragma unroll
    for (int jp = 0; jp < Lay::NPAIR; ++jp) ids[jp] = trow.entry(min(t0 + pair_key(jp), last_pair) >> bs_shift);
  };
  auto load_tile = [&](int t0) {
    if (!loader) return;
#pragma unroll
    for (int jp = 0; jp < Lay::NPAIR; ++jp) {
      const int te = min(t0 + pair_key(jp), last_pair);
      PA_FLAG_IF((unsigned)ids[jp] >= (unsigned)a.num_blocks, kViolationTableId);
      const int blk = ((unsigned)ids[jp] < (unsigned)a.num_blocks) ? ids[jp] : 0;
      const size_t off =
          ((((size_t)blk * a.num_kv_heads + g) * block_size + (te & bmask)) * D + pair_dch(jp) * 8) * 2;
      kreg[2 * jp] = ld16(kpool + off);
      kreg[2 * jp + 1] = ld16(kpool + off + D * 2);
      vreg[2 * jp] = ld16(vpool + off);
      vreg[2 * jp + 1] = ld16(vpool + off + D * 2);
    }
  };
  // Keys at or past L (only in the tile that holds the context's end) get
  // V = 0: their slots may hold anything, and a zero weight times a NaN is NaN.
  // The tile that holds the context's end (TAIL) is stored by its own copy of
  // the code, so that the other tiles carry no selects for it.
  auto store_tile_as = [&](auto tail_tag, int buf, int t0) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    if (!loader) return;
    char* kb = lds + buf * Lay::kBufBytes;
    char* vb = kb + Lay::kKBytes;
#pragma unroll
    for (int jp = 0; jp < Lay::NPAIR; ++jp) {
      const int key = pair_key(jp), dch = pair_dch(jp);
      *reinterpret_cast<u32x4*>(kb + key * Lay::kRowB + dch * 16) = kreg[2 * jp];
      *reinterpret_cast<u32x4*>(kb + (key + 1) * Lay::kRowB + dch * 16) = kreg[2 * jp + 1];
      u32x4 v0 = vreg[2 * jp], v1 = vreg[2 * jp + 1];
      if constexpr (TAIL) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        v0 = t0 + key < L ? v0 : z;
        v1 = t0 + key + 1 < L ? v1 : z;
      }
      if constexpr (PA_PREFILL_VTR != 0) {
        *reinterpret_cast<u32x4*>(vb + key * Lay::kVrB + dch * 16) = v0;
        *reinterpret_cast<u32x4*>(vb + (key + 1) * Lay::kVrB + dch * 16) = v1;
        continue;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // element e of both keys: low halves (even e) or high halves (odd e)
        const uint32_t w = (e & 1) ? __builtin_amdgcn_perm(v1[e >> 1], v0[e >> 1], 0x07060302u)
                                   : __builtin_amdgcn_perm(v1[e >> 1], v0[e >> 1], 0x05040100u);
        const int row = dch * 8 + e;
        *reinterpret_cast<uint32_t*>(vb + row * Lay::kVtB + ((pair_pos(jp) ^ vt_swizzle(row)) << 2)) = w;
      }
    }
  };
  auto store_tile = [&](int buf, int t0) {
    if (t0 + kPfKeys > L)   // uniform
      store_tile_as(std::true_type{}, buf, t0);
    else
      store_tile_as(std::false_type{}, buf, t0);
  };

  // Row sums come from the matrix cores: a 16 x 32 operand of ones times the
  // rounded P^T gives every row of the product the sum of P over the keys,
  // so lane l holds its query row's sum in each of its 4 accumulators, and
  // the sum is of the same rounded weights that multiply V.
  float m_run[NG];
  f32x4 oacc[NG][NDT], lacc[NG];
#pragma unroll
  for (int grp = 0; grp < NG; ++grp) {
    m_run[grp] = kNegInf;
    lacc[grp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[grp][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t one2 = pack2<T>(1.f, 1.f);
  const u32x4 ones = {one2, one2, one2, one2};
  // the wave's smallest position: a tile whose keys all lie at or below it
  // is seen whole by every row of the wave and needs no causal mask
  const int wave_first = L - n + min(qb * QB + wave * TPW, n - 1);

  const int ntiles = (kend + kPfKeys - 1) / kPfKeys;
  load_ids(0);
  load_tile(0);
  store_tile(0, 0);
  if (ntiles > 1) load_ids(kPfKeys);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int t0 = it * kPfKeys;
    if (it + 1 < ntiles) load_tile(t0 + kPfKeys);
    if (it + 2 < ntiles) load_ids(t0 + 2 * kPfKeys);
    if (t0 <= wave_last) {   // wave-uniform: some row of this wave sees a key of the tile
      const char* kb = lds + (it & 1) * Lay::kBufBytes;
      const char* vb = kb + Lay::kKBytes;
      f32x4 st[NG][kPfSub];
#pragma unroll
      for (int grp = 0; grp < NG; ++grp)
#pragma unroll
        for (int sub = 0; sub < kPfSub; ++sub) st[grp][sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
#pragma unroll
        for (int sub = 0; sub < kPfSub; ++sub) {
          const u32x4 ak =
              *reinterpret_cast<const u32x4*>(kb + (16 * sub + c) * Lay::kRowB + (32 * kc + 8 * gq) * 2);
#pragma unroll
          for (int grp = 0; grp < NG; ++grp) st[grp][sub] = mfma_16x16x32<T>(ak, qop[grp][kc], st[grp][sub]);
        }
      }
#if PA_PREFILL_SCHED > 0
      // K operands PA_PREFILL_SCHED reads ahead of their products
      __builtin_amdgcn_sched_group_barrier(0x100, PA_PREFILL_SCHED, 0);
#pragma unroll
      for (int r = 0; r < NKC * kPfSub; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, NG, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#endif
      // lane holds keys 16 sub + 4 gq + i; k-slot 8 gq + j of PV product h
      // (keys [32 h, 32 h + 32)) means key 32 h + 4 gq + j (j < 4) or
      // 32 h + 16 + 4 gq + j - 4.  Scores stay raw (scale > 0 after the sign
      // went into Q); the scale enters the max once and each exponent as one
      // fused multiply-add.
      const bool diag = t0 + kPfKeys - 1 > wave_first;   // wave-uniform
      u32x4 pb[NG][kPfSub / 2];
      const int kt = t0 + 4 * gq;
#pragma unroll
      for (int grp = 0; grp < NG; ++grp) {
        float sc[4 * kPfSub];
#pragma unroll
        for (int sub = 0; sub < kPfSub; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[4 * sub + i] = st[grp][sub][i];
        if (diag) {   // key kt + 16 sub + i is seen when 16 sub + i <= pos - kt
          const int dpos = pos[grp] - kt;
#pragma unroll
          for (int sub = 0; sub < kPfSub; ++sub)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sc[4 * sub + i] = (16 * sub + i <= dpos) ? sc[4 * sub + i] : kNegInf;
        }
        float tmax = sc[0];
#pragma unroll
        for (int i = 1; i < 4 * kPfSub; ++i) tmax = fmaxf(tmax, sc[i]);
        tmax *= sp;   // -inf stays -inf
        // The 4 lanes of a row share m_run, and it moves only when a score of
        // the row exceeds it by more than 2^kPfLazy, so each lane tests its own
        // scores and the row-wide max is formed only when some lane asks.
        // Every row sees key 0 in the first tile (so m_run is finite after it,
        // and a masked score's exponent is -inf, giving 0).
        if (__any(tmax > m_run[grp] + kPfLazy)) {
          const float rmax = row_max4(tmax);
          const bool grow = rmax > m_run[grp] + kPfLazy;   // the same in the row's 4 lanes
          const float m_new = grow ? rmax : m_run[grp];
          const float alpha = grow ? fast_exp2(m_run[grp] - m_new) : 1.f;
          m_run[grp] = m_new;
          lacc[grp] *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) oacc[grp][dt] *= alpha;
        }
        const float nm = -m_run[grp];
        float p[4 * kPfSub];
#pragma unroll
        for (int i = 0; i < 4 * kPfSub; ++i) p[i] = fast_exp2(fmaf(sc[i], sp, nm));
#pragma unroll
        for (int h = 0; h < kPfSub / 2; ++h) {
          pb[grp][h][0] = pack2<T>(p[8 * h + 0], p[8 * h + 1]);
          pb[grp][h][1] = pack2<T>(p[8 * h + 2], p[8 * h + 3]);
          pb[grp][h][2] = pack2<T>(p[8 * h + 4], p[8 * h + 5]);
          pb[grp][h][3] = pack2<T>(p[8 * h + 6], p[8 * h + 7]);
        }
      }
      // V^T operands one step ahead of their products, so LDS latency
      // overlaps the matrix cores instead of preceding each product
      constexpr int NVS = NDT * (kPfSub / 2);
      // row 16 dt + c of V^T (c < 16) has swizzle sw = vt_swizzle(16 dt), and
      // lane (c, gq) of half h reads dwords (16 h + 4 gq) ^ sw .. + 3 =
      // 16 (h ^ sw / 16) + 4 (gq ^ (sw / 4) % 4) .. + 3: the row base, a
      // constant and one of four lane offsets
      const char* vlane = vb + c * Lay::kVtB;
      // Transposing read (row-major V): within each 16-lane group, lane j
      // receives value j % 4 of the 8-byte chunks addressed by lanes j / 4,
      // 4 + j / 4, 8 + j / 4 and 12 + j / 4.  Lane (c, gq) addresses chunk
      // c % 4 (d = 16 dt + 4 (c % 4) ..) of key row 32 h + 4 gq + c / 4, so
      // lane c receives d = 16 dt + c of keys 32 h + 4 gq .. + 3 (k-slots
      // 8 gq .. 8 gq + 3); the same 16 rows further gives keys 32 h + 16 + 4 gq
      // .. + 3 (k-slots 8 gq + 4 ..).
      typedef short v4i16 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
      const char* vtr = vb + (4 * gq + (c >> 2)) * Lay::kVrB + 8 * (c & 3);
      auto read_v = [&](int step) {
        const int h = step / NDT, dt = step % NDT;
        if constexpr (PA_PREFILL_VTR != 0) {
          const char* src = vtr + 32 * h * Lay::kVrB + 32 * dt;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)src);
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(src + 16 * Lay::kVrB));
          const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
          return u32x4{l2.x, l2.y, h2.x, h2.y};
        }
        const int sw = vt_swizzle(16 * dt);
        const char* src = vlane + 16 * dt * Lay::kVtB + 64 * (h ^ (sw >> 4)) + 16 * (gq ^ ((sw >> 2) & 3));
        return *reinterpret_cast<const u32x4*>(src);
      };
      u32x4 av = read_v(0);
#pragma unroll
      for (int grp = 0; grp < NG; ++grp)
#pragma unroll
        for (int h = 0; h < kPfSub / 2; ++h) lacc[grp] = mfma_16x16x32<T>(ones, pb[grp][h], lacc[grp]);
      // step = h NDT + dt: consecutive products accumulate into different d
      // tiles, so a product's dependence on the same tile's previous one is
      // NDT products back (the matrix-core latency stays covered)
#pragma unroll
      for (int step = 0; step < NVS; ++step) {
        const u32x4 nxt = read_v(step + 1 < NVS ? step + 1 : step);
        const int h = step / NDT, dt = step % NDT;
#pragma unroll
        for (int grp = 0; grp < NG; ++grp) oacc[grp][dt] = mfma_16x16x32<T>(av, pb[grp][h], oacc[grp][dt]);
        av = nxt;
      }
#if PA_PREFILL_SCHED > 0
      // keep each V^T read PA_PREFILL_SCHED products ahead of its use (two
      // transposing reads per operand with row-major V)
      constexpr int kVReads = PA_PREFILL_VTR ? 2 : 1;
      __builtin_amdgcn_sched_group_barrier(0x100, kVReads * PA_PREFILL_SCHED, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NG * (kPfSub / 2), 0);
#pragma unroll
      for (int step = 0; step < NVS; ++step) {
        __builtin_amdgcn_sched_group_barrier(0x008, NG, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, kVReads, 0);
      }
#endif
    }
    if (it + 1 < ntiles) store_tile((it + 1) & 1, t0 + kPfKeys);   // the other buffer: free since the last barrier
    __syncthreads();
  }

#pragma unroll
  for (int grp = 0; grp < NG; ++grp) {
    if (!row_ok[grp]) continue;
    const float inv = 1.f / lacc[grp][0];
    char* orow = reinterpret_cast<char*>(a.out) +
                 (((size_t)(q0 + tq[grp]) * a.num_q_heads + (size_t)g * G + hh) * D) * 2;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint2 w;
      w.x = pack2<T>(oacc[grp][dt][0] * inv, oacc[grp][dt][1] * inv);
      w.y = pack2<T>(oacc[grp][dt][2] * inv, oacc[grp][dt][3] * inv);
      *reinterpret_cast<uint2*>(orow + (16 * dt + 4 * gq) * 2) = w;
    }
  }
}

template <class T, int D, int NW>
static hipError_t prefill_waves(const PrefillArgs& a, int bs, int group, hipStream_t st) {
  int shift = 0;
  while ((1 << shift) < bs) ++shift;
  const int QB = NW * 16 * kPfGroups / group;
  PrefillArgs args = a;
  args.qblocks = (a.max_query_len + QB - 1) / QB;
  const uint64_t units = (uint64_t)a.num_seqs * a.num_kv_heads * args.qblocks;
  if (units == 0) return hipSuccess;
  if (units > 0x7fffffffull) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)units), block(NW * kWave);
  switch (group) {
    case 1: hipLaunchKernelGGL((prefill_kernel<T, D, 1, NW>), grid, block, 0, st, args, bs, shift); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<T, D, 2, NW>), grid, block, 0, st, args, bs, shift); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<T, D, 4, NW>), grid, block, 0, st, args, bs, shift); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<T, D, 8, NW>), grid, block, 0, st, args, bs, shift); break;
    case 16: hipLaunchKernelGGL((prefill_kernel<T, D, 16, NW>), grid, block, 0, st, args, bs, shift); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class T, int D>
static hipError_t prefill_group(const PrefillArgs& a, int bs, int group, hipStream_t st) {
  return prefill_waves<T, D, kPfWaves>(a, bs, group, st);
}

PA_VIOLATIONS_GETTER(debug_violations_prefill)

hipError_t launch_prefill(const PrefillArgs& a, Elem elem, int head_dim, int block_size, int group,
                          hipStream_t stream) {
  if (elem == Elem::BF16) {
    return head_dim == 128 ? prefill_group<BF16, 128>(a, block_size, group, stream)
                           : prefill_group<BF16, 64>(a, block_size, group, stream);
  }
  if (elem == Elem::F16) {
    return head_dim == 128 ? prefill_group<F16, 128>(a, block_size, group, stream)
                           : prefill_group<F16, 64>(a, block_size, group, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
