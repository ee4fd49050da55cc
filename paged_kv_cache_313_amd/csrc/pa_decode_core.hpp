// Decode attention over a paged KV cache (gfx950, wave64): the kernels.
// Included by one instantiation unit per storage type (pa_decode_{f32,f16,bf16}.hip).
//
// One query token per sequence attends over the sequence's context, whose K/V
// rows sit in fixed-size physical blocks reached through the sequence's block
// table (vLLM/PagedAttention paged-KV analysis page, section 3.1: the kernel is
// changed to read non-contiguous blocks; the simplified sketch walks the table
// block by block and loads K and V of each physical page).  The sketch
// normalises per block; the operation reached here is one softmax over the
// whole context, evaluated as an online softmax: running maxima, running sums
// and un-normalised accumulators are rescaled by exp(m_old - m_new) when a max
// grows.  Scores are kept in the log2 domain (scale * log2(e) folded in) so
// every exponential is one v_exp_f32.
//
// A *segment* is a token range [tok0, tok1) of one sequence for one group of
// query heads sharing a KV head, and one wave runs it from start to end: it
// stages the segment's block-table slice in its own LDS window (taking the
// table->block dependent load off the tile path), streams the 16-token tiles
// with the next tile's loads in flight, reduces across its lanes and writes
// the result itself.  Waves never wait for one another, so a wave starting a
// segment does not stall its neighbours.  Three ways to cut the work:
//  * unit mode, no split: one segment per (sequence, head group);
//  * unit mode, fixed partitions of P tokens: one segment per (sequence, head
//    group, partition), partials merged by decode_merge_parts_kernel;
//  * balanced mode: the grid holds exactly the waves the GPU keeps resident,
//    and each takes an equal share of the flattened (sequence, head group,
//    tile) space, so ragged batches finish together; a (sequence, head group)
//    shared by several waves is merged by decode_merge_balanced_kernel.
#pragma once

#include <type_traits>

#include "pa_common.hpp"
#include "pa_launch.hpp"

namespace pa {

constexpr int kTile = 16;      // tokens per tile
constexpr int kTblWin = 256;   // block-table entries a wave stages in LDS at a time
// A lane rescales its accumulators only when a score exceeds its running max
// by more than this (log2 units), so every p <= 2^8 and sums stay far from
// fp32 overflow; the result is the same up to rounding.
constexpr float kLazy = 8.f;
// Tiles in flight per wave (tile_loop's ring): the current one and the next.
// Rings of 3 and 4 (8 KiB tiles, fewer resident waves for their registers)
// streamed no faster on the GQA batches.
#ifndef PA_TILE_RING
#define PA_TILE_RING 2
#endif
constexpr int kRing = PA_TILE_RING;

// Cache policy of the K/V loads.  A tile read once per call is loaded with
// the non-temporal hint.  Blocks that the neighbouring sequences s-1 or s+1
// map at the same logical position (the prompt blocks that the samples or
// beams of one request share; a scheduler keeps those sequences together, so
// their waves run at about the same time) are loaded with the default policy,
// so that the neighbours hit in L2 or the MALL.  Shared blocks form a prefix
// of each table, and the tile loop is run twice -- over the window's leading
// shared blocks, then over the rest -- so that no branch sits between a
// tile's loads and their use.  This holds for the balanced grid (one
// workgroup per CU, long ranges per wave).  Unit-mode grids (many resident
// waves, one short segment each) load every tile with the default policy:
// there the hint made a 64-sequence MHA batch 32 % slower.  The policy does
// not change any result.

// Stage table entries [first, first+count) of sequence s (1 <= count <=
// kTblWin) into this wave's LDS window (ids clamped into the pool:
// memory-safe on bad tables) and return how many leading entries are shared
// with a neighbour, whose entries count only below its own block count.  All
// loads are issued before any is used: every index is clamped into its row
// (a row has at least one entry), so none needs a guard.  LDS
// operations of one wave complete in order; the wait makes the entries
// visible to every lane before the wave reads them.
template <int BS, bool SPLIT>
__device__ __forceinline__ int stage_table_wave(int32_t* tbl, const DecodeArgs& a, const TableView& row, int s,
                                                int first, int count, int lane) {
  if constexpr (!SPLIT) {   // unit mode: every tile under the default policy
    for (int i = lane; i < count; i += kWave) {
      const int e = row.entry(first + i);
      PA_FLAG_IF((unsigned)e >= (unsigned)a.num_blocks, kViolationTableId);
      tbl[i] = ((unsigned)e < (unsigned)a.num_blocks) ? e : 0;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    return count;
  }
  constexpr int NI = kTblWin / kWave;
  const bool has_prev = s > 0, has_next = s + 1 < a.num_seqs;
  const int sp = has_prev ? s - 1 : s, sn = has_next ? s + 1 : s;
  const int lp = a.context_lens[sp], ln = a.context_lens[sn];   // issued with the entries below
  const TableView rprev = table_view(a, sp);
  const TableView rnext = table_view(a, sn);
  int e[NI], ep[NI], en[NI];
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int j = first + min(lane + k * kWave, count - 1);
    e[k] = row.entry_sel(j);
    ep[k] = rprev.entry_sel(min(j, rprev.capacity - 1));
    en[k] = rnext.entry_sel(min(j, rnext.capacity - 1));
  }
  // the neighbours' lengths clamped as clamp_len does, in blocks
  auto nblk = [&](int L, const TableView& v) {
    L = min(max(L, 0), min(v.capacity * BS, a.max_context_len));
    return (L + BS - 1) / BS;
  };
  const int nprev = has_prev ? nblk(lp, rprev) : 0;
  const int nnext = has_next ? nblk(ln, rnext) : 0;
  int lead = count;   // first entry not shared (wave-uniform: from ballots)
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int i = lane + k * kWave;
    bool unshared = false;
    if (i < count) {
      const int j = first + i;
      unshared = !((j < nprev && ep[k] == e[k]) || (j < nnext && en[k] == e[k]));
      PA_FLAG_IF((unsigned)e[k] >= (unsigned)a.num_blocks, kViolationTableId);
      tbl[i] = ((unsigned)e[k] < (unsigned)a.num_blocks) ? e[k] : 0;
    }
    const uint64_t m = __ballot(unshared);
    if (lead == count && m != 0) lead = k * kWave + (int)__builtin_ctzll(m);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  return lead;
}

// The table window a wave last staged: consecutive segments of a wave are
// mostly the same sequence under another KV head and need the same entries,
// so a window that still covers the next one is reused (one dependent global
// round trip less per segment start).
struct TblCache {
  int s = -1, first = 0, count = 0, shared = 0;
};

// Entries [fblk, fblk + nent) of sequence s, staged unless the cached window
// holds them; returns the LDS address of entry fblk and sets `nshared` to the
// number of leading entries from fblk that are shared with a neighbour.
template <int BS, bool SPLIT>
__device__ __forceinline__ int32_t* staged_window(const DecodeArgs& a, int32_t* tbl, TblCache& tc,
                                                  const TableView& row, int s, int fblk, int nent, int lane,
                                                  int& nshared) {
  if (!(tc.s == s && tc.first <= fblk && fblk + nent <= tc.first + tc.count)) {
    tc.shared = stage_table_wave<BS, SPLIT>(tbl, a, row, s, fblk, nent, lane);
    tc.s = s;
    tc.first = fblk;
    tc.count = nent;
  }
  nshared = min(max(tc.shared - (fblk - tc.first), 0), nent);
  return tbl + (fblk - tc.first);
}

// Tiles of a window of nent blocks (starting off0 tokens into its first
// block) that lie wholly in its first nshared blocks: all of them when every
// block is shared.
template <int BS>
__device__ __forceinline__ int shared_tiles(int nshared, int nent, int off0, int ntiles) {
  if (nshared >= nent) return ntiles;
  const int t = (nshared * BS - off0) / kTile;
  return t < 0 ? 0 : (t > ntiles ? ntiles : t);
}

using PolicyDefault = std::integral_constant<int, kAuxDefault>;
using PolicyStream = std::integral_constant<int, kStreamAux>;

// Walk tiles 0 .. ntiles-1 keeping the next NB-1 tiles' K/V loads in flight
// while the current one is computed.  The loop runs over NB tiles at a time
// with a ring of NB buffers and has a single exit, so that no path (not even
// a structurized, never-taken one) returns to the loop head with the
// prefetches outstanding; that lets the compiler's vmcnt waits leave the newer
// loads in flight.  Loads are unconditional: a prefetch past the last tile
// re-reads it (an L2 hit) instead of branching.  After the loop fewer than NB
// tiles remain, and they are exactly the ones already in buf[0 ..].
template <class Buf, int NB = 2, class Load, class Compute>
__device__ __forceinline__ void tile_loop(int ntiles, Load&& load, Compute&& compute) {
  static_assert(NB >= 2, "ring");
  if (ntiles <= 0) return;
  const int last = ntiles - 1;
  Buf buf[NB];
#pragma unroll
  for (int j = 0; j + 1 < NB; ++j) load(min(j, last), buf[j]);
  int ti = 0;
  for (; ti + NB <= ntiles; ti += NB) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      load(min(ti + j + NB - 1, last), buf[(j + NB - 1) % NB]);
      compute(ti + j, buf[j]);
    }
  }
#pragma unroll
  for (int j = 0; j + 1 < NB; ++j)
    if (ti + j < ntiles) compute(ti + j, buf[j]);
}

// Tiles [0, nsh) of a window with the default cache policy, then tiles
// [nsh, ntiles) with the non-temporal one: two loops, so that every load of a
// loop has a fixed policy and nothing but the loop's own exit separates a
// prefetch from its use.  SPLIT is false for unit-mode kernels: one loop, all
// tiles under the default policy.
template <class Buf, bool SPLIT, class Load, class Compute>
__device__ __forceinline__ void run_window(int ntiles, int nsh, Load& load, Compute& compute) {
  if constexpr (!SPLIT) {   // unit mode: one loop, default policy
    tile_loop<Buf, kRing>(ntiles, [&](int ti, Buf& b) { load(PolicyDefault{}, ti, b); }, compute);
    return;
  }
  if (nsh > 0)
    tile_loop<Buf, kRing>(nsh, [&](int ti, Buf& b) { load(PolicyDefault{}, ti, b); },
                          [&](int ti, const Buf& b) { compute(ti, b); });
  tile_loop<Buf, kRing>(ntiles - nsh, [&](int ti, Buf& b) { load(PolicyStream{}, nsh + ti, b); },
                        [&](int ti, const Buf& b) { compute(nsh + ti, b); });
}

// Byte offsets, from the start of a KV head's slice of the pool, of the
// 16-token tile that starts `rel` tokens after the first staged block.  The
// block id is wave-uniform, so the offsets live in SGPRs and each lane adds a
// constant 32-bit offset: no per-lane address arithmetic on the tile path.
// With block_size >= 16 the tile lies in one block (lo == hi); with 8 its
// tokens [8, 16) are in the next block, which may be past the window's last
// staged entry only when every one of those tokens is masked (then lo is
// reused).
template <int BS, int ROWB>
__device__ __forceinline__ void tile_offsets(const int32_t* tbl, int rel, int nent, size_t blk_stride,
                                             size_t& lo, size_t& hi) {
  if constexpr (BS >= 16) {
    const int b = __builtin_amdgcn_readfirstlane(tbl[rel / BS]);
    lo = hi = (size_t)b * blk_stride + (size_t)(rel % BS) * ROWB;
  } else {
    const int e = rel / BS;
    const int b0 = __builtin_amdgcn_readfirstlane(tbl[e]);
    const int b1 = e + 1 < nent ? __builtin_amdgcn_readfirstlane(tbl[e + 1]) : b0;
    lo = (size_t)b0 * blk_stride;
    hi = (size_t)b1 * blk_stride;
  }
}

// Where a segment's result goes: the output rows (direct) or partial rows
// prow0 + hh * pstride of the workspace (m, l, un-normalised acc).  With
// part > 0 the segment [tok0, tok1) is a run of consecutive `part`-token
// partitions (tok0 a multiple of part), each with its own result: partition
// k of the run goes to partial rows prow0 + k + hh * pstride, and the
// running state restarts at each partition boundary.
struct Dest {
  bool direct;
  size_t prow0, pstride;
  int part;
};

// The destination of partition k of a run (k = 0 for a single result).
__device__ __forceinline__ Dest dest_part(const Dest& d, int k) {
  Dest r = d;
  r.prow0 += (size_t)k;
  return r;
}

// Write n consecutive results of head row `orow`, starting at element d0.
template <class T, int N>
__device__ __forceinline__ void emit_chunk(const DecodeArgs& a, const Dest& dst, size_t orow, int hh,
                                           int d0, int D, const float* acc, float l) {
  if (dst.direct) {
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < N; ++e) store_elem<T>(a.out, orow * D + d0 + e, acc[e] * inv);
  } else {   // partial rows are 16-byte aligned and d0 is a multiple of 4
    const size_t pr = dst.prow0 + (size_t)hh * dst.pstride;
    static_assert(N % 4 == 0, "whole 16-byte chunks");
#pragma unroll
    for (int e = 0; e < N; e += 4)
      st16(a.ws_o + pr * D + d0 + e, u32x4{__float_as_uint(acc[e]), __float_as_uint(acc[e + 1]),
                                           __float_as_uint(acc[e + 2]), __float_as_uint(acc[e + 3])});
  }
}

__device__ __forceinline__ void emit_ml(const DecodeArgs& a, const Dest& dst, int hh, float m, float l) {
  if (!dst.direct) {
    const size_t pr = dst.prow0 + (size_t)hh * dst.pstride;
    a.ws_m[pr] = m;
    a.ws_l[pr] = l;
  }
}

// Results of the resident-grid kernels, buffered in LDS per wave.  A global
// store in the middle of the K/V stream is costly: vmcnt counts loads and
// stores in issue order, so the wait for the next tile's loads also waits for
// the store's acknowledgement, which queues behind the read stream (measured:
// about 7 us per flushed partition on the long-context batch).  So each
// segment's or partition's (acc, m, l) goes to a slot of the wave's LDS
// buffer, and the slots are written out together when the buffer is full and
// when the wave has finished all its work: partial rows to the workspace,
// whole results (acc / l, rounded once to the output type) to the output.
template <int H, int D>
struct PartBuf {
  static constexpr int kBytes = 32768;                      // per wave
  static constexpr int kSlotBytes = H * (D + 2) * 4 + 8;
  static constexpr int kCap = kBytes / kSlotBytes;          // slots (3 at H 16, D 128)
  static_assert(kCap >= 1, "one slot at least");
  static constexpr size_t kDirect = (size_t)1 << 63;        // row tag: an output row
  float* o;        // [kCap][H][D], 16-byte aligned
  float* ml;       // [kCap][H][2]: m, l
  size_t* row;     // [kCap]: head 0's partial row (head hh: + hh * pstride), or
                   // kDirect | its output row (head hh: + hh)
  size_t pstride;
  int count;
  __device__ __forceinline__ void init(char* lds, size_t stride) {
    o = reinterpret_cast<float*>(lds);
    ml = o + kCap * H * D;
    row = reinterpret_cast<size_t*>(ml + kCap * H * 2);
    pstride = stride;
    count = 0;
  }
  // Write the buffered slots out (16-byte chunks of whole rows per
  // instruction) and empty the buffer.
  template <class T>
  __device__ __forceinline__ void flush(const DecodeArgs& a, int lane) {
    constexpr int CPR = D / 4;
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's slot writes have landed
    __builtin_amdgcn_wave_barrier();
    for (int k = 0; k < count; ++k) {
      const size_t tag = row[k];
      const size_t r0 = tag & ~kDirect;
      if (tag & kDirect) {   // wave-uniform
        for (int idx = lane; idx < H * CPR; idx += kWave) {
          const int hh = idx / CPR, ch = idx % CPR;
          const float inv = 1.f / ml[(k * H + hh) * 2 + 1];
          const f32x4 v = *reinterpret_cast<const f32x4*>(o + (k * H + hh) * D + 4 * ch);
#pragma unroll
          for (int e = 0; e < 4; ++e) store_elem<T>(a.out, (r0 + hh) * D + 4 * ch + e, v[e] * inv);
        }
        continue;
      }
      for (int idx = lane; idx < H * CPR; idx += kWave) {
        const int hh = idx / CPR, ch = idx % CPR;
        st16(a.ws_o + (r0 + (size_t)hh * pstride) * D + 4 * ch,
             *reinterpret_cast<const u32x4*>(o + (k * H + hh) * D + 4 * ch));
      }
      if (lane < H) {
        const size_t r = r0 + (size_t)lane * pstride;
        a.ws_m[r] = ml[(k * H + lane) * 2];
        a.ws_l[r] = ml[(k * H + lane) * 2 + 1];
      }
    }
    count = 0;
    __builtin_amdgcn_s_waitcnt(0xc07f);   // reads done before the slots are reused
    __builtin_amdgcn_wave_barrier();
  }
  // The slot for the next result (flushing first when the buffer is full).
  template <class T>
  __device__ __forceinline__ int take(const DecodeArgs& a, int lane) {
    if (count == kCap) flush<T>(a, lane);
    return count;
  }
  // n consecutive results (n a multiple of 4) of head hh, from element d0
  template <int N>
  __device__ __forceinline__ void chunk(int slot, int hh, int d0, const float* v) {
    static_assert(N % 4 == 0, "whole 16-byte chunks");
#pragma unroll
    for (int e = 0; e < N; e += 4)
      *reinterpret_cast<u32x4*>(o + (slot * H + hh) * D + d0 + e) =
          u32x4{__float_as_uint(v[e]), __float_as_uint(v[e + 1]), __float_as_uint(v[e + 2]),
                __float_as_uint(v[e + 3])};
  }
  __device__ __forceinline__ void set_ml(int slot, int hh, float m, float l) {
    ml[(slot * H + hh) * 2] = m;
    ml[(slot * H + hh) * 2 + 1] = l;
  }
};

template <class T, int D, int H>
__device__ __forceinline__ void store_zero_rows(const DecodeArgs& a, int s, int h0, int lane) {
  for (int idx = lane; idx < H * D; idx += kWave)
    store_elem<T>(a.out, ((size_t)s * a.num_q_heads + h0) * D + idx, 0.f);
}

// ============================================================================
// VALU core: any dtype, H q heads (1, 2 or 4) of one KV head.
// Lane layout per tile: token slot tt = lane / 4, quarter qp = lane % 4; the
// lane holds the row bytes [16 (4 j + qp), +16) for j < NL, i.e. D/4
// elements.  QK^T: v_dot2c_f32_{f16,bf16} (fp32 FMA for fp32) in four
// independent chains, then a quad sum; P.V: v_fma_mix_f32 for fp16, fp32 FMAs
// otherwise.  Each token slot keeps its own running max, sum and accumulator,
// so the tile loop needs no cross-lane reduction beyond the quad's dot sum;
// the slots are merged with the log-sum-exp rule at the end of the segment.
// ============================================================================
template <int NL>
struct ValuBuf {
  u32x4 k[NL], v[NL];
};

// Resident workgroups per CU of the VALU core's balanced grid (0: as many as
// its resources allow, 3 for MHA fp16).  One was 2.6 % faster than three on
// the OPT-13B-shaped MHA batch: fewer, longer ranges pay fewer segment starts.
#ifndef PA_VALU_WG_PER_CU
#define PA_VALU_WG_PER_CU 1
#endif
template <class T, int D, int BS, int H>
struct ValuCore {
  static constexpr int EB = T::bytes;
  static constexpr int ROWB = D * EB;
  static constexpr int NL = ROWB / 64;    // 16-byte loads per lane per token row
  static constexpr int NE = 16 / EB;      // elements per 16 bytes
  static constexpr int DPL = NL * NE;     // elements per lane (= D / 4)
  static constexpr int HEADS = H;
  static constexpr int kBalancedWgPerCu = PA_VALU_WG_PER_CU;
  static_assert(DPL * 4 == D, "layout");
  static_assert(kTblWin * BS % kTile == 0, "window");

  // q heads h0 .. h0+H-1 of sequence s over tokens [tok0, tok1), run by one
  // wave; tbl is the wave's LDS window.
  template <bool SPLIT, bool PARTS = false, bool BUF = PARTS>
  __device__ static void run(const DecodeArgs& a, int32_t* tbl_lds, TblCache& tc, int s, int h0, int tok0,
                             int tok1, const Dest& dst, PartBuf<H, D>* pb = nullptr) {
    const int lane = threadIdx.x & (kWave - 1);
    const int G = a.num_q_heads / a.num_kv_heads;
    const int g = h0 / G;
    const int tt = lane >> 2, qp = lane & 3;

    u32x4 qraw[H][NL];  // the lane's D/4 query elements of each head, as stored
#pragma unroll
    for (int hh = 0; hh < H; ++hh) {
      const char* qrow = reinterpret_cast<const char*>(a.query) +
                         ((size_t)s * a.num_q_heads + h0 + hh) * ROWB + qp * 16;
#pragma unroll
      for (int j = 0; j < NL; ++j) qraw[hh][j] = ld16(qrow + j * 64);
    }
    float m_run[H], l_run[H], acc[H][DPL];
    auto reset = [&]() {
#pragma unroll
      for (int hh = 0; hh < H; ++hh) {
        m_run[hh] = kNegInf;
        l_run[hh] = 0.f;
#pragma unroll
        for (int i = 0; i < DPL; ++i) acc[hh][i] = 0.f;
      }
    };
    reset();
    // with PARTS: the end of the current partition and its index in the run
    int pend = tok0 + dst.part, pk = 0;

    // merge the 16 token slots (lanes with equal qp): rescale to the common
    // max, then sum; slots that saw no token have m = -inf and weigh 0.
    // Within a 16-lane row the slots of one qp sit 4 lanes apart: two row
    // rotates (by 4, then 8) sum them into each lane, and at row positions
    // 0..3 in the order of a butterfly over lane ^ 4, lane ^ 8; the lane
    // swaps then add the other rows.  Lanes 0..3 hold the results.
    auto finish = [&](const Dest& d) {
      constexpr bool buffered = BUF;   // results go to the wave's LDS buffer
      int slot = 0;
      if constexpr (BUF) slot = pb->template take<T>(a, lane);
#pragma unroll
      for (int hh = 0; hh < H; ++hh) {
        float M = m_run[hh];
        M = fmaxf(M, row_ror<4>(M));
        M = fmaxf(M, row_ror<8>(M));
        M = swap_pair_max<16>(M);
        M = swap_pair_max<32>(M);
        const float f = m_run[hh] == kNegInf ? 0.f : fast_exp2(m_run[hh] - M);
        float l = l_run[hh] * f;
        l += row_ror<4>(l);
        l += row_ror<8>(l);
        l = swap_pair_sum<16>(l);
        l = swap_pair_sum<32>(l);
        float r[DPL];
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
          float x = acc[hh][i] * f;
          x += row_ror<4>(x);
          x += row_ror<8>(x);
          x = swap_pair_sum<16>(x);
          r[i] = swap_pair_sum<32>(x);
        }
        const size_t orow = (size_t)s * a.num_q_heads + h0 + hh;
        if (tt == 0) {  // lanes 0..3 hold the whole row
#pragma unroll
          for (int j = 0; j < NL; ++j) {
            if (buffered)
              pb->template chunk<NE>(slot, hh, (4 * j + qp) * NE, &r[j * NE]);
            else
              emit_chunk<T, NE>(a, d, orow, hh, (4 * j + qp) * NE, D, &r[j * NE], l);
          }
        }
        if (lane == 0) {
          if (buffered)
            pb->set_ml(slot, hh, M, l);
          else
            emit_ml(a, d, hh, M, l);
        }
      }
      if constexpr (BUF) {
        if (lane == 0)
          pb->row[slot] = d.direct ? (PartBuf<HEADS, D>::kDirect | ((size_t)s * a.num_q_heads + h0)) : d.prow0;
        ++pb->count;
      }
    };

    const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (size_t)g * BS * ROWB;
    const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (size_t)g * BS * ROWB;
    const size_t blk_stride = (size_t)a.num_kv_heads * BS * ROWB;
    const TableView trow = table_view(a, s);
    // lane's row within the tile's block region, and which block (block_size 8)
    const uint32_t lane_off = (uint32_t)((BS >= 16 ? tt : (tt & 7)) * ROWB + qp * 16);
    const bool hi_blk = BS < 16 && tt >= 8;

    // windows of at most kTblWin blocks; a segment may start inside a block
    // (balanced mode, block_size 32): off0 is that start within its block
    for (int wb = tok0; wb < tok1;) {
      const int fblk = wb / BS;
      const int off0 = wb - fblk * BS;
      const int we = min((fblk + kTblWin) * BS, tok1);
      const int nent = (we - 1) / BS - fblk + 1;
      int nshared;
      const int32_t* tbl = staged_window<BS, SPLIT>(a, tbl_lds, tc, trow, s, fblk, nent, lane, nshared);

      auto load = [&](auto pol, int ti, ValuBuf<NL>& buf) {
        constexpr int AUX = decltype(pol)::value;
        size_t lo, hi;
        tile_offsets<BS, ROWB>(tbl, off0 + ti * kTile, nent, blk_stride, lo, hi);
        if constexpr (BS >= 16) {  // one block region: SGPR base + lane offset
          // the resource ends at the window's last token: rows past it read
          // as zeros without a memory access (they are masked below)
          const uint32_t tb = (uint32_t)min(kTile, we - (wb + ti * kTile)) * ROWB;
          const rsrc_t rk = make_rsrc(kbase + lo, tb);
          const rsrc_t rv = make_rsrc(vbase + lo, tb);
#pragma unroll
          for (int j = 0; j < NL; ++j) buf.k[j] = buf_ld16_aux<AUX>(rk, lane_off + j * 64);
#pragma unroll
          for (int j = 0; j < NL; ++j) buf.v[j] = buf_ld16_aux<AUX>(rv, lane_off + j * 64);
        } else {  // block_size 8: tokens 8..15 come from the next block
          const size_t off = (hi_blk ? hi : lo) + lane_off;
#pragma unroll
          for (int j = 0; j < NL; ++j) buf.k[j] = ld16_aux<AUX>(kbase + off + j * 64);
#pragma unroll
          for (int j = 0; j < NL; ++j) buf.v[j] = ld16_aux<AUX>(vbase + off + j * 64);
        }
      };
      auto compute = [&](int ti, const ValuBuf<NL>& buf) {
        const bool valid = wb + ti * kTile + tt < we;
        float pr[H];
#pragma unroll
        for (int hh = 0; hh < H; ++hh) {
          float d[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < NL; ++j) Dot16<T>::run(qraw[hh][j], buf.k[j], d);
          float dot = (d[0] + d[1]) + (d[2] + d[3]);
          dot += xor_lane<1>(dot);
          dot += xor_lane<2>(dot);
          const float sc = valid ? dot * a.scale_log2 : kNegInf;
          const bool grow = sc > m_run[hh] + kLazy;   // true for a slot's first token
          if (__any(grow)) {
            const float m_new = grow ? sc : m_run[hh];
            const float alpha = grow ? fast_exp2(m_run[hh] - m_new) : 1.f;
            l_run[hh] *= alpha;
#pragma unroll
            for (int i = 0; i < DPL; ++i) acc[hh][i] *= alpha;
            m_run[hh] = m_new;
          }
          pr[hh] = valid ? fast_exp2(sc - m_run[hh]) : 0.f;
          l_run[hh] += pr[hh];
        }
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const u32x4 z = {0u, 0u, 0u, 0u};
          const u32x4 vj = valid ? buf.v[j] : z;   // tail slots may hold NaN
#pragma unroll
          for (int hh = 0; hh < H; ++hh) Axpy16<T>::run(pr[hh], vj, &acc[hh][j * NE]);
        }
        if constexpr (PARTS) {   // a partition ends inside the run: write it, start the next
          if (wb + ti * kTile + kTile == pend && pend < tok1) {
            finish(dest_part(dst, pk));
            reset();
            pend += dst.part;
            ++pk;
          }
        }
      };
      const int ntiles = (we - wb + kTile - 1) / kTile;
      run_window<ValuBuf<NL>, SPLIT>(ntiles, shared_tiles<BS>(nshared, nent, off0, ntiles), load, compute);
      wb = we;
    }

    finish(dest_part(dst, pk));
  }
};

// ============================================================================
// MFMA core for grouped queries (f16/bf16, G = Hq/Hkv in {2, 4, 8, 16}).
//
// Scores of a 16-token tile: S^T[t][n] = sum_d K[t][d] Q[n % G][d] with
// v_mfma_f32_16x16x32_{bf16,f16}: A = the K tile (row m = token, loaded
// straight from HBM, 16 bytes per lane), B = the G query rows replicated
// 16/G times across the 16 columns.  The contraction order over d is free as
// long as A and B agree, so lane (gr = lane/16, w = lane%16) feeds chunk
// 4i + gr of token w to MFMA i: every load instruction reads 64 contiguous
// bytes of 16 token rows.  The result lands as S[token 4 gr + r][head w % G],
// r = 0..3, in every lane -- the same 4 tokens that the lane's V loads cover.
// P.V stays on the VALU in fp32: each lane holds one 16-byte chunk of d for
// its tokens, fetches p of the other heads from its quad (DPP) or row, and
// accumulates G x 8 fp32 values.  Each row gr keeps its own running max per
// head (no cross-row reduction per tile); rows merge at the end.
// ============================================================================
template <class T, int G>
__device__ __forceinline__ float bcast_head(float x, int h, int lane) {
  if constexpr (G <= 4) {
    switch (h) {
      case 0: return quad_bcast<0>(x);
      case 1: return quad_bcast<1>(x);
      case 2: return quad_bcast<2>(x);
      default: return quad_bcast<3>(x);
    }
  } else {
    return __shfl(x, (lane & ~15) + h, kWave);
  }
}

template <int NQK, int NVI>
struct MfmaBuf {
  u32x4 k[NQK], v[NVI];
};

#ifndef PA_MFMA_WG_PER_CU
#define PA_MFMA_WG_PER_CU 1
#endif
template <class T, int D, int BS, int G>
struct MfmaCore {
  static constexpr int ROWB = D * 2;
  static constexpr int NQK = D / 32;   // MFMAs per tile (k = 32 per MFMA)
  static constexpr int CPR = D / 8;    // 16-byte chunks per token row
  static constexpr int NVI = D / 32;   // V chunks per lane per tile (16 * CPR / 64)
  static constexpr int HEADS = G;
  // Balanced grid: one workgroup per CU.  With 8 KiB tiles and one tile
  // prefetched per wave, more resident waves only add concurrent streams: on
  // the Llama-3-8B-shaped batch 1 workgroup per CU streamed 1-2 % faster than
  // 2 or 3, and equal on the long-context batch.
  static constexpr int kBalancedWgPerCu = PA_MFMA_WG_PER_CU;
  static_assert(16 % G == 0 && G >= 2, "group");
  static_assert(kTblWin * BS % kTile == 0, "window");

  // the G q heads h0 .. h0+G-1 (KV head h0 / G) of sequence s over tokens
  // [tok0, tok1), run by one wave; tbl is the wave's LDS window.
  template <bool SPLIT, bool PARTS = false, bool BUF = PARTS>
  __device__ static void run(const DecodeArgs& a, int32_t* tbl_lds, TblCache& tc, int s, int h0, int tok0,
                             int tok1, const Dest& dst, PartBuf<G, D>* pb = nullptr) {
    const int lane = threadIdx.x & (kWave - 1);
    const int gr = lane >> 4, w = lane & 15;
    const int g = h0 / G;

    u32x4 qop[NQK];  // B operand: query row of head w % G, chunk 4 i + gr
    {
      const char* qrow = reinterpret_cast<const char*>(a.query) +
                         ((size_t)s * a.num_q_heads + h0 + (w % G)) * ROWB;
#pragma unroll
      for (int i = 0; i < NQK; ++i) qop[i] = ld16(qrow + (4 * i + gr) * 16);
    }
    float m_run, l_run;   // head w % G, tokens of row gr
    float acc[G][8];      // row gr, d = 8 * (w % CPR) + e
    auto reset = [&]() {
      m_run = kNegInf;
      l_run = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    };
    reset();
    // with PARTS: the end of the current partition and its index in the run
    int pend = tok0 + dst.part, pk = 0;

    // merge the four rows: rescale each to the head's common max, then sum;
    // every row then holds all sums, and row gr writes the heads h with
    // h % 4 == gr
    auto finish = [&](const Dest& d) {
      constexpr bool buffered = BUF;   // results go to the wave's LDS buffer
      int slot = 0;
      if constexpr (BUF) slot = pb->template take<T>(a, lane);
      float M = m_run;
      M = swap_pair_max<16>(M);
      M = swap_pair_max<32>(M);
      const float f = m_run == kNegInf ? 0.f : fast_exp2(m_run - M);
      float l = l_run * f;
      l = swap_pair_sum<16>(l);
      l = swap_pair_sum<32>(l);
      float r[G][8];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float fh = bcast_head<T, G>(f, h, lane);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float x = acc[h][e] * fh;
          if constexpr (CPR == 8) x += row_ror<8>(x);   // lane ^ 8 within the row
          x = swap_pair_sum<16>(x);
          r[h][e] = swap_pair_sum<32>(x);
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float lh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), h));
        const float mh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(M), h));
        const size_t orow = (size_t)s * a.num_q_heads + h0 + h;
        if (gr == (h & 3) && w < CPR) {
          if (buffered)
            pb->template chunk<8>(slot, h, 8 * w, r[h]);
          else
            emit_chunk<T, 8>(a, d, orow, h, 8 * w, D, r[h], lh);
        }
        if (lane == 0) {
          if (buffered)
            pb->set_ml(slot, h, mh, lh);
          else
            emit_ml(a, d, h, mh, lh);
        }
      }
      if constexpr (BUF) {
        if (lane == 0)
          pb->row[slot] = d.direct ? (PartBuf<HEADS, D>::kDirect | ((size_t)s * a.num_q_heads + h0)) : d.prow0;
        ++pb->count;
      }
    };

    const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (size_t)g * BS * ROWB;
    const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (size_t)g * BS * ROWB;
    const size_t blk_stride = (size_t)a.num_kv_heads * BS * ROWB;
    const TableView trow = table_view(a, s);
    // K: token w of the tile, chunk 4 i + gr (i = instruction);
    // V: token 4 gr + w / CPR + 16 j / CPR, chunk w % CPR (j = instruction)
    const int tv0 = 4 * gr + w / CPR;
    const uint32_t k_off = (uint32_t)((BS >= 16 ? w : (w & 7)) * ROWB + gr * 16);
    const uint32_t v_off = (uint32_t)((BS >= 16 ? tv0 : (tv0 & 7)) * ROWB + (w % CPR) * 16);
    const bool k_hi = BS < 16 && w >= 8;
    const bool v_hi = BS < 16 && gr >= 2;

    for (int wb = tok0; wb < tok1;) {
      const int fblk = wb / BS;
      const int off0 = wb - fblk * BS;
      const int we = min((fblk + kTblWin) * BS, tok1);
      const int nent = (we - 1) / BS - fblk + 1;
      int nshared;
      const int32_t* tbl = staged_window<BS, SPLIT>(a, tbl_lds, tc, trow, s, fblk, nent, lane, nshared);

      auto load = [&](auto pol, int ti, MfmaBuf<NQK, NVI>& buf) {
        constexpr int AUX = decltype(pol)::value;
        size_t lo, hi;
        tile_offsets<BS, ROWB>(tbl, off0 + ti * kTile, nent, blk_stride, lo, hi);
        if constexpr (BS >= 16) {  // one block region: SGPR base + lane offset
          // the resource ends at the window's last token: rows past it read
          // as zeros without a memory access (they are masked below)
          const uint32_t tb = (uint32_t)min(kTile, we - (wb + ti * kTile)) * ROWB;
          const rsrc_t rk = make_rsrc(kbase + lo, tb);
          const rsrc_t rv = make_rsrc(vbase + lo, tb);
#pragma unroll
          for (int i = 0; i < NQK; ++i) buf.k[i] = buf_ld16_aux<AUX>(rk, k_off + i * 64);
#pragma unroll
          for (int j = 0; j < NVI; ++j) buf.v[j] = buf_ld16_aux<AUX>(rv, v_off + (16 * j / CPR) * ROWB);
        } else {  // block_size 8: tokens 8..15 come from the next block
          const char* kb = kbase + (k_hi ? hi : lo) + k_off;
          const char* vb = vbase + (v_hi ? hi : lo) + v_off;
#pragma unroll
          for (int i = 0; i < NQK; ++i) buf.k[i] = ld16_aux<AUX>(kb + i * 64);
#pragma unroll
          for (int j = 0; j < NVI; ++j) buf.v[j] = ld16_aux<AUX>(vb + (16 * j / CPR) * ROWB);
        }
      };
      auto compute = [&](int ti, const MfmaBuf<NQK, NVI>& buf) {
        const int ts = wb + ti * kTile;
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NQK; ++i) sacc = mfma_16x16x32<T>(buf.k[i], qop[i], sacc);

        float sc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = (ts + 4 * gr + r < we) ? sacc[r] * a.scale_log2 : kNegInf;
        const float tmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        const bool grow = tmax > m_run + kLazy;   // true for the row's first valid token
        if (__any(grow)) {
          const float m_new = grow ? tmax : m_run;
          const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float ah = bcast_head<T, G>(alpha, h, lane);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= ah;
          }
        }
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pr[r] = sc[r] == kNegInf ? 0.f : fast_exp2(sc[r] - m_run);
          l_run += pr[r];
        }
#pragma unroll
        for (int j = 0; j < NVI; ++j) {
          const int idx = w + 16 * j;
          const int rt = idx / CPR;   // token of the group: uniform for D = 128
          const bool vvalid = ts + 4 * gr + rt < we;
          const u32x4 z = {0u, 0u, 0u, 0u};
          const u32x4 vj = vvalid ? buf.v[j] : z;   // tail slots may hold NaN
          float vf[8];
          Unpack<T>::run(vj, vf);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            float ph;
            if constexpr (CPR == 16) {
              ph = bcast_head<T, G>(pr[j], h, lane);
            } else {  // D = 64: rows hold two tokens of the group, lanes w < 8 and w >= 8
              const float pa_ = bcast_head<T, G>(pr[2 * j], h, lane);
              const float pb_ = bcast_head<T, G>(pr[2 * j + 1], h, lane);
              ph = (w < 8) ? pa_ : pb_;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
          }
        }
        if constexpr (PARTS) {   // a partition ends inside the run: write it, start the next
          if (ts + kTile == pend && pend < tok1) {
            finish(dest_part(dst, pk));
            reset();
            pend += dst.part;
            ++pk;
          }
        }
      };
      const int ntiles = (we - wb + kTile - 1) / kTile;
      run_window<MfmaBuf<NQK, NVI>, SPLIT>(ntiles, shared_tiles<BS>(nshared, nent, off0, ntiles), load, compute);
      wb = we;
    }

    finish(dest_part(dst, pk));
  }
};

// ============================================================================
// MFMA core with P.V on the matrix cores too (f16/bf16, head_dim 128, large
// groups).  Scores as in MfmaCore: lane (gr = lane / 16, w = lane % 16) ends
// a tile holding S[token 4 gr + r][head w % G], r = 0..3, and its V loads
// hold tokens 4 gr + j (j = 0..3) at d = 8 w .. 8 w + 7.  Both are already
// operands of O^T[d][head] += V^T P^T as v_mfma_f32_16x16x16_{bf16,f16}
// products: B = the lane's 4 probabilities (k = token 4 gr + r, column =
// head w % G), and A for product dt (dt = 0..7) = element dt of the lane's
// 4 V chunks (row w, k = the same tokens), once output row i of product dt is
// taken to stand for d = 8 i + dt.  Two byte permutes form each A; no value
// crosses lanes.  The product sums over the 16 tokens of all four rows, so
// the running max is per head over the whole tile (two lane swaps), and lane
// (gr, w) ends holding O[head w % G][d] for d in [32 gr, 32 gr + 32).  The
// probabilities are rounded to the input type for the product (and the row
// sums add the same rounded values), as in the prefill kernel.  Per tile and
// wave: 4 + 8 matrix-core products and about 60 vector instructions, where
// MfmaCore's P.V needs G x 36 (2,300 at G = 16).
// ============================================================================
#ifndef PA_PV_MFMA_MIN_GROUP
#define PA_PV_MFMA_MIN_GROUP 4
#endif
// KM > 1 (grouped decode): the 16 query columns hold the G heads of KM
// consecutive sequences, which read the same K/V tiles (a shared prefix);
// column w is sequence s + (w % (G KM)) / G, head h0 + w % G, so one tile
// load and one set of products serve all of them.  Each column's
// arithmetic is the same as with KM = 1.
template <class T, int D, int BS, int G, int KM = 1>
struct MfmaPvCore {
  static_assert(D == 128, "lane layout of the V chunks");
  static constexpr int ROWB = D * 2;
  static constexpr int NQK = D / 32;   // score products per tile (k = 32)
  static constexpr int NVI = 4;        // V chunks per lane per tile: tokens 4 gr .. 4 gr + 3
  static constexpr int NDT = 8;        // P.V products per tile (elements of a chunk)
  static constexpr int HEADS = G;
  static constexpr int MEMBERS = KM;
  static constexpr int kBalancedWgPerCu = PA_MFMA_WG_PER_CU;
  static_assert(16 % (G * KM) == 0 && G >= 2, "group");
  static_assert(kTblWin * BS % kTile == 0, "window");

  // km (KM > 1): sequences s .. s + km - 1 take part (km <= KM); the other
  // columns repeat sequence s and write nothing.
  template <bool SPLIT, bool PARTS = false, bool BUF = PARTS>
  __device__ static void run(const DecodeArgs& a, int32_t* tbl_lds, TblCache& tc, int s, int h0, int tok0,
                             int tok1, const Dest& dst, PartBuf<G, D>* pb = nullptr, int km = 1) {
    static_assert(KM == 1 || !BUF, "grouped units write their partial rows directly");
    const int lane = threadIdx.x & (kWave - 1);
    const int gr = lane >> 4, w = lane & 15;
    const int g = h0 / G;
    const int mi = (w % (G * KM)) / G;   // column w's sequence s + mi
    const bool col_on = KM == 1 || (w < G * KM && mi < km);

    u32x4 qop[NQK];  // B operand of the scores: query row of head w % G, chunk 4 i + gr
    {
      const int qs = KM == 1 ? s : s + (mi < km ? mi : 0);
      const char* qrow = reinterpret_cast<const char*>(a.query) +
                         ((size_t)qs * a.num_q_heads + h0 + (w % G)) * ROWB;
#pragma unroll
      for (int i = 0; i < NQK; ++i) qop[i] = ld16(qrow + (4 * i + gr) * 16);
    }
    float m_run, l_run;   // head w % G: max over the tiles so far, sum over row gr's tokens
    f32x4 oacc[NDT];      // O[head w % G][8 (4 gr + r) + dt] in oacc[dt][r]
    auto reset = [&]() {
      m_run = kNegInf;
      l_run = 0.f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    reset();
    int pend = tok0 + dst.part, pk = 0;   // with PARTS: end of the current partition, its index

    // the four rows' sums add up to the head's; lanes w < G write head w,
    // d = 32 gr .. 32 gr + 31 (row gr = 0 writes m and l)
    auto finish = [&](const Dest& d) {
      int slot = 0;
      if constexpr (BUF) slot = pb->template take<T>(a, lane);
      float l = swap_pair_sum<16>(l_run);
      l = swap_pair_sum<32>(l);
      float v[32];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) v[8 * r + dt] = oacc[dt][r];
      if (KM == 1 && w < G) {
        const size_t orow = (size_t)s * a.num_q_heads + h0 + w;
        if constexpr (BUF) {
          pb->template chunk<32>(slot, w, 32 * gr, v);
          if (gr == 0) pb->set_ml(slot, w, m_run, l);
        } else {
          emit_chunk<T, 32>(a, d, orow, w, 32 * gr, D, v, l);
          if (gr == 0) emit_ml(a, d, w, m_run, l);
        }
      } else if (KM > 1 && col_on) {   // row (s + mi, h0 + w % G), partial row prow0 + hh pstride
        const int hh = mi * a.num_q_heads + w % G;
        const size_t orow = ((size_t)s + mi) * a.num_q_heads + h0 + w % G;
        emit_chunk<T, 32>(a, d, orow, hh, 32 * gr, D, v, l);
        if (gr == 0) emit_ml(a, d, hh, m_run, l);
      }
      if constexpr (BUF) {
        if (lane == 0)
          pb->row[slot] = d.direct ? (PartBuf<HEADS, D>::kDirect | ((size_t)s * a.num_q_heads + h0)) : d.prow0;
        ++pb->count;
      }
    };

    const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (size_t)g * BS * ROWB;
    const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (size_t)g * BS * ROWB;
    const size_t blk_stride = (size_t)a.num_kv_heads * BS * ROWB;
    const TableView trow = table_view(a, s);
    // K: token w of the tile, chunk 4 i + gr; V: token 4 gr + j, chunk w
    const uint32_t k_off = (uint32_t)((BS >= 16 ? w : (w & 7)) * ROWB + gr * 16);
    const uint32_t v_off = (uint32_t)((BS >= 16 ? 4 * gr : ((4 * gr) & 7)) * ROWB + w * 16);
    const bool k_hi = BS < 16 && w >= 8;
    const bool v_hi = BS < 16 && gr >= 2;

    for (int wb = tok0; wb < tok1;) {
      const int fblk = wb / BS;
      const int off0 = wb - fblk * BS;
      const int we = min((fblk + kTblWin) * BS, tok1);
      const int nent = (we - 1) / BS - fblk + 1;
      int nshared;
      const int32_t* tbl = staged_window<BS, SPLIT>(a, tbl_lds, tc, trow, s, fblk, nent, lane, nshared);

      auto load = [&](auto pol, int ti, MfmaBuf<NQK, NVI>& buf) {
        constexpr int AUX = decltype(pol)::value;
        size_t lo, hi;
        tile_offsets<BS, ROWB>(tbl, off0 + ti * kTile, nent, blk_stride, lo, hi);
        if constexpr (BS >= 16) {  // one block region: SGPR base + lane offset
          // the resource ends at the window's last token: rows past it read
          // as zeros without a memory access (they are masked below)
          const uint32_t tb = (uint32_t)min(kTile, we - (wb + ti * kTile)) * ROWB;
          const rsrc_t rk = make_rsrc(kbase + lo, tb);
          const rsrc_t rv = make_rsrc(vbase + lo, tb);
#pragma unroll
          for (int i = 0; i < NQK; ++i) buf.k[i] = buf_ld16_aux<AUX>(rk, k_off + i * 64);
#pragma unroll
          for (int j = 0; j < NVI; ++j) buf.v[j] = buf_ld16_aux<AUX>(rv, v_off + j * ROWB);
        } else {  // block_size 8: tokens 8..15 come from the next block
          const char* kb = kbase + (k_hi ? hi : lo) + k_off;
          const char* vb = vbase + (v_hi ? hi : lo) + v_off;
#pragma unroll
          for (int i = 0; i < NQK; ++i) buf.k[i] = ld16_aux<AUX>(kb + i * 64);
#pragma unroll
          for (int j = 0; j < NVI; ++j) buf.v[j] = ld16_aux<AUX>(vb + j * ROWB);
        }
      };
      auto compute = [&](int ti, const MfmaBuf<NQK, NVI>& buf) {
        const int ts = wb + ti * kTile;
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NQK; ++i) sacc = mfma_16x16x32<T>(buf.k[i], qop[i], sacc);

        float sc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = (ts + 4 * gr + r < we) ? sacc[r] * a.scale_log2 : kNegInf;
        float tmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        tmax = swap_pair_max<16>(tmax);   // the head's max over the tile's 16 tokens
        tmax = swap_pair_max<32>(tmax);
        const bool grow = tmax > m_run + kLazy;   // true for the first tile
        if (__any(grow)) {
          const float m_new = grow ? tmax : m_run;
          const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
        }
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = sc[r] == kNegInf ? 0.f : fast_exp2(sc[r] - m_run);
        u32x2 pb_op;   // B operand: the 4 probabilities rounded to the input type
        pb_op[0] = pack2<T>(pr[0], pr[1]);
        pb_op[1] = pack2<T>(pr[2], pr[3]);
        {
          float r0, r1, r2, r3;   // the row sum adds the rounded weights that multiply V
          unpack2<T>(pb_op[0], r0, r1);
          unpack2<T>(pb_op[1], r2, r3);
          l_run += (r0 + r1) + (r2 + r3);
        }
        u32x4 vz[NVI];
#pragma unroll
        for (int j = 0; j < NVI; ++j) {
          const u32x4 z = {0u, 0u, 0u, 0u};
          vz[j] = (ts + 4 * gr + j < we) ? buf.v[j] : z;   // tail slots may hold NaN
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          // element dt of tokens 4 gr + 0 .. 3: low halves (even dt) or high halves (odd dt)
          const uint32_t sel = (dt & 1) ? 0x07060302u : 0x05040100u;
          u32x2 av;
          av[0] = __builtin_amdgcn_perm(vz[1][dt >> 1], vz[0][dt >> 1], sel);
          av[1] = __builtin_amdgcn_perm(vz[3][dt >> 1], vz[2][dt >> 1], sel);
          oacc[dt] = mfma_16x16x16<T>(av, pb_op, oacc[dt]);
        }
        if constexpr (PARTS) {   // a partition ends inside the run: write it, start the next
          if (ts + kTile == pend && pend < tok1) {
            finish(dest_part(dst, pk));
            reset();
            pend += dst.part;
            ++pk;
          }
        }
      };
      const int ntiles = (we - wb + kTile - 1) / kTile;
      run_window<MfmaBuf<NQK, NVI>, SPLIT>(ntiles, shared_tiles<BS>(nshared, nent, off0, ntiles), load, compute);
      wb = we;
    }

    finish(dest_part(dst, pk));
  }
};

// ============================================================================
// Unit-mode kernel: wave = (sequence, head group, partition), sequence the
// fastest index.  xcd_unit spreads runs of neighbouring workgroups over the
// XCDs.
// ============================================================================
template <class Core, class T, int D, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_unit_kernel(DecodeArgs a, int block_size) {
  constexpr int H = Core::HEADS;
  __shared__ int32_t s_tbl[NW][kTblWin];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t u = xcd_unit(blockIdx.x, gridDim.x) * NW + wave;
  const int S = a.num_seqs, C = a.head_chunks;
  if (u >= (uint32_t)S * C * a.num_parts) return;
  const int s = (int)(u % (uint32_t)S);
  const uint32_t rest = u / (uint32_t)S;
  const int c = (int)(rest % (uint32_t)C);
  const int p = (int)(rest / (uint32_t)C);
  const int h0 = c * H;
  const int L = clamp_len(a, s, block_size);
  const int P = a.partition_size;
  const int t0 = p * P;
  if (L == 0) {
    if (p == 0) store_zero_rows<T, D, H>(a, s, h0, lane);
    return;
  }
  if (t0 >= L) return;
  const int t1 = min(t0 + P, L);
  // partial rows: (s, h, p) -> ((s * Hq + h) * NP + p)
  const Dest dst{!a.split || L <= P, ((size_t)s * a.num_q_heads + h0) * a.num_parts + p,
                 (size_t)a.num_parts, 0};
  TblCache tc;
  Core::template run<false>(a, s_tbl[wave], tc, s, h0, t0, t1, dst);
}

// ============================================================================
// Grouped decode: the partition units of decode_unit_kernel, except that the
// partitions of a prefix group's shared tokens run once per KM of its
// sequences (CoreK), which read each shared K/V tile once for all of them.
// The grid holds the shared units first -- (group, member chunk, head
// group, partition), member chunk fastest, so the units that read one tile
// are neighbours on one XCD -- then the private units in decode_unit_kernel's
// order, which skip the partitions their group's shared units cover.  Every
// partial row is the one the plain partition pass would write, so the
// partition merge (launch_merge_parts) combines them unchanged.
// ============================================================================

// Shared tokens of group grp: group_shared[grp] rounded down to whole
// partitions, within the grid's shared partitions, and short of every
// member's length (each member keeps a private partition, so its merge has
// at least two parts, the shared units never write its output, and the
// unit's first member, whose table it reads, holds every shared block; a
// group with an empty member shares nothing).
__device__ __forceinline__ int group_shared_tokens(const DecodeArgs& a, const GroupArgs& ga, int grp, int first,
                                                   int end, int block_size) {
  const int P = a.partition_size;
  int sh = ga.group_shared[grp];
  sh = sh < 0 ? 0 : sh - sh % P;
  sh = min(sh, ga.shared_parts * P);
  for (int s = max(first, 0); s < end; ++s) sh = min(sh, (clamp_len(a, s, block_size) - 1) / P * P);
  return sh < 0 ? 0 : sh;
}

// Group of sequence s (its members first .. end - 1), or false when no group
// holds it.  group_start is non-decreasing from 0 (caller's contract).
__device__ __forceinline__ bool find_group(const GroupArgs& ga, int s, int& grp, int& first, int& end) {
  int lo = 0, hi = ga.num_groups;   // group_start[lo] <= s < group_start[hi] when s is in a group
  if (ga.num_groups <= 0 || s < ga.group_start[0] || s >= ga.group_start[ga.num_groups]) return false;
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (ga.group_start[mid] <= s) lo = mid; else hi = mid;
  }
  grp = lo;
  first = ga.group_start[lo];
  end = ga.group_start[lo + 1];
  return true;
}

template <class Core, class CoreK, class T, int D, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_group_kernel(DecodeArgs a, GroupArgs ga, int block_size) {
  constexpr int H = Core::HEADS;
  constexpr int KM = CoreK::MEMBERS;
  __shared__ int32_t s_tbl[NW][kTblWin];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t u = xcd_unit(blockIdx.x, gridDim.x) * NW + wave;
  const int S = a.num_seqs, C = a.head_chunks, P = a.partition_size;
  const uint32_t MC = (uint32_t)((ga.max_group_size + KM - 1) / KM);
  const uint32_t nsh = MC * (uint32_t)ga.num_groups * (uint32_t)C * (uint32_t)ga.shared_parts;
  TblCache tc;
  if (u < nsh) {
    const int mc = (int)(u % MC);
    uint32_t rest = u / MC;
    const int grp = (int)(rest % (uint32_t)ga.num_groups);
    rest /= (uint32_t)ga.num_groups;
    const int c = (int)(rest % (uint32_t)C);
    const int p = (int)(rest / (uint32_t)C);
    const int first = ga.group_start[grp], end = min(ga.group_start[grp + 1], S);
    const int s0 = first + mc * KM;
    const int km = min(KM, end - s0);
    if (first < 0 || km <= 0) return;
    const int t0 = p * P;
    if (t0 >= group_shared_tokens(a, ga, grp, first, end, block_size)) return;
    const int h0 = c * H;
    // rows (s0 + i, h0 + j, p) -> ((s0 + i) Hq + h0 + j) NP + p = prow0 + (i Hq + j) NP
    const Dest dst{false, ((size_t)s0 * a.num_q_heads + h0) * a.num_parts + p, (size_t)a.num_parts, 0};
    CoreK::template run<false>(a, s_tbl[wave], tc, s0, h0, t0, t0 + P, dst, nullptr, km);
    return;
  }
  const uint32_t v = u - nsh;
  if (v >= (uint32_t)S * C * a.num_parts) return;
  const int s = (int)(v % (uint32_t)S);
  const uint32_t rest = v / (uint32_t)S;
  const int c = (int)(rest % (uint32_t)C);
  const int p = (int)(rest / (uint32_t)C);
  const int h0 = c * H;
  const int L = clamp_len(a, s, block_size);
  if (L == 0) {
    if (p == 0) store_zero_rows<T, D, H>(a, s, h0, lane);
    return;
  }
  const int t0 = p * P;
  if (t0 >= L) return;
  int grp, first, end;
  // members past the grid's member chunks keep their shared tokens to themselves
  if (find_group(ga, s, grp, first, end) && s - first < (int)MC * KM &&
      t0 < group_shared_tokens(a, ga, grp, first, min(end, S), block_size))
    return;   // a shared unit's partition
  const int t1 = min(t0 + P, L);
  const Dest dst{L <= P, ((size_t)s * a.num_q_heads + h0) * a.num_parts + p, (size_t)a.num_parts, 0};
  Core::template run<false>(a, s_tbl[wave], tc, s, h0, t0, t1, dst);
}

// ============================================================================
// Balanced-mode kernel.  Flattened space: each (sequence, head group) with
// nt = ceil(L_s / 16) > 0 tiles costs X + nt units -- X for starting a
// segment (its query, its first tiles' latency, its epilogue), then its
// tiles -- so sequence s owns [C cum[s], C cum[s+1]) with cum the prefix of
// C (X + nt) and head groups major.  Of ntot units, wave w of W takes
// [w ntot / W, (w+1) ntot / W): waves whose range holds many short segments
// get fewer tiles, and all finish together.  A (sequence, head group) whose
// tiles all fall in one range is written directly; the first and the last
// segment of a range, when they are pieces of a larger one, go to partial
// slots 2w and 2w+1 (H rows each).  Each XCD gets a contiguous run of waves
// (so samples sharing a prompt's blocks meet in one L2); workgroup 0 also
// stores cum for the merge.
// ============================================================================
#ifndef PA_SEG_COST
#define PA_SEG_COST 2
#endif
// Segment start cost in tiles.  Swept with the kernels that buffer results in
// LDS (X = 0 / 1 / 2 / 3): OPT-13B-shaped MHA batch 169.8 / 162.7 / 155.2 /
// 156.9 us, the GQA batches within 0.3 % of each other.
constexpr int kSegCost = PA_SEG_COST;
__device__ __forceinline__ int64_t range_start(int64_t w, int64_t ntot, int64_t W) {
  return w * ntot / W;
}

// Workgroup b runs on XCD b % 8: give XCD x the contiguous logical range
// [x q + min(x, r), ...) of the n workgroups (q = n / 8, r = n % 8).
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t b, uint32_t n) {
  const uint32_t q = n / kNumXcd, r = n % kNumXcd;
  const uint32_t x = b % kNumXcd, k = b / kNumXcd;
  return x * q + (x < r ? x : r) + k;
}

template <int NT, bool PARTS = false>
__device__ __forceinline__ void tile_prefix(const DecodeArgs& a, int block_size, int32_t* s_cum,
                                            int32_t* s_wave) {
  // s_cum[s] = sum_{s' < s} cost(s'), cost = X + ceil(L / 16) (0 for an
  // empty sequence; with PARTS, X for each of its ceil(L / P) partitions),
  // s = 0..S: each thread sums a contiguous run of sequences, then the runs
  // are offset by a shuffle scan within each wave and the totals of the
  // waves before it
  static_assert(NT % kWave == 0, "whole waves");
  const int S = a.num_seqs;
  const int per = (S + NT - 1) / NT;
  const int lo = threadIdx.x * per, hi = min(lo + per, S);
  int sum = 0;
  for (int s = lo; s < hi; ++s) {
    const int L = clamp_len(a, s, block_size);
    const int nt = (L + kTile - 1) / kTile;
    s_cum[s] = sum;   // local exclusive prefix, offset below
    const int starts = PARTS ? (L + a.partition_size - 1) / a.partition_size : 1;
    sum += nt > 0 ? nt + starts * kSegCost : 0;
  }
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  int x = sum;   // inclusive scan over the wave's lanes
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) s_wave[wv] = x;
  __syncthreads();
  int base = x - sum, total = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) {
    const int t = s_wave[i];
    base += i < wv ? t : 0;
    total += t;
  }
  for (int s = lo; s < hi; ++s) s_cum[s] += base;
  if (threadIdx.x == 0) s_cum[S] = total;
  __syncthreads();
}

template <class Core, class T, int D, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_balanced_kernel(DecodeArgs a, int block_size) {
  constexpr int H = Core::HEADS;
  __shared__ int32_t s_cum[kBalancedMaxSeqs + 1];
  __shared__ int32_t s_wave[NW];
  __shared__ int32_t s_tbl[NW][kTblWin];
  using Buf = PartBuf<H, D>;
  __shared__ __align__(16) char s_pbuf[NW][Buf::kBytes];
  const int S = a.num_seqs, C = a.head_chunks;
  tile_prefix<NW * kWave>(a, block_size, s_cum, s_wave);
  // sequences with no tile own no range: their rows are zeros, written here
  for (int s = blockIdx.x; s < S; s += gridDim.x)
    if (s_cum[s + 1] == s_cum[s])
      for (int idx = threadIdx.x; idx < a.num_q_heads * D; idx += NW * kWave)
        store_elem<T>(a.out, (size_t)s * a.num_q_heads * D + idx, 0.f);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t W = (int64_t)gridDim.x * NW;
  const int64_t w = (int64_t)xcd_contiguous(blockIdx.x, gridDim.x) * NW + wave;
  const int64_t ntot = (int64_t)C * s_cum[S];
  int64_t f = range_start(w, ntot, W);
  const int64_t fb = range_start(w + 1, ntot, W);
  // The merge descriptor of boundary w (1 <= w < W, at position f): the head
  // group [A0, A0 + cost) whose real tiles [A0 + X, A0 + cost) it is the first
  // to split (wave w - 1 holds the first of them), or A0 = -1.  Every
  // boundary's descriptor is written by its wave in every call, so the merge
  // never reads one left by an earlier call.
  int64_t desc[4] = {-1, ntot, 0, 0};
  if (w >= 1 && f > 0 && f < ntot) {
    int lo = 0, hi = S - 1;   // the last s with C cum[s] <= f - 1
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)C * s_cum[mid] <= f - 1) lo = mid; else hi = mid - 1;
    }
    const int cost = s_cum[lo + 1] - s_cum[lo];
    const int cm = (int)((f - 1 - (int64_t)C * s_cum[lo]) / cost);
    const int64_t A0 = (int64_t)C * s_cum[lo] + (int64_t)cm * cost;
    const int64_t A = A0 + kSegCost, B = A0 + cost;
    if (A < f && f < B && range_start(w - 1, ntot, W) <= A) {
      desc[0] = A0;
      desc[2] = (int64_t)lo * a.num_q_heads + (int64_t)cm * H;
      desc[3] = (B * W - 1) / ntot - (w - 1) + 1;   // waves w - 1 .. w_hi
    }
  }
  const int lane = threadIdx.x & (kWave - 1);
  auto write_desc = [&]() {
    if (w >= 1 && lane == 0) {
      int64_t* d = a.ws_desc + 4 * w;
      d[0] = desc[0];
      d[1] = desc[1];
      d[2] = desc[2];
      d[3] = desc[3];
    }
  };
  if (f >= fb) {
    write_desc();
    return;
  }
  // the sequence holding tile f: the last s with C cum[s] <= f (empty
  // sequences share their successor's cum and are skipped)
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)C * s_cum[mid] <= f) lo = mid; else hi = mid - 1;
  }
  int s = lo;
  int ntc = s_cum[s + 1] - s_cum[s];        // cost of one head group of s: X + nt
  const int64_t rel = f - (int64_t)C * s_cum[s];
  int c = (int)(rel / ntc);
  int u = (int)(rel - (int64_t)c * ntc);    // position within that cost
  bool first = true;
  TblCache tc;
  Buf pb;
  pb.init(s_pbuf[wave], 1);
  while (f < fb) {
    const int n = (int)min((int64_t)(ntc - u), fb - f);
    const int nt = ntc - kSegCost;
    const int t0 = max(u - kSegCost, 0), t1 = min(u + n - kSegCost, nt);
    if (t1 > t0) {   // the range holds real tiles of this head group
      const int L = clamp_len(a, s, block_size);
      const int tok0 = t0 * kTile, tok1 = min(t1 * kTile, L);
      const size_t slot = 2 * (size_t)w + (first ? 0 : 1);
      const Dest dst{t0 == 0 && t1 == nt, slot * H, 1, 0};
      Core::template run<true, false, true>(a, s_tbl[wave], tc, s, c * H, tok0, tok1, dst, &pb);
      first = false;
    }
    f += n;
    u += n;
    if (u == ntc && f < fb) {  // next head group, or the next sequence with tiles
      u = 0;
      if (++c == C) {
        c = 0;
        do {
          ++s;
        } while (s_cum[s + 1] == s_cum[s]);
      }
      ntc = s_cum[s + 1] - s_cum[s];
    }
  }
  pb.template flush<T>(a, lane);   // results of the wave's segments, after its last loads
  write_desc();
}

// ============================================================================
// Fixed partitions on the resident grid.  The same units as the unit-mode
// split -- partition p of (sequence s, head group c) covers tokens
// [p P, min((p + 1) P, L)), each computed by one wave from start to end and
// written as a partial row (or directly when the sequence fits one
// partition) -- but the grid holds only the waves the GPU keeps resident,
// and each takes a contiguous run of whole units in (sequence, head group,
// partition) order.  Runs are cut by cost: a unit costs X + its tiles, so
// waves finish together up to one unit.  A wave walks the consecutive
// partitions of a head group in one tile loop (its query loaded once, its
// table windows of up to 256 entries, the next tile in flight across each
// partition boundary), writing each partition's result and restarting the
// running state at the boundary; K/V tiles stream with the non-temporal
// hint (shared blocks keep the default policy), as in the balanced split.
// Partials wait in a per-wave LDS buffer (PartBuf) and are written out in
// bursts.  Flattened position of unit (s, c, p):
// C cum[s] + c cost(s) + p (X + P / 16), cost(s) = ceil(L / 16) + X ceil(L / P).
// A wave owns the units that start in [w ntot / W, (w + 1) ntot / W).
// Arithmetic per unit is that of the unit-mode kernel, so both give the same
// bits; decode_merge_parts_kernel merges the partials.
// ============================================================================
template <class Core, class T, int D, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_parts_resident_kernel(DecodeArgs a, int block_size) {
  constexpr int H = Core::HEADS;
  __shared__ int32_t s_cum[kBalancedMaxSeqs + 1];
  __shared__ int32_t s_wave[NW];
  __shared__ int32_t s_tbl[NW][kTblWin];
  using Buf = PartBuf<H, D>;
  __shared__ __align__(16) char s_pbuf[NW][Buf::kBytes];
  const int S = a.num_seqs, C = a.head_chunks, P = a.partition_size;
  const int PT = P / kTile;                 // tiles of a full partition
  tile_prefix<NW * kWave, true>(a, block_size, s_cum, s_wave);
  for (int s = blockIdx.x; s < S; s += gridDim.x)   // empty sequences: zero rows
    if (s_cum[s + 1] == s_cum[s])
      for (int idx = threadIdx.x; idx < a.num_q_heads * D; idx += NW * kWave)
        store_elem<T>(a.out, (size_t)s * a.num_q_heads * D + idx, 0.f);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t W = (int64_t)gridDim.x * NW;
  const int64_t w = (int64_t)xcd_contiguous(blockIdx.x, gridDim.x) * NW + wave;
  const int64_t ntot = (int64_t)C * s_cum[S];
  const int64_t f = range_start(w, ntot, W);
  const int64_t fb = range_start(w + 1, ntot, W);
  if (f >= fb) return;
  int lo = 0, hi = S - 1;   // the sequence holding position f (empty ones skipped)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)C * s_cum[mid] <= f) lo = mid; else hi = mid - 1;
  }
  int s = lo;
  int cost = s_cum[s + 1] - s_cum[s];
  const int64_t rel = f - (int64_t)C * s_cum[s];
  int c = (int)(rel / cost);
  const int r = (int)(rel - (int64_t)c * cost);
  int p = (r + kSegCost + PT - 1) / (kSegCost + PT);   // first unit starting at or after r
  int64_t ustart = (int64_t)C * s_cum[s] + (int64_t)c * cost + (int64_t)p * (kSegCost + PT);
  int L = clamp_len(a, s, block_size);
  int np = (L + P - 1) / P;
  TblCache tc;
  Buf pb;
  pb.init(s_pbuf[wave], (size_t)a.num_parts);
  const int lane = threadIdx.x & (kWave - 1);
  for (;;) {
    if (p >= np) {   // next head group, or the next sequence with tiles
      p = 0;
      if (++c == C) {
        c = 0;
        do {
          ++s;
        } while (s < S && s_cum[s + 1] == s_cum[s]);
        if (s >= S) break;
        cost = s_cum[s + 1] - s_cum[s];
        L = clamp_len(a, s, block_size);
        np = (L + P - 1) / P;
      }
      ustart = (int64_t)C * s_cum[s] + (int64_t)c * cost;
    }
    if (ustart >= fb) break;
    // this head group's partitions p .. pl that start before fb, as one run
    const int64_t sc0 = ustart - (int64_t)p * (kSegCost + PT);
    const int pl = (int)min((int64_t)np - 1, (fb - sc0 + kSegCost + PT - 1) / (kSegCost + PT) - 1);
    const int h0 = c * H;
    const Dest dst{np == 1, ((size_t)s * a.num_q_heads + h0) * a.num_parts + p, (size_t)a.num_parts, P};
    Core::template run<true, true>(a, s_tbl[wave], tc, s, h0, p * P, min(pl * P + P, L), dst, &pb);
    ustart += (int64_t)(pl + 1 - p) * (kSegCost + PT);
    p = pl + 1;
  }
  pb.template flush<T>(a, lane);   // the K/V stream is over: nothing waits on these stores
}

// ============================================================================
// Merges.  Partition mode, per (sequence, q head): M = max_p m_p,
// w_p = 2^(m_p - M), out = sum_p w_p o_p / sum_p w_p l_p (o_p un-normalised).
// One workgroup of kPartMergeWaves waves per row.  A lane owns one 16-byte
// chunk of d, and the RPI = 64 / (D / 4) lane groups of a wave take different
// partitions, so one load instruction reads RPI partial rows; wave k takes
// partitions RPI k + j + q RPI W (j its lane group), 4 per lane in flight.
// Each wave first forms M from all m_p; the waves' sums meet in LDS and are
// added in wave order.
// ============================================================================
constexpr int kPartMergeWaves = 4;
template <class T, int D>
__global__ __launch_bounds__(kPartMergeWaves * kWave) void decode_merge_parts_kernel(DecodeArgs a,
                                                                                   int block_size) {
  constexpr int CH = D / 4;                 // 16-byte chunks of a partial row
  constexpr int RPI = kWave / CH;           // partial rows per load instruction
  constexpr int STEP = RPI * kPartMergeWaves;
  constexpr int U = 4;
  __shared__ f32x4 s_num[kPartMergeWaves][CH];
  __shared__ float s_den[kPartMergeWaves];
  const int row = blockIdx.x;               // s * Hq + h
  const int s = row / a.num_q_heads;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int L = clamp_len(a, s, block_size);
  const int P = a.partition_size;
  const int np = (L + P - 1) / P;
  if (np <= 1) return;                      // written directly by the partition pass
  const size_t base = (size_t)row * a.num_parts;
  float M = kNegInf;
  for (int p = lane; p < np; p += kWave) M = fmaxf(M, a.ws_m[base + p]);
  M = fmaxf(M, xor_lane<1>(M));
  M = fmaxf(M, xor_lane<2>(M));
  M = fmaxf(M, xor_lane<4>(M));
  M = fmaxf(M, xor_lane<8>(M));
  M = fmaxf(M, xor_lane<16>(M));
  M = fmaxf(M, xor_lane<32>(M));
  const int ch = lane % CH, j = lane / CH;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int p0 = RPI * wave + j; p0 < np; p0 += U * STEP) {
    f32x4 o[U];
    float wgt[U], l[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * STEP;
      const int pc = p < np ? p : p0;        // in range; weight 0 below
      o[u] = *reinterpret_cast<const f32x4*>(a.ws_o + (base + pc) * D + 4 * ch);
      wgt[u] = p < np ? fast_exp2(a.ws_m[base + pc] - M) : 0.f;
      l[u] = a.ws_l[base + pc];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) num[e] = fmaf(wgt[u], o[u][e], num[e]);
      den = fmaf(wgt[u], l[u], den);
    }
  }
  // lane groups j of the wave hold other partitions of the same chunk
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (RPI >= 4) num[e] += xor_lane<16>(num[e]);
    num[e] += xor_lane<32>(num[e]);
  }
  if constexpr (RPI >= 4) den += xor_lane<16>(den);
  den += xor_lane<32>(den);
  if (j == 0) s_num[wave][ch] = num;
  if (lane == 0) s_den[wave] = den;
  __syncthreads();
  if (wave == 0 && lane < CH) {
    f32x4 t = s_num[0][lane];
    float dt = s_den[0];
#pragma unroll
    for (int k = 1; k < kPartMergeWaves; ++k) {
      const f32x4 x = s_num[k][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] += x[e];
      dt += s_den[k];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) store_elem<T>(a.out, (size_t)row * D + 4 * lane + e, t[e] / dt);
  }
}

// The same merge for calls of at most 8 partitions per sequence at head_dim
// 128 (short contexts, prefix-shared samples), where a workgroup per row
// spends its launch on two or three partial rows: here a wave merges two
// rows, 32 lanes per row and one 16-byte chunk per lane.  It forms the same
// sums in the same order as decode_merge_parts_kernel, where partition p
// falls to wave p / 2 and lane half p % 2 (each wave adds its two products,
// then the four wave sums are added in wave order, absent partitions adding
// +0), so the two kernels give the same bits.
constexpr int kFewParts = 8;
template <class T, int D>
__global__ __launch_bounds__(4 * kWave) void decode_merge_few_kernel(DecodeArgs a, int block_size) {
  static_assert(D == 128, "32 lanes of 4 floats per row");
  const int lane = threadIdx.x & (kWave - 1);
  const size_t row = ((size_t)blockIdx.x * 4 + threadIdx.x / kWave) * 2 + (lane >> 5);   // s * Hq + h
  if (row >= (size_t)a.num_seqs * a.num_q_heads) return;
  const int s = (int)(row / (size_t)a.num_q_heads);
  const int L = clamp_len(a, s, block_size);
  const int P = a.partition_size;
  const int np = min((L + P - 1) / P, kFewParts);
  if (np <= 1) return;                      // written directly by the partition pass
  const size_t base = row * a.num_parts;
  const int ch = lane & 31;
  float m[kFewParts];
  float M = kNegInf;
#pragma unroll
  for (int p = 0; p < kFewParts; ++p) {
    m[p] = p < np ? a.ws_m[base + p] : kNegInf;
    M = fmaxf(M, m[p]);
  }
  f32x4 t = {0.f, 0.f, 0.f, 0.f};
  float dt = 0.f;
#pragma unroll
  for (int k = 0; k < kFewParts / 2; ++k) {
    f32x4 half[2];
    float dh[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int p = 2 * k + j;
      half[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      dh[j] = 0.f;
      if (p < np) {
        const float w = fast_exp2(m[p] - M);
        const f32x4 o = *reinterpret_cast<const f32x4*>(a.ws_o + (base + p) * D + 4 * ch);
#pragma unroll
        for (int e = 0; e < 4; ++e) half[j][e] = fmaf(w, o[e], 0.f);
        dh[j] = fmaf(w, a.ws_l[base + p], 0.f);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float n = half[0][e] + half[1][e];
      t[e] = k == 0 ? n : t[e] + n;
    }
    const float dn = dh[0] + dh[1];
    dt = k == 0 ? dn : dt + dn;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) store_elem<T>(a.out, row * D + 4 * ch + e, t[e] / dt);
}

// Merge launch of the fixed-partition passes.
template <class T, int D>
static hipError_t launch_merge_parts(const DecodeArgs& a, int bs, hipStream_t st) {
  const uint32_t rows = (uint32_t)a.num_seqs * a.num_q_heads;
  if constexpr (D == 128) {
    if (a.num_parts <= kFewParts) {
      hipLaunchKernelGGL((decode_merge_few_kernel<T, D>), dim3((rows + 7) / 8), dim3(4 * kWave), 0, st, a, bs);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_merge_parts_kernel<T, D>), dim3(rows), dim3(kPartMergeWaves * kWave), 0, st, a, bs);
  return hipGetLastError();
}

// Balanced mode: the head groups whose tiles were split between waves are
// found from the wave boundaries.  Boundary w (1 <= w < W, at position
// b = range_start(w) of the flattened space) merges the head group whose
// tiles [A, B) it is the first to split: A < b < B and wave w - 1 holds A.
// Decode wave w has already found that head group and left it in boundary
// w's descriptor (output row, cost start A0, piece count), so the merge
// starts with one load instead of a search of the prefix sums.  Head groups
// written whole need nothing, so the launch is sized by the boundaries,
// however many sequences there are.  The waves that shared [A, B)
// are w_lo = w - 1 .. w_hi; wave w left its piece in slot 2w + (its range
// starts at or after the head group's cost start A0 = A - X ? 0 : 1), and
// waves with an empty range wrote nothing.  Per head, lane p holds piece p
// (64 at a time) for the max and the sum, then all lanes walk the pieces with
// slot and weight read from lane j (loads unrolled by 8), each accumulating
// D/64 outputs.  Lanes without a piece point at w_lo's piece (always written
// in this call) with weight 0, so nothing left in the workspace by an earlier
// call is read.
constexpr int kMergeWaves = 4;
// The H heads of a boundary's head group go to min(H, 4) waves of one
// workgroup (each taking every min(H, 4)-th head), and a workgroup serves
// 4 / min(H, 4) boundaries.
template <int H>
constexpr int kMergeHeadWaves = H < kMergeWaves ? H : kMergeWaves;
template <int H>
constexpr int kMergeBoundaries = kMergeWaves / kMergeHeadWaves<H>;

template <class T, int D, int H>
__global__ __launch_bounds__(kMergeWaves * kWave) void decode_merge_balanced_kernel(DecodeArgs a,
                                                                                   int block_size,
                                                                                   int nwaves) {
  constexpr int EPL = D / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t W = nwaves;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (wave / kMergeHeadWaves<H> >= kMergeBoundaries<H>) return;
  const int64_t w = (int64_t)blockIdx.x * kMergeBoundaries<H> + wave / kMergeHeadWaves<H>;
  if (w < 1 || w >= W) return;
  const int64_t* desc = a.ws_desc + 4 * w;   // written by decode wave w in this call
  const int64_t A0 = desc[0];
  if (A0 < 0) return;
  const int64_t ntot = desc[1];
  const size_t orow = (size_t)desc[2];
  const int k = (int)desc[3];
  const int64_t w_lo = w - 1;
  const int slot_lo = (int)(2 * w_lo + (range_start(w_lo, ntot, W) >= A0 ? 0 : 1));
  auto piece_slot = [&](int p, bool& ok) {
    const int64_t w = w_lo + p;
    const int64_t ws = range_start(w, ntot, W);
    ok = p < k && ws != range_start(w + 1, ntot, W);
    return ok ? (int)(2 * w + (ws >= A0 ? 0 : 1)) : slot_lo;
  };
  for (int hh = wave % kMergeHeadWaves<H>; hh < H; hh += kMergeHeadWaves<H>) {
    float M = kNegInf;
    for (int p0 = 0; p0 < k; p0 += kWave) {
      bool ok;
      const int slot = piece_slot(p0 + lane, ok);
      M = fmaxf(M, a.ws_m[(size_t)slot * H + hh]);
    }
    M = fmaxf(M, xor_lane<1>(M));
    M = fmaxf(M, xor_lane<2>(M));
    M = fmaxf(M, xor_lane<4>(M));
    M = fmaxf(M, xor_lane<8>(M));
    M = fmaxf(M, xor_lane<16>(M));
    M = fmaxf(M, xor_lane<32>(M));
    float den = 0.f, num[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) num[e] = 0.f;
    for (int p0 = 0; p0 < k; p0 += kWave) {
      bool ok;
      const int slot = piece_slot(p0 + lane, ok);
      const float wgt = ok ? fast_exp2(a.ws_m[(size_t)slot * H + hh] - M) : 0.f;
      den = fmaf(wgt, a.ws_l[(size_t)slot * H + hh], den);
      const int cnt = min(kWave, k - p0);
      constexpr int U = 8;
      for (int j0 = 0; j0 < cnt; j0 += U) {
        float ov[U][EPL];
        float wj[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = min(j0 + u, cnt - 1);
          const int sj = __builtin_amdgcn_readlane(slot, j);
          wj[u] = j0 + u < cnt ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), j)) : 0.f;
          const float* o = a.ws_o + ((size_t)sj * H + hh) * D + lane;
#pragma unroll
          for (int e = 0; e < EPL; ++e) ov[u][e] = o[e * kWave];
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int e = 0; e < EPL; ++e) num[e] = fmaf(wj[u], ov[u][e], num[e]);
      }
    }
    den += xor_lane<1>(den);
    den += xor_lane<2>(den);
    den += xor_lane<4>(den);
    den += xor_lane<8>(den);
    den += xor_lane<16>(den);
    den += xor_lane<32>(den);
#pragma unroll
    for (int e = 0; e < EPL; ++e) store_elem<T>(a.out, (orow + hh) * D + e * kWave + lane, num[e] / den);
  }
}

// ============================================================================
// dispatch
// ============================================================================
#ifndef PA_WAVES_PER_UNIT
#define PA_WAVES_PER_UNIT 4
#endif
constexpr int kWavesPerGroup = PA_WAVES_PER_UNIT;

template <class Core, class T, int D>
static hipError_t run_core(const DecodeArgs& a, int bs, hipStream_t st) {
  constexpr int NW = kWavesPerGroup;
  constexpr int H = Core::HEADS;
  if (a.mode == kModeBalanced) {
    auto kern = decode_balanced_kernel<Core, T, D, NW>;
    int nwg = 0;
    hipError_t e = balanced_grid(reinterpret_cast<const void*>(kern), NW * kWave, Core::kBalancedWgPerCu,
                                 kBalancedMaxWaves / NW, &nwg);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(nwg), dim3(NW * kWave), 0, st, a, bs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const uint32_t waves = (uint32_t)nwg * NW;
    constexpr uint32_t BPW = kMergeBoundaries<H>;
    hipLaunchKernelGGL((decode_merge_balanced_kernel<T, D, H>), dim3((waves + BPW - 1) / BPW),
                       dim3(kMergeWaves * kWave), 0, st, a, bs, (int)waves);
    return hipGetLastError();
  }
  if (a.split && a.num_seqs <= kBalancedMaxSeqs) {   // fixed partitions on the resident grid
    auto kern = decode_parts_resident_kernel<Core, T, D, NW>;
    int nwg = 0;
    hipError_t e = balanced_grid(reinterpret_cast<const void*>(kern), NW * kWave, Core::kBalancedWgPerCu,
                                 kBalancedMaxWaves / NW, &nwg);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(nwg), dim3(NW * kWave), 0, st, a, bs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge_parts<T, D>(a, bs, st);
  }
  const uint64_t units = (uint64_t)a.num_seqs * a.head_chunks * a.num_parts;
  const uint32_t groups = (uint32_t)((units + NW - 1) / NW);
  hipLaunchKernelGGL((decode_unit_kernel<Core, T, D, NW>), dim3(groups), dim3(NW * kWave), 0, st, a, bs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.split) return e;
  return launch_merge_parts<T, D>(a, bs, st);
}

// Grouped decode (prefix groups given, fixed partitions): the group kernel,
// then the partition merge.
template <class T, int D, int BS, int G>
static hipError_t run_grouped(const DecodeArgs& a, const GroupArgs& ga, hipStream_t st) {
  constexpr int NW = kWavesPerGroup;
  using Core = MfmaPvCore<T, D, BS, G>;
  using CoreK = MfmaPvCore<T, D, BS, G, 16 / G>;
  constexpr int KM = CoreK::MEMBERS;
  const uint64_t mc = ((uint64_t)ga.max_group_size + KM - 1) / KM;
  const uint64_t units = mc * (uint64_t)ga.num_groups * a.head_chunks * ga.shared_parts +
                         (uint64_t)a.num_seqs * a.head_chunks * a.num_parts;
  if (units > 0x7fffffffull) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_group_kernel<Core, CoreK, T, D, NW>), dim3((uint32_t)((units + NW - 1) / NW)),
                     dim3(NW * kWave), 0, st, a, ga, BS);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge_parts<T, D>(a, BS, st);
}

// Grouped queries: P.V on the matrix cores for head_dim 128 and groups of at
// least PA_PV_MFMA_MIN_GROUP, MfmaCore otherwise.  The vector P.V of MfmaCore,
// G x 36 instructions per V chunk, bounds the call at larger groups (65 % of
// the HBM peak at G = 8, 32 % at G = 16 on the Llama-3-8B-shaped batch); at
// G = 4 the HBM-bound batches time the same either way (Llama-3-8B 670.4
// against 672.5 us, long context 831.4 against 830.9 us), and where shared
// blocks come from the caches the matrix-core form is 4 % faster
// (prefix-shared decode 237.3 against 247.7 us).
// With prefix groups on other cores the plain partition pass runs: the
// same results, without the shared reads.
template <class T, int D, int BS, int G>
static hipError_t run_gqa(const DecodeArgs& a, const GroupArgs* ga, hipStream_t st) {
  if constexpr (D == 128 && G >= PA_PV_MFMA_MIN_GROUP) {
    if (ga && a.split && a.mode == kModeUnit) return run_grouped<T, D, BS, G>(a, *ga, st);
    return run_core<MfmaPvCore<T, D, BS, G>, T, D>(a, BS, st);
  } else {
    return run_core<MfmaCore<T, D, BS, G>, T, D>(a, BS, st);
  }
}

template <class T, int D, int BS>
static hipError_t dispatch_bs(const DecodeArgs& a, int group, hipStream_t st, const GroupArgs* ga) {
  if constexpr (!std::is_same<T, F32>::value) {
    switch (group) {
      case 2: return run_gqa<T, D, BS, 2>(a, ga, st);
      case 4: return run_gqa<T, D, BS, 4>(a, ga, st);
      case 8: return run_gqa<T, D, BS, 8>(a, ga, st);
      case 16: return run_gqa<T, D, BS, 16>(a, ga, st);
      default: break;   // group 1: VALU
    }
  }
  switch (a.num_q_heads / a.head_chunks) {
    case 1: return run_core<ValuCore<T, D, BS, 1>, T, D>(a, BS, st);
    default: break;
  }
  if constexpr (std::is_same<T, F32>::value) {  // fp32 groups: 2 or 4 heads per unit
    switch (a.num_q_heads / a.head_chunks) {
      case 2: return run_core<ValuCore<T, D, BS, 2>, T, D>(a, BS, st);
      case 4: return run_core<ValuCore<T, D, BS, 4>, T, D>(a, BS, st);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

template <class T, int D>
static hipError_t dispatch_d(const DecodeArgs& a, int bs, int group, hipStream_t st, const GroupArgs* ga) {
  switch (bs) {
    case 8: return dispatch_bs<T, D, 8>(a, group, st, ga);
    case 16: return dispatch_bs<T, D, 16>(a, group, st, ga);
    case 32: return dispatch_bs<T, D, 32>(a, group, st, ga);
    default: return hipErrorInvalidValue;
  }
}

template <class T>
static hipError_t dispatch_t(const DecodeArgs& a, int head_dim, int bs, int group, hipStream_t st,
                             const GroupArgs* ga) {
  switch (head_dim) {
    case 64: return dispatch_d<T, 64>(a, bs, group, st, ga);
    case 128: return dispatch_d<T, 128>(a, bs, group, st, ga);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
