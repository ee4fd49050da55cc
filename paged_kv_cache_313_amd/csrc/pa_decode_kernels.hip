// Decode attention over a paged KV cache (gfx950, wave64).
//
// One query token per sequence attends over the sequence's context, whose K/V
// rows sit in fixed-size physical blocks reached through the sequence's block
// table (vLLM/PagedAttention paged-KV analysis page, section 3.1: the kernel is
// changed to read non-contiguous blocks; the simplified sketch walks the table
// block by block and loads K and V of each physical page).  The sketch
// normalises per block; the operation reached here is one softmax over the
// whole context, evaluated as an online softmax: a running max m, a running
// sum l and an un-normalised accumulator are rescaled by exp(m_old - m_new)
// whenever the max grows.  Scores are kept in the log2 domain
// (scale * log2(e) folded in) so every exponential is one v_exp_f32.
//
// A *segment* is a token range [tok0, tok1) of one sequence for one group of
// query heads sharing a KV head.  A workgroup of NW waves runs a segment: the
// segment's block-table slice is staged in LDS (taking the table->block
// dependent load off the tile path), the waves take interleaved 16-token
// tiles, and at the end the waves merge through LDS.  Three ways to cut the
// work into segments:
//  * unit mode, no split: one workgroup per (sequence, head group);
//  * unit mode, fixed partitions of P tokens: one workgroup per (sequence,
//    head group, partition), partials merged by decode_merge_parts_kernel;
//  * balanced mode: the grid holds exactly the workgroups the GPU keeps
//    resident, and each takes an equal share of the flattened
//    (sequence, head group, tile) space, so ragged batches finish together;
//    a (sequence, head group) shared by several workgroups is merged by
//    decode_merge_balanced_kernel.
#include <type_traits>

#include "pa_common.hpp"
#include "pa_launch.hpp"

namespace pa {

constexpr int kTile = 16;      // tokens per tile
constexpr int kTblWin = 256;   // block-table entries staged in LDS at a time

template <int NW>
__device__ __forceinline__ void stage_table(int32_t* s_tbl, const int32_t* row, int first, int count,
                                            int num_blocks) {
  for (int i = threadIdx.x; i < count; i += NW * kWave) {
    const int e = row[first + i];
    s_tbl[i] = ((unsigned)e < (unsigned)num_blocks) ? e : 0;  // memory-safe clamp
  }
}

// Walk the 16-token tiles assigned to this wave (tiles wave, wave+NW, ...),
// keeping the next tile's K/V loads in flight while the current one is
// computed.  The loop runs over pairs of tiles with ping-pong buffers and has a
// single exit, so that no path (not even a structurized, never-taken one)
// returns to the loop head with the prefetch outstanding; that lets the
// compiler's vmcnt waits leave the newer loads in flight.  Loads are
// unconditional: a prefetch past the wave's last tile re-reads that tile (an
// L2 hit) instead of branching.
template <int NW, class Buf, class Load, class Compute>
__device__ __forceinline__ void tile_loop(int ntiles, int wave, Load&& load, Compute&& compute) {
  if (wave >= ntiles) return;
  const int n = (ntiles - wave + NW - 1) / NW;   // tiles of this wave
  const int last = wave + (n - 1) * NW;
  Buf a, b;
  int ti = wave;
  load(ti, a);
  for (int k = 0; k + 2 <= n; k += 2) {
    load(min(ti + NW, last), b);
    compute(ti, a);
    load(min(ti + 2 * NW, last), a);
    compute(ti + NW, b);
    ti += 2 * NW;
  }
  if (n & 1) compute(ti, a);
}

// Byte offsets, from the start of a KV head's slice of the pool, of the
// 16-token tile that starts `rel` tokens after the first staged block.  The block id is
// wave-uniform, so the offsets live in SGPRs and each lane adds a constant
// 32-bit offset: no per-lane address arithmetic on the tile path.  With
// block_size >= 16 the tile lies in one block (lo == hi); with 8 its tokens
// [8, 16) are in the next block, which may be past the window's last staged
// entry only when every one of those tokens is masked (then lo is reused).
template <int BS, int ROWB>
__device__ __forceinline__ void tile_offsets(const int32_t* s_tbl, int rel, int nent,
                                             size_t blk_stride, size_t& lo, size_t& hi) {
  if constexpr (BS >= 16) {
    const int b = __builtin_amdgcn_readfirstlane(s_tbl[rel / BS]);
    lo = hi = (size_t)b * blk_stride + (size_t)(rel % BS) * ROWB;
  } else {
    const int e = rel / BS;
    const int b0 = __builtin_amdgcn_readfirstlane(s_tbl[e]);
    const int b1 = e + 1 < nent ? __builtin_amdgcn_readfirstlane(s_tbl[e + 1]) : b0;
    lo = (size_t)b0 * blk_stride;
    hi = (size_t)b1 * blk_stride;
  }
}

// Per-wave results of a segment, merged across the workgroup's waves.
template <int H, int D, int NW>
struct SegSmem {
  int32_t tbl[kTblWin];
  float m[NW][H], l[NW][H];
  float acc[NW][H][D];
};

// Merge the NW waves' (m, l, acc) and write H rows: the output (direct) or a
// partial (m, l, un-normalised acc) at workspace rows prow0 + hh * pstride.
template <class T, int D, int H, int NW>
__device__ __forceinline__ void emit_rows(const DecodeArgs& a, const SegSmem<H, D, NW>& sm, int s,
                                          int h0, bool direct, size_t prow0, size_t pstride) {
  for (int idx = threadIdx.x; idx < H * D; idx += NW * kWave) {
    const int hh = idx / D, d = idx - (idx / D) * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.m[w][hh]);
    float lt = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(sm.m[w][hh] - M);   // a wave with no tile has m = -inf: f = 0
      lt += f * sm.l[w][hh];
      o += f * sm.acc[w][hh][d];
    }
    if (direct) {
      store_elem<T>(a.out, ((size_t)s * a.num_q_heads + h0 + hh) * D + d, o / lt);
    } else {
      const size_t pr = prow0 + (size_t)hh * pstride;
      a.ws_o[pr * D + d] = o;
      if (d == 0) {
        a.ws_m[pr] = M;
        a.ws_l[pr] = lt;
      }
    }
  }
}

template <class T, int D, int H, int NW>
__device__ __forceinline__ void store_zero_rows(const DecodeArgs& a, int s, int h0) {
  for (int idx = threadIdx.x; idx < H * D; idx += NW * kWave)
    store_elem<T>(a.out, ((size_t)s * a.num_q_heads + h0) * D + idx, 0.f);
}

// ============================================================================
// VALU core: any dtype, H q heads (1, 2 or 4) of one KV head.
// Lane layout per tile: token tt = lane / 4, quarter qp = lane % 4; the lane
// holds the row bytes [16 (4 j + qp), +16) for j < NL, i.e. D/4 elements.
// ============================================================================
template <int NL>
struct ValuBuf {
  u32x4 k[NL], v[NL];
};

template <class T, int D, int BS, int H, int NW>
struct ValuCore {
  static constexpr int EB = T::bytes;
  static constexpr int ROWB = D * EB;
  static constexpr int NL = ROWB / 64;    // 16-byte loads per lane per token row
  static constexpr int NE = 16 / EB;      // elements per 16 bytes
  static constexpr int DPL = NL * NE;     // elements per lane (= D / 4)
  static constexpr int HEADS = H;
  static_assert(DPL * 4 == D, "layout");
  static_assert(kTblWin * BS % kTile == 0, "window");
  // bytes a tile's buffer resource spans: its 16 rows (8 per block at block_size 8)
  static constexpr uint32_t kTileBytes = (BS >= 16 ? kTile : BS) * ROWB;
  using Smem = SegSmem<H, D, NW>;

  // q heads h0 .. h0+H-1 of sequence s over tokens [tok0, tok1); leaves the
  // per-wave results in sm and ends with a barrier.
  __device__ static void run(const DecodeArgs& a, Smem& sm, int s, int h0, int tok0, int tok1) {
    const int lane = threadIdx.x & (kWave - 1);
    // wave-uniform by construction; readfirstlane tells the compiler so that
    // the tile loop runs on scalar branches (no exec-mask flow blocks)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int G = a.num_q_heads / a.num_kv_heads;
    const int g = h0 / G;
    const int tt = lane >> 2, qp = lane & 3;

    float qf[H][DPL];  // query rows in fp32, the lane's D/4 elements
#pragma unroll
    for (int hh = 0; hh < H; ++hh) {
      const char* qrow = reinterpret_cast<const char*>(a.query) +
                         ((size_t)s * a.num_q_heads + h0 + hh) * ROWB + qp * 16;
#pragma unroll
      for (int j = 0; j < NL; ++j) Unpack<T>::run(ld16(qrow + j * 64), &qf[hh][j * NE]);
    }
    float m_run[H], l_run[H], acc[H][DPL];
#pragma unroll
    for (int hh = 0; hh < H; ++hh) {
      m_run[hh] = kNegInf;
      l_run[hh] = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[hh][i] = 0.f;
    }

    const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (size_t)g * BS * ROWB;
    const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (size_t)g * BS * ROWB;
    const size_t blk_stride = (size_t)a.num_kv_heads * BS * ROWB;
    const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks_per_seq;
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
      __syncthreads();
      stage_table<NW>(sm.tbl, trow, fblk, nent, a.num_blocks);
      __syncthreads();

      auto load = [&](int ti, ValuBuf<NL>& buf) {
        size_t lo, hi;
        tile_offsets<BS, ROWB>(sm.tbl, off0 + ti * kTile, nent, blk_stride, lo, hi);
        if constexpr (BS >= 16) {  // one block region: SGPR base + lane offset
          const rsrc_t rk = make_rsrc(kbase + lo, kTileBytes);
          const rsrc_t rv = make_rsrc(vbase + lo, kTileBytes);
#pragma unroll
          for (int j = 0; j < NL; ++j) buf.k[j] = buf_ld16(rk, lane_off + j * 64);
#pragma unroll
          for (int j = 0; j < NL; ++j) buf.v[j] = buf_ld16(rv, lane_off + j * 64);
        } else {  // block_size 8: tokens 8..15 come from the next block
          const size_t off = (hi_blk ? hi : lo) + lane_off;
#pragma unroll
          for (int j = 0; j < NL; ++j) buf.k[j] = ld16(kbase + off + j * 64);
#pragma unroll
          for (int j = 0; j < NL; ++j) buf.v[j] = ld16(vbase + off + j * 64);
        }
      };
      auto compute = [&](int ti, const ValuBuf<NL>& buf) {
        const bool valid = wb + ti * kTile + tt < we;
        float kf[DPL];
#pragma unroll
        for (int j = 0; j < NL; ++j) Unpack<T>::run(buf.k[j], &kf[j * NE]);
        float pr[H];
#pragma unroll
        for (int hh = 0; hh < H; ++hh) {
          float dot = 0.f;
#pragma unroll
          for (int i = 0; i < DPL; ++i) dot = fmaf(qf[hh][i], kf[i], dot);
          dot += xor_lane<1>(dot);
          dot += xor_lane<2>(dot);
          const float sc = valid ? dot * a.scale_log2 : kNegInf;
          float tmax = sc;
          tmax = fmaxf(tmax, xor_lane<4>(tmax));
          tmax = fmaxf(tmax, xor_lane<8>(tmax));
          tmax = fmaxf(tmax, xor_lane<16>(tmax));
          tmax = fmaxf(tmax, xor_lane<32>(tmax));
          const float m_new = fmaxf(m_run[hh], tmax);
          if (m_new > m_run[hh]) {  // same value in every lane: a uniform branch
            const float alpha = fast_exp2(m_run[hh] - m_new);
            l_run[hh] *= alpha;
#pragma unroll
            for (int i = 0; i < DPL; ++i) acc[hh][i] *= alpha;
            m_run[hh] = m_new;
          }
          pr[hh] = fast_exp2(sc - m_run[hh]);
          l_run[hh] += pr[hh];
        }
        float vf[DPL];
#pragma unroll
        for (int j = 0; j < NL; ++j) Unpack<T>::run(buf.v[j], &vf[j * NE]);
#pragma unroll
        for (int i = 0; i < DPL; ++i) vf[i] = valid ? vf[i] : 0.f;  // tail slots may hold NaN
#pragma unroll
        for (int hh = 0; hh < H; ++hh)
#pragma unroll
          for (int i = 0; i < DPL; ++i) acc[hh][i] = fmaf(pr[hh], vf[i], acc[hh][i]);
      };
      tile_loop<NW, ValuBuf<NL>>((we - wb + kTile - 1) / kTile, wave, load, compute);
      wb = we;
    }

    // sum over the 16 token slots of the wave (lanes with equal qp)
#pragma unroll
    for (int hh = 0; hh < H; ++hh) {
      float l = l_run[hh];
      l += xor_lane<4>(l);
      l += xor_lane<8>(l);
      l += xor_lane<16>(l);
      l += xor_lane<32>(l);
      l_run[hh] = l;
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        float x = acc[hh][i];
        x += xor_lane<4>(x);
        x += xor_lane<8>(x);
        x += xor_lane<16>(x);
        x += xor_lane<32>(x);
        acc[hh][i] = x;
      }
    }
    if (lane < 4) {
#pragma unroll
      for (int hh = 0; hh < H; ++hh)
#pragma unroll
        for (int j = 0; j < NL; ++j)
#pragma unroll
          for (int e = 0; e < NE; ++e) sm.acc[wave][hh][(4 * j + qp) * NE + e] = acc[hh][j * NE + e];
      if (lane == 0) {
#pragma unroll
        for (int hh = 0; hh < H; ++hh) {
          sm.m[wave][hh] = m_run[hh];
          sm.l[wave][hh] = l_run[hh];
        }
      }
    }
    __syncthreads();
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
// accumulates G x 8 fp32 values.
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

template <int NQK, int NVI>
struct MfmaBuf {
  u32x4 k[NQK], v[NVI];
};

template <class T, int D, int BS, int G, int NW>
struct MfmaCore {
  static constexpr int ROWB = D * 2;
  static constexpr int NQK = D / 32;   // MFMAs per tile (k = 32 per MFMA)
  static constexpr int CPR = D / 8;    // 16-byte chunks per token row
  static constexpr int NVI = D / 32;   // V chunks per lane per tile (16 * CPR / 64)
  static constexpr int HEADS = G;
  static_assert(16 % G == 0 && G >= 2, "group");
  static_assert(kTblWin * BS % kTile == 0, "window");
  static constexpr uint32_t kTileBytes = (BS >= 16 ? kTile : BS) * ROWB;
  using Smem = SegSmem<G, D, NW>;

  // the G q heads h0 .. h0+G-1 (KV head h0 / G) of sequence s over tokens
  // [tok0, tok1); leaves the per-wave results in sm and ends with a barrier.
  __device__ static void run(const DecodeArgs& a, Smem& sm, int s, int h0, int tok0, int tok1) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int gr = lane >> 4, w = lane & 15;
    const int g = h0 / G;

    u32x4 qop[NQK];  // B operand: query row of head w % G, chunk 4 i + gr
    {
      const char* qrow = reinterpret_cast<const char*>(a.query) +
                         ((size_t)s * a.num_q_heads + h0 + (w % G)) * ROWB;
#pragma unroll
      for (int i = 0; i < NQK; ++i) qop[i] = ld16(qrow + (4 * i + gr) * 16);
    }
    float m_run = kNegInf, l_run = 0.f;  // for head w % G
    float acc[G][8];                     // d = 8 * (w % CPR) + e
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

    const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (size_t)g * BS * ROWB;
    const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (size_t)g * BS * ROWB;
    const size_t blk_stride = (size_t)a.num_kv_heads * BS * ROWB;
    const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks_per_seq;
    // K: token w of the tile, chunk 4 i + gr (i = instruction);
    // V: token 4 gr + w / CPR + 16 j / CPR, chunk w % CPR (j = instruction)
    const int tv0 = 4 * gr + w / CPR;
    const uint32_t k_off = (uint32_t)((BS >= 16 ? w : (w & 7)) * ROWB + gr * 16);
    const uint32_t v_off = (uint32_t)((BS >= 16 ? tv0 : (tv0 & 7)) * ROWB + (w % CPR) * 16);
    const bool k_hi = BS < 16 && w >= 8;
    const bool v_hi = BS < 16 && gr >= 2;

    // windows of at most kTblWin blocks; a segment may start inside a block
    // (balanced mode, block_size 32): off0 is that start within its block
    for (int wb = tok0; wb < tok1;) {
      const int fblk = wb / BS;
      const int off0 = wb - fblk * BS;
      const int we = min((fblk + kTblWin) * BS, tok1);
      const int nent = (we - 1) / BS - fblk + 1;
      __syncthreads();
      stage_table<NW>(sm.tbl, trow, fblk, nent, a.num_blocks);
      __syncthreads();

      auto load = [&](int ti, MfmaBuf<NQK, NVI>& buf) {
        size_t lo, hi;
        tile_offsets<BS, ROWB>(sm.tbl, off0 + ti * kTile, nent, blk_stride, lo, hi);
        if constexpr (BS >= 16) {  // one block region: SGPR base + lane offset
          const rsrc_t rk = make_rsrc(kbase + lo, kTileBytes);
          const rsrc_t rv = make_rsrc(vbase + lo, kTileBytes);
#pragma unroll
          for (int i = 0; i < NQK; ++i) buf.k[i] = buf_ld16(rk, k_off + i * 64);
#pragma unroll
          for (int j = 0; j < NVI; ++j) buf.v[j] = buf_ld16(rv, v_off + (16 * j / CPR) * ROWB);
        } else {  // block_size 8: tokens 8..15 come from the next block
          const char* kb = kbase + (k_hi ? hi : lo) + k_off;
          const char* vb = vbase + (v_hi ? hi : lo) + v_off;
#pragma unroll
          for (int i = 0; i < NQK; ++i) buf.k[i] = ld16(kb + i * 64);
#pragma unroll
          for (int j = 0; j < NVI; ++j) buf.v[j] = ld16(vb + (16 * j / CPR) * ROWB);
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
        tmax = fmaxf(tmax, xor_lane<16>(tmax));
        tmax = fmaxf(tmax, xor_lane<32>(tmax));
        const float m_new = fmaxf(m_run, tmax);
        if (__any(m_new > m_run)) {
          const float alpha = fast_exp2(m_run - m_new);
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
          pr[r] = fast_exp2(sc[r] - m_run);
          l_run += pr[r];
        }
#pragma unroll
        for (int j = 0; j < NVI; ++j) {
          const int idx = w + 16 * j;
          const int rt = idx / CPR;   // token of the group: uniform for D = 128
          float vf[8];
          Unpack<T>::run(buf.v[j], vf);
          const bool vvalid = ts + 4 * gr + rt < we;
#pragma unroll
          for (int e = 0; e < 8; ++e) vf[e] = vvalid ? vf[e] : 0.f;
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
      };
      tile_loop<NW, MfmaBuf<NQK, NVI>>((we - wb + kTile - 1) / kTile, wave, load, compute);
      wb = we;
    }

    // l: sum over the four token groups; acc: sum over lanes holding the same chunk
    l_run += xor_lane<16>(l_run);
    l_run += xor_lane<32>(l_run);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = acc[h][e];
        if constexpr (CPR == 8) x += xor_lane<8>(x);
        x += xor_lane<16>(x);
        x += xor_lane<32>(x);
        acc[h][e] = x;
      }
    if (gr == 0 && w < CPR) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.acc[wave][h][8 * w + e] = acc[h][e];
    }
    if (lane < G) {
      sm.m[wave][lane] = m_run;
      sm.l[wave][lane] = l_run;
    }
    __syncthreads();
  }
};

// ============================================================================
// Unit-mode kernel: workgroup = (sequence, head group, partition).  Sequence
// is the fastest index of the logical unit; xcd_unit spreads runs of
// neighbouring units over the XCDs.
// ============================================================================
template <class Core, class T, int D, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_unit_kernel(DecodeArgs a, int block_size) {
  constexpr int H = Core::HEADS;
  __shared__ typename Core::Smem sm;
  const uint32_t u = xcd_unit(blockIdx.x, gridDim.x);
  const int S = a.num_seqs, C = a.head_chunks;
  const int s = (int)(u % (uint32_t)S);
  const uint32_t rest = u / (uint32_t)S;
  const int c = (int)(rest % (uint32_t)C);
  const int p = (int)(rest / (uint32_t)C);
  const int h0 = c * H;
  const int L = clamp_len(a, s, block_size);
  const int P = a.partition_size;
  const int t0 = p * P;
  if (L == 0) {
    if (p == 0) store_zero_rows<T, D, H, NW>(a, s, h0);
    return;
  }
  if (t0 >= L) return;
  const int t1 = min(t0 + P, L);
  const bool direct = !a.split || L <= P;
  Core::run(a, sm, s, h0, t0, t1);
  // partial rows: (s, h, p) -> ((s * Hq + h) * NP + p)
  emit_rows<T, D, H, NW>(a, sm, s, h0, direct,
                         ((size_t)s * a.num_q_heads + h0) * a.num_parts + p, (size_t)a.num_parts);
}

// ============================================================================
// Balanced-mode kernel.  Flattened space: sequence s owns tiles
// [C cum[s], C cum[s+1]) (C head groups of ceil(L_s / 16) tiles each, head
// group major).  Of ntot tiles, workgroup w takes [w ntot / W, (w+1) ntot / W).  A (sequence, head
// group) wholly inside the range is written directly; the first and the last
// segment of the range, when they are pieces of a larger one, go to partial
// slots 2w and 2w+1 (H rows each).  Workgroup 0 also stores cum for the merge.
// ============================================================================
__device__ __forceinline__ int64_t range_start(int64_t w, int64_t ntot, int64_t W) {
  return w * ntot / W;
}

template <int NT>
__device__ __forceinline__ void tile_prefix(const DecodeArgs& a, int block_size, int32_t* s_cum,
                                            int32_t* s_part) {
  // s_cum[s] = sum_{s' < s} ceil(L_s' / 16), s = 0..S, by a block-wide scan
  const int S = a.num_seqs;
  const int per = (S + NT - 1) / NT;
  const int lo = threadIdx.x * per, hi = min(lo + per, S);
  int sum = 0;
  for (int s = lo; s < hi; ++s) {
    const int nt = (clamp_len(a, s, block_size) + kTile - 1) / kTile;
    s_cum[s] = sum;   // local exclusive prefix, offset below
    sum += nt;
  }
  s_part[threadIdx.x] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < NT; ++i) {
      const int x = s_part[i];
      s_part[i] = run;
      run += x;
    }
    s_cum[S] = run;
  }
  __syncthreads();
  const int base = s_part[threadIdx.x];
  for (int s = lo; s < hi; ++s) s_cum[s] += base;
  __syncthreads();
}

template <class Core, class T, int D, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_balanced_kernel(DecodeArgs a, int block_size) {
  constexpr int H = Core::HEADS;
  __shared__ typename Core::Smem sm;
  __shared__ int32_t s_cum[kBalancedMaxSeqs + 1];
  __shared__ int32_t s_part[NW * kWave];
  const int S = a.num_seqs, C = a.head_chunks;
  tile_prefix<NW * kWave>(a, block_size, s_cum, s_part);
  if (blockIdx.x == 0)
    for (int s = threadIdx.x; s <= S; s += NW * kWave) a.ws_cum[s] = s_cum[s];

  const int64_t W = gridDim.x, w = blockIdx.x;
  const int64_t ntot = (int64_t)C * s_cum[S];
  int64_t f = range_start(w, ntot, W);
  const int64_t fb = range_start(w + 1, ntot, W);
  if (f >= fb) return;
  // the sequence holding tile f: the last s with C cum[s] <= f (empty
  // sequences share their successor's cum and are skipped)
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)C * s_cum[mid] <= f) lo = mid; else hi = mid - 1;
  }
  int s = lo;
  int nt = s_cum[s + 1] - s_cum[s];
  const int64_t rel = f - (int64_t)C * s_cum[s];
  int c = (int)(rel / nt);
  int t = (int)(rel - (int64_t)c * nt);
  bool first = true;
  while (f < fb) {
    const int n = (int)min((int64_t)(nt - t), fb - f);
    const int L = clamp_len(a, s, block_size);
    const int tok0 = t * kTile, tok1 = min((t + n) * kTile, L);
    Core::run(a, sm, s, c * H, tok0, tok1);
    const bool whole = t == 0 && t + n == nt;
    const size_t slot = 2 * (size_t)w + (first ? 0 : 1);
    emit_rows<T, D, H, NW>(a, sm, s, c * H, whole, slot * H, 1);
    first = false;
    f += n;
    t += n;
    if (t == nt && f < fb) {  // next head group, or the next sequence with tiles
      t = 0;
      if (++c == C) {
        c = 0;
        do {
          ++s;
        } while (s_cum[s + 1] == s_cum[s]);
      }
      nt = s_cum[s + 1] - s_cum[s];
    }
  }
}

// ============================================================================
// Merges.  Partition mode, per (sequence, q head): M = max_p m_p,
// w_p = 2^(m_p - M), out = sum_p w_p o_p / sum_p w_p l_p (o_p un-normalised).
// One wave per row: lane p reads (m_p, l_p) for 64 partitions at a time; the
// lanes then walk the partitions with the weight read from lane j, each lane
// accumulating D/64 output elements, loads unrolled for memory parallelism.
// ============================================================================
template <class T, int D>
__global__ __launch_bounds__(kWave) void decode_merge_parts_kernel(DecodeArgs a, int block_size) {
  constexpr int EPL = D / kWave;            // output elements per lane
  const int row = blockIdx.x;               // s * Hq + h
  const int s = row / a.num_q_heads;
  const int lane = threadIdx.x;
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
  float den = 0.f, num[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) num[e] = 0.f;
  for (int p0 = 0; p0 < np; p0 += kWave) {
    const int p = p0 + lane;
    const float wgt = p < np ? fast_exp2(a.ws_m[base + p] - M) : 0.f;
    den = p < np ? fmaf(wgt, a.ws_l[base + p], den) : den;
    const int cnt = min(kWave, np - p0);
    const float* o = a.ws_o + (base + p0) * D + lane;
    int j = 0;
    for (; j + 4 <= cnt; j += 4) {
      float ov[4][EPL];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < EPL; ++e) ov[u][e] = o[(size_t)(j + u) * D + e * kWave];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), j + u));
#pragma unroll
        for (int e = 0; e < EPL; ++e) num[e] = fmaf(wj, ov[u][e], num[e]);
      }
    }
    for (; j < cnt; ++j) {
      const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), j));
#pragma unroll
      for (int e = 0; e < EPL; ++e) num[e] = fmaf(wj, o[(size_t)j * D + e * kWave], num[e]);
    }
  }
  den += xor_lane<1>(den);
  den += xor_lane<2>(den);
  den += xor_lane<4>(den);
  den += xor_lane<8>(den);
  den += xor_lane<16>(den);
  den += xor_lane<32>(den);
#pragma unroll
  for (int e = 0; e < EPL; ++e) store_elem<T>(a.out, (size_t)row * D + e * kWave + lane, num[e] / den);
}

// Balanced mode, per (sequence, head group): the workgroups that shared its
// tile range [A, B) are w_lo .. w_hi (w_lo: the last workgroup whose range
// starts at or before A); workgroup w left its piece in slot
// 2w + (its range starts at or after A ? 0 : 1).  Empty sequences get zeros.
template <class T, int D, int H>
__global__ __launch_bounds__(256) void decode_merge_balanced_kernel(DecodeArgs a, int block_size,
                                                                    int nwg) {
  const int C = a.head_chunks;
  const int s = blockIdx.x / C, c = blockIdx.x - (blockIdx.x / C) * C;
  const int L = clamp_len(a, s, block_size);
  const int nt = (L + kTile - 1) / kTile;
  const size_t orow = (size_t)s * a.num_q_heads + (size_t)c * H;
  if (nt == 0) {
    for (int idx = threadIdx.x; idx < H * D; idx += blockDim.x) store_elem<T>(a.out, orow * D + idx, 0.f);
    return;
  }
  const int64_t W = nwg;
  const int64_t ntot = (int64_t)C * a.ws_cum[a.num_seqs];
  const int64_t A = (int64_t)C * a.ws_cum[s] + (int64_t)c * nt, B = A + nt;
  const int64_t w_lo = ((A + 1) * W - 1) / ntot, w_hi = (B * W - 1) / ntot;
  if (w_lo == w_hi) return;                 // one workgroup wrote it directly
  // workgroups with an empty range (more workgroups than tiles) wrote nothing
  for (int idx = threadIdx.x; idx < H * D; idx += blockDim.x) {
    const int hh = idx / D, d = idx - (idx / D) * D;
    float M = kNegInf;
    for (int64_t w = w_lo; w <= w_hi; ++w) {
      const int64_t ws = range_start(w, ntot, W);
      if (ws == range_start(w + 1, ntot, W)) continue;
      const size_t slot = 2 * (size_t)w + (ws >= A ? 0 : 1);
      M = fmaxf(M, a.ws_m[slot * H + hh]);
    }
    float num = 0.f, den = 0.f;
    for (int64_t w = w_lo; w <= w_hi; ++w) {
      const int64_t ws = range_start(w, ntot, W);
      if (ws == range_start(w + 1, ntot, W)) continue;
      const size_t slot = 2 * (size_t)w + (ws >= A ? 0 : 1);
      const size_t r = slot * H + hh;
      const float f = fast_exp2(a.ws_m[r] - M);
      den = fmaf(f, a.ws_l[r], den);
      num = fmaf(f, a.ws_o[r * D + d], num);
    }
    store_elem<T>(a.out, (orow + hh) * D + d, num / den);
  }
}

// ============================================================================
// dispatch
// ============================================================================
#ifndef PA_WAVES_PER_UNIT
#define PA_WAVES_PER_UNIT 4
#endif
constexpr int kWavesPerUnit = PA_WAVES_PER_UNIT;

template <class Core, class T, int D>
static hipError_t run_core(const DecodeArgs& a, int bs, hipStream_t st) {
  constexpr int NW = kWavesPerUnit;
  constexpr int H = Core::HEADS;
  if (a.mode == kModeBalanced) {
    auto kern = decode_balanced_kernel<Core, T, D, NW>;
    int nwg = 0;
    hipError_t e = balanced_grid(reinterpret_cast<const void*>(kern), NW * kWave, &nwg);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(nwg), dim3(NW * kWave), 0, st, a, bs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_balanced_kernel<T, D, H>), dim3((uint32_t)a.num_seqs * a.head_chunks),
                       dim3(256), 0, st, a, bs, nwg);
    return hipGetLastError();
  }
  const uint32_t units = (uint32_t)a.num_seqs * a.head_chunks * a.num_parts;
  hipLaunchKernelGGL((decode_unit_kernel<Core, T, D, NW>), dim3(units), dim3(NW * kWave), 0, st, a, bs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.split) return e;
  hipLaunchKernelGGL((decode_merge_parts_kernel<T, D>), dim3((uint32_t)a.num_seqs * a.num_q_heads),
                     dim3(kWave), 0, st, a, bs);
  return hipGetLastError();
}

template <class T, int D, int BS>
static hipError_t dispatch_bs(const DecodeArgs& a, int group, hipStream_t st) {
  constexpr int NW = kWavesPerUnit;
  if constexpr (!std::is_same<T, F32>::value) {
    switch (group) {
      case 2: return run_core<MfmaCore<T, D, BS, 2, NW>, T, D>(a, BS, st);
      case 4: return run_core<MfmaCore<T, D, BS, 4, NW>, T, D>(a, BS, st);
      case 8: return run_core<MfmaCore<T, D, BS, 8, NW>, T, D>(a, BS, st);
      case 16: return run_core<MfmaCore<T, D, BS, 16, NW>, T, D>(a, BS, st);
      default: break;   // group 1: VALU
    }
  }
  switch (a.num_q_heads / a.head_chunks) {
    case 1: return run_core<ValuCore<T, D, BS, 1, NW>, T, D>(a, BS, st);
    default: break;
  }
  if constexpr (std::is_same<T, F32>::value) {  // fp32 groups: 2 or 4 heads per unit
    switch (a.num_q_heads / a.head_chunks) {
      case 2: return run_core<ValuCore<T, D, BS, 2, NW>, T, D>(a, BS, st);
      case 4: return run_core<ValuCore<T, D, BS, 4, NW>, T, D>(a, BS, st);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

template <class T, int D>
static hipError_t dispatch_d(const DecodeArgs& a, int bs, int group, hipStream_t st) {
  switch (bs) {
    case 8: return dispatch_bs<T, D, 8>(a, group, st);
    case 16: return dispatch_bs<T, D, 16>(a, group, st);
    case 32: return dispatch_bs<T, D, 32>(a, group, st);
    default: return hipErrorInvalidValue;
  }
}

template <class T>
static hipError_t dispatch_t(const DecodeArgs& a, int head_dim, int bs, int group, hipStream_t st) {
  switch (head_dim) {
    case 64: return dispatch_d<T, 64>(a, bs, group, st);
    case 128: return dispatch_d<T, 128>(a, bs, group, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs& a, Elem elem, int head_dim, int block_size, int group,
                         hipStream_t st) {
  switch (elem) {
    case Elem::F32: return dispatch_t<F32>(a, head_dim, block_size, group, st);
    case Elem::F16: return dispatch_t<F16>(a, head_dim, block_size, group, st);
    case Elem::BF16: return dispatch_t<BF16>(a, head_dim, block_size, group, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
