// Decode attention over a paged KV cache (gfx950, wave64).
//
// One query token per sequence attends over the sequence's context, whose K/V
// rows sit in fixed-size physical blocks reached through the sequence's block
// table (vLLM/PagedAttention paged-KV analysis page, section 3.1: the kernel is
// changed to read non-contiguous blocks, the simplified sketch walks the table
// block by block and loads K and V of each physical page).  The sketch
// normalises per block; the operation reached here is one softmax over the
// whole context, evaluated as an online softmax: a running max m, a running
// sum l and an un-normalised accumulator are rescaled by exp(m_old - m_new)
// whenever the max grows.  Scores are kept in the log2 domain
// (scale * log2(e) folded in) so every exponential is one v_exp_f32.
//
// Work unit = (sequence, KV head or q-head chunk, context partition).  A
// workgroup of NW waves takes one unit; its waves take interleaved 16-token
// tiles, so one wave-wide load instruction moves whole 64-byte row segments of
// 16 different tokens.  The unit's block-table slice is staged in LDS first,
// which takes the table->block dependent load off the per-tile path.  At the
// end the waves merge through LDS.  A partition that is the whole sequence
// writes the output directly; otherwise it writes (m, l, acc) to the workspace
// and decode_merge_kernel applies the log-sum-exp rescale across partitions.
#include <type_traits>

#include "pa_common.hpp"
#include "pa_launch.hpp"

namespace pa {

constexpr int kTile = 16;      // tokens per tile
constexpr int kTblWin = 256;   // block-table entries staged in LDS at a time

// Unit index -> (sequence, head chunk, partition); sequence is the fastest index.
struct Unit {
  int s, c, p;
};
__device__ __forceinline__ Unit unit_of(uint32_t u, int S, int C) {
  Unit r;
  r.s = (int)(u % (uint32_t)S);
  const uint32_t rest = u / (uint32_t)S;
  r.c = (int)(rest % (uint32_t)C);
  r.p = (int)(rest / (uint32_t)C);
  return r;
}

template <int NW>
__device__ __forceinline__ void stage_table(int32_t* s_tbl, const int32_t* row, int first, int count,
                                            int num_blocks) {
  for (int i = threadIdx.x; i < count; i += NW * kWave) {
    const int e = row[first + i];
    s_tbl[i] = ((unsigned)e < (unsigned)num_blocks) ? e : 0;  // memory-safe clamp
  }
}

// Merge the NW waves' (m, l, acc) held in LDS and write the unit's result.
template <class T, int D, int H, int NW>
__device__ __forceinline__ void merge_waves_and_store(const DecodeArgs& a, const float (*s_m)[H],
                                                      const float (*s_l)[H],
                                                      const float (*s_acc)[H][D], int s, int h0,
                                                      int p, bool direct) {
  for (int idx = threadIdx.x; idx < H * D; idx += NW * kWave) {
    const int hh = idx / D, d = idx - (idx / D) * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][hh]);
    float lt = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(s_m[w][hh] - M);
      lt += f * s_l[w][hh];
      o += f * s_acc[w][hh][d];
    }
    const size_t row = (size_t)s * a.num_q_heads + h0 + hh;
    if (direct) {
      store_elem<T>(a.out, row * D + d, o / lt);
    } else {
      const size_t pr = row * a.num_parts + p;
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
// VALU kernel: any dtype, H q heads (1, 2 or 4) of one KV head per unit.
// Lane layout per tile: token tt = lane / 4, quarter qp = lane % 4; the lane
// holds the row bytes [16 (4 j + qp), +16) for j < NL, i.e. D/4 elements.
// ============================================================================
template <class T, int D, int BS, int H, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_valu_kernel(DecodeArgs a) {
  constexpr int EB = T::bytes;
  constexpr int ROWB = D * EB;
  constexpr int NL = ROWB / 64;            // 16-byte loads per lane per token row
  constexpr int NE = 16 / EB;              // elements per 16 bytes
  constexpr int DPL = NL * NE;             // elements per lane (= D / 4)
  static_assert(DPL * 4 == D, "layout");
  static_assert(kTblWin * BS % kTile == 0, "window");

  __shared__ int32_t s_tbl[kTblWin];
  __shared__ float s_m[NW][H], s_l[NW][H];
  __shared__ float s_acc[NW][H][D];

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int S = a.num_seqs;
  const Unit un = unit_of(xcd_unit(blockIdx.x, gridDim.x), S, a.head_chunks);
  const int s = un.s, p = un.p, h0 = un.c * H;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int g = h0 / G;
  const int L = clamp_len(a, s, BS);
  const int P = a.partition_size;
  const int t0 = p * P;
  if (L == 0) {
    if (p == 0) store_zero_rows<T, D, H, NW>(a, s, h0);
    return;
  }
  if (t0 >= L) return;
  const int t1 = min(t0 + P, L);
  const bool direct = !a.split || L <= P;

  const int tt = lane >> 2, qp = lane & 3;

  // query rows in fp32, the lane's D/4 elements of each of the H heads
  float qf[H][DPL];
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

  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (size_t)g * BS * ROWB + qp * 16;
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (size_t)g * BS * ROWB + qp * 16;
  const size_t blk_stride = (size_t)a.num_kv_heads * BS * ROWB;
  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks_per_seq;

  for (int wb = t0; wb < t1; wb += kTblWin * BS) {
    const int we = min(wb + kTblWin * BS, t1);
    __syncthreads();
    stage_table<NW>(s_tbl, trow, wb / BS, (we - wb + BS - 1) / BS, a.num_blocks);
    __syncthreads();
    const int ntiles = (we - wb + kTile - 1) / kTile;
    for (int ti = wave; ti < ntiles; ti += NW) {
      const int pos = wb + ti * kTile + tt;
      const bool valid = pos < we;
      const int rel = valid ? pos - wb : 0;
      const size_t phys = (size_t)s_tbl[rel / BS];
      const size_t roff = phys * blk_stride + (size_t)(rel % BS) * ROWB;
      u32x4 kr[NL], vr[NL];
#pragma unroll
      for (int j = 0; j < NL; ++j) kr[j] = ld16(kbase + roff + j * 64);
#pragma unroll
      for (int j = 0; j < NL; ++j) vr[j] = ld16(vbase + roff + j * 64);

      float kf[DPL];
#pragma unroll
      for (int j = 0; j < NL; ++j) Unpack<T>::run(kr[j], &kf[j * NE]);
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
      for (int j = 0; j < NL; ++j) Unpack<T>::run(vr[j], &vf[j * NE]);
#pragma unroll
      for (int i = 0; i < DPL; ++i) vf[i] = valid ? vf[i] : 0.f;  // tail slots may hold NaN
#pragma unroll
      for (int hh = 0; hh < H; ++hh)
#pragma unroll
        for (int i = 0; i < DPL; ++i) acc[hh][i] = fmaf(pr[hh], vf[i], acc[hh][i]);
    }
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
        for (int e = 0; e < NE; ++e) s_acc[wave][hh][(4 * j + qp) * NE + e] = acc[hh][j * NE + e];
    if (lane == 0) {
#pragma unroll
      for (int hh = 0; hh < H; ++hh) {
        s_m[wave][hh] = m_run[hh];
        s_l[wave][hh] = l_run[hh];
      }
    }
  }
  __syncthreads();
  merge_waves_and_store<T, D, H, NW>(a, s_m, s_l, s_acc, s, h0, p, direct);
}

// ============================================================================
// MFMA kernel for grouped queries (f16/bf16, G = Hq/Hkv in {2, 4, 8, 16}).
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

template <class T, int D, int BS, int G, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int ROWB = D * 2;
  constexpr int NQK = D / 32;   // MFMAs per tile (k = 32 per MFMA)
  constexpr int CPR = D / 8;    // 16-byte chunks per token row
  constexpr int NVI = D / 32;   // V chunks per lane per tile (16 * CPR / 64)
  static_assert(16 % G == 0 && G >= 2, "group");
  static_assert(kTblWin * BS % kTile == 0, "window");

  __shared__ int32_t s_tbl[kTblWin];
  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ float s_acc[NW][G][D];

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int gr = lane >> 4, w = lane & 15;
  const int S = a.num_seqs;
  const Unit un = unit_of(xcd_unit(blockIdx.x, gridDim.x), S, a.num_kv_heads);
  const int s = un.s, g = un.c, p = un.p;
  const int h0 = g * G;
  const int L = clamp_len(a, s, BS);
  const int P = a.partition_size;
  const int t0 = p * P;
  if (L == 0) {
    if (p == 0) store_zero_rows<T, D, G, NW>(a, s, h0);
    return;
  }
  if (t0 >= L) return;
  const int t1 = min(t0 + P, L);
  const bool direct = !a.split || L <= P;

  // B operand: query row of head w % G, chunk 4 i + gr
  u32x4 qop[NQK];
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

  for (int wb = t0; wb < t1; wb += kTblWin * BS) {
    const int we = min(wb + kTblWin * BS, t1);
    __syncthreads();
    stage_table<NW>(s_tbl, trow, wb / BS, (we - wb + BS - 1) / BS, a.num_blocks);
    __syncthreads();
    const int ntiles = (we - wb + kTile - 1) / kTile;
    for (int ti = wave; ti < ntiles; ti += NW) {
      const int ts = wb + ti * kTile;
      // ---- K: token w of the tile, chunks 4 i + gr
      u32x4 kop[NQK];
      {
        const int pos = ts + w;
        const int rel = pos < we ? pos - wb : 0;
        const size_t off = (size_t)s_tbl[rel / BS] * blk_stride + (size_t)(rel % BS) * ROWB;
#pragma unroll
        for (int i = 0; i < NQK; ++i) kop[i] = ld16(kbase + off + (4 * i + gr) * 16);
      }
      // ---- V: chunk (w + 16 j) % CPR of token 4 gr + (w + 16 j) / CPR
      u32x4 vop[NVI];
#pragma unroll
      for (int j = 0; j < NVI; ++j) {
        const int idx = w + 16 * j;
        const int pos = ts + 4 * gr + idx / CPR;
        const int rel = pos < we ? pos - wb : 0;
        const size_t off = (size_t)s_tbl[rel / BS] * blk_stride + (size_t)(rel % BS) * ROWB;
        vop[j] = ld16(vbase + off + (idx % CPR) * 16);
      }

      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NQK; ++i) sacc = mfma_16x16x32<T>(kop[i], qop[i], sacc);

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
        Unpack<T>::run(vop[j], vf);
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
    }
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
      for (int e = 0; e < 8; ++e) s_acc[wave][h][8 * w + e] = acc[h][e];
  }
  if (lane < G) {
    s_m[wave][lane] = m_run;
    s_l[wave][lane] = l_run;
  }
  __syncthreads();
  merge_waves_and_store<T, D, G, NW>(a, s_m, s_l, s_acc, s, h0, p, direct);
}

// ============================================================================
// Merge of the partitions of one (sequence, q head): M = max_p m_p,
// w_p = 2^(m_p - M), out = sum_p w_p o_p / sum_p w_p l_p (o_p un-normalised).
// ============================================================================
template <class T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a, int block_size) {
  const int row = blockIdx.x;               // s * Hq + h
  const int s = row / a.num_q_heads;
  const int d = threadIdx.x;
  const int L = clamp_len(a, s, block_size);
  const int P = a.partition_size;
  const int np = (L + P - 1) / P;
  if (np <= 1) return;                      // written directly by the partition pass
  const size_t base = (size_t)row * a.num_parts;
  float M = kNegInf;
  for (int p = 0; p < np; ++p) M = fmaxf(M, a.ws_m[base + p]);
  float num = 0.f, den = 0.f;
  for (int p = 0; p < np; ++p) {
    const float f = fast_exp2(a.ws_m[base + p] - M);
    den = fmaf(f, a.ws_l[base + p], den);
    num = fmaf(f, a.ws_o[(base + p) * D + d], num);
  }
  store_elem<T>(a.out, (size_t)row * D + d, num / den);
}

// ============================================================================
// dispatch
// ============================================================================
constexpr int kWavesPerUnit = 4;

template <class T, int D, int BS, int H>
static hipError_t run_valu(const DecodeArgs& a, hipStream_t st) {
  const uint32_t units = (uint32_t)a.num_seqs * a.head_chunks * a.num_parts;
  hipLaunchKernelGGL((decode_valu_kernel<T, D, BS, H, kWavesPerUnit>), dim3(units),
                     dim3(kWavesPerUnit * kWave), 0, st, a);
  return hipGetLastError();
}

template <class T, int D, int BS, int G>
static hipError_t run_mfma(const DecodeArgs& a, hipStream_t st) {
  const uint32_t units = (uint32_t)a.num_seqs * a.num_kv_heads * a.num_parts;
  hipLaunchKernelGGL((decode_mfma_kernel<T, D, BS, G, kWavesPerUnit>), dim3(units),
                     dim3(kWavesPerUnit * kWave), 0, st, a);
  return hipGetLastError();
}

template <class T, int D, int BS>
static hipError_t dispatch_bs(const DecodeArgs& a, int group, hipStream_t st) {
  constexpr bool mfma_ok = !std::is_same<T, F32>::value;
  if (mfma_ok && group >= 2) {
    if constexpr (mfma_ok) {
      switch (group) {
        case 2: return run_mfma<T, D, BS, 2>(a, st);
        case 4: return run_mfma<T, D, BS, 4>(a, st);
        case 8: return run_mfma<T, D, BS, 8>(a, st);
        case 16: return run_mfma<T, D, BS, 16>(a, st);
        default: return hipErrorInvalidValue;
      }
    }
  }
  const int H = a.num_q_heads / a.head_chunks;
  switch (H) {
    case 1: return run_valu<T, D, BS, 1>(a, st);
    case 2: return run_valu<T, D, BS, 2>(a, st);
    case 4: return run_valu<T, D, BS, 4>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <class T, int D>
static hipError_t dispatch_d(const DecodeArgs& a, int bs, int group, hipStream_t st) {
  hipError_t e;
  switch (bs) {
    case 8: e = dispatch_bs<T, D, 8>(a, group, st); break;
    case 16: e = dispatch_bs<T, D, 16>(a, group, st); break;
    case 32: e = dispatch_bs<T, D, 32>(a, group, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || !a.split) return e;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((uint32_t)a.num_seqs * a.num_q_heads), dim3(D),
                     0, st, a, bs);
  return hipGetLastError();
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
