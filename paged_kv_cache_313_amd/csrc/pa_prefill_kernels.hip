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
// Work unit: one workgroup of 4 waves per (sequence, KV head, block of query
// tokens).  The 64 query rows of a workgroup are (token, head) pairs of the G
// heads sharing the KV head, heads fastest: each wave owns 16 of them.  Keys
// advance 32 at a time through double-buffered LDS tiles: K row-major, V
// transposed (d-major), both gathered through the block table by all 256
// threads, the next tile's loads in flight while the current one is used.
//
// Per 32-key tile, each wave computes
//   S^T[key][row] = K Q^T          (A = K from LDS, B = its query rows, kept
//                                   in registers for the whole unit)
// so that lane l holds the scores of query row l % 16 for keys
// 4 (l / 16) + {0..3} and 16 + 4 (l / 16) + {0..3}: exactly the 8 k-values
// that lane supplies as the B operand of
//   O^T[d][row] += V^T P^T          (A = V^T from LDS)
// once k-slot 8 (l / 16) + j is taken to mean those keys (the contraction
// order is free as long as A and B agree).  The probabilities never leave the
// lane, and a query row's statistics are shared by the 4 lanes l % 16 = row:
// two butterflies reduce a max or a sum.  Online softmax in the log2 domain
// with a lazy rescale (a row's reference max moves only when a score exceeds
// it by more than 2^8), P rounded to the input type for the MFMA, fp32
// accumulation.
#include "pa_common.hpp"
#include "pa_launch.hpp"

namespace pa {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfRows = kPfWaves * 16;   // query rows (token, head) per workgroup
constexpr int kPfKeys = 32;              // keys per tile
constexpr float kPfLazy = 8.f;

template <int D>
struct PfLayout {
  static constexpr int kRowB = D * 2 + 16;           // K row pitch in LDS (bytes), padded
  static constexpr int kVtB = kPfKeys * 2 + 8;       // V^T row pitch in LDS (bytes), padded
  static constexpr int kKBytes = kPfKeys * kRowB;
  static constexpr int kBufBytes = kKBytes + D * kVtB;
  static constexpr int CPR = D / 8;                  // 16-byte chunks per token row
  static constexpr int NCH = kPfKeys * CPR / kPfThreads;   // chunks per thread per tile
  static_assert(NCH * kPfThreads == kPfKeys * CPR, "tile split");
};

template <class T, int D, int G>
__global__ __launch_bounds__(kPfThreads) void prefill_kernel(PrefillArgs a, int block_size, int bs_shift) {
  using Lay = PfLayout<D>;
  constexpr int QB = kPfRows / G;          // query tokens per workgroup
  constexpr int TPW = 16 / G;              // query tokens per wave
  constexpr int NKC = D / 32;              // k-chunks of the score MFMA
  constexpr int NDT = D / 16;              // 16-row d tiles of the output
  __shared__ __align__(16) char lds[2 * Lay::kBufBytes];

  // unit: (sequence, KV head, query block), query block fastest, dealt to
  // XCDs in runs so that one sequence's blocks share an L2
  const uint32_t u = xcd_unit(blockIdx.x, gridDim.x);
  const int qb = (int)(u % (uint32_t)a.qblocks);
  const int sg = (int)(u / (uint32_t)a.qblocks);
  const int g = sg % a.num_kv_heads;
  const int s = sg / a.num_kv_heads;
  if (s >= a.num_seqs) return;
  // memory safety on inconsistent inputs: rows outside [0, num_tokens), more
  // new tokens than the context holds, or a query block past the sequence's
  // new tokens leave the unit idle (and those rows unwritten)
  const int q0 = a.query_start[s];
  const int n = a.query_start[s + 1] - q0;
  const int L = min(a.context_lens[s], a.max_blocks_per_seq * block_size);
  if (q0 < 0 || n <= 0 || n > a.num_tokens - q0 || qb * QB >= n || n > L) return;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int c = lane & 15, gq = lane >> 4;

  // this lane's query row (column c of the wave's MFMA tiles)
  const int tq = qb * QB + wave * TPW + c / G;      // token index among the n new ones
  const int hh = c % G;
  const bool row_ok = tq < n;
  const int pos = L - n + (row_ok ? tq : n - 1);
  const int wave_last = L - n + min(qb * QB + (wave + 1) * TPW, n) - 1;   // wave's largest position
  const int kend = L - n + min(qb * QB + QB, n);                          // keys the unit needs

  u32x4 qop[NKC];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const char* qrow = reinterpret_cast<const char*>(a.query) +
                       (((size_t)(q0 + (row_ok ? tq : 0)) * a.num_q_heads + (size_t)g * G + hh) * D) * 2;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) qop[kc] = row_ok ? ld16(qrow + (32 * kc + 8 * gq) * 2) : z;
  }

  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const char* kpool = reinterpret_cast<const char*>(a.k_pool);
  const char* vpool = reinterpret_cast<const char*>(a.v_pool);
  const int bmask = block_size - 1;

  u32x4 kreg[Lay::NCH], vreg[Lay::NCH];
  bool vok[Lay::NCH];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int j = 0; j < Lay::NCH; ++j) {
      const int ch = j * kPfThreads + tid;
      const int key = ch / Lay::CPR, dch = ch % Lay::CPR;
      const int t = t0 + key;
      const int tt = min(t, L - 1);
      int blk = trow[tt >> bs_shift];
      blk = ((unsigned)blk < (unsigned)a.num_blocks) ? blk : 0;
      const size_t off = ((((size_t)blk * a.num_kv_heads + g) * block_size + (tt & bmask)) * D + dch * 8) * 2;
      kreg[j] = ld16(kpool + off);
      vreg[j] = ld16(vpool + off);
      vok[j] = t < L;
    }
  };
  auto store_tile = [&](int buf) {
    char* kb = lds + buf * Lay::kBufBytes;
    char* vb = kb + Lay::kKBytes;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < Lay::NCH; ++j) {
      const int ch = j * kPfThreads + tid;
      const int key = ch / Lay::CPR, dch = ch % Lay::CPR;
      *reinterpret_cast<u32x4*>(kb + key * Lay::kRowB + dch * 16) = kreg[j];
      const u32x4 v = vok[j] ? vreg[j] : z;      // slots past the context may hold anything
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t x = (uint16_t)(v[e >> 1] >> ((e & 1) * 16));
        *reinterpret_cast<uint16_t*>(vb + (dch * 8 + e) * Lay::kVtB + key * 2) = x;
      }
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x4 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = (kend + kPfKeys - 1) / kPfKeys;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int t0 = it * kPfKeys;
    if (it + 1 < ntiles) load_tile(t0 + kPfKeys);
    if (t0 <= wave_last) {   // wave-uniform: some row of this wave sees a key of the tile
      const char* kb = lds + (it & 1) * Lay::kBufBytes;
      const char* vb = kb + Lay::kKBytes;
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(kb + c * Lay::kRowB + (32 * kc + 8 * gq) * 2);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(kb + (16 + c) * Lay::kRowB + (32 * kc + 8 * gq) * 2);
        s0 = mfma_16x16x32<T>(a0, qop[kc], s0);
        s1 = mfma_16x16x32<T>(a1, qop[kc], s1);
      }
      float sc[8];
      const int kt = t0 + 4 * gq;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[i] = (kt + i <= pos) ? s0[i] * a.scale_log2 : kNegInf;
        sc[4 + i] = (kt + 16 + i <= pos) ? s1[i] * a.scale_log2 : kNegInf;
      }
      float tmax = sc[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, sc[i]);
      tmax = fmaxf(tmax, xor_lane<16>(tmax));
      tmax = fmaxf(tmax, xor_lane<32>(tmax));
      const bool grow = tmax > m_run + kPfLazy;    // always true on a row's first key
      if (__any(grow)) {
        const float m_new = grow ? tmax : m_run;
        const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
      }
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = sc[i] == kNegInf ? 0.f : fast_exp2(sc[i] - m_run);
        l_run += p[i];
      }
      u32x4 pb;
      pb[0] = pack2<T>(p[0], p[1]);
      pb[1] = pack2<T>(p[2], p[3]);
      pb[2] = pack2<T>(p[4], p[5]);
      pb[3] = pack2<T>(p[6], p[7]);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const char* vrow = vb + (16 * dt + c) * Lay::kVtB;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + (4 * gq) * 2);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (16 + 4 * gq) * 2);
        const u32x4 av = {lo.x, lo.y, hi.x, hi.y};
        oacc[dt] = mfma_16x16x32<T>(av, pb, oacc[dt]);
      }
    }
    if (it + 1 < ntiles) store_tile((it + 1) & 1);   // the other buffer: free since the last barrier
    __syncthreads();
  }

  l_run += xor_lane<16>(l_run);
  l_run += xor_lane<32>(l_run);
  if (!row_ok) return;
  const float inv = 1.f / l_run;
  char* orow = reinterpret_cast<char*>(a.out) +
               (((size_t)(q0 + tq) * a.num_q_heads + (size_t)g * G + hh) * D) * 2;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    uint2 w;
    w.x = pack2<T>(oacc[dt][0] * inv, oacc[dt][1] * inv);
    w.y = pack2<T>(oacc[dt][2] * inv, oacc[dt][3] * inv);
    *reinterpret_cast<uint2*>(orow + (16 * dt + 4 * gq) * 2) = w;
  }
}

template <class T, int D>
static hipError_t prefill_group(const PrefillArgs& a, int bs, int group, hipStream_t st) {
  int shift = 0;
  while ((1 << shift) < bs) ++shift;
  const int QB = kPfRows / group;
  PrefillArgs args = a;
  args.qblocks = (a.max_query_len + QB - 1) / QB;
  const uint64_t units = (uint64_t)a.num_seqs * a.num_kv_heads * args.qblocks;
  if (units == 0) return hipSuccess;
  if (units > 0x7fffffffull) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)units), block(kPfThreads);
  switch (group) {
    case 1: hipLaunchKernelGGL((prefill_kernel<T, D, 1>), grid, block, 0, st, args, bs, shift); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<T, D, 2>), grid, block, 0, st, args, bs, shift); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<T, D, 4>), grid, block, 0, st, args, bs, shift); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<T, D, 8>), grid, block, 0, st, args, bs, shift); break;
    case 16: hipLaunchKernelGGL((prefill_kernel<T, D, 16>), grid, block, 0, st, args, bs, shift); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

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
