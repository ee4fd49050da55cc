// Host-side KV block manager: physical block allocation, per-sequence block
// tables, reference-counted sharing with copy-on-write, release on finish
// (vLLM/PagedAttention paged-KV analysis page, sections 2.2, 2.3, 3.2, 3.3;
// vLLM entity page, "what it is"), and whole-request swap for preemption
// (Cross-Paper Synthesis page, section 3).
//
// Free blocks live in a three-level bitmap (bit set = free): level 0 has one
// bit per block, level 1 one bit per non-empty level-0 word, level 2 one bit
// per non-empty level-1 word.  Taking the lowest free block is three
// count-trailing-zeros steps after a scan of level 2 (16 words for 4M
// blocks); returning one sets three bits.  A batch of appends logs every
// change it makes and rolls them back if the pool runs dry or an output
// buffer fills, so a failed call leaves the manager as it was.
#include <climits>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pa_block_manager.h"

#define PA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

class FreeBitmap {
 public:
  void init(int32_t n) {
    n_ = n;
    const size_t w0 = ((size_t)n + 63) / 64, w1 = (w0 + 63) / 64, w2 = (w1 + 63) / 64;
    l0_.assign(w0, ~0ull);
    if (n % 64) l0_[w0 - 1] = (1ull << (n % 64)) - 1;
    l1_.assign(w1, 0);
    for (size_t i = 0; i < w0; ++i) l1_[i / 64] |= 1ull << (i % 64);
    l2_.assign(w2, 0);
    for (size_t i = 0; i < w1; ++i) l2_[i / 64] |= 1ull << (i % 64);
    count_ = n;
  }
  int32_t count() const { return count_; }
  bool is_free(int32_t b) const { return (l0_[b >> 6] >> (b & 63)) & 1; }

  // lowest free block, or -1
  int32_t take() {
    for (size_t k = 0; k < l2_.size(); ++k) {
      if (!l2_[k]) continue;
      const size_t i1 = k * 64 + __builtin_ctzll(l2_[k]);
      const size_t i0 = i1 * 64 + __builtin_ctzll(l1_[i1]);
      const int32_t b = (int32_t)(i0 * 64 + __builtin_ctzll(l0_[i0]));
      clear(b);
      return b;
    }
    return -1;
  }
  void clear(int32_t b) {
    const size_t i0 = (size_t)b >> 6;
    l0_[i0] &= ~(1ull << (b & 63));
    if (!l0_[i0]) {
      const size_t i1 = i0 >> 6;
      l1_[i1] &= ~(1ull << (i0 & 63));
      if (!l1_[i1]) l2_[i1 >> 6] &= ~(1ull << (i1 & 63));
    }
    --count_;
  }
  // Lowest aligned run of h free blocks (h a power of two); returns its
  // first block or -1.  A linear scan of the block bitmap: large pages are
  // taken once per prompt.
  int32_t find_run(int32_t h) const {
    if (h <= 64) {
      const uint64_t m = h == 64 ? ~0ull : ((1ull << h) - 1);
      for (size_t i = 0; i < l0_.size(); ++i) {
        const uint64_t w = l0_[i];
        if (!w) continue;
        for (int off = 0; off < 64; off += h)
          if (((w >> off) & m) == m && (int64_t)i * 64 + off + h <= n_) return (int32_t)(i * 64 + off);
      }
      return -1;
    }
    const size_t words = (size_t)h / 64;
    for (size_t i = 0; i + words <= l0_.size(); i += words) {
      size_t k = 0;
      while (k < words && l0_[i + k] == ~0ull) ++k;
      if (k == words && (int64_t)(i + words) * 64 <= n_) return (int32_t)(i * 64);
    }
    return -1;
  }
  void put(int32_t b) {
    const size_t i0 = (size_t)b >> 6, i1 = i0 >> 6;
    l0_[i0] |= 1ull << (b & 63);
    l1_[i1] |= 1ull << (i0 & 63);
    l2_[i1 >> 6] |= 1ull << (i1 & 63);
    ++count_;
  }

 private:
  int32_t n_ = 0, count_ = 0;
  std::vector<uint64_t> l0_, l1_, l2_;
};

struct Sequence {
  std::vector<int32_t> table;   // every block, large pages' blocks first
  int64_t len = 0;
  int32_t num_large = 0;        // large pages at the start of the table
  int32_t large_h = 0;          // their size in blocks
};

struct SwappedOut {
  int64_t len = 0;
  int32_t nblocks = 0;
};

// one reversible change made by an append batch
struct Undo {
  enum Kind : uint8_t { kTake, kRefDec, kTableSet, kTablePush, kLen } kind;
  int32_t block;      // kTake, kRefDec; old entry for kTableSet
  int32_t index;      // kTableSet
  Sequence* seq;      // kTableSet, kTablePush, kLen
  int64_t old_len;    // kLen
};

}  // namespace

struct pa_block_manager {
  int32_t num_blocks = 0, block_size = 0;
  int64_t next_id = 0;
  int64_t blocks_in_use = 0;
  std::vector<int32_t> ref;
  FreeBitmap free;
  std::unordered_map<int64_t, Sequence> seqs;        // resident
  std::unordered_map<int64_t, SwappedOut> swapped;   // preempted to host memory
  std::vector<Undo> log;   // reused by every append batch

  int32_t take() {
    const int32_t b = free.take();
    if (b >= 0) {
      ref[b] = 1;
      ++blocks_in_use;
    }
    return b;
  }
  void release_ref(int32_t b) {
    if (--ref[b] == 0) {
      free.put(b);
      --blocks_in_use;
    }
  }
  void rollback() {
    for (size_t i = log.size(); i-- > 0;) {
      const Undo& u = log[i];
      switch (u.kind) {
        case Undo::kTake:
          ref[u.block] = 0;
          free.put(u.block);
          --blocks_in_use;
          break;
        case Undo::kRefDec: ++ref[u.block]; break;
        case Undo::kTableSet: u.seq->table[u.index] = u.block; break;
        case Undo::kTablePush: u.seq->table.pop_back(); break;
        case Undo::kLen: u.seq->len = u.old_len; break;
      }
    }
    log.clear();
  }
};

PA_EXPORT pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager** out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (num_blocks < 1 || block_size < 1) return PA_ERR_SHAPE;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager;
  if (!bm) return PA_ERR_CAPACITY;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->ref.assign((size_t)num_blocks, 0);
    bm->free.init(num_blocks);
  } catch (...) {
    delete bm;
    return PA_ERR_CAPACITY;
  }
  *out = bm;
  return PA_OK;
}

PA_EXPORT void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

PA_EXPORT pa_status pa_bm_add_sequence(pa_block_manager* bm, int64_t* seq_id) {
  if (!bm || !seq_id) return PA_ERR_NULL;
  try {
    bm->seqs.emplace(bm->next_id, Sequence{});
  } catch (...) {
    return PA_ERR_CAPACITY;
  }
  *seq_id = bm->next_id++;
  return PA_OK;
}

PA_EXPORT pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t* child) {
  if (!bm || !child) return PA_ERR_NULL;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return PA_ERR_SEQUENCE;
  const Sequence* par = &it->second;   // element pointers survive a rehash
  try {
    Sequence copy = *par;
    bm->seqs.emplace(bm->next_id, std::move(copy));
  } catch (...) {
    return PA_ERR_CAPACITY;
  }
  for (int32_t b : par->table) ++bm->ref[b];
  *child = bm->next_id++;
  return PA_OK;
}

PA_EXPORT pa_status pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return PA_ERR_NULL;
  if (bm->swapped.erase(seq_id)) return PA_OK;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_SEQUENCE;
  for (int32_t b : it->second.table) bm->release_ref(b);
  bm->seqs.erase(it);
  return PA_OK;
}

PA_EXPORT pa_status pa_bm_append_slots(pa_block_manager* bm, const int64_t* seq_ids,
                                       const int32_t* num_new, int32_t num_seqs,
                                       int64_t* slot_mapping, int64_t slot_capacity,
                                       int32_t* block_mapping, int32_t pair_capacity,
                                       int32_t* num_pairs) {
  if (!bm || !num_pairs) return PA_ERR_NULL;
  if (num_seqs < 0 || slot_capacity < 0 || pair_capacity < 0) return PA_ERR_SHAPE;
  if (num_seqs > 0 && (!seq_ids || !num_new)) return PA_ERR_NULL;
  // validate everything that can be checked up front
  int64_t total = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (num_new[i] < 0) return PA_ERR_SHAPE;
    if (bm->seqs.find(seq_ids[i]) == bm->seqs.end()) return PA_ERR_SEQUENCE;
    total += num_new[i];
  }
  if (total > slot_capacity) return PA_ERR_CAPACITY;
  if (total > 0 && !slot_mapping) return PA_ERR_NULL;
  if (pair_capacity > 0 && !block_mapping) return PA_ERR_NULL;

  const int32_t bs = bm->block_size;
  bm->log.clear();
  try {   // at most one length entry per batch entry and three per token: no growth below
    bm->log.reserve((size_t)num_seqs + 3 * (size_t)total);
  } catch (...) {
    return PA_ERR_CAPACITY;
  }
  int64_t k = 0;
  int32_t pairs = 0;
  pa_status st = PA_OK;
  try {
    for (int32_t i = 0; i < num_seqs && st == PA_OK; ++i) {
      Sequence& s = bm->seqs.find(seq_ids[i])->second;
      if (num_new[i] > 0) bm->log.push_back({Undo::kLen, 0, 0, &s, s.len});
      for (int32_t n = 0; n < num_new[i]; ++n) {
        const int64_t p = s.len;
        const int64_t j = p / bs;
        const int32_t o = (int32_t)(p % bs);
        if (o == 0) {
          const int32_t b = bm->take();
          if (b < 0) { st = PA_ERR_NO_BLOCKS; break; }
          bm->log.push_back({Undo::kTake, b, 0, nullptr, 0});
          s.table.push_back(b);
          bm->log.push_back({Undo::kTablePush, 0, 0, &s, 0});
        } else if (bm->ref[s.table[j]] > 1) {
          const int32_t old = s.table[j];
          if (pairs >= pair_capacity) { st = PA_ERR_CAPACITY; break; }
          const int32_t fresh = bm->take();
          if (fresh < 0) { st = PA_ERR_NO_BLOCKS; break; }
          bm->log.push_back({Undo::kTake, fresh, 0, nullptr, 0});
          --bm->ref[old];   // still >= 1: another table holds it
          bm->log.push_back({Undo::kRefDec, old, 0, nullptr, 0});
          s.table[j] = fresh;
          bm->log.push_back({Undo::kTableSet, old, (int32_t)j, &s, 0});
          block_mapping[2 * pairs] = old;
          block_mapping[2 * pairs + 1] = fresh;
          ++pairs;
        }
        slot_mapping[k++] = (int64_t)s.table[j] * bs + o;
        s.len = p + 1;
      }
    }
  } catch (...) {   // a table could not grow; its block is logged, the push is not
    st = PA_ERR_CAPACITY;
  }
  if (st != PA_OK) {
    bm->rollback();
    return st;
  }
  bm->log.clear();
  *num_pairs = pairs;
  return PA_OK;
}

PA_EXPORT pa_status pa_bm_append_prompt_large(pa_block_manager* bm, int64_t seq_id, int32_t num_tokens,
                                              int32_t pages_per_large, int64_t* slot_mapping,
                                              int64_t slot_capacity) {
  if (!bm) return PA_ERR_NULL;
  if (num_tokens < 0 || pages_per_large < 1 || pages_per_large > 1024 ||
      (pages_per_large & (pages_per_large - 1)) != 0)
    return PA_ERR_SHAPE;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_SEQUENCE;
  Sequence& s = it->second;
  if (s.len != 0 || !s.table.empty()) return PA_ERR_SHAPE;
  if (slot_capacity < num_tokens) return PA_ERR_CAPACITY;
  if (num_tokens > 0 && !slot_mapping) return PA_ERR_NULL;
  const int32_t H = pages_per_large, bs = bm->block_size;
  const int64_t page_tokens = (int64_t)H * bs;
  const int32_t nl = (int32_t)(num_tokens / page_tokens);
  try {
    bm->log.clear();
    bm->log.reserve(1 + (size_t)nl * H * 2);
    s.table.reserve((size_t)nl * H + (size_t)((num_tokens - nl * page_tokens + bs - 1) / bs));
  } catch (...) {
    return PA_ERR_CAPACITY;
  }
  bm->log.push_back({Undo::kLen, 0, 0, &s, s.len});
  for (int32_t k = 0; k < nl; ++k) {
    const int32_t first = bm->free.find_run(H);
    if (first < 0) {
      bm->rollback();
      return PA_ERR_NO_BLOCKS;
    }
    for (int32_t i = 0; i < H; ++i) {
      bm->free.clear(first + i);
      bm->ref[first + i] = 1;
      ++bm->blocks_in_use;
      bm->log.push_back({Undo::kTake, first + i, 0, nullptr, 0});
      s.table.push_back(first + i);
      bm->log.push_back({Undo::kTablePush, 0, 0, &s, 0});
    }
  }
  for (int64_t t = 0; t < (int64_t)nl * page_tokens; ++t)
    slot_mapping[t] = (int64_t)s.table[t / bs] * bs + t % bs;
  s.len = (int64_t)nl * page_tokens;
  // the rest goes where an append puts it; that call rolls back its own part
  const int64_t sid = seq_id;
  const int32_t rest = (int32_t)(num_tokens - s.len);
  int32_t pairs = 0;
  std::vector<Undo> mine;
  mine.swap(bm->log);
  const pa_status st = pa_bm_append_slots(bm, &sid, &rest, 1, slot_mapping + s.len, slot_capacity - s.len,
                                          nullptr, 0, &pairs);
  mine.swap(bm->log);
  if (st != PA_OK) {
    bm->rollback();
    return st;
  }
  bm->log.clear();
  s.num_large = nl;
  s.large_h = nl > 0 ? H : 0;
  return PA_OK;
}

PA_EXPORT pa_status pa_bm_block_tables_hier(const pa_block_manager* bm, const int64_t* seq_ids,
                                            int32_t num_seqs, int32_t pages_per_large,
                                            int32_t max_large_per_seq, int32_t max_small_per_seq,
                                            int32_t* large_tables, int32_t* num_large, int32_t* small_tables,
                                            int32_t* context_lens) {
  if (!bm) return PA_ERR_NULL;
  if (num_seqs < 0 || max_large_per_seq < 0 || max_small_per_seq < 0 || pages_per_large < 1) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!seq_ids || !num_large || !small_tables || !context_lens || (max_large_per_seq > 0 && !large_tables))
    return PA_ERR_NULL;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return PA_ERR_SEQUENCE;
    const Sequence& s = it->second;
    const int32_t nl = s.large_h == pages_per_large ? s.num_large : 0;
    if (nl > max_large_per_seq || (int64_t)s.table.size() - (int64_t)nl * pages_per_large > max_small_per_seq ||
        s.len > INT32_MAX)
      return PA_ERR_CAPACITY;
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Sequence& s = bm->seqs.find(seq_ids[i])->second;
    const int32_t nl = s.large_h == pages_per_large ? s.num_large : 0;
    int32_t* lrow = large_tables + (size_t)i * max_large_per_seq;
    for (int32_t k = 0; k < max_large_per_seq; ++k)
      lrow[k] = k < nl ? s.table[(size_t)k * pages_per_large] / pages_per_large : -1;
    int32_t* srow = small_tables + (size_t)i * max_small_per_seq;
    const size_t off = (size_t)nl * pages_per_large, n = s.table.size() - off;
    for (size_t j = 0; j < (size_t)max_small_per_seq; ++j) srow[j] = j < n ? s.table[off + j] : -1;
    num_large[i] = nl;
    context_lens[i] = (int32_t)s.len;
  }
  return PA_OK;
}

PA_EXPORT pa_status pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids,
                                       int32_t num_seqs, int32_t max_blocks_per_seq,
                                       int32_t* block_tables, int32_t* context_lens) {
  if (!bm) return PA_ERR_NULL;
  if (num_seqs < 0 || max_blocks_per_seq < 0) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!seq_ids || !block_tables || !context_lens) return PA_ERR_NULL;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return PA_ERR_SEQUENCE;
    if ((int64_t)it->second.table.size() > max_blocks_per_seq || it->second.len > INT32_MAX)
      return PA_ERR_CAPACITY;
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Sequence& s = bm->seqs.find(seq_ids[i])->second;
    int32_t* row = block_tables + (size_t)i * max_blocks_per_seq;
    const size_t n = s.table.size();
    if (n) std::memcpy(row, s.table.data(), n * sizeof(int32_t));
    for (size_t j = n; j < (size_t)max_blocks_per_seq; ++j) row[j] = -1;
    context_lens[i] = (int32_t)s.len;
  }
  return PA_OK;
}

PA_EXPORT pa_status pa_bm_swap_out(pa_block_manager* bm, int64_t seq_id, int32_t* block_ids,
                                   int32_t capacity, int32_t* num_ids) {
  if (!bm || !num_ids) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_SEQUENCE;
  const std::vector<int32_t>& table = it->second.table;
  const size_t n = table.size();
  if (n > (size_t)(capacity < 0 ? 0 : capacity)) return PA_ERR_CAPACITY;
  if (n && !block_ids) return PA_ERR_NULL;
  try {
    bm->swapped.emplace(seq_id, SwappedOut{it->second.len, (int32_t)n});
  } catch (...) {
    return PA_ERR_CAPACITY;
  }
  if (n) std::memcpy(block_ids, table.data(), n * sizeof(int32_t));
  for (int32_t b : table) bm->release_ref(b);
  bm->seqs.erase(it);
  *num_ids = (int32_t)n;
  return PA_OK;
}

PA_EXPORT pa_status pa_bm_swap_in(pa_block_manager* bm, int64_t seq_id, int32_t* block_ids,
                                  int32_t capacity, int32_t* num_ids) {
  if (!bm || !num_ids) return PA_ERR_NULL;
  auto it = bm->swapped.find(seq_id);
  if (it == bm->swapped.end()) return PA_ERR_SEQUENCE;
  const int32_t n = it->second.nblocks;
  if (n > capacity) return PA_ERR_CAPACITY;
  if (n && !block_ids) return PA_ERR_NULL;
  if (bm->free.count() < n) return PA_ERR_NO_BLOCKS;
  Sequence s;
  try {
    s.table.reserve((size_t)n);
    bm->seqs.reserve(bm->seqs.size() + 1);
  } catch (...) {
    return PA_ERR_CAPACITY;
  }
  s.len = it->second.len;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = bm->take();   // cannot fail: n blocks are free
    s.table.push_back(b);
    block_ids[i] = b;
  }
  bm->seqs.emplace(seq_id, std::move(s));   // no rehash: reserved above
  bm->swapped.erase(it);
  *num_ids = n;
  return PA_OK;
}

PA_EXPORT int32_t pa_bm_num_free_blocks(const pa_block_manager* bm) {
  return bm ? bm->free.count() : -1;
}

PA_EXPORT pa_status pa_bm_sequence_length(const pa_block_manager* bm, int64_t seq_id, int64_t* length) {
  if (!bm || !length) return PA_ERR_NULL;
  auto sw = bm->swapped.find(seq_id);
  if (sw != bm->swapped.end()) {
    *length = sw->second.len;
    return PA_OK;
  }
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_SEQUENCE;
  *length = it->second.len;
  return PA_OK;
}

PA_EXPORT pa_status pa_bm_utilisation(const pa_block_manager* bm, int64_t* tokens, int64_t* slots) {
  if (!bm || !tokens || !slots) return PA_ERR_NULL;
  int64_t t = 0;
  for (const auto& kv : bm->seqs) t += kv.second.len;
  *tokens = t;
  *slots = bm->blocks_in_use * bm->block_size;
  return PA_OK;
}

PA_EXPORT pa_status pa_bm_refcounts(const pa_block_manager* bm, int32_t* refcounts, int32_t count) {
  if (!bm || !refcounts) return PA_ERR_NULL;
  if (count != bm->num_blocks) return PA_ERR_SHAPE;
  std::memcpy(refcounts, bm->ref.data(), (size_t)count * sizeof(int32_t));
  return PA_OK;
}
