"""CPU oracle for the paged-KV decode path (fp64, NumPy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or dtype converters); the only
thing both sides read is the seeded input arrays from ``workloads``.

What it computes, and where the pages define it:

* KV append -- a newly generated token's K and V are written into the slot of
  its sequence's current block (paged-KV analysis page, section 3.2, the
  copy-on-write paragraph on generating a token; vLLM entity page, "what it
  is": blocks are taken on demand).  Slot = physical_block * block_size +
  offset.  Plain byte copy.
* Block copy -- copy-on-write: before a sequence writes into a block that other
  sequences still reference, the block is duplicated (paged-KV analysis page,
  sections 2.3 and 3.2; Cross-Paper Synthesis page, section 2).  Plain byte
  copy of every head and slot of the block, from the pre-call state.
* Decode attention -- one query token per sequence attends over the
  sequence's context, whose K/V sit in fixed-size physical blocks reached
  through the sequence's block table (paged-KV analysis page, section 3.1,
  the simplified attention sketch, and section 2.2).  That sketch normalises
  per block and has no scale and no tail mask; it is marked as simplified,
  and the method reaches ordinary attention over the whole context, so the
  oracle is that definition written out: gather the first L tokens in logical
  order, s_t = scale * <q, k_t>, w_t = exp(s_t - max s) / sum, out = sum w_t v_t.
  Query head h reads KV head h // (Hq / Hkv) (consecutive grouping; the pages
  name grouped-query attention only as an orthogonal model change, Cross-Paper
  Synthesis page, section 2).
* Partitioned decode -- the same attention evaluated per 512-token slice and
  merged by the log-sum-exp rescale (not on the pages; it is the split that
  long contexts need).  Exactly equal to the dense result up to rounding.
* Prefill over a cached prefix -- the new tokens of a request attend
  causally over its whole paged context, shared prefix pages included
  (paged-KV analysis page, sections 3.2 and 4.1).  Token at position p reads
  tokens t <= p.  Written out as masked dense attention per (sequence, head).
* Two-level tables -- large pages (aligned runs of H blocks) for a prompt,
  small blocks for what follows (Cross-Paper Synthesis page, section 5):
  expanded into a flat table, then the definitions above.
* Swap out / swap in -- preemption evicts all blocks of a request to host
  memory and brings them back later (Cross-Paper Synthesis page, section 3);
  the host copy is block-first (vLLM entity page, key observations).  Byte
  copies.
* Utilisation readout -- effective memory utilisation = sum of sequence
  lengths / (allocated blocks * page size) (paged-KV analysis page, section
  4.2).

Every floating-point value is upcast exactly to float64 before any
arithmetic.  Pins against independent facts live in ``tests/test_oracle.py``.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

DTYPES = ("f32", "f16", "bf16")


# ----------------------------------------------------------------------------
# exact upcast of the storage formats
# ----------------------------------------------------------------------------

def infer_dtype(arr: np.ndarray) -> str:
    if arr.dtype == np.float32:
        return "f32"
    if arr.dtype == np.float16:
        return "f16"
    if arr.dtype == np.uint16:
        return "bf16"
    raise TypeError(f"unsupported storage dtype {arr.dtype}")


def upcast(arr: np.ndarray, dtype: str | None = None) -> np.ndarray:
    """Storage array -> float64, exactly (bf16 is held as uint16 bit patterns:
    the bf16 value is the float32 whose upper half is those bits)."""
    dtype = dtype or infer_dtype(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(arr, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(arr, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# append and copy-on-write (byte copies)
# ----------------------------------------------------------------------------

def kv_append(k_pool: np.ndarray, v_pool: np.ndarray, key: np.ndarray, value: np.ndarray,
              slot_mapping: np.ndarray, block_size: int) -> None:
    """Write token i's K/V rows into slot ``slot_mapping[i]`` of the pools (in
    place).  A negative slot means the token is not stored.  Pools are
    ``[num_blocks, num_kv_heads, block_size, head_dim]``; key/value are
    ``[num_tokens, num_kv_heads, head_dim]``."""
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        block, offset = divmod(int(slot), block_size)
        k_pool[block, :, offset, :] = key[i]
        v_pool[block, :, offset, :] = value[i]


def block_copy(k_pool: np.ndarray, v_pool: np.ndarray, block_mapping: np.ndarray) -> None:
    """Copy-on-write: for every (src, dst) pair, block dst of both pools
    becomes a copy of block src as it was before the call (in place)."""
    pairs = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    k_src = {int(s): k_pool[int(s)].copy() for s, _ in pairs}
    v_src = {int(s): v_pool[int(s)].copy() for s, _ in pairs}
    for src, dst in pairs:
        k_pool[int(dst)] = k_src[int(src)]
        v_pool[int(dst)] = v_src[int(src)]


def swap_out(k_pool: np.ndarray, v_pool: np.ndarray, block_ids, host: np.ndarray) -> None:
    """Preemption moves every block of a request out of HBM at once
    (Cross-Paper Synthesis page, section 3, the preemption item).  The host
    copy is block-first -- entry i holds block block_ids[i]'s K tile then its V
    tile, so one request's KV is one contiguous run (vLLM entity page, key
    observations: block-first layout for KV movement).  host has shape
    [n, 2, Hkv, block_size, D]; entries whose id is outside the pool are left
    as they are."""
    ids = np.asarray(block_ids, dtype=np.int64).reshape(-1)
    for i, b in enumerate(ids):
        if 0 <= b < k_pool.shape[0]:
            host[i, 0] = k_pool[b]
            host[i, 1] = v_pool[b]


def swap_in(host: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_ids) -> None:
    """The way back: block block_ids[i] of both pools receives entry i of the
    block-first host copy (ids outside the pool are skipped)."""
    ids = np.asarray(block_ids, dtype=np.int64).reshape(-1)
    for i, b in enumerate(ids):
        if 0 <= b < k_pool.shape[0]:
            k_pool[b] = host[i, 0]
            v_pool[b] = host[i, 1]


# ----------------------------------------------------------------------------
# decode attention
# ----------------------------------------------------------------------------

def kv_head_of(q_head: int, num_q_heads: int, num_kv_heads: int) -> int:
    """Consecutive grouping: q heads [g*G, (g+1)*G) share KV head g."""
    return q_head // (num_q_heads // num_kv_heads)


def gather_tokens(pool: np.ndarray, table_row: np.ndarray, length: int, block_size: int,
                  kv_head: int) -> np.ndarray:
    """Rows of the first ``length`` tokens of one KV head, in logical order:
    token t lives in physical block ``table_row[t // block_size]`` at offset
    ``t % block_size``."""
    rows = []
    for t in range(length):
        block = int(table_row[t // block_size])
        rows.append(pool[block, kv_head, t % block_size, :])
    if not rows:
        return pool[:0, kv_head, 0, :]
    return np.stack(rows)


def gather_tokens_fast(pool: np.ndarray, table_row: np.ndarray, length: int, block_size: int,
                       kv_head: int) -> np.ndarray:
    """Same as :func:`gather_tokens`, block at a time (used for large inputs;
    pinned against the token-at-a-time version in the tests)."""
    nb = -(-length // block_size)
    if nb == 0:
        return pool[:0, kv_head, 0, :]
    blocks = pool[np.asarray(table_row[:nb], dtype=np.int64), kv_head]   # [nb, bs, D]
    return blocks.reshape(nb * block_size, pool.shape[-1])[:length]


def attention_weights(scores: np.ndarray) -> np.ndarray:
    """Softmax over the last axis: w_t = exp(s_t - max s) / sum_u exp(s_u - max s)."""
    m = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - m)
    return e / e.sum(axis=-1, keepdims=True)


def attend(q_rows: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """Dense single-query attention for G query rows sharing one K/V set.
    q_rows [G, D], keys/values [L, D] (float64) -> [G, D].  L = 0 gives zeros."""
    if keys.shape[0] == 0:
        return np.zeros((q_rows.shape[0], values.shape[1]), dtype=np.float64)
    scores = (q_rows @ keys.T) * scale                   # [G, L]
    return attention_weights(scores) @ values            # [G, D]


def decode_group(query, k_pool, v_pool, block_tables, context_lens, scale, block_size, dtype,
                 seq: int, kv_head: int, fast: bool = True) -> np.ndarray:
    """Output rows [G, D] (float64) of the q heads of sequence ``seq`` that read
    KV head ``kv_head``."""
    Hq, Hkv = query.shape[1], k_pool.shape[1]
    G = Hq // Hkv
    L = int(context_lens[seq])
    gather = gather_tokens_fast if fast else gather_tokens
    keys = upcast(gather(k_pool, block_tables[seq], L, block_size, kv_head), dtype)
    values = upcast(gather(v_pool, block_tables[seq], L, block_size, kv_head), dtype)
    heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == kv_head]
    q_rows = upcast(query[seq, heads], dtype)
    scale64 = float(np.float32(scale))
    assert len(heads) == G
    return attend(q_rows, keys, values, scale64)


def decode_attention(query, k_pool, v_pool, block_tables, context_lens, scale, block_size,
                     dtype=None, seqs=None, fast: bool = True) -> np.ndarray:
    """Decode attention for every (sequence, q head); float64 [S, Hq, D].
    ``seqs`` restricts the work to some sequences (other rows are NaN)."""
    dtype = dtype or infer_dtype(query)
    S, Hq, D = query.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    out = np.full((S, Hq, D), np.nan, dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        for g in range(Hkv):
            out[s, g * G:(g + 1) * G] = decode_group(query, k_pool, v_pool, block_tables,
                                                     context_lens, scale, block_size, dtype,
                                                     s, g, fast=fast)
    return out


def prefill_attention(query, k_pool, v_pool, block_tables, context_lens, query_start, scale,
                      block_size, dtype=None, seqs=None) -> np.ndarray:
    """Multi-token attention over a paged, partly cached context; float64
    [T, Hq, D].

    When a request's prompt shares a cached prefix, only its new tokens run
    through prefill, reading the prefix's KV pages instead of recomputing
    them (paged-KV analysis page, section 3.2 and the TTFT row of section
    4.1).  Sequence s has context_lens[s] = L tokens in its pages, the last
    n = query_start[s+1] - query_start[s] of which are its new tokens (already
    appended); query row query_start[s] + j is the token at position
    p = L - n + j, and attends causally, to tokens t <= p:
        out = sum_{t<=p} exp(s_t - max) v_t / sum_{t<=p} exp(s_t - max),
        s_t = scale * <q, k_t>.
    n = 1 is decode attention.  ``seqs`` restricts the work (other rows NaN)."""
    dtype = dtype or infer_dtype(query)
    T, Hq, D = query.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    scale64 = float(np.float32(scale))
    out = np.full((T, Hq, D), np.nan, dtype=np.float64)
    starts = np.asarray(query_start, dtype=np.int64)
    for s in (range(len(starts) - 1) if seqs is None else seqs):
        q0, q1 = int(starts[s]), int(starts[s + 1])
        n, L = q1 - q0, int(context_lens[s])
        if n == 0:
            continue
        pos = np.arange(L - n, L)                                  # positions of the new tokens
        for g in range(Hkv):
            keys = upcast(gather_tokens_fast(k_pool, block_tables[s], L, block_size, g), dtype)
            values = upcast(gather_tokens_fast(v_pool, block_tables[s], L, block_size, g), dtype)
            for h in range(g * G, (g + 1) * G):
                q = upcast(query[q0:q1, h], dtype)                 # [n, D]
                scores = (q @ keys.T) * scale64                    # [n, L]
                scores[np.arange(L)[None, :] > pos[:, None]] = -np.inf
                out[q0:q1, h] = attention_weights(scores) @ values
    return out


def expand_hier_tables(large_tables, num_large, small_tables, pages_per_large: int) -> np.ndarray:
    """Two-level (hierarchical) block tables as one flat block table.

    The pages propose two page granularities at once, like an OS's huge and
    small pages: large pages where a sequence's prompt is written in one go
    (fewer table entries), small blocks where it grows token by token (less
    fragmentation) (Cross-Paper Synthesis page, section 5, the adaptive block
    size item).  Reading: a large page is an aligned run of H =
    pages_per_large consecutive blocks of the one pool, large page P covering
    blocks [P H, P H + H).  Sequence s's first num_large[s] * H logical blocks
    live in its large pages, the rest in its small blocks:
        entry j = large_tables[s][j // H] * H + j % H      if j < num_large[s] * H
                = small_tables[s][j - num_large[s] * H]    otherwise."""
    large_tables = np.asarray(large_tables)
    small_tables = np.asarray(small_tables)
    S = small_tables.shape[0]
    H = int(pages_per_large)
    width = int(np.max(np.asarray(num_large))) * H + small_tables.shape[1] if S else 0
    flat = np.full((S, width), -1, dtype=np.int64)
    for s in range(S):
        nl = int(num_large[s])
        for j in range(nl * H):
            flat[s, j] = int(large_tables[s, j // H]) * H + j % H
        flat[s, nl * H:nl * H + small_tables.shape[1]] = small_tables[s]
    return flat


def decode_attention_hier(query, k_pool, v_pool, large_tables, num_large, small_tables, pages_per_large,
                          context_lens, scale, block_size, dtype=None, seqs=None) -> np.ndarray:
    """Decode attention through two-level tables: the flat expansion above,
    then the same definition as :func:`decode_attention`."""
    flat = expand_hier_tables(large_tables, num_large, small_tables, pages_per_large)
    return decode_attention(query, k_pool, v_pool, flat, context_lens, scale, block_size, dtype, seqs=seqs)


def prefill_attention_hier(query, k_pool, v_pool, large_tables, num_large, small_tables, pages_per_large,
                           context_lens, query_start, scale, block_size, dtype=None, seqs=None) -> np.ndarray:
    flat = expand_hier_tables(large_tables, num_large, small_tables, pages_per_large)
    return prefill_attention(query, k_pool, v_pool, flat, context_lens, query_start, scale, block_size, dtype,
                             seqs=seqs)


def attend_partitioned(q_rows, keys, values, scale, partition_size: int) -> np.ndarray:
    """Attention over [0, L) split into partitions [p*P, min((p+1)*P, L)):
    partition p gives its max m_p, its sum l_p = sum exp(s - m_p) and its
    normalised output o_p; the merge takes M = max m_p, w_p = l_p exp(m_p - M)
    and returns sum_p w_p o_p / sum_p w_p."""
    L = keys.shape[0]
    if L == 0:
        return np.zeros((q_rows.shape[0], values.shape[1]), dtype=np.float64)
    parts = []
    for start in range(0, L, partition_size):
        stop = min(start + partition_size, L)
        s = (q_rows @ keys[start:stop].T) * scale                 # [G, n]
        m = s.max(axis=-1)                                        # [G]
        e = np.exp(s - m[:, None])
        l_p = e.sum(axis=-1)
        o_p = (e @ values[start:stop]) / l_p[:, None]
        parts.append((m, l_p, o_p))
    M = np.max(np.stack([m for m, _, _ in parts]), axis=0)
    num = np.zeros_like(parts[0][2])
    den = np.zeros_like(parts[0][1])
    for m, l_p, o_p in parts:
        w = l_p * np.exp(m - M)
        num += w[:, None] * o_p
        den += w
    return num / den[:, None]


def decode_attention_partitioned(query, k_pool, v_pool, block_tables, context_lens, scale,
                                 block_size, partition_size, dtype=None, seqs=None) -> np.ndarray:
    dtype = dtype or infer_dtype(query)
    S, Hq, D = query.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    scale64 = float(np.float32(scale))
    out = np.full((S, Hq, D), np.nan, dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        L = int(context_lens[s])
        for g in range(Hkv):
            keys = upcast(gather_tokens_fast(k_pool, block_tables[s], L, block_size, g), dtype)
            values = upcast(gather_tokens_fast(v_pool, block_tables[s], L, block_size, g), dtype)
            q_rows = upcast(query[s, g * G:(g + 1) * G], dtype)
            out[s, g * G:(g + 1) * G] = attend_partitioned(q_rows, keys, values, scale64,
                                                           partition_size)
    return out


# ----------------------------------------------------------------------------
# utilisation readout
# ----------------------------------------------------------------------------

def kv_utilisation(context_lens, allocated_blocks: int, block_size: int) -> Fraction:
    """Effective KV memory utilisation: tokens actually stored over token
    slots allocated (paged-KV analysis page, section 4.2), as an exact ratio."""
    total = sum(int(x) for x in context_lens)
    return Fraction(total, int(allocated_blocks) * int(block_size))


def blocks_needed(context_lens, block_size: int) -> int:
    return sum(-(-int(x) // block_size) for x in context_lens)
