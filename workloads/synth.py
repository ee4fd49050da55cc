"""Seeded synthetic inputs for the paged-KV decode path.

This module draws random numbers and lays them out in the storage formats the
path consumes: element arrays (fp32, fp16, or bf16 held as uint16 bit
patterns), physical K/V block pools ``[num_blocks, num_kv_heads, block_size,
head_dim]``, per-sequence block tables, context lengths, slot mappings for the
append and (src, dst) pairs for copy-on-write.  It contains none of the
attention, append or copy arithmetic: both the GPU tests and the CPU oracle
read the arrays built here, and each side computes from them on its own.

Paging model (vLLM/PagedAttention pages, "PagedAttention core idea" and
"paging mechanism" sections): a sequence's tokens are cut into fixed-size
logical blocks, each mapped by the sequence's block table to an arbitrary
physical block of a shared pool.  Physical ids are drawn without replacement
from a seeded permutation, so consecutive logical blocks are scattered.

Seeding: every random stream is a child ``SeedSequence(seed, spawn_key=(k,))``
with a fixed ``k`` per purpose, so any sequence's K/V can be regenerated alone
and the content of a logical token does not depend on the block size or on
the physical permutation.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
ELT_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
# quiet-NaN bit patterns used to poison every pool slot that no sequence owns
POISON_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}
_BITS_VIEW = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}

# stream ids (spawn keys) of the child generators
S_LENS, S_PERM, S_QUERY, S_NEWTOK, S_MISC = 0, 1, 2, 3, 4
S_SEQ_BASE = 1_000           # per-sequence (or per-prompt) K/V content
S_SUFFIX_BASE = 2_000_000    # per-sample suffix K/V (prefix-sharing workload)

CONFIG_SEED_BASE = 313_000


def child_rng(seed: int, key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(key,)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = POISON_BITS["bf16"]
    return out


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 draws -> the storage array of ``dtype`` (RNE rounding)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def poison_array(shape, dtype: str) -> np.ndarray:
    a = np.empty(shape, dtype=STORAGE[dtype])
    a.view(_BITS_VIEW[dtype]).fill(POISON_BITS[dtype])
    return a


def default_scale(head_dim: int) -> float:
    """1/sqrt(head_dim) rounded to float32 (the value both sides are given)."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))


@dataclass
class Batch:
    """One synthetic decode step in host memory (storage dtypes)."""

    name: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    query: np.ndarray            # [S, Hq, D]
    k_pool: np.ndarray           # [NB, Hkv, bs, D]
    v_pool: np.ndarray           # [NB, Hkv, bs, D]
    block_tables: np.ndarray     # int32 [S, max_blocks_per_seq], unused = -1
    context_lens: np.ndarray     # int32 [S]: tokens attended to (after any append)
    partition_size: int = 512
    # optional append (applied before attention)
    new_key: Optional[np.ndarray] = None      # [T, Hkv, D]
    new_value: Optional[np.ndarray] = None    # [T, Hkv, D]
    slot_mapping: Optional[np.ndarray] = None  # int64 [T], <0 = skip
    # optional copy-on-write pairs (applied before the append)
    block_mapping: Optional[np.ndarray] = None  # int32 [N, 2] (src, dst)
    meta: dict = field(default_factory=dict)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def elt_bytes(self) -> int:
        return ELT_BYTES[self.dtype]

    def kv_bytes(self) -> int:
        """K+V bytes of the valid tokens read by one decode step."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_dim * 2 * self.elt_bytes


def _alloc_tables(lens_blocks: np.ndarray, perm: np.ndarray, max_blocks: int) -> np.ndarray:
    """Deal physical ids from ``perm`` to sequences in order; unused entries -1."""
    S = len(lens_blocks)
    tables = np.full((S, max_blocks), -1, dtype=np.int32)
    pos = 0
    for s in range(S):
        nb = int(lens_blocks[s])
        tables[s, :nb] = perm[pos:pos + nb]
        pos += nb
    return tables


def _fill_sequence(pool_k, pool_v, table_row, k_log, v_log, block_size, dtype):
    """Place logical-order K/V [L, H, D] of one sequence into its physical blocks."""
    L = k_log.shape[0]
    nb = -(-L // block_size)
    if nb == 0:
        return
    H, D = k_log.shape[1], k_log.shape[2]
    for src, pool in ((k_log, pool_k), (v_log, pool_v)):
        padded = poison_array((nb * block_size, H, D), dtype)
        padded[:L] = src
        tiles = padded.reshape(nb, block_size, H, D).transpose(0, 2, 1, 3)
        # whole blocks are rewritten, so unused tail slots stay poisoned
        pool[table_row[:nb]] = tiles


def _draw_kv(seed, key, L, H, D, dtype):
    rng = child_rng(seed, key)
    k = to_storage(rng.standard_normal((L, H, D), dtype=np.float32), dtype)
    v = to_storage(rng.standard_normal((L, H, D), dtype=np.float32), dtype)
    return k, v


def make_decode_batch(seed: int, *, num_seqs: int, num_q_heads: int, num_kv_heads: int,
                      head_dim: int, dtype: str, block_size: int, context_lens,
                      num_blocks: Optional[int] = None, headroom: float = 0.10,
                      append: bool = False, table_layout: str = "shuffled",
                      partition_size: int = 512, scale: Optional[float] = None,
                      name: str = "custom", threads: int = 8) -> Batch:
    """Build a ragged decode batch.

    ``context_lens`` are the lengths the attention runs over.  With
    ``append=True`` the pool holds ``context_lens - 1`` tokens per sequence and
    the batch carries one new token per sequence, to be written at position
    ``context_lens - 1`` through ``slot_mapping`` before attending.
    """
    if dtype not in DTYPES:
        raise ValueError(dtype)
    S = int(num_seqs)
    lens = np.asarray(context_lens, dtype=np.int64).reshape(S)
    if (lens < 0).any():
        raise ValueError("negative context length")
    if append and (lens < 1).any():
        raise ValueError("append needs context_lens >= 1")
    bs = int(block_size)
    blocks_per_seq = -(-lens // bs)
    needed = int(blocks_per_seq.sum())
    if num_blocks is None:
        num_blocks = max(needed, int(math.ceil(needed * (1.0 + headroom))))
    if num_blocks < needed:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {needed}")
    max_blocks = max(1, int(blocks_per_seq.max()) if S else 1)

    if table_layout == "shuffled":
        perm = child_rng(seed, S_PERM).permutation(num_blocks).astype(np.int32)
    elif table_layout == "identity":
        perm = np.arange(num_blocks, dtype=np.int32)
    else:
        raise ValueError(table_layout)
    tables = _alloc_tables(blocks_per_seq, perm, max_blocks)

    Hkv, D = int(num_kv_heads), int(head_dim)
    q = to_storage(child_rng(seed, S_QUERY).standard_normal((S, num_q_heads, D), dtype=np.float32), dtype)
    k_pool = poison_array((num_blocks, Hkv, bs, D), dtype)
    v_pool = poison_array((num_blocks, Hkv, bs, D), dtype)
    stored = lens - 1 if append else lens

    def work(s):
        k, v = _draw_kv(seed, S_SEQ_BASE + s, int(stored[s]), Hkv, D, dtype)
        _fill_sequence(k_pool, v_pool, tables[s], k, v, bs, dtype)

    if S:
        with ThreadPoolExecutor(max_workers=max(1, min(threads, S))) as ex:
            list(ex.map(work, range(S)))

    batch = Batch(name=name, dtype=dtype, num_seqs=S, num_q_heads=int(num_q_heads),
                  num_kv_heads=Hkv, head_dim=D, block_size=bs, num_blocks=int(num_blocks),
                  scale=default_scale(D) if scale is None else float(np.float32(scale)),
                  query=q, k_pool=k_pool, v_pool=v_pool, block_tables=tables,
                  context_lens=lens.astype(np.int32), partition_size=partition_size)
    if append:
        rng = child_rng(seed, S_NEWTOK)
        batch.new_key = to_storage(rng.standard_normal((S, Hkv, D), dtype=np.float32), dtype)
        batch.new_value = to_storage(rng.standard_normal((S, Hkv, D), dtype=np.float32), dtype)
        pos = stored
        blk = tables[np.arange(S), pos // bs].astype(np.int64)
        batch.slot_mapping = blk * bs + pos % bs
    return batch


def make_prefix_shared_batch(seed: int, *, num_prompts: int = 64, samples: int = 8,
                             prefix_len: int = 1032, suffix_len: int = 256,
                             num_q_heads: int = 32, num_kv_heads: int = 8, head_dim: int = 128,
                             dtype: str = "bf16", block_size: int = 16, headroom: float = 0.10,
                             partition_size: int = 512, name: str = "prefix_shared",
                             threads: int = 8) -> Batch:
    """Parallel sampling over shared prompts with copy-on-write.

    Each prompt's ``prefix_len`` tokens sit in blocks shared by all of its
    ``samples`` sequences (reference count = samples).  Every sample then
    appends its own ``suffix_len`` tokens.  The first write of a sample lands
    in the prompt's last, partly filled block when ``prefix_len`` is not a
    multiple of the block size; a writer that finds that block's reference
    count above one gets a private copy first (one (src, dst) pair), and the
    last writer, finding a count of one, writes in place.  All copies are
    gathered into ``block_mapping`` so that one call performs them.

    Sequence ``s = prompt * samples + j``.  The returned batch is the state
    *before* the step: pools hold only the prompts; the step is block copy ->
    append of all suffix tokens -> decode over ``prefix_len + suffix_len``.
    """
    bs = int(block_size)
    P, N = int(num_prompts), int(samples)
    S = P * N
    Hkv, D = int(num_kv_heads), int(head_dim)
    L = prefix_len + suffix_len
    shared_nb = -(-prefix_len // bs)
    total_nb = -(-L // bs)
    partial_last = prefix_len % bs != 0

    # physical block accounting (refcounts) for the whole step
    cow_per_prompt = (N - 1) if (partial_last and N > 1 and suffix_len > 0) else 0
    private_per_seq = total_nb - shared_nb
    needed = P * shared_nb + P * cow_per_prompt + S * private_per_seq
    num_blocks = max(needed, int(math.ceil(needed * (1.0 + headroom))))
    perm = child_rng(seed, S_PERM).permutation(num_blocks).astype(np.int32)
    free = list(perm[::-1])  # pop() hands out perm[0], perm[1], ...

    def alloc():
        return int(free.pop())

    refcount = {}
    tables = np.full((S, total_nb), -1, dtype=np.int32)
    prompt_blocks = []
    for p in range(P):
        blocks = [alloc() for _ in range(shared_nb)]
        for b in blocks:
            refcount[b] = N
        prompt_blocks.append(blocks)
        for j in range(N):
            tables[p * N + j, :shared_nb] = blocks
    pairs = []
    for p in range(P):
        for j in range(N):
            s = p * N + j
            if suffix_len > 0 and partial_last:
                b = int(tables[s, shared_nb - 1])
                if refcount[b] > 1:
                    nbk = alloc()
                    refcount[b] -= 1
                    refcount[nbk] = 1
                    pairs.append((b, nbk))
                    tables[s, shared_nb - 1] = nbk
            for lb in range(shared_nb, total_nb):
                tables[s, lb] = alloc()

    q = to_storage(child_rng(seed, S_QUERY).standard_normal((S, num_q_heads, D), dtype=np.float32), dtype)
    k_pool = poison_array((num_blocks, Hkv, bs, D), dtype)
    v_pool = poison_array((num_blocks, Hkv, bs, D), dtype)

    def fill_prompt(p):
        k, v = _draw_kv(seed, S_SEQ_BASE + p, prefix_len, Hkv, D, dtype)
        _fill_sequence(k_pool, v_pool, np.asarray(prompt_blocks[p], dtype=np.int32), k, v, bs, dtype)

    with ThreadPoolExecutor(max_workers=max(1, min(threads, P))) as ex:
        list(ex.map(fill_prompt, range(P)))

    new_k = np.empty((S * suffix_len, Hkv, D), dtype=STORAGE[dtype])
    new_v = np.empty_like(new_k)
    slots = np.empty(S * suffix_len, dtype=np.int64)
    pos = np.arange(prefix_len, L)

    def fill_suffix(s):
        k, v = _draw_kv(seed, S_SUFFIX_BASE + s, suffix_len, Hkv, D, dtype)
        new_k[s * suffix_len:(s + 1) * suffix_len] = k
        new_v[s * suffix_len:(s + 1) * suffix_len] = v
        slots[s * suffix_len:(s + 1) * suffix_len] = tables[s, pos // bs].astype(np.int64) * bs + pos % bs

    with ThreadPoolExecutor(max_workers=max(1, min(threads, S))) as ex:
        list(ex.map(fill_suffix, range(S)))

    batch = Batch(name=name, dtype=dtype, num_seqs=S, num_q_heads=int(num_q_heads),
                  num_kv_heads=Hkv, head_dim=D, block_size=bs, num_blocks=num_blocks,
                  scale=default_scale(D), query=q, k_pool=k_pool, v_pool=v_pool,
                  block_tables=tables, context_lens=np.full(S, L, dtype=np.int32),
                  partition_size=partition_size, new_key=new_k, new_value=new_v,
                  slot_mapping=slots,
                  block_mapping=np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    batch.meta.update(num_prompts=P, samples=N, prefix_len=prefix_len, suffix_len=suffix_len,
                      shared_blocks_per_prompt=shared_nb,
                      unique_blocks=P * shared_nb + P * cow_per_prompt + S * private_per_seq)
    return batch


# --------------------------------------------------------------------------
# The five workloads.  ``scale_down`` options shrink them for fast tests while
# keeping their structure (ragged lengths, shuffled pools, append, CoW, split).
# --------------------------------------------------------------------------

def config1(**kw) -> Batch:
    """Tiny MHA decode: 4 seqs, 8 heads, D=64, fp32, bs 16, lens {5,17,33,64},
    32-block pool assigned by a seeded permutation, scale 1/8."""
    seed = CONFIG_SEED_BASE + 1
    args = dict(num_seqs=4, num_q_heads=8, num_kv_heads=8, head_dim=64, dtype="f32",
                block_size=16, context_lens=[5, 17, 33, 64], num_blocks=32,
                name="tiny_mha_f32", partition_size=0)
    args.update(kw)
    return make_decode_batch(seed, **args)


def config2_lens(num_seqs=64, sigma=1.0, median=512, lo=16, hi=2048, seed=None):
    rng = child_rng(CONFIG_SEED_BASE + 2 if seed is None else seed, S_LENS)
    z = rng.standard_normal(num_seqs)
    return np.clip(np.rint(median * np.exp(sigma * z)), lo, hi).astype(np.int64)


def config2(num_seqs=64, **kw) -> Batch:
    """OPT-13B-shaped MHA decode: 40 heads, D=128, fp16, bs 16, lognormal lens
    (median 512, sigma 1, clipped to [16, 2048]), 20k-block shuffled pool."""
    seed = CONFIG_SEED_BASE + 2
    args = dict(num_seqs=num_seqs, num_q_heads=40, num_kv_heads=40, head_dim=128, dtype="f16",
                block_size=16, context_lens=config2_lens(num_seqs), num_blocks=20_000,
                name="opt13b_mha_f16")
    args.update(kw)
    return make_decode_batch(seed, **args)


def config3_lens(num_seqs=256, lo=1024, hi=8192, seed=None):
    rng = child_rng(CONFIG_SEED_BASE + 3 if seed is None else seed, S_LENS)
    return rng.integers(lo, hi, size=num_seqs, endpoint=True).astype(np.int64)


def config3(num_seqs=256, lo=1024, hi=8192, **kw) -> Batch:
    """Llama-3-8B-shaped GQA decode: 32 q heads over 8 KV heads, D=128, bf16,
    bs 16, 256 seqs with lens uniform in [1024, 8192] before the append of one
    new token per sequence (attention then runs over L + 1)."""
    seed = CONFIG_SEED_BASE + 3
    lens = config3_lens(num_seqs, lo, hi) + 1
    args = dict(num_seqs=num_seqs, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                block_size=16, context_lens=lens, append=True, name="llama3_8b_gqa_bf16")
    args.update(kw)
    return make_decode_batch(seed, **args)


def config4(**kw) -> Batch:
    """Prefix-shared parallel sampling: 64 prompts x 8 samples, GQA 32/8, D=128,
    bf16, bs 16, 1032-token shared prompt (64 full blocks + one half-filled),
    256-token private suffixes, 448 CoW pairs."""
    return make_prefix_shared_batch(CONFIG_SEED_BASE + 4, **kw)


def config5_lens(num_seqs=16, lo=32768, hi=131072, seed=None):
    rng = child_rng(CONFIG_SEED_BASE + 5 if seed is None else seed, S_LENS)
    return rng.integers(lo, hi, size=num_seqs, endpoint=True).astype(np.int64)


def config5(block_size=16, num_seqs=16, lo=32768, hi=131072, **kw) -> Batch:
    """Long-context split decode: 16 seqs, GQA 32/8, D=128, bf16, lens uniform
    in [32768, 131072], block size 8/16/32, 512-token partitions + reduce."""
    seed = CONFIG_SEED_BASE + 5
    args = dict(num_seqs=num_seqs, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                block_size=block_size, context_lens=config5_lens(num_seqs, lo, hi),
                partition_size=512, name=f"long_ctx_gqa_bf16_bs{block_size}")
    args.update(kw)
    return make_decode_batch(seed, **args)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


S_HIER = 5   # stream id of the two-level layout's placement draws


def to_hierarchical(b: Batch, pages_per_large: int, prompt_tokens, seed: int = 0):
    """The same logical content as ``b`` laid out with two-level tables.

    Sequence s keeps its first ``prompt_tokens[s] // (H * bs)`` full large
    pages' worth of tokens in large pages -- aligned runs of H = pages_per_large
    blocks placed at random aligned positions of the pool -- and the rest of
    its blocks as small blocks at random free positions.  Block contents are
    copied over, unused blocks stay poisoned and any append slots are moved
    with their blocks.  Returns (batch, large_tables, num_large): the batch's
    block_tables are the small tables."""
    H, bs, S = int(pages_per_large), b.block_size, b.num_seqs
    lens = b.context_lens.astype(np.int64)
    nblk = -(-lens // bs)
    nl = np.array([min(int(prompt_tokens[s]), int(lens[s])) // (H * bs) for s in range(S)], dtype=np.int64)
    n_small = nblk - nl * H
    nlp_total = int(nl.sum())
    need = nlp_total * H + int(n_small.sum())
    nb = max(b.num_blocks, -(-need // H) * H + H)
    rng = child_rng(seed, S_HIER)
    slots_lp = rng.permutation(nb // H)[:nlp_total]              # aligned large-page positions
    used = np.zeros(nb, dtype=bool)
    for P in slots_lp:
        used[P * H:(P + 1) * H] = True
    free_small = rng.permutation(np.flatnonzero(~used))[:int(n_small.sum())]
    large = np.full((S, max(1, int(nl.max()) if S else 1)), -1, dtype=np.int32)
    small = np.full((S, max(1, int(n_small.max()) if S else 1)), -1, dtype=np.int32)
    newphys = {}
    kl = ks = 0
    for s in range(S):
        large[s, :nl[s]] = slots_lp[kl:kl + nl[s]]
        kl += int(nl[s])
        small[s, :n_small[s]] = free_small[ks:ks + n_small[s]]
        ks += int(n_small[s])
        for j in range(int(nblk[s])):
            new = int(large[s, j // H]) * H + j % H if j < nl[s] * H else int(small[s, j - nl[s] * H])
            newphys[int(b.block_tables[s, j])] = new
    old_ids = np.fromiter(newphys.keys(), dtype=np.int64)
    new_ids = np.fromiter(newphys.values(), dtype=np.int64)
    k_pool = poison_array((nb,) + b.k_pool.shape[1:], b.dtype)
    v_pool = poison_array((nb,) + b.v_pool.shape[1:], b.dtype)
    k_pool[new_ids] = b.k_pool[old_ids]
    v_pool[new_ids] = b.v_pool[old_ids]
    slot_mapping = None
    if b.slot_mapping is not None:
        sm = b.slot_mapping.astype(np.int64)
        blk, off = sm // bs, sm % bs
        remap = np.array([newphys.get(int(x), -1) for x in blk], dtype=np.int64)
        slot_mapping = np.where((sm >= 0) & (remap >= 0), remap * bs + off, -1).astype(np.int64)
    hb = Batch(name=b.name + f"_hier{H}", dtype=b.dtype, num_seqs=S, num_q_heads=b.num_q_heads,
               num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, block_size=bs, num_blocks=nb, scale=b.scale,
               query=b.query, k_pool=k_pool, v_pool=v_pool, block_tables=small, context_lens=b.context_lens,
               partition_size=b.partition_size, new_key=b.new_key, new_value=b.new_value,
               slot_mapping=slot_mapping, block_mapping=None,
               meta={**b.meta, "pages_per_large": H, "num_large_pages": nlp_total})
    return hb, large, nl.astype(np.int32)
