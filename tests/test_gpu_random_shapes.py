"""Seeded random shapes through the decode step and the prefill call, every
output against the oracle.  Each case draws the storage type, head size,
block size, group size, number of KV heads, batch size, a length mix (empty
and one-token sequences, short ragged ones, ones crossing table windows),
the split mode and whether the step appends a token; prefill cases draw a
mix of cached prefixes and new tokens (fresh prompts, single tokens, chunks
spanning several query-block bands); two-level-table cases lay a random
decode step out with large pages of a random size and compare bit for bit
with the flat layout.  The hand-picked cases of the other files stay; these
reach combinations that no one picked."""

import numpy as np
import pytest
import torch

import oracle.pa_oracle as O
import paged_kv_cache_313_amd as P
from workloads import synth as W
from workloads import torch_io

from gpu_util import MANT_BITS, check_close, gpu_out_f64, gpu_step, note, oracle_out, oracle_pools, pv_extra

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16")


def draw_lens(rng, S, lo):
    kind = rng.random(S)
    lens = np.where(kind < 0.1, 0, np.where(kind < 0.2, 1, np.where(kind < 0.7, rng.integers(2, 300, S),
                                                                     rng.integers(300, 3000, S))))
    return np.maximum(lens, lo).astype(int).tolist()


def decode_case(seed):
    rng = np.random.default_rng(seed)
    dtype = DTYPES[rng.integers(3)]
    D, bs = int(rng.choice([64, 128])), int(rng.choice([8, 16, 32]))
    G, Hkv = int(rng.choice([1, 2, 4, 8, 16])), int(rng.integers(1, 4))
    S = int(rng.integers(1, 40))
    append = bool(rng.random() < 0.5)
    part = int(rng.choice([0, 4 * bs, 512, -1]))
    lens = draw_lens(rng, S, 1 if append else 0)
    return dict(dtype=dtype, D=D, bs=bs, G=G, Hkv=Hkv, lens=lens, append=append, part=part)


@pytest.mark.parametrize("seed", range(1000, 1064))
def test_random_decode_step(seed):
    c = decode_case(seed)
    b = W.make_decode_batch(seed, num_seqs=len(c["lens"]), num_q_heads=c["G"] * c["Hkv"], num_kv_heads=c["Hkv"],
                            head_dim=c["D"], dtype=c["dtype"], block_size=c["bs"], context_lens=c["lens"],
                            append=c["append"])
    note(f"random decode seed={seed} {c}")
    d = torch_io.to_device(b)
    out = gpu_step(b, d, partition_size=c["part"])
    got = gpu_out_f64(out, c["dtype"])
    check_close(got, oracle_out(b), c["dtype"], f"random decode {seed}", extra=pv_extra(b))
    for s in np.flatnonzero(np.asarray(c["lens"]) == 0):
        assert (got[s] == 0).all()
    if c["append"]:   # the appended rows landed where the oracle put them
        ko, vo = oracle_pools(b)
        assert torch_io.torch_to_storage(d.k_pool, c["dtype"]).tobytes() == ko.tobytes()
        assert torch_io.torch_to_storage(d.v_pool, c["dtype"]).tobytes() == vo.tobytes()


@pytest.mark.parametrize("seed", range(2000, 2032))
def test_random_prefill(seed):
    rng = np.random.default_rng(seed)
    dtype = ("f16", "bf16")[rng.integers(2)]
    D, bs = int(rng.choice([64, 128])), int(rng.choice([8, 16, 32]))
    G, Hkv = int(rng.choice([1, 2, 4, 8, 16])), int(rng.integers(1, 3))
    S = int(rng.integers(1, 7))
    lens, news = [], []
    for _ in range(S):
        L = int(rng.integers(1, 2200))
        kind = rng.random()
        n = L if kind < 0.3 else (1 if kind < 0.45 else int(rng.integers(1, L + 1)))
        lens.append(L)
        news.append(n)
    b = W.make_decode_batch(seed, num_seqs=S, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
                            block_size=bs, context_lens=lens)
    starts = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = W.to_storage(rng.standard_normal((int(starts[-1]), G * Hkv, D), dtype=np.float32), dtype)
    note(f"random prefill seed={seed} {dtype} D={D} bs={bs} G={G} Hkv={Hkv} lens={lens} news={news}")
    d = torch_io.to_device(b)
    out = P.prefill_attention(torch_io.storage_to_torch(q, dtype, "cuda"), d.k_pool, d.v_pool, d.block_tables,
                              d.context_lens, torch.from_numpy(starts).cuda(), b.scale, int(max(news)))
    torch.cuda.synchronize()
    ref = O.prefill_attention(q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, starts, b.scale, bs, dtype)
    # the weights are rounded to the input type before the products: 2^-m times
    # the oracle over |V| bounds what that adds
    vabs = W.to_storage(np.abs(O.upcast(b.v_pool, dtype)).astype(np.float32), dtype)
    mean = O.prefill_attention(q, b.k_pool, vabs, b.block_tables, b.context_lens, starts, b.scale, bs, dtype)
    check_close(gpu_out_f64(out, dtype), ref, dtype, f"random prefill {seed}", extra=2.0 ** -MANT_BITS[dtype] * mean)


@pytest.mark.parametrize("seed", range(3000, 3024))
def test_random_decode_two_level_tables_bit_identical_to_flat(seed):
    """A random decode case (with an appended token) laid out flat and with
    large pages of a random size holding a random share of each prompt: the
    two calls give the same bits, in the case's split mode."""
    c = decode_case(seed)
    rng = np.random.default_rng(seed + 7)
    lens = [max(L, 1) for L in c["lens"]]
    H = int(rng.choice([1, 2, 4, 16, 64]))
    prompts = [int(rng.integers(0, L + 1)) for L in lens]
    b = W.make_decode_batch(seed, num_seqs=len(lens), num_q_heads=c["G"] * c["Hkv"], num_kv_heads=c["Hkv"],
                            head_dim=c["D"], dtype=c["dtype"], block_size=c["bs"], context_lens=lens, append=True)
    hb, large, nl = W.to_hierarchical(b, H, prompts, seed=seed + 1)
    note(f"random two-level decode seed={seed} H={H} {c}")
    flat = gpu_step(b, torch_io.to_device(b), partition_size=c["part"])
    d = torch_io.to_device(hb)
    P.kv_append(d.new_key, d.new_value, d.k_pool, d.v_pool, d.slot_mapping)
    hier = P.decode_attention_hier(d.query, d.k_pool, d.v_pool, d.block_tables, torch.from_numpy(large).cuda(),
                                   torch.from_numpy(nl).cuda(), H, d.context_lens, hb.scale, hb.max_context_len,
                                   c["part"])
    torch.cuda.synchronize()
    dt = c["dtype"]
    assert torch_io.torch_to_storage(flat, dt).tobytes() == torch_io.torch_to_storage(hier, dt).tobytes()
