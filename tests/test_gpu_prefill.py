"""GPU parity of pa_prefill_attention (causal multi-token attention over a
paged, partly cached context) against the oracle: every dtype, head size,
block size and group size, ragged mixes of cached prefix and new tokens
(fresh prompts, one token, chunks spanning several query blocks and key
tiles), NaN-poisoned unused slots, rows the call must not write, and a
chunked-prefill batch at serving size on sampled rows."""

import numpy as np
import pytest
import torch

import oracle.pa_oracle as O
import paged_kv_cache_313_amd as P
from workloads import synth as W
from workloads import torch_io

from gpu_util import check_close, gpu_out_f64, note

pytestmark = pytest.mark.gpu

ULPS = 2
MANT = {"f16": 10, "bf16": 7}


def p_rounding(q, b, starts, seqs=None):
    """Allowance for rounding the probabilities to the input type before the
    products with V and with the ones that form the row sums: each weight
    carries a relative error of at most half an ulp, u = 2^-(m+1), and the
    normaliser is the sum of the same rounded weights, so each normalised
    weight is off by at most 2u / (1 - u) relatively and the output by at most
    that times sum_t w_t |v_t| / sum_t w_t -- the oracle over |V| gives that
    weighted mean exactly.  2^-m covers 2u / (1 - u) up to a term of order u^2,
    which the 2-ulp part of the bound absorbs."""
    kabs = b.k_pool
    vabs = W.to_storage(np.abs(O.upcast(b.v_pool, b.dtype)).astype(np.float32), b.dtype)
    mean = O.prefill_attention(q, kabs, vabs, b.block_tables, b.context_lens, starts, b.scale, b.block_size,
                               b.dtype, seqs=seqs)
    return 2.0 ** -MANT[b.dtype] * mean


def case(dtype, D, bs, G, lens, news, Hkv=2, seed=0):
    b = W.make_decode_batch(seed, num_seqs=len(lens), num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D,
                            dtype=dtype, block_size=bs, context_lens=lens)
    rng = np.random.default_rng(seed + 1)
    starts = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = W.to_storage(rng.standard_normal((int(starts[-1]), G * Hkv, D), dtype=np.float32), dtype)
    return b, q, starts


def run(b, q, starts, max_query_len=None, out=None):
    d = torch_io.to_device(b)
    qd = torch_io.storage_to_torch(q, b.dtype, "cuda")
    res = P.prefill_attention(qd, d.k_pool, d.v_pool, d.block_tables, d.context_lens,
                              torch.from_numpy(starts).cuda(), b.scale,
                              int(np.diff(starts).max()) if max_query_len is None else max_query_len, out=out)
    torch.cuda.synchronize()
    return res


LENS = [1, 17, 100, 300, 700, 64]
NEWS = [1, 17, 33, 64, 130, 1]
CASES = [(dt, D, bs, G) for dt in ("f16", "bf16") for D in (64, 128) for bs in (8, 16, 32) for G in (1, 4)]
CASES += [("bf16", 128, 16, 2), ("bf16", 128, 16, 8), ("bf16", 128, 16, 16), ("f16", 64, 8, 16)]


# A host bound far above the real n: the grid holds 8 bands of query blocks,
# handed out from the band nearest the context's end, and the blocks past a
# sequence's new tokens have no rows and exit.
LOOSE_MAX_QUERY = 4096


@pytest.mark.parametrize("max_query_len", [None, LOOSE_MAX_QUERY], ids=["tight", "loose"])
@pytest.mark.parametrize("dtype,D,bs,G", CASES)
def test_prefill_matches_oracle(dtype, D, bs, G, max_query_len):
    b, q, starts = case(dtype, D, bs, G, LENS, NEWS, seed=D + bs + G)
    note(f"prefill dtype={dtype} D={D} bs={bs} G={G} max_query_len={max_query_len}")
    out = run(b, q, starts, max_query_len=max_query_len)
    ref = O.prefill_attention(q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, starts, b.scale,
                              b.block_size, dtype)
    check_close(gpu_out_f64(out, dtype), ref, dtype, f"prefill {dtype}/D{D}/bs{bs}/G{G}", ulps=ULPS,
                extra=p_rounding(q, b, starts))


@pytest.mark.parametrize("max_query_len", [None, LOOSE_MAX_QUERY], ids=["tight", "loose"])
def test_fresh_prompts_and_whole_context(max_query_len):
    """n = L for every sequence: plain causal prefill through the pages."""
    lens = [5, 31, 32, 33, 129]
    b, q, starts = case("bf16", 128, 16, 4, lens, lens, seed=3)
    note(f"prefill fresh prompts max_query_len={max_query_len}")
    out = run(b, q, starts, max_query_len=max_query_len)
    ref = O.prefill_attention(q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, starts, b.scale, 16, "bf16")
    check_close(gpu_out_f64(out, "bf16"), ref, "bf16", "fresh prompts", ulps=ULPS, extra=p_rounding(q, b, starts))
    # the first token of each fresh prompt sees only itself: exactly its value row
    o = torch_io.torch_to_storage(out, "bf16")
    for s in range(len(lens)):
        blk = b.block_tables[s, 0]
        for h in range(q.shape[1]):
            assert o[starts[s], h].tobytes() == b.v_pool[blk, h // 4, 0].tobytes()


def test_rows_not_to_write_are_left_alone():
    """A sequence claiming more new tokens than its context, and tokens past
    max_query_len, are not written."""
    lens, news = [40, 10, 200], [8, 12, 100]          # sequence 1: n > L
    b, q, starts = case("f16", 64, 16, 4, lens, news, seed=5)
    qd = torch_io.storage_to_torch(q, "f16", "cuda")
    sentinel = torch.full_like(qd, 7.0)
    note("prefill untouched rows")
    out = run(b, q, starts, max_query_len=64, out=sentinel)
    o = out.float().cpu().numpy()
    assert (o[starts[1]:starts[2]] == 7.0).all()
    assert (o[starts[2] + 64:starts[3]] == 7.0).all()
    ref = O.prefill_attention(q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, starts, b.scale, 16, "f16",
                              seqs=[0])
    got = gpu_out_f64(out, "f16")
    ex = p_rounding(q, b, starts, seqs=[0, 2])
    check_close(got[starts[0]:starts[1]], ref[starts[0]:starts[1]], "f16", "seq 0", ulps=ULPS,
                extra=ex[starts[0]:starts[1]])
    # sequence 2's first 64 rows only see keys below their own positions
    ref2 = O.prefill_attention(q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, starts, b.scale, 16, "f16",
                               seqs=[2])
    check_close(got[starts[2]:starts[2] + 64], ref2[starts[2]:starts[2] + 64], "f16", "seq 2 head", ulps=ULPS,
                extra=ex[starts[2]:starts[2] + 64])


def test_long_fresh_prompts_several_bands():
    """Fresh prompts of 2,600 and 700 tokens, GQA 8/2, D 128, bf16: 41 query
    blocks of 64 tokens for the long one, so 5 full bands of 8 and a band of
    1, and fewer bands for the short one; every output vs the oracle."""
    lens = [2600, 700]
    b, q, starts = case("bf16", 128, 16, 4, lens, lens, seed=13)
    note("prefill long fresh prompt")
    out = run(b, q, starts)
    ref = O.prefill_attention(q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, starts, b.scale, 16, "bf16")
    check_close(gpu_out_f64(out, "bf16"), ref, "bf16", "long fresh prompt", ulps=ULPS,
                extra=p_rounding(q, b, starts))


def test_chunked_prefill_at_serving_size():
    """8 sequences with 512-token chunks on 2K-8K cached contexts, GQA 32/8,
    D 128, bf16: every output element of 4 sampled sequences vs the oracle."""
    rng = np.random.default_rng(11)
    lens = rng.integers(2048, 8193, size=8).tolist()
    news = [512] * 8
    b, q, starts = case("bf16", 128, 16, 4, lens, news, Hkv=8, seed=11)
    note("prefill serving size")
    out = run(b, q, starts)
    seqs = [0, 3, 5, 7]
    ref = O.prefill_attention(q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, starts, b.scale, 16, "bf16",
                              seqs=seqs)
    got = gpu_out_f64(out, "bf16")
    ex = p_rounding(q, b, starts, seqs=seqs)
    for s in seqs:
        sl = slice(starts[s], starts[s + 1])
        check_close(got[sl], ref[sl], "bf16", f"seq {s}", ulps=ULPS, extra=ex[sl])


def test_ragged_long_chunks_across_bands():
    """Sequences bringing 1,500, 700, 2,100, 64 and 1 new tokens on contexts
    of 4,000, 700 (fresh), 3,000, 5,000 and 900 tokens, GQA 16/4, D 128,
    bf16: 33 query blocks of 64 tokens for the longest, so the grid has 5
    bands and in most of them the shorter sequences' blocks have no rows and
    exit; every output of every sequence vs the oracle."""
    lens, news = [4000, 700, 3000, 5000, 900], [1500, 700, 2100, 64, 1]
    b, q, starts = case("bf16", 128, 16, 4, lens, news, Hkv=4, seed=21)
    note("prefill ragged long chunks")
    out = run(b, q, starts)
    ref = O.prefill_attention(q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, starts, b.scale, 16, "bf16")
    check_close(gpu_out_f64(out, "bf16"), ref, "bf16", "ragged long chunks", ulps=ULPS,
                extra=p_rounding(q, b, starts))
