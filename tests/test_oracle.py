"""Pins for the CPU oracle, each against something other than the oracle itself.

* an independent library routine: torch's scaled_dot_product_attention in
  float64 on contiguous K/V regenerated straight from the seeded streams
  (never from the pool), with grouped heads expanded by repeat_interleave;
* a hand-derived worked example and an exact utilisation ratio
  (``tests/golden``);
* closed forms (one token, zero query, equal keys, two tokens);
* brute force in pure Python on tiny shapes;
* invariances the paging definition fixes (physical permutation, shared vs
  copied prefix, partitioned == dense);
* planted mistakes (a transposed head map, the literal per-block softmax of the
  simplified sketch, a dropped scale, keys read one slot off their values) that the pins must
  catch.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle.pa_oracle as O
from workloads import synth as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def small_batch(seed=7, S=5, Hq=8, Hkv=2, D=16, dtype="f32", bs=4, lens=None, **kw):
    if lens is None:
        lens = np.random.default_rng(seed).integers(1, 40, size=S)
    return W.make_decode_batch(seed, num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                               dtype=dtype, block_size=bs, context_lens=lens, **kw)


def oracle_out(b, **kw):
    return O.decode_attention(b.query, b.k_pool, b.v_pool, b.block_tables, b.context_lens,
                              b.scale, b.block_size, b.dtype, **kw)


def sdpa_reference(b, seed):
    """Dense attention from K/V regenerated in logical order (no pool, no table)."""
    S, Hq, D = b.query.shape
    G = Hq // b.num_kv_heads
    out = np.zeros((S, Hq, D))
    scale = float(np.float32(b.scale))
    for s in range(S):
        L = int(b.context_lens[s])
        k, v = W._draw_kv(seed, W.S_SEQ_BASE + s, L, b.num_kv_heads, D, b.dtype)
        kt = torch.from_numpy(O.upcast(k, b.dtype)).permute(1, 0, 2).repeat_interleave(G, dim=0)
        vt = torch.from_numpy(O.upcast(v, b.dtype)).permute(1, 0, 2).repeat_interleave(G, dim=0)
        qt = torch.from_numpy(O.upcast(b.query[s], b.dtype))[:, None, :]
        o = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None], scale=scale)
        out[s] = o[0, :, 0, :].numpy()
    return out


# ---------------------------------------------------------------- dtype decode

def test_upcast_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F80], dtype=np.uint16)
    got = O.upcast(bits, "bf16")
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 1.0 + 2.0 ** -7
    assert got[3] == 0.0 and np.signbit(got[4]) and np.isinf(got[5])
    h = np.array([1.0, -0.5, 65504.0, 2.0 ** -24], dtype=np.float16)
    assert list(O.upcast(h, "f16")) == [1.0, -0.5, 65504.0, 2.0 ** -24]


def test_generator_bf16_rounding_is_rne():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6: even (1+2^-6) wins.
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -3.0], dtype=np.float32)
    got = O.upcast(W.f32_to_bf16_bits(x), "bf16")
    assert list(got) == [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -3.0]


# ---------------------------------------------------------------- golden values

def test_golden_hand_attention():
    g = json.load(open(os.path.join(GOLDEN, "hand_attention.json")))
    q = np.array([g["query"]])
    k = np.array(g["keys"])
    v = np.array(g["values"])
    w = O.attention_weights(q @ k.T * g["scale"])[0]
    np.testing.assert_allclose(w, g["weights"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.attend(q, k, v, g["scale"])[0], g["out"], rtol=0, atol=1e-14)


def test_golden_hand_attention_through_pool():
    """The same example stored in a shuffled fp32 pool and read through a table."""
    g = json.load(open(os.path.join(GOLDEN, "hand_attention.json")))
    bs, nb = 2, 6
    k_pool = W.poison_array((nb, 1, bs, 2), "f32")
    v_pool = W.poison_array((nb, 1, bs, 2), "f32")
    table = np.array([[4, 1, -1]], dtype=np.int32)
    for t in range(3):
        k_pool[table[0, t // bs], 0, t % bs] = g["keys"][t]
        v_pool[table[0, t // bs], 0, t % bs] = g["values"][t]
    q = np.array([[g["query"]]], dtype=np.float32)
    out = O.decode_attention(q, k_pool, v_pool, table, np.array([3]), g["scale"], bs, "f32")
    # keys are rounded to fp32 (ln 2, ln 3 move by < 3e-8), hence the looser bound
    np.testing.assert_allclose(out[0, 0], g["out"], rtol=0, atol=1e-7)


def test_golden_utilisation_config1():
    g = json.load(open(os.path.join(GOLDEN, "utilisation_config1.json")))
    assert O.blocks_needed(g["context_lens"], g["block_size"]) == g["blocks"]
    assert O.kv_utilisation(g["context_lens"], g["blocks"], g["block_size"]) == Fraction(g["utilisation"])
    b = W.config1()
    used = int((b.block_tables >= 0).sum())
    assert O.kv_utilisation(b.context_lens, used, b.block_size) == Fraction(g["utilisation"])


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("dtype,bs,Hq,Hkv,D", [
    ("f32", 4, 4, 4, 8), ("f16", 8, 8, 2, 16), ("bf16", 16, 8, 2, 32), ("bf16", 32, 12, 3, 16),
    ("f32", 16, 8, 8, 64),
])
def test_matches_sdpa_on_contiguous_kv(dtype, bs, Hq, Hkv, D):
    seed = 11
    b = small_batch(seed=seed, S=6, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, bs=bs,
                    lens=[1, bs - 1, bs, bs + 1, 3 * bs + 5, 70])
    np.testing.assert_allclose(oracle_out(b), sdpa_reference(b, seed), rtol=0, atol=1e-12)


def test_config1_matches_sdpa():
    b = W.config1()
    np.testing.assert_allclose(oracle_out(b), sdpa_reference(b, W.CONFIG_SEED_BASE + 1),
                               rtol=0, atol=1e-12)


def test_gather_fast_equals_token_by_token():
    b = small_batch(dtype="bf16", bs=8)
    for s in range(b.num_seqs):
        L = int(b.context_lens[s])
        for g in range(b.num_kv_heads):
            a = O.gather_tokens(b.k_pool, b.block_tables[s], L, b.block_size, g)
            c = O.gather_tokens_fast(b.k_pool, b.block_tables[s], L, b.block_size, g)
            assert a.tobytes() == c.tobytes()
    np.testing.assert_array_equal(oracle_out(b, fast=False), oracle_out(b, fast=True))


# ---------------------------------------------------------------- closed forms

def test_single_token_returns_value_row_exactly():
    b = small_batch(dtype="bf16", lens=[1, 1, 1], S=3, bs=16)
    out = oracle_out(b)
    G = b.num_q_heads // b.num_kv_heads
    for s in range(3):
        blk = b.block_tables[s, 0]
        for h in range(b.num_q_heads):
            assert np.array_equal(out[s, h], O.upcast(b.v_pool[blk, h // G, 0], "bf16"))


def test_zero_query_gives_mean_of_values():
    b = small_batch(dtype="f16", lens=[9, 33], S=2)
    b.query[:] = 0
    out = oracle_out(b)
    G = b.num_q_heads // b.num_kv_heads
    for s in range(2):
        L = int(b.context_lens[s])
        for h in range(b.num_q_heads):
            vals = [O.upcast(b.v_pool[b.block_tables[s, t // b.block_size], h // G, t % b.block_size], "f16")
                    for t in range(L)]
            np.testing.assert_allclose(out[s, h], np.mean(vals, axis=0), rtol=0, atol=1e-13)


def test_equal_keys_gives_mean_of_values():
    b = small_batch(dtype="f32", lens=[13], S=1)
    b.k_pool[:] = 0.5
    out = oracle_out(b)
    vals = np.stack([O.upcast(b.v_pool[b.block_tables[0, t // b.block_size], :, t % b.block_size], "f32")
                     for t in range(13)])  # [L, Hkv, D]
    G = b.num_q_heads // b.num_kv_heads
    for h in range(b.num_q_heads):
        np.testing.assert_allclose(out[0, h], vals[:, h // G].mean(axis=0), rtol=0, atol=1e-13)


def test_two_tokens_logistic_form():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 8))
    k = rng.standard_normal((2, 8))
    v = rng.standard_normal((2, 8))
    scale = 0.3
    s0, s1 = (scale * math.fsum(q[0] * k[0]), scale * math.fsum(q[0] * k[1]))
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    expect = sig(s0 - s1) * v[0] + sig(s1 - s0) * v[1]
    np.testing.assert_allclose(O.attend(q, k, v, scale)[0], expect, rtol=0, atol=1e-14)


def test_weights_sum_to_one():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((4, 1000)) * 30
    w = O.attention_weights(s)
    np.testing.assert_allclose(w.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    assert (w >= 0).all()


def test_empty_context_gives_zeros():
    b = small_batch(lens=[0, 5], S=2)
    out = oracle_out(b)
    assert (out[0] == 0).all() and np.isfinite(out[1]).all()


# ---------------------------------------------------------------- brute force

def brute_force(q, keys, values, scale):
    """Pure-Python scalar enumeration: no NumPy arithmetic."""
    scores = [scale * math.fsum(a * b for a, b in zip(q, k)) for k in keys]
    m = max(scores)
    e = [math.exp(x - m) for x in scores]
    z = math.fsum(e)
    return [math.fsum(e[t] * values[t][d] for t in range(len(keys))) / z for d in range(len(values[0]))]


@settings(max_examples=60, deadline=None)
@given(L=st.integers(1, 4), D=st.integers(1, 4), seed=st.integers(0, 2 ** 31 - 1),
       mag=st.sampled_from([0.1, 1.0, 10.0]))
def test_brute_force_tiny(L, D, seed, mag):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, D)) * mag
    k = rng.standard_normal((L, D)) * mag
    v = rng.standard_normal((L, D))
    expect = brute_force(q[0].tolist(), k.tolist(), v.tolist(), 0.7)
    np.testing.assert_allclose(O.attend(q, k, v, 0.7)[0], expect, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- invariances

def relabel(b, seed=99):
    """Move every physical block to a new id and rewrite the tables to match."""
    perm = np.random.default_rng(seed).permutation(b.num_blocks)
    k2 = np.empty_like(b.k_pool)
    v2 = np.empty_like(b.v_pool)
    k2[perm] = b.k_pool
    v2[perm] = b.v_pool
    t2 = np.where(b.block_tables >= 0, perm[np.maximum(b.block_tables, 0)], -1).astype(np.int32)
    return k2, v2, t2


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_physical_permutation_invariance(dtype):
    b = small_batch(dtype=dtype, bs=8, S=6)
    k2, v2, t2 = relabel(b)
    a = oracle_out(b)
    c = O.decode_attention(b.query, k2, v2, t2, b.context_lens, b.scale, b.block_size, dtype)
    assert np.array_equal(a, c)


def test_identity_and_shuffled_tables_agree():
    kw = dict(seed=21, S=4, dtype="bf16", bs=8, lens=[7, 40, 64, 3])
    a = oracle_out(small_batch(table_layout="shuffled", **kw))
    c = oracle_out(small_batch(table_layout="identity", **kw))
    assert np.array_equal(a, c)


@pytest.mark.parametrize("P", [8, 16, 48, 512])
def test_partitioned_equals_dense(P):
    b = small_batch(dtype="bf16", bs=8, S=6, lens=[1, 7, 8, 9, 100, 257])
    dense = oracle_out(b)
    part = O.decode_attention_partitioned(b.query, b.k_pool, b.v_pool, b.block_tables,
                                          b.context_lens, b.scale, b.block_size, P, "bf16")
    np.testing.assert_allclose(part, dense, rtol=0, atol=1e-12)


def small_prefix_batch():
    return W.make_prefix_shared_batch(17, num_prompts=3, samples=4, prefix_len=20, suffix_len=11,
                                      num_q_heads=4, num_kv_heads=2, head_dim=8, dtype="bf16",
                                      block_size=8)


def run_step(b, k_pool, v_pool, tables, block_mapping):
    O.block_copy(k_pool, v_pool, block_mapping)
    O.kv_append(k_pool, v_pool, b.new_key, b.new_value, b.slot_mapping, b.block_size)
    return O.decode_attention(b.query, k_pool, v_pool, tables, b.context_lens, b.scale,
                              b.block_size, b.dtype)


def test_shared_prefix_equals_copied_prefix():
    """Refcounted sharing + CoW must give the same outputs as giving every
    sample its own full copy of the prompt."""
    b = small_prefix_batch()
    N = b.meta["samples"]
    nshared = b.meta["shared_blocks_per_prompt"]
    assert len(b.block_mapping) == b.meta["num_prompts"] * (N - 1)
    shared_out = run_step(b, b.k_pool.copy(), b.v_pool.copy(), b.block_tables, b.block_mapping)

    # fully copied layout: fresh blocks hold each sample's private prompt copy
    extra = b.num_seqs * nshared
    k = np.concatenate([b.k_pool, W.poison_array((extra,) + b.k_pool.shape[1:], "bf16")])
    v = np.concatenate([b.v_pool, W.poison_array((extra,) + b.v_pool.shape[1:], "bf16")])
    tables = b.block_tables.copy()
    nxt = b.num_blocks
    for s in range(b.num_seqs):
        p = s // N
        src_row = b.block_tables[p * N + N - 1]   # the in-place writer keeps the originals
        for lb in range(nshared):
            k[nxt] = b.k_pool[src_row[lb]]
            v[nxt] = b.v_pool[src_row[lb]]
            tables[s, lb] = nxt
            nxt += 1
    slots = b.slot_mapping.copy()
    for i, slot in enumerate(slots):
        s = i // b.meta["suffix_len"]
        blk, off = divmod(int(slot), b.block_size)
        lb = list(b.block_tables[s]).index(blk)
        slots[i] = tables[s, lb] * b.block_size + off
    O.kv_append(k, v, b.new_key, b.new_value, slots, b.block_size)
    copied_out = O.decode_attention(b.query, k, v, tables, b.context_lens, b.scale, b.block_size, "bf16")
    assert np.array_equal(shared_out, copied_out)


# ---------------------------------------------------------------- append / copy

def test_append_roundtrip_and_untouched_bytes():
    b = small_batch(dtype="bf16", bs=8, S=4, lens=[5, 8, 9, 30], append=True)
    k0, v0 = b.k_pool.copy(), b.v_pool.copy()
    slots = b.slot_mapping.copy()
    slots[2] = -1                     # token 2 is skipped
    k, v = b.k_pool.copy(), b.v_pool.copy()
    O.kv_append(k, v, b.new_key, b.new_value, slots, b.block_size)
    changed = np.zeros(k.shape[:3], dtype=bool)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), b.block_size)
        assert k[blk, :, off].tobytes() == b.new_key[i].tobytes()
        assert v[blk, :, off].tobytes() == b.new_value[i].tobytes()
        changed[blk, :, off] = True
    assert k[~changed].tobytes() == k0[~changed].tobytes()
    assert v[~changed].tobytes() == v0[~changed].tobytes()
    # gathering through the table returns the appended token at position L-1
    s = 1
    L = int(b.context_lens[s])
    row = O.gather_tokens(k, b.block_tables[s], L, b.block_size, 0)
    assert row[L - 1].tobytes() == b.new_key[s, 0].tobytes()


def test_block_copy_reads_pre_call_state():
    b = small_batch(dtype="f16", bs=4, S=3)
    k, v = b.k_pool.copy(), b.v_pool.copy()
    pairs = np.array([[0, 5], [5, 7], [2, 3]], dtype=np.int32)   # 5 is both dst and src
    O.block_copy(k, v, pairs)
    assert k[5].tobytes() == b.k_pool[0].tobytes()
    assert k[7].tobytes() == b.k_pool[5].tobytes()
    assert v[3].tobytes() == b.v_pool[2].tobytes()
    others = [i for i in range(b.num_blocks) if i not in (5, 7, 3)]
    assert k[others].tobytes() == b.k_pool[others].tobytes()


# ---------------------------------------------------------------- planted mistakes

def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    seed = 11
    b = small_batch(seed=seed, S=4, Hq=8, Hkv=2, D=16, dtype="f32", bs=4, lens=[3, 9, 17, 30])
    ref = sdpa_reference(b, seed)
    check = lambda: np.testing.assert_allclose(oracle_out(b), ref, rtol=0, atol=1e-12)
    check()

    with monkeypatch.context() as m:       # transposed head grouping
        m.setattr(O, "kv_head_of", lambda h, hq, hkv: h % hkv)
        assert _fails(check)

    def per_block(scores, bs=b.block_size):  # the sketch's literal per-block softmax, summed
        out = np.zeros_like(scores)
        for st_ in range(0, scores.shape[-1], bs):
            sl = scores[..., st_:st_ + bs]
            e = np.exp(sl - sl.max(axis=-1, keepdims=True))
            out[..., st_:st_ + bs] = e / e.sum(axis=-1, keepdims=True)
        return out
    with monkeypatch.context() as m:
        m.setattr(O, "attention_weights", per_block)
        assert _fails(check)

    orig_attend = O.attend
    with monkeypatch.context() as m:       # dropped scale
        m.setattr(O, "attend", lambda q, k, v, scale: orig_attend(q, k, v, 1.0))
        assert _fails(check)

    orig_fast = O.gather_tokens_fast
    # keys read one slot off from their values (attention is invariant to a
    # shared reordering of K and V, so only a K/V mismatch is a real mistake)
    def shifted(pool, row, L, bs, g):
        rows = orig_fast(pool, row, L, bs, g)
        return np.roll(rows, 1, axis=0) if pool is b.k_pool else rows
    with monkeypatch.context() as m:
        m.setattr(O, "gather_tokens_fast", shifted)
        assert _fails(check)


# -- swap out / swap in -------------------------------------------------------

def _pools(seed=0, nb=12, hkv=2, bs=4, d=8):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((nb, hkv, bs, d))
    v = rng.standard_normal((nb, hkv, bs, d))
    return k, v


def test_swap_out_layout_is_block_first():
    k, v = _pools()
    ids = [7, 2, 9]
    host = np.zeros((3, 2) + k.shape[1:])
    O.swap_out(k, v, ids, host)
    flat = host.reshape(3, -1)
    for i, b in enumerate(ids):   # one contiguous run per block: its K tile, then its V tile
        assert np.array_equal(flat[i], np.concatenate([k[b].ravel(), v[b].ravel()]))


def test_swap_round_trip_equals_block_copy():
    k, v = _pools(1)
    k2, v2 = k.copy(), v.copy()
    src, dst = [3, 0, 8], [5, 11, 1]
    host = np.zeros((3, 2) + k.shape[1:])
    O.swap_out(k, v, src, host)
    O.swap_in(host, k, v, dst)
    O.block_copy(k2, v2, np.array(list(zip(src, dst))))
    assert np.array_equal(k, k2) and np.array_equal(v, v2)


def test_swap_in_restores_clobbered_blocks_and_skips_bad_ids():
    k, v = _pools(2)
    k0, v0 = k.copy(), v.copy()
    ids = [4, 6, -1, 99]
    host = np.full((4, 2) + k.shape[1:], 7.0)
    O.swap_out(k, v, ids, host)
    assert (host[2:] == 7.0).all()                # out-of-pool ids leave their entries
    k[[4, 6]] = np.nan
    v[[4, 6]] = np.nan
    O.swap_in(host, k, v, ids)
    assert np.array_equal(k, k0) and np.array_equal(v, v0)


# -- prefill over a cached prefix ----------------------------------------------

def _prefill_case(seed, lens, news, Hq=4, Hkv=2, D=16, bs=4, dtype="f32"):
    rng = np.random.default_rng(seed)
    S = len(lens)
    nbs = [-(-L // bs) for L in lens]
    NB = sum(nbs) + 3
    perm = rng.permutation(NB)
    tables = np.full((S, max(nbs)), -1, dtype=np.int32)
    k = 0
    for s, nb in enumerate(nbs):
        tables[s, :nb] = perm[k:k + nb]
        k += nb
    kp = W.to_storage(rng.standard_normal((NB, Hkv, bs, D), dtype=np.float32), dtype)
    vp = W.to_storage(rng.standard_normal((NB, Hkv, bs, D), dtype=np.float32), dtype)
    starts = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = W.to_storage(rng.standard_normal((int(starts[-1]), Hq, D), dtype=np.float32), dtype)
    return q, kp, vp, tables, np.array(lens, dtype=np.int32), starts, bs


def test_prefill_is_bottom_right_causal_sdpa():
    """The new tokens are the last rows of ordinary causal attention over the
    whole sequence: torch SDPA (fp64, is_causal) over all L positions, with
    the cached prefix's queries filled at random, keeps the last n rows."""
    lens, news = [37, 5, 64], [9, 5, 1]
    q, kp, vp, tables, L, starts, bs = _prefill_case(3, lens, news)
    Hq, Hkv, D = q.shape[1], kp.shape[1], q.shape[2]
    out = O.prefill_attention(q, kp, vp, tables, L, starts, 0.25, bs)
    rng = np.random.default_rng(9)
    for s in range(len(lens)):
        n, Ls = news[s], lens[s]
        full_q = rng.standard_normal((Ls, Hq, D))
        full_q[Ls - n:] = q[starts[s]:starts[s + 1]]
        for g in range(Hkv):
            kk = torch.from_numpy(O.gather_tokens(kp, tables[s], Ls, bs, g).astype(np.float64))
            vv = torch.from_numpy(O.gather_tokens(vp, tables[s], Ls, bs, g).astype(np.float64))
            for h in range(g * (Hq // Hkv), (g + 1) * (Hq // Hkv)):
                qq = torch.from_numpy(full_q[:, h])
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qq[None, None], kk[None, None], vv[None, None], is_causal=True, scale=0.25)[0, 0]
                assert np.allclose(out[starts[s]:starts[s + 1], h], ref[Ls - n:].numpy(), atol=1e-12, rtol=0)


def test_prefill_of_one_token_is_decode():
    lens = [1, 17, 40]
    q, kp, vp, tables, L, starts, bs = _prefill_case(5, lens, [1, 1, 1], dtype="bf16")
    a = O.prefill_attention(q, kp, vp, tables, L, starts, 0.3, bs, "bf16")
    b = O.decode_attention(q, kp, vp, tables, L, 0.3, bs, "bf16")
    assert np.allclose(a, b, atol=1e-12, rtol=0)      # same sums, BLAS may order them differently


def test_prefill_first_token_of_fresh_prompt_is_its_value():
    """With no cached prefix (n = L) the first new token sees only itself."""
    q, kp, vp, tables, L, starts, bs = _prefill_case(7, [12], [12])
    out = O.prefill_attention(q, kp, vp, tables, L, starts, 0.5, bs)
    blk = tables[0, 0]
    for h in range(q.shape[1]):
        assert np.array_equal(out[0, h], vp[blk, h // 2, 0].astype(np.float64))


def test_prefill_brute_force_tiny():
    q, kp, vp, tables, L, starts, bs = _prefill_case(11, [6, 3], [4, 3], Hq=2, Hkv=1, D=3, bs=2)
    out = O.prefill_attention(q, kp, vp, tables, L, starts, 0.7, bs)
    for s in range(2):
        n, Ls = int(starts[s + 1] - starts[s]), int(L[s])
        for j in range(n):
            p = Ls - n + j
            for h in range(2):
                num = np.zeros(3)
                den = 0.0
                for t in range(p + 1):
                    b, o = tables[s, t // bs], t % bs
                    sc = float(np.float32(0.7))       # the scale argument is an fp32 value
                    w = math.exp(sc * float(np.dot(q[starts[s] + j, h].astype(np.float64), kp[b, 0, o])))
                    num += w * vp[b, 0, o].astype(np.float64)
                    den += w
                assert np.allclose(out[starts[s] + j, h], num / den, atol=1e-12, rtol=0)


def test_prefill_planted_mistakes_are_caught():
    """An off-by-one causal mask, or the mask anchored at the prefix start
    (top-left), changes the output."""
    q, kp, vp, tables, L, starts, bs = _prefill_case(13, [30], [8])
    good = O.prefill_attention(q, kp, vp, tables, L, starts, 0.25, bs)
    keys = O.gather_tokens(kp, tables[0], 30, bs, 0).astype(np.float64)
    vals = O.gather_tokens(vp, tables[0], 30, bs, 0).astype(np.float64)
    qq = q[:, 0].astype(np.float64)
    sc = (qq @ keys.T) * 0.25
    strict = sc.copy(); strict[np.arange(30)[None, :] >= np.arange(22, 30)[:, None]] = -np.inf
    topleft = sc.copy(); topleft[np.arange(30)[None, :] > np.arange(8)[:, None]] = -np.inf
    assert not np.allclose(O.attention_weights(strict) @ vals, good[:, 0])
    assert not np.allclose(O.attention_weights(topleft) @ vals, good[:, 0])


# -- two-level (large page + small block) tables --------------------------------

def test_hier_tables_hand_example():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hier_tables.json")))
    flat = O.expand_hier_tables(np.array(g["large_tables"]), g["num_large"], np.array(g["small_tables"]),
                                g["pages_per_large"])
    for s, want in enumerate(g["flat_prefixes"]):
        assert flat[s, :len(want)].tolist() == want


def test_hier_decode_reads_tokens_where_the_pages_put_them():
    """Brute force: write each token's K/V at the physical place the two-level
    rule gives (large page run, then small blocks), attend through the
    hierarchical tables, and compare with plain attention over the logical
    token sequence."""
    rng = np.random.default_rng(21)
    H, bs, D, NB = 2, 4, 8, 40
    L = [19, 6]
    nl = [2, 0]                                   # 2 large pages = 16 tokens for seq 0
    large = np.array([[7, 3], [-1, -1]])          # blocks 14,15 and 6,7
    small = np.array([[30, -1], [11, 25]])
    kp = np.full((NB, 1, bs, D), np.nan, dtype=np.float32)
    vp = np.full((NB, 1, bs, D), np.nan, dtype=np.float32)
    keys = [rng.standard_normal((n, D)).astype(np.float32).astype(np.float64) for n in L]
    vals = [rng.standard_normal((n, D)).astype(np.float32).astype(np.float64) for n in L]
    for s in range(2):
        for t in range(L[s]):
            j, o = divmod(t, bs)
            blk = large[s, j // H] * H + j % H if j < nl[s] * H else small[s, j - nl[s] * H]
            kp[blk, 0, o] = keys[s][t]
            vp[blk, 0, o] = vals[s][t]
    q = rng.standard_normal((2, 1, D)).astype(np.float32)
    out = O.decode_attention_hier(q, kp, vp, large, nl, small, H, np.array(L), 0.3, bs, "f32")
    for s in range(2):
        sc = keys[s] @ q[s, 0].astype(np.float64) * float(np.float32(0.3))
        w = np.exp(sc - sc.max())
        assert np.allclose(out[s, 0], (w @ vals[s]) / w.sum(), atol=1e-12, rtol=0)


def test_hierarchical_layout_keeps_logical_content():
    """The two-level layout generator moves blocks, not tokens: gathering each
    sequence through the expanded two-level tables returns the same K/V rows as
    the flat batch, and unused blocks stay poisoned."""
    b = W.make_decode_batch(4, num_seqs=5, num_q_heads=4, num_kv_heads=2, head_dim=16, dtype="bf16", block_size=8,
                            context_lens=[1, 64, 65, 200, 513], append=True)
    hb, large, nl = W.to_hierarchical(b, 4, prompt_tokens=[1, 64, 40, 199, 512], seed=2)
    assert nl.tolist() == [0, 2, 1, 6, 16]
    flat = O.expand_hier_tables(large, nl, hb.block_tables, 4)
    for s in range(b.num_seqs):
        L = int(b.context_lens[s])
        for g in range(2):
            old_k = O.gather_tokens(b.k_pool, b.block_tables[s], L, 8, g)
            new_k = O.gather_tokens(hb.k_pool, flat[s], L, 8, g)
            assert old_k.tobytes() == new_k.tobytes()
    used = set(int(x) for x in flat[flat >= 0])
    spare = [i for i in range(hb.num_blocks) if i not in used]
    assert np.isnan(O.upcast(hb.k_pool[spare], "bf16")).all()
    # append slots follow their blocks
    ko, vo = b.k_pool.copy(), b.v_pool.copy()
    O.kv_append(ko, vo, b.new_key, b.new_value, b.slot_mapping, 8)
    kn, vn = hb.k_pool.copy(), hb.v_pool.copy()
    O.kv_append(kn, vn, hb.new_key, hb.new_value, hb.slot_mapping, 8)
    for s in range(b.num_seqs):
        L = int(b.context_lens[s])
        assert O.gather_tokens(ko, b.block_tables[s], L, 8, 1).tobytes() == O.gather_tokens(kn, flat[s], L, 8, 1).tobytes()
