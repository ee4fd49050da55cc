"""GPU parity of the two-level-table entry points (pa_decode_attention_hier,
pa_prefill_attention_hier): the same logical batch laid out flat and with
large pages gives bit-identical outputs, in every split mode, and matches the
oracle; argument checks of the large-page arguments."""

import numpy as np
import pytest
import torch

import oracle.pa_oracle as O
import paged_kv_cache_313_amd as P
from workloads import synth as W
from workloads import torch_io

from gpu_util import check_close, gpu_out_f64, gpu_step, note, pv_extra

pytestmark = pytest.mark.gpu


def pair(dtype, D, bs, G, lens, prompts, H, seed=0, append=True):
    b = W.make_decode_batch(seed, num_seqs=len(lens), num_q_heads=2 * G, num_kv_heads=2, head_dim=D, dtype=dtype,
                            block_size=bs, context_lens=lens, append=append)
    hb, large, nl = W.to_hierarchical(b, H, prompts, seed=seed + 1)
    return b, hb, large, nl


def hier_step(hb, large, nl, H, partition):
    d = torch_io.to_device(hb)
    P.kv_append(d.new_key, d.new_value, d.k_pool, d.v_pool, d.slot_mapping)
    out = P.decode_attention_hier(d.query, d.k_pool, d.v_pool, d.block_tables, torch.from_numpy(large).cuda(),
                                  torch.from_numpy(nl).cuda(), H, d.context_lens, hb.scale, hb.max_context_len,
                                  partition)
    torch.cuda.synchronize()
    return out


LENS = [1, 40, 300, 1000, 2100]
PROMPTS = [1, 39, 290, 800, 2090]


@pytest.mark.parametrize("partition", [0, 64, -1])
@pytest.mark.parametrize("dtype,D,bs,G,H", [("bf16", 128, 16, 4, 16), ("f16", 64, 8, 1, 4), ("f32", 128, 32, 4, 2),
                                            ("bf16", 64, 16, 8, 64), ("f16", 128, 16, 1, 1), ("bf16", 128, 16, 16, 4)])
def test_decode_hier_bit_identical_to_flat(dtype, D, bs, G, H, partition):
    b, hb, large, nl = pair(dtype, D, bs, G, LENS, PROMPTS, H, seed=bs + H)
    note(f"hier decode {dtype} D={D} bs={bs} G={G} H={H} P={partition}")
    flat = gpu_step(b, torch_io.to_device(b), partition_size=partition)
    hier = hier_step(hb, large, nl, H, partition)
    assert torch_io.torch_to_storage(flat, dtype).tobytes() == torch_io.torch_to_storage(hier, dtype).tobytes()
    kp, vp = hb.k_pool.copy(), hb.v_pool.copy()
    O.kv_append(kp, vp, hb.new_key, hb.new_value, hb.slot_mapping, bs)
    ref = O.decode_attention_hier(hb.query, kp, vp, large, nl, hb.block_tables, H, hb.context_lens, hb.scale, bs,
                                  dtype)
    check_close(gpu_out_f64(hier, dtype), ref, dtype, "hier decode", extra=pv_extra(b))


@pytest.mark.parametrize("dtype,G,H", [("bf16", 4, 16), ("f16", 1, 4)])
def test_prefill_hier_bit_identical_to_flat(dtype, G, H):
    lens, news = [64, 300, 1000], [64, 37, 200]
    # every token already in the pages (no pending append)
    b, hb, large, nl = pair(dtype, 128, 16, G, lens, [L - n for L, n in zip(lens, news)], H, seed=7, append=False)
    starts = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = W.to_storage(np.random.default_rng(3).standard_normal((int(starts[-1]), 2 * G, 128), dtype=np.float32), dtype)
    qd = torch_io.storage_to_torch(q, dtype, "cuda")
    st = torch.from_numpy(starts).cuda()
    note(f"hier prefill {dtype} G={G} H={H}")
    d = torch_io.to_device(b)
    flat = P.prefill_attention(qd, d.k_pool, d.v_pool, d.block_tables, d.context_lens, st, b.scale, max(news))
    dh = torch_io.to_device(hb)
    hier = P.prefill_attention_hier(qd, dh.k_pool, dh.v_pool, dh.block_tables, torch.from_numpy(large).cuda(),
                                    torch.from_numpy(nl).cuda(), H, dh.context_lens, st, hb.scale, max(news))
    torch.cuda.synchronize()
    assert torch_io.torch_to_storage(flat, dtype).tobytes() == torch_io.torch_to_storage(hier, dtype).tobytes()
    ref = O.prefill_attention_hier(q, hb.k_pool, hb.v_pool, large, nl, hb.block_tables, H, hb.context_lens, starts,
                                   hb.scale, 16, dtype)
    check_close(gpu_out_f64(hier, dtype), ref, dtype, "hier prefill", ulps=2,
                extra=2.0 ** -(7 if dtype == "bf16" else 10) * np.abs(ref).max())


def test_hier_argument_checks():
    lib = P.load()
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((16, 1, 16, 128), dtype=torch.bfloat16, device="cuda")
    t = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    n = torch.zeros((1,), dtype=torch.int32, device="cuda")
    note("hier argument checks")
    for H, ml, large, status in [(3, 1, t, 2), (2048, 1, t, 2), (4, 0, t, 2), (4, 1, None, 1)]:
        st = lib.pa_decode_attention_hier(q.data_ptr(), q.data_ptr(), pool.data_ptr(), pool.data_ptr(), t.data_ptr(),
                                          None if large is None else large.data_ptr(), n.data_ptr(), n.data_ptr(),
                                          1, 4, 1, 128, 16, 2, ml, H, 16, 32, 0.1, 0, 2, None, 0, None)
        assert st == status, (H, ml, st)
