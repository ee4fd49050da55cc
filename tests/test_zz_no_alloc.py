"""pa_decode_attention_noalloc (the entry point for callers that cannot
allocate: its split writes partials to the library's static device scratch)
against pa_decode_attention with a caller workspace, on the same inputs: the
same kernels run, so the outputs must agree bit for bit, and both must meet
the oracle's bound.  Two calls in a row per case, the second on a smaller
batch, so that partials the first call left in the scratch are never read."""

import numpy as np
import pytest
import torch

import paged_kv_cache_313_amd as P
from workloads import synth as W
from workloads import torch_io

from gpu_util import check_close, gpu_out_f64, note, oracle_out, pv_extra

pytestmark = pytest.mark.gpu

CASES = [  # dtype, D, bs, G, partition, (first lens, second lens)
    ("bf16", 128, 16, 4, -1, ([3000, 17, 1, 800, 4100, 2048, 5, 640], [300, 16, 1])),
    ("f16", 128, 16, 1, -1, ([2100, 400, 1, 33, 1500], [64, 2])),
    ("bf16", 64, 32, 8, 64, ([700, 64, 65, 1, 1200], [130, 2, 64])),
    ("f32", 64, 8, 2, 512, ([1025, 512, 3, 2000], [513, 1])),
    ("bf16", 128, 8, 16, -1, ([5000, 2, 900], [100])),
    ("f16", 128, 16, 4, 0, ([300, 17], [16])),
]


def batch(dtype, D, bs, G, lens, seed):
    return W.make_decode_batch(seed, num_seqs=len(lens), num_q_heads=2 * G, num_kv_heads=2, head_dim=D,
                               dtype=dtype, block_size=bs, context_lens=lens)


@pytest.mark.parametrize("dtype,D,bs,G,partition,lens", CASES)
def test_noalloc_matches_workspace_entry_point(dtype, D, bs, G, partition, lens):
    for call, ls in enumerate(lens):
        b = batch(dtype, D, bs, G, ls, seed=40 + call)
        d = torch_io.to_device(b)
        note(f"noalloc call {call}: {dtype} D={D} bs={bs} G={G} P={partition} lens={ls}")
        ref_out = P.decode_attention(d.query, d.k_pool, d.v_pool, d.block_tables, d.context_lens, b.scale,
                                     b.max_context_len, partition)
        out = torch.full_like(d.query, float("nan"))
        P.decode_attention_noalloc(d.query, d.k_pool, d.v_pool, d.block_tables, d.context_lens, b.scale,
                                   b.max_context_len, partition, out=out)
        torch.cuda.synchronize()
        a = torch_io.torch_to_storage(out, dtype)
        r = torch_io.torch_to_storage(ref_out, dtype)
        assert a.tobytes() == r.tobytes(), f"call {call}: differs from pa_decode_attention"
        check_close(gpu_out_f64(out, dtype), oracle_out(b), dtype, f"noalloc call {call}", extra=pv_extra(b))


def test_noalloc_refuses_partials_beyond_the_scratch():
    b = batch("bf16", 128, 16, 4, [16, 16], seed=3)
    d = torch_io.to_device(b)
    out = torch.empty_like(d.query)
    # a declared bound of 524288 tokens in 16-token partitions: 2 seqs x 8 heads x 32768
    # partials of 130 floats, 272 MB > 64 MiB; rejected before any launch
    with pytest.raises(P.PagedKVError, match="WORKSPACE"):
        P.decode_attention_noalloc(d.query, d.k_pool, d.v_pool, d.block_tables, d.context_lens, b.scale,
                                   8 * 65536, 16, out=out)
