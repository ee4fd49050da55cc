"""The five workloads at full size, in the launch configurations bench.py
times.  Every output element of every sequence is compared with the oracle
(computed once per batch), the append/copy results bit for bit over the whole
pools, and every output row is checked finite (unused slots are NaN-poisoned).

Sizes: tiny MHA fp32 (4 seqs); OPT-13B-shaped MHA fp16 (64 seqs, 40 heads,
lognormal lengths up to 2048); Llama-3-8B-shaped GQA bf16 (256 seqs, 32/8
heads, lengths 1024..8192, plus one appended token each); prefix-shared
sampling (64 prompts x 8 samples, 448 CoW copies, 131072 appended tokens);
long-context split (16 seqs, lengths 32768..131072, block size 8/16/32), run
both in the balanced split the library picks and in the 512-token partitions
followed by the cross-partition rescale merge that the workload names."""

import gc

import numpy as np
import pytest
import torch

import paged_kv_cache_313_amd as P
from workloads import synth as W
from workloads import torch_io

from gpu_util import check_close, gpu_out_f64, gpu_step, note, oracle_out, oracle_pools, pv_extra

pytestmark = pytest.mark.gpu


def full_check(b, partitions=(None,), check_pools=False):
    """One step (copies, appends, decode) with the first partition choice,
    then decode alone with each further one; all outputs against the oracle."""
    d = torch_io.to_device(b)
    k_ref, v_ref = oracle_pools(b)
    ref = oracle_out(b, k_ref, v_ref)                 # every sequence
    extra = pv_extra(b, k_ref, v_ref)
    for i, part in enumerate(partitions):
        chosen = part if part is not None else P.choose_partition(b.num_seqs, b.num_kv_heads,
                                                                  b.max_context_len, b.block_size)
        note(f"{b.name}: S={b.num_seqs} maxL={b.max_context_len} bs={b.block_size} partition={chosen}")
        out = gpu_step(b, d, partition_size=chosen, copy_append=(i == 0))
        gout = gpu_out_f64(out, b.dtype)
        assert np.isfinite(gout).all()
        if i == 0 and check_pools:
            k = torch_io.torch_to_storage(d.k_pool, b.dtype)
            v = torch_io.torch_to_storage(d.v_pool, b.dtype)
            assert k.view(np.uint8).tobytes() == k_ref.view(np.uint8).tobytes()
            assert v.view(np.uint8).tobytes() == v_ref.view(np.uint8).tobytes()
            del k, v
        stats = check_close(gout, ref, b.dtype, f"{b.name}/P{chosen}", extra=extra)
        note(f"{b.name}: partition={chosen}: all {b.num_seqs} seqs checked, max_abs={stats['max_abs']:.3g}")
        del out
    del d
    torch.cuda.empty_cache()
    gc.collect()


def test_config1_tiny_mha_f32_all_outputs():
    full_check(W.config1(), partitions=(None, 0, 16, -1))


def test_config2_opt13b_mha_f16():
    full_check(W.config2(), partitions=(None, 0, 512))


def test_config3_llama3_gqa_bf16_with_append():
    full_check(W.config3(), partitions=(None, 512), check_pools=True)


@pytest.mark.parametrize("group", [8, 16])
def test_config3_larger_groups_matrix_core_pv(group):
    # the Llama-3-8B-shaped batch with 8 x group query heads: P.V on the matrix cores
    full_check(W.config3(num_q_heads=8 * group), partitions=(None, 512))


def test_config4_prefix_shared_cow_append():
    b = W.config4()
    assert len(b.block_mapping) == 448
    full_check(b, partitions=(None, 0), check_pools=True)


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_config5_long_context_balanced_and_512_token_partitions(bs):
    b = W.config5(block_size=bs)
    assert b.partition_size == 512
    full_check(b, partitions=(None, b.partition_size))
