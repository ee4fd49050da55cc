"""The five workloads at full size, in the launch configuration bench.py times
(partition chosen by the library).  Outputs are compared with the oracle
element by element on a sample of sequences (all heads of each), the
append/copy results bit for bit over the whole pools, and every output row is
checked finite (unused slots are NaN-poisoned).

Sizes: tiny MHA fp32 (4 seqs); OPT-13B-shaped MHA fp16 (64 seqs, 40 heads,
lognormal lengths up to 2048); Llama-3-8B-shaped GQA bf16 (256 seqs, 32/8
heads, lengths 1024..8192, plus one appended token each); prefix-shared
sampling (64 prompts x 8 samples, 448 CoW copies, 131072 appended tokens);
long-context split (16 seqs, lengths 32768..131072, block size 8/16/32)."""

import gc

import numpy as np
import pytest
import torch

from workloads import synth as W
from workloads import torch_io

from gpu_util import check_close, gpu_out_f64, gpu_step, note, oracle_out, oracle_pools, pick_seqs

pytestmark = pytest.mark.gpu


def full_check(b, nseq, check_pools=False):
    d = torch_io.to_device(b)
    note(f"{b.name}: S={b.num_seqs} maxL={b.max_context_len} bs={b.block_size}")
    out = gpu_step(b, d)
    gout = gpu_out_f64(out, b.dtype)
    assert np.isfinite(gout).all()
    k_ref, v_ref = oracle_pools(b)
    if check_pools:
        k = torch_io.torch_to_storage(d.k_pool, b.dtype)
        v = torch_io.torch_to_storage(d.v_pool, b.dtype)
        assert k.view(np.uint8).tobytes() == k_ref.view(np.uint8).tobytes()
        assert v.view(np.uint8).tobytes() == v_ref.view(np.uint8).tobytes()
        del k, v
    seqs = list(range(b.num_seqs)) if nseq >= b.num_seqs else pick_seqs(b, nseq)
    ref = oracle_out(b, k_ref, v_ref, seqs=seqs)
    stats = check_close(gout[seqs], ref[seqs], b.dtype, b.name)
    note(f"{b.name}: {len(seqs)} seqs checked, max_abs={stats['max_abs']:.3g}")
    del d, out
    torch.cuda.empty_cache()
    gc.collect()


def test_config1_tiny_mha_f32_all_outputs():
    full_check(W.config1(), 4)


def test_config2_opt13b_mha_f16():
    full_check(W.config2(), 12)


def test_config3_llama3_gqa_bf16_with_append():
    full_check(W.config3(), 16, check_pools=True)


def test_config4_prefix_shared_cow_append():
    b = W.config4()
    assert len(b.block_mapping) == 448
    full_check(b, 16, check_pools=True)


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_config5_long_context_split(bs):
    full_check(W.config5(block_size=bs), 4)
