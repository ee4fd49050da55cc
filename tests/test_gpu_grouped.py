"""pa_decode_attention_grouped: the decode of samples that share a prompt's
blocks, each shared tile read once for up to 16 / G samples.  Every case is
compared with pa_decode_attention at the same fixed partition size, which
must give the same bits (each partial result is computed by the same
arithmetic, and the same merge combines them), and with the oracle."""

import numpy as np
import pytest
import torch

import paged_kv_cache_313_amd as P
from workloads import synth as W
from workloads import torch_io

from gpu_util import check_close, gpu_out_f64, gpu_step, note, oracle_out, pv_extra

pytestmark = pytest.mark.gpu


def shared_batch(seed, dtype, G, bs, prompts, samples, prefix, suffix, part, Hkv=2):
    return W.make_prefix_shared_batch(seed, num_prompts=prompts, samples=samples, prefix_len=prefix,
                                      suffix_len=suffix, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=128,
                                      dtype=dtype, block_size=bs, partition_size=part, threads=4)


def grouped_vs_plain(b, d, part, gs, gsh, max_group=None, max_shared=None):
    max_group = int(np.diff(gs).max(initial=1)) if max_group is None else max_group
    max_shared = int(gsh.max(initial=0)) if max_shared is None else max_shared
    plain = P.decode_attention(d.query, d.k_pool, d.v_pool, d.block_tables, d.context_lens, b.scale,
                               b.max_context_len, part)
    got = torch.full_like(d.query, float("nan"))
    P.decode_attention_grouped(d.query, d.k_pool, d.v_pool, d.block_tables, d.context_lens,
                               torch.from_numpy(gs).cuda(), torch.from_numpy(gsh).cuda(), max_group, max_shared,
                               b.scale, b.max_context_len, part, out=got)
    torch.cuda.synchronize()
    return plain, got


def check(b, plain, got, what):
    dt = b.dtype
    assert torch_io.torch_to_storage(got, dt).tobytes() == torch_io.torch_to_storage(plain, dt).tobytes(), \
        f"{what}: differs from pa_decode_attention"
    check_close(gpu_out_f64(got, dt), oracle_out(b), dt, what, extra=pv_extra(b))


CASES = [  # dtype, G, bs, prompts, samples, prefix, suffix, partition
    ("bf16", 4, 16, 6, 8, 1032, 256, 512),   # the prefix-shared workload's shape, fewer prompts
    ("f16", 4, 8, 3, 5, 700, 100, 256),      # 5 samples: member chunks of 4 and 1
    ("bf16", 8, 32, 4, 3, 2048, 64, 512),    # group 8: 2 samples per shared unit
    ("bf16", 16, 16, 2, 4, 1024, 40, 512),   # group 16: 1 sample per shared unit
    ("bf16", 4, 16, 4, 9, 1500, 1, 128),     # 3 member chunks, one private token, many partitions
    ("f16", 2, 16, 3, 4, 600, 50, 256),      # group 2: the plain partition pass
]


@pytest.mark.parametrize("dtype,G,bs,prompts,samples,prefix,suffix,part", CASES)
def test_grouped_decode_matches_partition_pass_and_oracle(dtype, G, bs, prompts, samples, prefix, suffix, part):
    b = shared_batch(900 + G + bs, dtype, G, bs, prompts, samples, prefix, suffix, part)
    d = torch_io.to_device(b)
    note(f"grouped decode {dtype} G={G} bs={bs} {prompts}x{samples} prefix={prefix} suffix={suffix} P={part}")
    gpu_step(b, d, decode=False)   # copy-on-write copies and the suffix appends
    gs, gsh = P.prefix_groups(b.block_tables, b.context_lens, bs)
    assert len(gs) == prompts + 1 and (gsh > 0).all()
    plain, got = grouped_vs_plain(b, d, part, gs, gsh)
    check(b, plain, got, f"grouped {dtype} G={G} bs={bs}")


def test_grouped_decode_ragged_members_and_bounds():
    """Members shorter than the shared prefix (the call shortens the shared
    part so that each member keeps a private partition), an empty member
    (its group then shares nothing), a
    declared shared length that is not a whole number of partitions, host
    bounds below the true group size and shared length (members past the
    bound, and shared tokens past it, run as ordinary partitions), a group
    of one and sequences outside every group."""
    b = shared_batch(950, "bf16", 4, 16, 4, 6, 1100, 200, 256)
    lens = b.context_lens.copy()
    lens[1] = 300        # shorter than the prefix: its group shares one partition
    lens[8] = 1025       # just past four partitions
    lens[11] = 1         # one token, alone in its group
    lens[14] = 0         # empty: its group shares nothing
    b.context_lens = lens
    d = torch_io.to_device(b)
    note("grouped decode ragged members and bounds")
    gpu_step(b, d, decode=False)
    part = 256
    # groups: prompt 0 whole, prompt 1 split into a group of 5 and a group of one,
    # prompt 2 with a declared share that is not whole partitions, prompt 3 outside every group
    gs = np.array([0, 6, 11, 12, 18], np.int32)
    gsh = np.array([1024, 1024, 1024, 1000], np.int32)
    for mg, ms in ((6, 1024), (3, 1024), (6, 512), (6, 0)):
        plain, got = grouped_vs_plain(b, d, part, gs, gsh, max_group=mg, max_shared=ms)
        check(b, plain, got, f"ragged groups, max_group_size {mg}, max_shared_len {ms}")
        assert (gpu_out_f64(got, "bf16")[14] == 0).all()


def test_grouped_decode_without_groups_and_unsplit():
    """No groups at all, and a batch that fits one partition (no split): the
    plain paths run."""
    b = shared_batch(960, "bf16", 4, 16, 2, 4, 200, 40, 256)
    d = torch_io.to_device(b)
    note("grouped decode without groups / unsplit")
    gpu_step(b, d, decode=False)
    none_s, none_h = np.zeros(1, np.int32), np.zeros(0, np.int32)
    plain, got = grouped_vs_plain(b, d, 256, none_s, none_h, max_group=1, max_shared=0)
    check(b, plain, got, "no groups")
    gs, gsh = P.prefix_groups(b.block_tables, b.context_lens, 16)
    plain, got = grouped_vs_plain(b, d, 512, gs, gsh)
    check(b, plain, got, "one partition")


def test_grouped_decode_config4_full_size():
    """The prefix-shared workload at full size (64 prompts x 8 samples): bit
    for bit against 512-token partitions, the oracle on sampled sequences."""
    b = W.config4()
    d = torch_io.to_device(b)
    note("grouped decode, prefix-shared workload at full size")
    gpu_step(b, d, decode=False)
    gs, gsh = P.prefix_groups(b.block_tables, b.context_lens, b.block_size)
    assert len(gs) == 65 and (gsh == 1024).all()
    plain, got = grouped_vs_plain(b, d, 512, gs, gsh)
    dt = b.dtype
    assert torch_io.torch_to_storage(got, dt).tobytes() == torch_io.torch_to_storage(plain, dt).tobytes()
    seqs = [0, 7, 8, 255, 300, 511]
    ref = oracle_out(b, seqs=seqs)
    ex = pv_extra(b, seqs=seqs)
    check_close(gpu_out_f64(got, dt)[seqs], ref[seqs], dt, "prefix-shared full size", extra=ex[seqs])
