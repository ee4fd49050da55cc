#!/usr/bin/env python3
"""Decode-step benchmark of the paged-KV hot path on one MI355X.

A step is one pass of the whole path over one synthetic batch, with inputs
already resident in HBM: copy-on-write block copies (prefix-shared workload
only), the KV append of the step's new tokens, and paged decode attention
(partition pass + merge).  Default workload: the Llama-3-8B-shaped GQA batch
(256 sequences, 32 q / 8 KV heads, head_dim 128, bf16, 16-token blocks,
lengths uniform in [1024, 8192] plus one appended token each).

Prints ONE JSON line: seq-steps/s (value), KV-read GB/s and the fraction of
the 8 TB/s HBM peak for the decode call (roofline), and the CPU oracle timed
on the host cores over the same batch (cpu_baseline).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "decode seq-steps/s + achieved KV-read GB/s (% of MI355X HBM peak), 1 GPU"
# rocprofv3 HBM byte counters of the decode call, one file per workload (and
# per non-default partition choice), written by --ingest-counters
PROFILE_STEMS = {1: "decode_tiny_mha_f32", 2: "decode_mha_opt13b", 3: "decode_gqa_llama3_8b",
                 4: "decode_prefix_shared_sampling", 5: "decode_long_context"}


def counters_file(config, block_size=16, partition=None):
    """profiles/<workload>[_bs<block size>][_p<partition>]_counters.json; the
    suffix _p<P> only when the partition is not the library's choice."""
    stem = PROFILE_STEMS[config] + (f"_bs{block_size}" if config == 5 else "")
    if partition is not None:
        stem += f"_p{partition}"
    return os.path.join(ROOT, "profiles", stem + "_counters.json")
SETTLE_S = 0.06   # seconds of whole steps before the timed region (clock settling)
KERNEL_SOURCES = ["paged_kv_cache_313_amd/csrc/pa_decode_core.hpp",
                  "paged_kv_cache_313_amd/csrc/pa_common.hpp"]

WORKLOADS = {
    1: "tiny MHA decode: 4 seqs, 8 heads, D64, fp32, bs16, lens {5,17,33,64}",
    2: "OPT-13B-shaped MHA decode: 64 seqs, 40 heads, D128, fp16, bs16, lognormal lens (median 512, [16,2048])",
    3: "Llama-3-8B-shaped GQA decode: 256 seqs, 32q/8kv heads, D128, bf16, bs16, lens U[1024,8192] + 1 appended token",
    4: "prefix-shared sampling: 64 prompts x 8 samples, GQA 32/8, D128, bf16, bs16, 1032-token shared prompt, 448 CoW copies, 256-token suffix append, decode over 1288",
    5: "long-context split decode: 16 seqs, GQA 32/8, D128, bf16, lens U[32768,131072], 512-token partitions",
}


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, choices=sorted(WORKLOADS))
    ap.add_argument("--block-size", type=int, default=16, help="block size of the long-context workload")
    ap.add_argument("--partition", type=int, default=None, help="partition size (default: library choice)")
    ap.add_argument("--table-layout", default="shuffled", choices=["shuffled", "identity", "hier"],
                    help="physical layout: shuffled blocks, identity (contiguous) tables, or two-level tables "
                         "with the prompt in 256-token large pages")
    ap.add_argument("--group", type=int, default=None, choices=[2, 4, 8, 16],
                    help="GQA group size of the Llama-3-8B-shaped workload (query heads = 8 x group; default 4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-swap", action="store_true", help="skip the swap (preemption traffic) leg")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill leg")
    ap.add_argument("--no-aux", action="store_true",
                    help="skip the cold-cache, achievable-read, step-latency and block-manager legs (profiled runs)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of HIP-graph replays")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only time pa_prefill_attention on the chunked-prefill workload and print its line")
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="minimum wall time of the oracle timing")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (5 times), the "
                         "reference kernel for scaling HBM byte counters, and exit")
    ap.add_argument("--ingest-grouped-counters", metavar="DIR", default=None,
                    help="only read FETCH_SIZE / WRITE_SIZE passes (and the copy calibration) under DIR of a "
                         "--config 4 run with its grouped leg, write the grouped decode's HBM bytes per call to "
                         "the profiles counters file, and exit (no GPU)")
    ap.add_argument("--ingest-counters", metavar="DIR", default=None,
                    help="only read rocprofv3 --pmc csv output under DIR/{fetch,write,calf,calw} (FETCH_SIZE and "
                         "WRITE_SIZE passes of the default decode bench and of --calibrate-copy-mib 1024), write "
                         "the decode call's HBM bytes to the profiles counters file, and exit (no GPU)")
    return ap.parse_args()


def calibrate_copy(mib):
    import torch
    n = mib << 20
    x = torch.ones(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n, "launches": 5}), flush=True)


def _pmc_per_dispatch(root, counter):
    """Mean of `counter` per dispatch, by kernel name, over every
    *counter_collection.csv under `root` (one row per dispatch and counter)."""
    import csv
    import glob
    sums, counts = {}, {}
    files = glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {root}")
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                k = row["Kernel_Name"]
                sums[k] = sums.get(k, 0.0) + float(row["Counter_Value"])
                counts[k] = counts.get(k, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


def _counter_passes(root):
    """FETCH_SIZE / WRITE_SIZE per dispatch (KiB) under root/{fetch,write},
    the scale factors from the plain 1 GiB copy under root/{calf,calw}, and a
    picker of the one kernel whose name holds a tag."""
    calib = 1 << 30
    fetch, write = _pmc_per_dispatch(os.path.join(root, "fetch"), "FETCH_SIZE"), \
        _pmc_per_dispatch(os.path.join(root, "write"), "WRITE_SIZE")
    calf, calw = _pmc_per_dispatch(os.path.join(root, "calf"), "FETCH_SIZE"), \
        _pmc_per_dispatch(os.path.join(root, "calw"), "WRITE_SIZE")
    copy_k = max(calf, key=calf.get)
    cal = {"copy_bytes": calib, "copy_kernel": copy_k, "fetch_kib": calf[copy_k], "write_kib": calw[copy_k],
           "fetch_factor": (calib / 1024) / calf[copy_k], "write_factor": (calib / 1024) / calw[copy_k]}

    def pick(d, tag):
        ks = [k for k in d if tag in k]
        if len(ks) != 1:
            raise SystemExit(f"expected one kernel named like {tag!r}, found {ks}")
        return ks[0]
    return fetch, write, cal, pick


GROUPED_COUNTERS = os.path.join(ROOT, "profiles", "decode_prefix_shared_sampling_grouped_counters.json")


def ingest_grouped_counters(root, out_path=GROUPED_COUNTERS):
    """The grouped decode's HBM bytes per call (its group kernel and its
    merge), from FETCH_SIZE / WRITE_SIZE passes over a prefix-shared run
    that includes bench's grouped leg, keyed by the kernel sources' hash."""
    fetch, write, cal, pick = _counter_passes(root)
    ff, wf = cal["fetch_factor"], cal["write_factor"]
    gk = pick(fetch, "decode_group_kernel")
    mk = pick(fetch, "decode_merge_few_kernel" if any("decode_merge_few_kernel" in k for k in fetch)
              else "decode_merge_parts_kernel")
    out = {"source_sha": source_sha(), "kernel": gk, "merge_kernel": mk, "calibration": cal,
           "fetch_bytes_per_call": (fetch[gk] + fetch[mk]) * 1024 * ff,
           "write_bytes_per_call": (write[gk] + write[mk]) * 1024 * wf,
           "group_kernel_fetch_bytes": fetch[gk] * 1024 * ff, "group_kernel_write_bytes": write[gk] * 1024 * wf}
    out["hbm_bytes_per_call"] = out["fetch_bytes_per_call"] + out["write_bytes_per_call"]
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))
    return out


def ingest_counters(root, config=3, partition=-1, out_path=None, block_size=16, explicit_partition=False):
    """Turn FETCH_SIZE / WRITE_SIZE passes (KiB per dispatch) into bytes per
    decode call, each scaled by what the same counter reads for a plain copy of
    known size, and store them keyed by the kernel sources' hash.  `partition`
    names the decode kernels: -1 the balanced kernel + its merge, P > 0 the
    unit kernel + the partition merge, 0 the unit kernel alone."""
    fetch, write, calib, pick = _counter_passes(root)
    ff, wf = calib["fetch_factor"], calib["write_factor"]
    if partition == -1:
        dk, mk = pick(fetch, "decode_balanced_kernel"), pick(fetch, "decode_merge_balanced_kernel")
    elif partition > 0:   # fixed partitions: the resident-grid kernel (the unit kernel above 4096 sequences)
        resident = [k for k in fetch if "decode_parts_resident_kernel" in k]
        dk = pick(fetch, "decode_parts_resident_kernel" if resident else "decode_unit_kernel")
        few = any("decode_merge_few_kernel" in k for k in fetch)   # at most 8 partitions
        mk = pick(fetch, "decode_merge_few_kernel" if few else "decode_merge_parts_kernel")
    else:
        dk, mk = pick(fetch, "decode_unit_kernel"), None
    dec_f, dec_w = fetch[dk] * 1024 * ff, write[dk] * 1024 * wf
    mrg_f, mrg_w = (fetch[mk] * 1024 * ff, write[mk] * 1024 * wf) if mk else (0.0, 0.0)
    out = {"config": config, "partition": partition, "block_size": block_size, "source_sha": source_sha(),
           "kernel": dk, "fetch_kib_per_dispatch": fetch[dk], "write_kib_per_dispatch": write[dk],
           "calibration": calib,
           "merge_kernel": None if mk is None else {
               "name": mk, "fetch_kib_per_dispatch": fetch[mk], "write_kib_per_dispatch": write[mk],
               "fetch_bytes": mrg_f, "write_bytes": mrg_w},
           "decode_kernel_bytes": dec_f + dec_w, "fetch_bytes_per_launch": dec_f + mrg_f,
           "write_bytes_per_launch": dec_w + mrg_w, "hbm_bytes_per_launch": dec_f + dec_w + mrg_f + mrg_w,
           "note": "hbm_bytes_per_launch covers one pa_decode_attention call: the decode kernel and its merge"}
    path = out_path or counters_file(config, block_size, partition if explicit_partition else None)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))
    return out


LARGE_PAGE_BLOCKS = 16   # two-level layout: 256-token large pages at bs 16


def make_batch(args):
    from workloads import synth as W
    kw = {}
    hier = args.table_layout == "hier"
    if args.config in (2, 3, 5):
        kw["table_layout"] = "shuffled" if hier else args.table_layout
    if args.group is not None:
        if args.config != 3:
            raise SystemExit("--group applies to the Llama-3-8B-shaped workload (--config 3)")
        kw["num_q_heads"] = 8 * args.group
    if args.config == 5:
        b = W.config5(block_size=args.block_size, **kw)
    else:
        b = W.CONFIGS[args.config](**kw)
    if hier:
        if b.block_mapping is not None and len(b.block_mapping):
            raise SystemExit("--table-layout hier: not for the copy-on-write workload")
        # everything before the step's appended token is the prompt: large pages
        hb, large, nl = W.to_hierarchical(b, LARGE_PAGE_BLOCKS, b.context_lens - 1, seed=313009)
        hb.meta["hier"] = (large, nl, LARGE_PAGE_BLOCKS)
        return hb
    return b


# ----------------------------------------------------------------------------- CPU oracle leg
_CPU_BATCH = None


def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _cpu_seq(s):
    import numpy as np
    import oracle.pa_oracle as O
    b = _CPU_BATCH
    G = b.num_q_heads // b.num_kv_heads
    out = np.empty((b.num_q_heads, b.head_dim))
    for g in range(b.num_kv_heads):
        out[g * G:(g + 1) * G] = O.decode_group(b.query, b._k_after, b._v_after, b.block_tables,
                                                b.context_lens, b.scale, b.block_size, b.dtype, s, g)
    return s, out


def cgroup_cpu_limit():
    """CPUs granted by the cgroup's CPU quota (cgroup v2 cpu.max or v1
    cfs_quota/period), or None when unlimited or unreadable."""
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        return None if quota == "max" else int(quota) / int(period)
    except (OSError, ValueError):
        pass
    try:
        with open("/sys/fs/cgroup/cpu/cpu.cfs_quota_us") as f:
            quota = int(f.read())
        with open("/sys/fs/cgroup/cpu/cpu.cfs_period_us") as f:
            period = int(f.read())
        return None if quota <= 0 else quota / period
    except (OSError, ValueError):
        return None


def cpu_share():
    """Worker processes for the oracle: the CPUs this process may run on
    (sched_getaffinity), cut to the cgroup quota and to OMP_NUM_THREADS when
    the host sets them (a shared GPU host states each job's CPU share that way)."""
    aff = len(os.sched_getaffinity(0))
    quota = cgroup_cpu_limit()
    omp = os.environ.get("OMP_NUM_THREADS", "")
    cores = aff
    if quota:
        cores = min(cores, max(1, int(quota)))
    if omp.isdigit() and int(omp) > 0:
        cores = min(cores, int(omp))
    return max(1, cores), {"affinity_cpus": aff, "cgroup_cpu_limit": quota, "omp_num_threads": omp or None}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_single_core(b, min_seconds=2.0, max_passes=20):
    """The oracle over the whole batch in this process on one core (one BLAS
    thread): seq-steps/s.  Used for the small workloads only."""
    import numpy as np
    import oracle.pa_oracle as O
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except Exception:
        limit = None
    try:
        G = b.num_q_heads // b.num_kv_heads
        out = np.empty((b.num_seqs, b.num_q_heads, b.head_dim))
        passes = 0
        t0 = time.perf_counter()
        while True:
            for s in range(b.num_seqs):
                for g in range(b.num_kv_heads):
                    out[s, g * G:(g + 1) * G] = O.decode_group(b.query, b._k_after, b._v_after, b.block_tables,
                                                               b.context_lens, b.scale, b.block_size, b.dtype,
                                                               s, g)
            passes += 1
            el = time.perf_counter() - t0
            if el >= min_seconds or passes >= max_passes:
                break
    finally:
        if limit is not None:
            limit.restore_original_limits()
    return {"value": b.num_seqs * passes / el, "unit": "seq-steps/s", "cores": 1,
            "sample": f"all {b.num_seqs} sequences, {passes} passes in {el:.2f} s, 1 process x 1 BLAS thread"}


def cpu_baseline(b, min_seconds, single_core=False):
    """The fp64 oracle, unchanged, over the whole batch: the step's CoW copies
    and appends, then attention for every sequence, sequences dealt
    longest-first to one worker process per CPU of this job's share (one BLAS
    thread each)."""
    import multiprocessing as mp

    import numpy as np
    import oracle.pa_oracle as O
    global _CPU_BATCH
    cores, share = cpu_share()
    if "hier" in b.meta:     # the oracle reads two-level tables through their flat expansion
        import dataclasses
        large, nl, H = b.meta["hier"]
        b = dataclasses.replace(b, block_tables=O.expand_hier_tables(large, nl, b.block_tables, H))
    # pools after the step (oracle copies + appends); the timed loop redoes them
    k, v = b.k_pool, b.v_pool
    if b.block_mapping is not None and len(b.block_mapping):
        k, v = k.copy(), v.copy()
        O.block_copy(k, v, b.block_mapping)
    if b.new_key is not None:
        if k is b.k_pool:
            k, v = k.copy(), v.copy()
        O.kv_append(k, v, b.new_key, b.new_value, b.slot_mapping, b.block_size)
    b._k_after, b._v_after = k, v
    _CPU_BATCH = b
    order = sorted(range(b.num_seqs), key=lambda s: -int(b.context_lens[s]))
    ctx = mp.get_context("fork")
    out = np.empty((b.num_seqs, b.num_q_heads, b.head_dim))
    passes = 0
    with ctx.Pool(cores, initializer=_cpu_worker_init) as pool:
        t0 = time.perf_counter()
        while True:
            if b.new_key is not None:   # redo the step's appends in place (idempotent)
                O.kv_append(k, v, b.new_key, b.new_value, b.slot_mapping, b.block_size)
            for s, o in pool.imap_unordered(_cpu_seq, order, chunksize=1):
                out[s] = o
            passes += 1
            el = time.perf_counter() - t0
            if el >= min_seconds or passes >= 50:
                break
    value = b.num_seqs * passes / el
    res = {"value": value, "unit": "seq-steps/s", "cores": cores, "kind": "oracle",
           "sample": f"all {b.num_seqs} sequences of the workload (step's CoW copies + appends + fp64 attention), "
                     f"{passes} passes in {el:.2f} s, {cores} worker processes x 1 BLAS thread",
           "kv_gbps_equiv": b.kv_bytes() * passes / el / 1e9,
           "cpu_model": cpu_model(), "cpu_share": share}
    if single_core:
        res["single_core"] = cpu_single_core(b)
    return res, out


# ----------------------------------------------------------------------------- GPU leg
def algorithmic_bytes(b):
    """Bytes the decode call must move: K/V of the valid tokens, query, output,
    block-table entries and lengths.  Partial results of a split are the
    implementation's overhead and are not counted."""
    import numpy as np
    L = b.context_lens.astype(np.int64)
    kv = b.kv_bytes()
    qo = 2 * b.num_seqs * b.num_q_heads * b.head_dim * b.elt_bytes
    nblk = -(-L // b.block_size)
    if "hier" in b.meta:       # large-page entries, small entries and the large-page counts
        _, nl, H = b.meta["hier"]
        nl = nl.astype(np.int64)
        tbl = int((nl + nblk - nl * H).sum()) * 4 + b.num_seqs * 8
    else:
        tbl = int(nblk.sum()) * 4 + b.num_seqs * 4
    return kv + qo + tbl, kv


def unique_kv_bytes(b):
    """K+V bytes of the distinct physical blocks the decode reads: a block that
    several sequences share (a prompt's blocks under parallel sampling) counts
    once, with the most valid tokens any of its readers uses.  Two-level
    layouts share nothing and equal the logical bytes."""
    import numpy as np
    if "hier" in b.meta:
        return b.kv_bytes()
    bs = b.block_size
    L = b.context_lens.astype(np.int64)
    nblk = -(-L // bs)
    blocks, toks = [], []
    for s in range(b.num_seqs):
        n = int(nblk[s])
        if n == 0:
            continue
        blocks.append(b.block_tables[s, :n].astype(np.int64))
        t = np.full(n, bs, dtype=np.int64)
        t[-1] = L[s] - (n - 1) * bs
        toks.append(t)
    if not blocks:
        return 0
    most = np.zeros(b.num_blocks, dtype=np.int64)
    np.maximum.at(most, np.concatenate(blocks), np.concatenate(toks))
    return int(most.sum()) * b.num_kv_heads * b.head_dim * 2 * b.elt_bytes


def decode_kernel_name(b, part):
    G = b.num_q_heads // b.num_kv_heads
    core = "ValuCore" if G == 1 or b.dtype == "f32" else ("MfmaPvCore" if G >= 4 and b.head_dim == 128 else "MfmaCore")
    if part == -1:
        return f"pa_decode_attention: decode_balanced_kernel<{core}> + decode_merge_balanced_kernel"
    if part and part > 0:
        if b.max_context_len <= part:   # one partition: no split, no merge
            return f"pa_decode_attention: decode_unit_kernel<{core}>"
        kern = "decode_parts_resident_kernel" if b.num_seqs <= 4096 else "decode_unit_kernel"
        few = b.head_dim == 128 and -(-b.max_context_len // part) <= 8   # at most 8 partitions
        return f"pa_decode_attention: {kern}<{core}> + {'decode_merge_few_kernel' if few else 'decode_merge_parts_kernel'}"
    return f"pa_decode_attention: decode_unit_kernel<{core}>"


def source_sha():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_from_profile(config, partition, block_size=16, explicit_partition=False):
    """The decode call's counter file for this workload, or None when there is
    none or the kernel sources changed since it was taken."""
    try:
        with open(counters_file(config, block_size, partition if explicit_partition else None)) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if (c.get("source_sha") != source_sha() or c.get("config") != config or c.get("partition") != partition
            or c.get("block_size", 16) != block_size):
        return None
    return c


def block_manager_leg(b, steps: int) -> dict:
    """Host cost of the native block manager for this batch's decode step:
    every sequence reserves one new slot (append_slots) and the batch's block
    tables are emitted (block_tables), through the Python binding."""
    import numpy as np

    import paged_kv_cache_313_amd as P

    S, bs = b.num_seqs, b.block_size
    lens = b.context_lens.astype(np.int64)
    need = int(((lens + steps + 1 + bs - 1) // bs).sum())
    bm = P.BlockManager(need + S, bs)
    ids = np.array([bm.add_sequence() for _ in range(S)], dtype=np.int64)
    t = time.perf_counter()
    bm.append_slots(ids, lens.astype(np.int32))          # the batch's existing context
    t_fill = time.perf_counter() - t
    ones = np.ones(S, dtype=np.int32)
    mb = int((lens.max() + steps + bs) // bs) + 1
    t_app, t_tab = [], []
    for _ in range(steps):
        t0 = time.perf_counter()
        bm.append_slots(ids, ones)
        t1 = time.perf_counter()
        bm.block_tables(ids, mb)
        t2 = time.perf_counter()
        t_app.append(t1 - t0)
        t_tab.append(t2 - t1)
    bm.close()
    return {"seqs": S, "append_slots_us": 1e6 * float(np.median(t_app)),
            "block_tables_us": 1e6 * float(np.median(t_tab)),
            "fill_context_ms": 1e3 * t_fill, "steps": steps,
            "what": "median host time per decode step of pa_bm_append_slots (1 token per sequence) and "
                    "pa_bm_block_tables (padded int32 tables), Python binding included"}


HOST_LINK_PEAK_GBPS = 64.0   # PCIe 5.0 x16, one direction
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of MI355X
PREFILL_WORKLOAD = ("chunked prefill over cached prefixes, Llama-3-8B-shaped: 16 seqs, 512 new tokens each "
                    "on 4096-token contexts (3584 cached), 32q/8kv heads, D128, bf16, bs16, causal")


def prefill_leg(reps: int = 20, parity_seqs=(0, 9), fresh: bool = True) -> dict:
    """pa_prefill_attention on the chunked-prefill workload: HIP-event time per
    call, causal TFLOP/s against the bf16 matrix-core peak, and every output
    of two sampled sequences against the oracle; with `fresh`, also the time
    on fresh prompts (`fresh_prompts`)."""
    import numpy as np
    import torch

    import paged_kv_cache_313_amd as P
    from workloads import synth as W
    from workloads import torch_io

    S, n, L, Hq, Hkv, D, bs = 16, 512, 4096, 32, 8, 128, 16
    b = W.make_decode_batch(313100, num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype="bf16",
                            block_size=bs, context_lens=[L] * S, name="prefill")
    rng = np.random.default_rng(313101)
    q = W.to_storage(rng.standard_normal((S * n, Hq, D), dtype=np.float32), "bf16")
    starts = np.arange(0, (S + 1) * n, n, dtype=np.int32)
    d = torch_io.to_device(b)
    qd = torch_io.storage_to_torch(q, "bf16", "cuda")
    st = torch.from_numpy(starts).cuda()
    out = torch.empty_like(qd)
    stream = torch.cuda.current_stream()
    f = lambda: P.prefill_attention(qd, d.k_pool, d.v_pool, d.block_tables, d.context_lens, st, b.scale, n,
                                    out=out, stream=stream)
    # warm-up: the leg follows the swap leg, during which the GPU is mostly
    # idle, and from there the first ~50 calls (~30 ms) ran up to 20 % slower
    # while the clock settled; 100 calls (~55 ms) reach the steady rate.
    for _ in range(100):
        f()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        f()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    keys = S * sum(L - n + j + 1 for j in range(n))          # (query token, key) pairs under the causal mask
    flops = 4.0 * D * keys * Hq                               # QK^T and PV, 2 flops per multiply-add
    tflops = flops / (ms * 1e-3) / 1e12
    parity = None
    if parity_seqs:
        import oracle.pa_oracle as O
        ref = O.prefill_attention(q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, starts, b.scale, bs,
                                  "bf16", seqs=list(parity_seqs))
        got = O.upcast(torch_io.torch_to_storage(out, "bf16"), "bf16")
        rows = np.concatenate([np.arange(starts[s], starts[s + 1]) for s in parity_seqs])
        err = np.abs(got[rows] - ref[rows])
        parity = {"max_abs_err": float(err.max()),
                  "within_tolerance": bool((err <= 2e-2 + 1e-2 * np.abs(ref[rows])).all()),
                  "checked": f"all outputs of sequences {list(parity_seqs)} vs the fp64 oracle"}
    del d, qd, st, out
    fresh = _fresh_prompt_prefill(reps) if fresh else None
    return {"workload": PREFILL_WORKLOAD, "ms": ms, "tflops": tflops, "flops_per_call": flops,
            "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                         "kernel": "pa_prefill_attention: prefill_kernel<BF16, 128, 4, 8> (8-wave workgroups)"},
            "parity": parity, "fresh_prompts": fresh}


def _fresh_prompt_prefill(reps: int) -> dict:
    """The same call on fresh prompts (no cached prefix: every token new),
    4 x 4096 tokens with the same heads, timed the same way after the chunked
    workload has warmed the clock.  Its outputs are checked against the oracle
    by the GPU tests (fresh prompts, several query-block bands), not here."""
    import numpy as np
    import torch

    import paged_kv_cache_313_amd as P
    from workloads import synth as W
    from workloads import torch_io

    S, L, Hq, Hkv, D, bs = 4, 4096, 32, 8, 128, 16
    b = W.make_decode_batch(313102, num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype="bf16",
                            block_size=bs, context_lens=[L] * S, name="prefill-fresh")
    rng = np.random.default_rng(313103)
    q = W.to_storage(rng.standard_normal((S * L, Hq, D), dtype=np.float32), "bf16")
    d = torch_io.to_device(b)
    qd = torch_io.storage_to_torch(q, "bf16", "cuda")
    st = torch.from_numpy(np.arange(0, (S + 1) * L, L, dtype=np.int32)).cuda()
    out = torch.empty_like(qd)
    stream = torch.cuda.current_stream()
    f = lambda: P.prefill_attention(qd, d.k_pool, d.v_pool, d.block_tables, d.context_lens, st, b.scale, L,
                                    out=out, stream=stream)
    for _ in range(30):
        f()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        f()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 4.0 * D * S * (L * (L + 1) // 2) * Hq
    tflops = flops / (ms * 1e-3) / 1e12
    return {"workload": f"fresh prompts: {S} x {L} tokens, no cached prefix, 32q/8kv heads, D128, bf16, bs16, causal",
            "ms": ms, "tflops": tflops, "frac_of_bf16_peak": tflops / MFMA_BF16_PEAK_TFLOPS}


def swap_leg(d, b, reps: int = 5, target_bytes: int = 1 << 30) -> dict:
    """Preemption traffic: pa_swap_out / pa_swap_in of about 1 GiB of whole
    blocks between the pools and a pinned block-first host buffer, timed with
    HIP events; out and in at once on two streams (both link directions); and
    a plain torch device-to-host copy of the same bytes as the link's
    achievable rate.  Swap-in writes back the bytes swap-out read, so the
    pools are left as they were."""
    import numpy as np
    import torch

    import paged_kv_cache_313_amd as P

    blk_bytes = 2 * b.num_kv_heads * b.block_size * b.head_dim * b.elt_bytes
    n = int(min(b.num_blocks // 2, max(1, target_bytes // blk_bytes)))
    rng = np.random.default_rng(7)
    perm = rng.permutation(b.num_blocks).astype(np.int32)
    ids_a = torch.from_numpy(perm[:n]).cuda()
    ids_b = torch.from_numpy(perm[n:2 * n]).cuda()
    host_a = P.swap_buffer(n, d.k_pool)
    host_b = P.swap_buffer(n, d.k_pool)
    nbytes = n * blk_bytes
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream()

    def timed(fn, stream):
        ms = []
        for _ in range(reps + 1):
            e0 = torch.cuda.Event(enable_timing=True); e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream); fn(); e1.record(stream)
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms[1:]))

    out_ms = timed(lambda: P.swap_out(d.k_pool, d.v_pool, ids_a, host_a, stream=s0), s0)
    in_ms = timed(lambda: P.swap_in(host_a, d.k_pool, d.v_pool, ids_a, stream=s0), s0)
    P.swap_out(d.k_pool, d.v_pool, ids_b, host_b, stream=s0)
    torch.cuda.synchronize()
    walls = []
    for _ in range(reps):
        t0 = time.perf_counter()
        P.swap_out(d.k_pool, d.v_pool, ids_a, host_a, stream=s0)
        P.swap_in(host_b, d.k_pool, d.v_pool, ids_b, stream=s1)
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
    duplex_ms = 1e3 * float(np.median(walls))
    flat_dev = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    flat_host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    d2h_ms = timed(lambda: flat_host.copy_(flat_dev, non_blocking=True), s0)
    h2d_ms = timed(lambda: flat_dev.copy_(flat_host, non_blocking=True), s0)
    gbps = lambda ms, k=1: k * nbytes / (ms * 1e-3) / 1e9
    return {"blocks": n, "bytes": nbytes, "block_bytes": blk_bytes,
            "swap_out_ms": out_ms, "swap_out_gbps": gbps(out_ms),
            "swap_in_ms": in_ms, "swap_in_gbps": gbps(in_ms),
            "duplex_ms": duplex_ms, "duplex_gbps": gbps(duplex_ms, 2),
            "plain_d2h_gbps": gbps(d2h_ms), "plain_h2d_gbps": gbps(h2d_ms),
            "link_peak_gbps_per_direction": HOST_LINK_PEAK_GBPS,
            "what": "random scattered blocks <-> pinned block-first host buffer, one launch per list; "
                    "duplex = swap-out and swap-in of two lists at once on two streams (wall time); "
                    "plain = one contiguous torch copy of the same bytes"}


def grouped_decode_leg(b, d, stream, alg_unique: int, step_decode_ms: float, K: int = 20,
                       partition_size: int = 1024) -> dict:
    """The prefix-shared batch through pa_decode_attention_grouped: the
    samples of a prompt read each shared K/V tile once per 16 / G of them
    instead of once each.  Groups come from the tables on the host (outside
    the timed region, as a block manager that forked the samples would hand
    them over).  Time per call over a HIP graph of K calls after the clock
    has settled, the distinct-bytes roofline, and the bit-for-bit check
    against pa_decode_attention with the same partitions."""
    import numpy as np
    import torch

    import paged_kv_cache_313_amd as P

    gs, gsh = P.prefix_groups(b.block_tables, b.context_lens, b.block_size)
    max_group, max_shared = int(np.diff(gs).max(initial=1)), int(gsh.max(initial=0))
    gsd, gshd = torch.from_numpy(gs).cuda(), torch.from_numpy(gsh).cuda()
    ws = torch.empty(max(16, P.decode_workspace_bytes(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim,
                                                      b.max_context_len, partition_size)),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d.query)

    def call(st):
        P.decode_attention_grouped(d.query, d.k_pool, d.v_pool, d.block_tables, d.context_lens, gsd, gshd,
                                   max_group, max_shared, b.scale, b.max_context_len, partition_size, out=out,
                                   workspace=ws, stream=st)

    call(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(stream)
    with torch.cuda.graph(g, stream=cs):
        for _ in range(K):
            call(cs)
    stream.wait_stream(cs)
    t_end = time.perf_counter() + SETTLE_S
    while True:
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            break
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / K
    plain = P.decode_attention(d.query, d.k_pool, d.v_pool, d.block_tables, d.context_lens, b.scale,
                               b.max_context_len, partition_size, workspace=ws)
    call(stream)
    torch.cuda.synchronize()
    same = bool(torch.equal(out.view(torch.int16), plain.view(torch.int16)))
    achieved = alg_unique / (ms * 1e-3) / 1e9
    traffic = None   # HBM bytes per call from rocprofv3 passes, while the kernel sources are unchanged
    try:
        with open(GROUPED_COUNTERS) as f:
            ctr = json.load(f)
        if ctr.get("source_sha") == source_sha():
            traffic = ctr["hbm_bytes_per_call"]
    except (OSError, ValueError):
        pass
    return {"ms": ms, "partition_size": partition_size, "groups": len(gsh), "max_group_size": max_group,
            "shared_tokens": max_shared, "achieved_gbps": achieved, "frac_of_hbm_peak": achieved / HBM_PEAK_GBPS,
            "speedup_vs_step_decode": step_decode_ms / ms, "bit_identical_to_partitions": same,
            "traffic": traffic, "traffic_over_algorithmic": None if traffic is None else traffic / alg_unique,
            "what": "pa_decode_attention_grouped over the step's pools (prompt groups from the tables), "
                    "HIP graph of K calls; bytes as roofline.algorithmic_bytes_per_launch"}


def cold_decode_leg(decode_call, stream, reps: int = 10, evict_bytes: int = 1 << 30) -> dict:
    """Decode time with nothing of the batch left in the caches: before each
    timed call a 1 GiB scratch buffer is read through (it evicts the 256 MB
    MALL and every L2 with clean lines, so no write-back competes with the
    call), then the call alone is timed with HIP events."""
    import numpy as np
    import torch

    scratch = torch.ones(evict_bytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty((), dtype=torch.int64, device="cuda")
    ms = []
    for i in range(reps + 1):
        torch.sum(scratch, dim=0, dtype=torch.int64, out=sink)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        decode_call()
        e1.record(stream)
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    del scratch, sink
    return {"decode_ms_median": float(np.median(ms[1:])), "reps": reps,
            "what": "median of per-call HIP-event times, each call after reading a 1 GiB scratch buffer"}


def step_latency_leg(step_fn, stream, graphs, n: int = 20) -> dict:
    """Percentiles of single-step latency: n steps, each bracketed by HIP
    events on the stream.  A read of a 64 MiB buffer is queued before each
    step (a 1 GiB one before the first), so that the host has queued the
    events and the step before the GPU reaches them and no launch gap is
    timed.  Steps replay a one-step HIP graph when graphs are in use."""
    import numpy as np
    import torch

    run = step_fn
    if graphs:
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(stream)
        with torch.cuda.graph(g, stream=cs):
            step_fn(cs)
        stream.wait_stream(cs)
        run = lambda st: g.replay()
    big = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    small = big[: 1 << 24]
    sink = torch.empty((), dtype=torch.int64, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    torch.sum(big, dim=0, dtype=torch.int64, out=sink)
    for e0, e1 in ev:
        torch.sum(small, dim=0, dtype=torch.int64, out=sink)
        e0.record(stream)
        run(stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    del big, small, sink
    return {"steps": n, "p10_ms": float(np.percentile(ms, 10)), "p50_ms": float(np.percentile(ms, 50)),
            "p90_ms": float(np.percentile(ms, 90)), "min_ms": float(ms.min()), "max_ms": float(ms.max()),
            "what": "per-step HIP-event times, each step queued behind a 64 MiB read so no launch gap is timed"}


def achievable_read_leg(stream, nbytes: int = 4 << 30, reps: int = 10) -> dict:
    """The box's achievable HBM read bandwidth: pa_stream_read sweeping a
    4 GiB buffer (16 times the MALL), reps back-to-back calls timed with HIP
    events on the stream, after two untimed ones."""
    import torch

    import paged_kv_cache_313_amd as P

    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    partials = torch.empty(P._lib.PA_STREAM_READ_PARTIALS, dtype=torch.int32, device="cuda")
    with torch.cuda.stream(stream):
        for _ in range(2):
            P.stream_read(buf, partials)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            P.stream_read(buf, partials)
        e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del buf, partials
    return {"gbps": nbytes / (ms * 1e-3) / 1e9, "bytes": nbytes, "ms": ms, "reps": reps,
            "what": "pa_stream_read: each workgroup sweeps a contiguous range of a 4 GiB buffer in 16-byte "
                    "loads, 8 in flight per thread; decode_frac_of_achievable = roofline.achieved / gbps"}


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the decode path here is a single-GPU kernel; sharding across GPUs is not implemented", file=sys.stderr)
        sys.exit(2)
    if args.ingest_grouped_counters:
        ingest_grouped_counters(args.ingest_grouped_counters)
        return
    if args.ingest_counters:
        part = args.partition if args.partition is not None else -1
        ingest_counters(args.ingest_counters, config=args.config, partition=part, block_size=args.block_size,
                        explicit_partition=args.partition is not None)
        return
    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib)
        return
    if args.prefill_only:
        import torch
        torch.cuda.set_device(0)
        leg = prefill_leg(reps=args.steps, parity_seqs=() if args.no_cpu_baseline else (0, 9), fresh=False)
        print(json.dumps({"metric": "prefill TFLOP/s (causal, bf16 matrix cores), 1 GPU", "value": leg["tflops"],
                          "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "higher_is_better": True,
                          "dtype": "bf16", "data": "synthetic", "config": {"workload": PREFILL_WORKLOAD},
                          **leg}), flush=True)
        return

    import numpy as np

    t_gen = time.perf_counter()
    b = make_batch(args)
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] workload {args.config} generated in {t_gen:.1f}s: {b.name}, S={b.num_seqs}, "
          f"KV bytes {b.kv_bytes() / 1e9:.3f} GB", file=sys.stderr, flush=True)

    cpu, cpu_out = None, None
    if not args.no_cpu_baseline:   # before any GPU call (forked workers)
        cpu, cpu_out = cpu_baseline(b, args.cpu_seconds, single_core=args.config in (1, 2))
        print(f"[bench] cpu oracle: {cpu['value']:.1f} seq-steps/s on {cpu['cores']} cores",
              file=sys.stderr, flush=True)

    import torch

    import oracle.pa_oracle as O
    import paged_kv_cache_313_amd as P
    from workloads import torch_io

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    d = torch_io.to_device(b, dev)
    part = args.partition if args.partition is not None else P.choose_partition(
        b.num_seqs, b.num_kv_heads, b.max_context_len, b.block_size)
    need = P.decode_workspace_bytes(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim,
                                    b.max_context_len, part)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    out = torch.empty_like(d.query)
    stream = torch.cuda.current_stream(dev)
    has_copy = b.block_mapping is not None and len(b.block_mapping) > 0
    hier = None
    if "hier" in b.meta:
        large, nl, H = b.meta["hier"]
        hier = (torch.from_numpy(large).to(dev), torch.from_numpy(nl).to(dev), H)
    has_append = b.new_key is not None

    def copy_only(st):
        P.block_copy(d.k_pool, d.v_pool, d.block_mapping, stream=st)

    def append_only(st):
        P.kv_append(d.new_key, d.new_value, d.k_pool, d.v_pool, d.slot_mapping, stream=st)

    def decode_only(st=None):
        st = stream if st is None else st
        if hier:
            P.decode_attention_hier(d.query, d.k_pool, d.v_pool, d.block_tables, hier[0], hier[1], hier[2],
                                    d.context_lens, b.scale, b.max_context_len, part, out=out, workspace=ws,
                                    stream=st)
        else:
            P.decode_attention(d.query, d.k_pool, d.v_pool, d.block_tables, d.context_lens, b.scale,
                               b.max_context_len, part, out=out, workspace=ws, stream=st)

    parts = ([copy_only] if has_copy else []) + ([append_only] if has_append else []) + [decode_only]

    def step_fn(st):
        for f in parts:
            f(st)

    def events_ms(run, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            run()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / n

    # The timed region is one HIP graph holding the K steps back to back (and
    # one per call kind, K calls each, for the per-call times): a single
    # launch, so host stalls cannot starve the GPU and no per-launch cost is
    # counted K times.  The library allocates, synchronises and clears
    # nothing, so its calls capture as they are.  Eager launches are the
    # fallback (--eager forces them).
    for _ in range(args.warmup):
        step_fn(stream)
    torch.cuda.synchronize()
    K = args.steps
    graphs = None
    if not args.eager:
        try:
            def capture(fn):
                g = torch.cuda.CUDAGraph()
                cs = torch.cuda.Stream()
                cs.wait_stream(stream)
                with torch.cuda.graph(g, stream=cs):
                    for _ in range(K):
                        fn(cs)
                stream.wait_stream(cs)
                return g
            graphs = {"step": capture(step_fn), "decode": capture(decode_only)}
            if has_append:
                graphs["append"] = capture(append_only)
            if has_copy:
                graphs["copy"] = capture(copy_only)
            graphs["step"].replay()   # warm the graph itself
            torch.cuda.synchronize()
        except Exception as exc:   # fall back to eager launches
            print(f"[bench] graph capture failed ({exc}); timing eager launches", file=sys.stderr, flush=True)
            graphs = None
            torch.cuda.synchronize()
    # Settle the clock: after lighter work the GPU takes a few tens of ms of
    # load to reach its steady clock (on the prefill the first ~30 ms of
    # calls ran up to 20 % slower), so whole steps run for SETTLE_S first.
    t_settle = time.perf_counter() + SETTLE_S
    while True:
        if graphs:
            graphs["step"].replay()
        else:
            step_fn(stream)
        torch.cuda.synchronize()
        if time.perf_counter() >= t_settle:
            break
    timing = f"one HIP graph of {K} steps" if graphs else "eager launches"
    print(f"[bench] warmup done ({args.warmup} steps), timing {K} steps ({timing})", file=sys.stderr, flush=True)

    def k_calls(kind, fn):
        if graphs:
            return graphs[kind].replay
        return lambda: [fn(stream) for _ in range(K)]

    run_steps = k_calls("step", step_fn)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) / K * 1e3
    # per-call times: K back-to-back calls of one kind, HIP events on the
    # stream, in step order (copies, appends, decode) so that the pools end in
    # the state a step leaves: a copy's source may be a block that an append
    # of the same step writes in place
    cp_ms = events_ms(k_calls("copy", copy_only), 1) / K if has_copy else None
    app_ms = events_ms(k_calls("append", append_only), 1) / K if has_append else None
    dec_ms = events_ms(k_calls("decode", decode_only), 1) / K
    alg_bytes, kv_bytes = algorithmic_bytes(b)
    uniq_kv = unique_kv_bytes(b)
    # the roofline counts each physical K/V byte once: blocks that several
    # sequences share (prefix-shared sampling) are one HBM read at best
    alg_unique = alg_bytes - kv_bytes + uniq_kv
    achieved = alg_unique / (dec_ms * 1e-3) / 1e9
    latency = None if args.no_aux else step_latency_leg(step_fn, stream, graphs, max(K, 20))

    cold = stream_leg = bm_leg = None
    if not args.no_aux:
        cold = cold_decode_leg(decode_only, stream)
        cold["kv_read_gbps"] = kv_bytes / (cold["decode_ms_median"] * 1e-3) / 1e9
        cold["pct_of_hbm_peak"] = 100.0 * alg_unique / (cold["decode_ms_median"] * 1e-3) / 1e9 / HBM_PEAK_GBPS
        stream_leg = achievable_read_leg(stream)
        stream_leg["decode_frac_of_achievable"] = achieved / stream_leg["gbps"]
        bm_leg = block_manager_leg(b, max(args.steps, 10))
    swap = None if args.no_swap else swap_leg(d, b)
    grouped = None
    if "samples" in b.meta and not args.no_aux:   # the prefix-shared batch
        grouped = grouped_decode_leg(b, d, stream, alg_unique, dec_ms, K)
    prefill = None if args.no_prefill else prefill_leg(parity_seqs=() if args.no_cpu_baseline else (0, 9))

    step_fn(stream)          # one whole step last: the output the parity check reads
    torch.cuda.synchronize()

    # parity of this run's output against the oracle run above (all sequences)
    parity = None
    if cpu_out is not None:
        got = O.upcast(torch_io.torch_to_storage(out, b.dtype), b.dtype)
        err = np.abs(got - cpu_out)
        if b.dtype == "f32":
            ok = bool(err.max() <= 1e-5)
        else:
            ok = bool((err <= 2e-2 + 1e-2 * np.abs(cpu_out)).all())
        parity = {"max_abs_err": float(err.max()), "within_tolerance": ok,
                  "checked": "all outputs vs the fp64 oracle"}

    explicit = args.partition is not None
    # counters were taken on the default workload shapes (shuffled tables, the
    # workload's own group size) only
    same_shape = args.group in (None, 4) and args.table_layout == "shuffled"
    ctr = counters_from_profile(args.config, part, b.block_size, explicit) if same_shape else None
    workload = WORKLOADS[args.config]
    if args.group is not None and args.group != 4:
        workload = workload.replace("32q/8kv heads", f"{8 * args.group}q/8kv heads")
    cfg = {"workload": workload, "num_seqs": b.num_seqs, "num_q_heads": b.num_q_heads,
           "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim, "block_size": b.block_size,
           "num_blocks": b.num_blocks, "partition_size": part, "table_layout": args.table_layout,
           "kv_bytes_per_step": kv_bytes, "unique_kv_bytes_per_step": uniq_kv,
           "tokens": int(b.context_lens.sum())}
    line = {
        "metric": METRIC,
        "value": b.num_seqs / (ms_per_step * 1e-3),
        "unit": "seq-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup, "settle_s": SETTLE_S,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": b.dtype,
        "data": "synthetic (seeded N(0,1) q/K/V, shuffled physical blocks)",
        "config": cfg,
        "kv_read_gbps": kv_bytes / (dec_ms * 1e-3) / 1e9,
        "pct_of_hbm_peak": 100.0 * achieved / HBM_PEAK_GBPS,
        "timing": timing,
        "decode_ms": dec_ms,
        "append_ms": app_ms,
        "block_copy_ms": cp_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None if ctr is None else ctr["hbm_bytes_per_launch"],
                     "kernel": decode_kernel_name(b, part),
                     "algorithmic_bytes_per_launch": alg_unique,
                     "logical_bytes_per_launch": alg_bytes,
                     "logical_gbps": alg_bytes / (dec_ms * 1e-3) / 1e9,
                     "fetched_bytes_per_launch": None if ctr is None else ctr.get("fetch_bytes_per_launch"),
                     "bytes": "algorithmic = K/V of the distinct physical blocks read (valid tokens) + query + "
                              "output + table entries + lengths; logical counts a shared block once per "
                              "sequence that reads it; traffic/fetched = rocprofv3 FETCH_SIZE + WRITE_SIZE of "
                              "the call, scaled by a plain copy's counts"},
        "step_latency": latency,
        "cpu_baseline": cpu,
        "parity": parity,
        "decode_cold_cache": cold,
        "achievable_read": stream_leg,
        "block_manager": bm_leg,
        "swap": swap,
        "prefill": prefill,
        "grouped_decode": grouped,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
