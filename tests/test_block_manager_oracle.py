"""Pins of the reference block manager (oracle/block_manager.py) against what
the paging definition fixes: every sequence, read back through its own table
after the copies and writes a batch asks for, holds exactly the tokens it was
given (its parent's prefix, then its own); reference counts equal the number
of tables that hold a block; copies happen exactly when a shared block is
written; closed-form block counts; the prefix-sharing workload's counts;
all-or-nothing batches; planted mistakes are caught."""

import json
import os
import random
from fractions import Fraction

import numpy as np
import pytest

from oracle.block_manager import BlockManager, OutOfBlocks, UnknownSequence

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class World:
    """A block manager plus a symbolic pool of token ids and each sequence's
    expected history; applies every batch the way the device would (copies
    from the pre-call state first, then the writes)."""

    def __init__(self, bm):
        self.bm = bm
        self.pool = np.full((bm.num_blocks, bm.block_size), -1, dtype=np.int64)
        self.hist = {}
        self.host = {}        # swapped-out sequences' blocks, block-first
        self.next_token = 0

    def add(self):
        sid = self.bm.add_sequence()
        self.hist[sid] = []
        return sid

    def fork(self, parent):
        sid = self.bm.fork(parent)
        self.hist[sid] = list(self.hist[parent])
        return sid

    def free(self, sid):
        self.bm.free_sequence(sid)
        del self.hist[sid]
        self.host.pop(sid, None)

    def prompt_large(self, sid, n, H):
        slots = self.bm.append_prompt_large(sid, n, H)
        assert len(slots) == n and len(set(slots)) == n
        for sl in slots:
            tok = self.next_token
            self.next_token += 1
            b, o = divmod(sl, self.bm.block_size)
            self.pool[b, o] = tok
            self.hist[sid].append(tok)
        return slots

    def swap_out(self, sid):
        ids = self.bm.swap_out(sid)
        self.host[sid] = self.pool[ids].copy()       # before anything reuses the blocks
        return ids

    def swap_in(self, sid):
        ids = self.bm.swap_in(sid)
        self.pool[ids] = self.host.pop(sid)
        return ids

    def append(self, seqs, counts):
        before = {b: self.bm.ref[b] for b in range(self.bm.num_blocks)}
        slots, pairs = self.bm.append_slots(seqs, counts)
        assert len(slots) == sum(counts)
        assert len(set(slots)) == len(slots), "two tokens of one batch share a slot"
        dsts = [d for _, d in pairs]
        assert len(set(dsts)) == len(dsts)
        assert not set(dsts) & {s for s, _ in pairs}
        for src, dst in pairs:       # only shared blocks are copied, into fresh ones
            assert before[src] >= 2 and before[dst] == 0
        snapshot = self.pool.copy()
        for src, dst in pairs:
            self.pool[dst] = snapshot[src]
        k = 0
        for sid, n in zip(seqs, counts):
            for _ in range(n):
                tok = self.next_token
                self.next_token += 1
                b, o = divmod(slots[k], self.bm.block_size)
                self.pool[b, o] = tok
                self.hist[sid].append(tok)
                k += 1
        return slots, pairs

    def check(self):
        bm = self.bm
        count = [0] * bm.num_blocks
        for sid, h in self.hist.items():
            if sid in self.host:
                assert sid in bm.swapped and sid not in bm.seqs and bm.length(sid) == len(h)
                assert len(self.host[sid]) == -(-len(h) // bm.block_size)
                continue
            s = bm.seqs[sid]
            assert s["len"] == len(h)
            assert len(s["table"]) == -(-len(h) // bm.block_size)
            for b in s["table"]:
                count[b] += 1
            got = [int(self.pool[s["table"][t // bm.block_size], t % bm.block_size]) for t in range(len(h))]
            assert got == h, f"sequence {sid} reads back other tokens"
            nl, H = s.get("nl", 0), s.get("H")
            for k in range(nl):                    # large pages: aligned runs, always full
                run = s["table"][k * H:(k + 1) * H]
                assert run[0] % H == 0 and run == list(range(run[0], run[0] + H))
            assert s["len"] >= nl * (H or 0) * bm.block_size
        assert count == bm.ref, "reference counts differ from table membership"
        assert sorted(bm.free) == [b for b in range(bm.num_blocks) if count[b] == 0]
        assert set(bm.seqs) | set(bm.swapped) == set(self.hist)
        assert not set(bm.seqs) & set(bm.swapped)


def random_ops(world, rng, steps, max_batch=6, max_tokens=40, swaps=True, large_pages=0):
    for _ in range(steps):
        live = sorted(s for s in world.hist if s not in world.host)
        out = sorted(world.host)
        r = rng.random()
        if not live or r < 0.15:
            sid = world.add()
            if large_pages and rng.random() < 0.5:
                try:
                    world.prompt_large(sid, rng.randint(0, 3 * large_pages * world.bm.block_size), large_pages)
                except OutOfBlocks:
                    pass
        elif r < 0.30:
            world.fork(rng.choice(live))
        elif r < 0.40 and len(live) > 1:
            world.free(rng.choice(live + out))
        elif swaps and r < 0.47:
            world.swap_out(rng.choice(live))
        elif swaps and r < 0.54 and out:
            try:
                world.swap_in(rng.choice(out))
            except OutOfBlocks:
                pass
        else:
            seqs = rng.sample(live, min(len(live), rng.randint(1, max_batch)))
            counts = [rng.choice([0, 1, 1, 1, rng.randint(1, max_tokens)]) for _ in seqs]
            try:
                world.append(seqs, counts)
            except OutOfBlocks:
                pass
        world.check()


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("bs", [1, 4, 16])
def test_random_histories_read_back_exactly(seed, bs):
    world = World(BlockManager(num_blocks=48, block_size=bs))
    random_ops(world, random.Random(seed), 150)


def test_no_sharing_closed_form():
    bs = 16
    bm = BlockManager(1000, bs)
    lens = [1, 15, 16, 17, 100, 257]
    seqs = [bm.add_sequence() for _ in lens]
    slots, pairs = bm.append_slots(seqs, lens)
    assert pairs == []
    need = sum(-(-L // bs) for L in lens)
    assert bm.blocks_in_use() == need
    assert bm.utilisation() == Fraction(sum(lens), need * bs)
    # lowest-first allocation on a fresh pool: sequence 0's blocks come first
    assert slots[:1] == [0] and slots[1] == bs  # seq 0 took block 0, seq 1 starts at block 1


def test_fork_then_each_writes_once():
    """k forks of a prompt whose last block is partly filled: the first k of
    the k + 1 writers copy it, the last writes in place."""
    bs, P, k = 16, 40, 5
    world = World(BlockManager(64, bs))
    root = world.add()
    world.append([root], [P])
    kids = [world.fork(root) for _ in range(k)]
    order = kids + [root]
    slots, pairs = world.append(order, [1] * (k + 1))
    world.check()
    shared_last = world.bm.seqs[root]["table"][-1]
    assert len(pairs) == k and all(src == shared_last for src, _ in pairs)
    assert slots[-1] == shared_last * bs + P % bs     # the last writer kept the block
    assert world.bm.blocks_in_use() == -(-P // bs) + k


def test_fork_at_block_boundary_needs_no_copy():
    world = World(BlockManager(64, 8))
    root = world.add()
    world.append([root], [24])
    kid = world.fork(root)
    _, pairs = world.append([kid, root], [1, 1])
    assert pairs == []
    world.check()


def test_prefix_sharing_workload_counts():
    """The prefix-shared sampling workload: 64 prompts of 1032 tokens, 8
    samples each (the prompt plus 7 forks), then 256 suffix tokens per sample
    one step at a time.  Counts in tests/golden/block_manager_prefix_sharing.json."""
    g = json.load(open(os.path.join(GOLDEN, "block_manager_prefix_sharing.json")))
    bs, prompts, samples, plen, suffix = g["block_size"], g["prompts"], g["samples"], g["prompt_len"], g["suffix_len"]
    bm = BlockManager(g["num_blocks"], bs)
    groups = []
    for _ in range(prompts):
        root = bm.add_sequence()
        bm.append_slots([root], [plen])
        groups.append([root] + [bm.fork(root) for _ in range(samples - 1)])
    assert bm.blocks_in_use() == g["blocks_after_prompts"]
    order = [sid for grp in groups for sid in grp[1:] + grp[:1]]   # forks first, the prompt's owner last
    _, pairs = bm.append_slots(order, [1] * len(order))
    assert len(pairs) == g["cow_pairs_first_step"]
    assert bm.blocks_in_use() == g["blocks_after_first_step"]
    for _ in range(suffix - 1):
        _, more = bm.append_slots(order, [1] * len(order))
        assert more == []
    assert bm.blocks_in_use() == g["blocks_at_end"]
    lens = [bm.length(s) for s in order]
    assert lens == [plen + suffix] * len(order)
    assert bm.utilisation() == Fraction(g["utilisation"][0], g["utilisation"][1])
    shared = [b for b in range(bm.num_blocks) if bm.ref[b] == samples]
    assert len(shared) == g["blocks_shared_by_all_samples"]


def test_batch_is_all_or_nothing():
    bm = BlockManager(10, 4)
    a, b = bm.add_sequence(), bm.add_sequence()
    bm.append_slots([a], [20])                  # 5 blocks
    state = (json.dumps(bm.seqs, sort_keys=True), list(bm.ref), sorted(bm.free))
    with pytest.raises(OutOfBlocks):
        bm.append_slots([a, b], [4, 20])          # needs 1 + 5 > 5 free
    assert (json.dumps(bm.seqs, sort_keys=True), list(bm.ref), sorted(bm.free)) == state
    bm.append_slots([a, b], [4, 16])              # exactly 5
    assert bm.num_free_blocks() == 0


def test_free_returns_blocks_lowest_first_reuse():
    bm = BlockManager(8, 2)
    a, b = bm.add_sequence(), bm.add_sequence()
    bm.append_slots([a, b], [4, 4])             # a: 0,1  b: 2,3
    bm.free_sequence(a)
    c = bm.add_sequence()
    slots, _ = bm.append_slots([c], [1])
    assert slots == [0]
    with pytest.raises(UnknownSequence):
        bm.free_sequence(a)


# -- planted mistakes: each must be caught by the checks above ---------------

class NoCopyBM(BlockManager):
    def append_slots(self, seqs, counts):
        real = self.ref
        self.ref = [min(r, 1) for r in real]     # pretend nothing is shared
        try:
            out = super().append_slots(seqs, counts)
        finally:
            fixed = self.ref
            self.ref = [max(r0, r1) if r0 > 1 else r1 for r0, r1 in zip(real, fixed)]
        return out


class LeakyCopyBM(BlockManager):
    def append_slots(self, seqs, counts):
        slots, pairs = super().append_slots(seqs, counts)
        for src, _ in pairs:
            self.ref[src] += 1                     # forgets to drop the old reference
        return slots, pairs


class KeepOnFreeBM(BlockManager):
    def free_sequence(self, sid):
        if sid in self.seqs:
            del self.seqs[sid]                     # never gives blocks back
        else:
            super().free_sequence(sid)


class ReversedSwapInBM(BlockManager):
    def swap_in(self, sid):
        ids = super().swap_in(sid)
        self.seqs[sid]["table"] = ids[::-1]      # table order lost on the way back
        return ids


@pytest.mark.parametrize("cls", [NoCopyBM, LeakyCopyBM, KeepOnFreeBM, ReversedSwapInBM])
def test_planted_mistakes_are_caught(cls):
    caught = False
    for seed in range(10):
        world = World(cls(num_blocks=64, block_size=4))
        try:
            random_ops(world, random.Random(seed), 200)
        except AssertionError:
            caught = True
            break
    assert caught


def test_swap_round_trip_and_errors():
    world = World(BlockManager(16, 4))
    a = world.add()
    world.append([a], [10])                       # 3 blocks
    b = world.fork(a)
    ids = world.swap_out(a)
    assert ids == [0, 1, 2] and world.bm.num_free_blocks() == 16 - 3   # b still holds them
    world.check()
    with pytest.raises(UnknownSequence):
        world.bm.append_slots([a], [1])
    with pytest.raises(UnknownSequence):
        world.bm.fork(a)
    world.append([b], [1])                        # b now owns block 2 alone: no copy
    back = world.swap_in(a)
    assert back == [3, 4, 5]                      # private copies, lowest first
    world.check()
    world.free(b)
    world.append([a], [3])
    world.check()
    # all-or-nothing: not enough blocks to come back
    c = world.add()
    world.append([c], [40])                       # 10 blocks: 3 + 10 of 16
    world.swap_out(a)
    d = world.add()
    world.append([d], [4 * 5])                    # 5 blocks: 15 of 16 used
    with pytest.raises(OutOfBlocks):
        world.swap_in(a)
    world.check()
    world.free(a)                                 # a swapped sequence can be dropped
    world.check()


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("bs,H", [(1, 4), (4, 2), (2, 8)])
def test_random_histories_with_large_pages(seed, bs, H):
    world = World(BlockManager(num_blocks=96, block_size=bs))
    random_ops(world, random.Random(100 + seed), 150, large_pages=H)


def test_large_pages_expand_to_the_flat_table():
    """block_tables_hier, expanded by the pool oracle's two-level rule, is the
    flat table; an aligned run is skipped while any of its blocks is taken."""
    import oracle.pa_oracle as O
    bm = BlockManager(64, 4)
    a = bm.add_sequence()
    bm.append_slots([a], [5])                       # blocks 0, 1: runs of 8 start at 8
    b = bm.add_sequence()
    slots = bm.append_prompt_large(b, 2 * 8 * 4 + 6, 8)
    assert slots[0] == 8 * 4 and bm.seqs[b]["table"][:16] == list(range(8, 24))
    assert bm.seqs[b]["table"][16:] == [2, 3]       # the rest: lowest free small blocks
    large, nl, small, lens = bm.block_tables_hier([a, b], 8, 2, 3)
    assert nl == [0, 2] and large[1] == [1, 2] and lens == [5, 70]
    flat = O.expand_hier_tables(np.array(large), nl, np.array(small), 8)
    for i, sid in enumerate([a, b]):
        t = bm.seqs[sid]["table"]
        assert flat[i, :len(t)].tolist() == t
    with pytest.raises(ValueError):
        bm.append_prompt_large(a, 40, 8)             # only into an empty sequence


class UnalignedLargeBM(BlockManager):
    def _take_run(self, H):
        got = [self._take() for _ in range(H)]        # lowest free blocks, not an aligned run
        return got[0] // H


def test_unaligned_large_pages_are_caught():
    caught = False
    for seed in range(10):
        world = World(UnalignedLargeBM(num_blocks=96, block_size=2))
        try:
            random_ops(world, random.Random(seed), 200, large_pages=4)
        except AssertionError:
            caught = True
            break
    assert caught
