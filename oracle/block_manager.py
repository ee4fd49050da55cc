"""Reference KV block manager (pure Python).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
native block manager in libpagedkv.

What it models, and where the pages define it:

* One global allocator owns the physical blocks of the KV pool, like an MMU
  owns page frames (paged-KV analysis page, section 2.3, the component table:
  KV block manager).
* Every sequence has its own block table that maps logical block j (tokens
  [j * block_size, (j + 1) * block_size)) to a physical block (same table,
  "Block Table"; section 2.2).
* Blocks are taken only when a sequence needs one, so only a sequence's last
  block can be partly filled (vLLM entity page, "what it is").
* Parallel samples, beams and common prompts share physical blocks through
  reference counts; a sequence about to write into a block that other
  sequences still reference first gets its own copy -- copy-on-write (vLLM
  entity page, "what it is"; paged-KV analysis page, section 3.2, the
  copy-on-write paragraph).
* A finished request gives its blocks back at once (paged-KV analysis page,
  section 3.3, continuous batching).
* Effective utilisation = sum of sequence lengths / (blocks in use * block
  size) (paged-KV analysis page, section 4.2).

Readings where the pages are silent:

* Allocation order: the lowest-numbered free block is taken first.  Any order
  is correct; fixing one makes two implementations comparable bit for bit.
* fork(parent) creates a sequence with the parent's length and a copy of its
  table; every block of the table gains one reference.  This is how parallel
  sampling and beam search share a prompt.
* append_slots(seqs, counts) reserves counts[i] new token positions at the end
  of sequence seqs[i], for i in order.  For each position p = current length:
    - p % block_size == 0: a fresh block is appended to the table;
    - else, if the last block has more than one reference: copy-on-write --
      a fresh block replaces it in this table, the pair (old, fresh) is
      emitted, and the old block loses one reference;
    - the slot emitted is table[p // block_size] * block_size + p % block_size.
  The copies must be applied (pre-call state) before the appends are written;
  a sequence later in the same batch that still shares the old block then
  finds it with fewer references.  A batch is all-or-nothing: if the free
  blocks do not cover it, nothing changes and OutOfBlocks is raised.
* free_sequence drops one reference from every block of the table; blocks
  left with none return to the free pool.
* Preemption evicts all of a request's blocks at once (Cross-Paper Synthesis
  page, section 3, the preemption item).  swap_out(seq) returns the table's
  blocks in table order -- the caller copies them to host memory before
  anything else writes them -- drops one reference from each, and leaves the
  sequence swapped: it keeps its length but holds no block, and only
  swap_in or free_sequence may name it.  swap_in(seq) takes as many fresh
  blocks as it held (lowest first, all-or-nothing) and returns them in table
  order; the caller copies the host data into them.  Blocks it shared before
  come back as private copies.  Utilisation counts resident sequences only.
* Large pages (Cross-Paper Synthesis page, section 5, the adaptive block size
  item): append_prompt_large(seq, n, H) writes an empty sequence's prompt of n
  tokens with its first n // (H * block_size) full large pages' worth of
  tokens in large pages -- for each, the lowest aligned run of H free blocks
  [P H, P H + H) -- and the rest as append_slots would place them.  The
  sequence's table still lists every block; its first num_large * H entries
  are the large pages' blocks, which block_tables_hier reports as large-page
  ids.  Large pages are always full, so no later write copies one; a swap-in
  brings the sequence back with small blocks only.
"""

from __future__ import annotations

import copy
import heapq
from fractions import Fraction


class OutOfBlocks(RuntimeError):
    pass


class UnknownSequence(KeyError):
    """No live sequence has this id, or it is swapped out where a resident
    one is needed (and the other way round)."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.ref = [0] * num_blocks
        self.free = list(range(num_blocks))      # a heap: lowest id on top
        heapq.heapify(self.free)
        self.seqs: dict[int, dict] = {}        # resident sequences
        self.swapped: dict[int, dict] = {}     # swapped out: length and block count
        self.next_id = 0

    # -- sequences ---------------------------------------------------------
    def add_sequence(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = {"table": [], "len": 0}
        return sid

    def _seq(self, sid: int) -> dict:
        """A resident sequence."""
        if sid not in self.seqs:
            raise UnknownSequence(sid)
        return self.seqs[sid]

    def fork(self, parent: int) -> int:
        p = self._seq(parent)
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = {"table": list(p["table"]), "len": p["len"], "nl": p.get("nl", 0), "H": p.get("H")}
        for b in p["table"]:
            self.ref[b] += 1
        return sid

    def _drop(self, table) -> None:
        for b in table:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                heapq.heappush(self.free, b)

    def free_sequence(self, sid: int) -> None:
        if sid in self.swapped:
            del self.swapped[sid]
            return
        s = self._seq(sid)
        self._drop(s["table"])
        del self.seqs[sid]

    def length(self, sid: int) -> int:
        if sid in self.swapped:
            return self.swapped[sid]["len"]
        return self._seq(sid)["len"]

    # -- preemption ----------------------------------------------------------
    def swap_out(self, sid: int) -> list:
        s = self._seq(sid)
        ids = list(s["table"])
        self._drop(ids)
        del self.seqs[sid]
        self.swapped[sid] = {"len": s["len"], "nblocks": len(ids)}
        return ids

    def swap_in(self, sid: int) -> list:
        if sid not in self.swapped:
            raise UnknownSequence(sid)
        w = self.swapped[sid]
        if len(self.free) < w["nblocks"]:
            raise OutOfBlocks()
        ids = [self._take() for _ in range(w["nblocks"])]
        del self.swapped[sid]
        self.seqs[sid] = {"table": ids, "len": w["len"]}
        return ids

    # -- allocation --------------------------------------------------------
    def _take(self) -> int:
        if not self.free:
            raise OutOfBlocks()
        b = heapq.heappop(self.free)
        self.ref[b] = 1
        return b

    def _take_run(self, H: int) -> int:
        """Lowest aligned run of H free blocks; returns its large-page id."""
        free = set(self.free)
        for P in range(self.num_blocks // H):
            if all(b in free for b in range(P * H, P * H + H)):
                for b in range(P * H, P * H + H):
                    self.ref[b] = 1
                self.free = [b for b in self.free if not (P * H <= b < P * H + H)]
                heapq.heapify(self.free)
                return P
        raise OutOfBlocks()

    def append_prompt_large(self, sid: int, n: int, H: int):
        """Slots of an empty sequence's n prompt tokens, full large pages first."""
        s = self._seq(sid)
        if s["len"] != 0 or n < 0 or H < 1:
            raise ValueError("prompt into an empty sequence only")
        nl = n // (H * self.block_size)
        saved = (copy.deepcopy(self.seqs), list(self.ref), list(self.free))
        try:
            pages = [self._take_run(H) for _ in range(nl)]
        except OutOfBlocks:
            self.seqs, self.ref, self.free = saved
            raise
        s["table"] = [P * H + i for P in pages for i in range(H)]
        s["len"] = nl * H * self.block_size
        s["nl"], s["H"] = nl, H
        slots = []
        for P in pages:
            slots += list(range(P * H * self.block_size, (P + 1) * H * self.block_size))
        try:
            rest, pairs = self.append_slots([sid], [n - s["len"]])
        except OutOfBlocks:
            self.seqs, self.ref, self.free = saved
            raise
        assert pairs == []
        return slots + rest

    def block_tables_hier(self, seqs, H: int, max_large: int, max_small: int):
        """(large ids, num_large, small tables, lengths); sequences written
        without large pages (or with another H) report num_large = 0."""
        large, nls, small, lens = [], [], [], []
        for sid in seqs:
            s = self._seq(sid)
            nl = s.get("nl", 0) if s.get("H") == H else 0
            lp = [s["table"][k * H] // H for k in range(nl)]
            sm = s["table"][nl * H:]
            if nl > max_large or len(sm) > max_small:
                raise ValueError("table widths too small")
            large.append(lp + [-1] * (max_large - nl))
            nls.append(nl)
            small.append(sm + [-1] * (max_small - len(sm)))
            lens.append(s["len"])
        return large, nls, small, lens

    def append_slots(self, seqs, counts):
        """Returns (slots, cow_pairs): one slot per new token in batch order,
        and the (src, dst) copies to apply before writing them."""
        if len(seqs) != len(counts):
            raise ValueError("seqs and counts differ in length")
        for sid, n in zip(seqs, counts):
            self._seq(sid)
            if n < 0:
                raise ValueError("negative token count")
        saved = (copy.deepcopy(self.seqs), list(self.ref), list(self.free))
        slots, pairs = [], []
        try:
            for sid, n in zip(seqs, counts):
                s = self.seqs[sid]
                for _ in range(n):
                    p = s["len"]
                    j, o = divmod(p, self.block_size)
                    if o == 0:
                        s["table"].append(self._take())
                    elif self.ref[s["table"][j]] > 1:
                        old = s["table"][j]
                        fresh = self._take()
                        self.ref[old] -= 1
                        s["table"][j] = fresh
                        pairs.append((old, fresh))
                    slots.append(s["table"][j] * self.block_size + o)
                    s["len"] = p + 1
        except OutOfBlocks:
            self.seqs, self.ref, self.free = saved
            raise
        return slots, pairs

    # -- read-outs ---------------------------------------------------------
    def block_tables(self, seqs, max_blocks_per_seq: int):
        """Padded tables (-1 past each sequence's last block) and lengths."""
        tables, lens = [], []
        for sid in seqs:
            s = self._seq(sid)
            if len(s["table"]) > max_blocks_per_seq:
                raise ValueError("max_blocks_per_seq too small")
            tables.append(s["table"] + [-1] * (max_blocks_per_seq - len(s["table"])))
            lens.append(s["len"])
        return tables, lens

    def num_free_blocks(self) -> int:
        return len(self.free)

    def blocks_in_use(self) -> int:
        return self.num_blocks - len(self.free)

    def utilisation(self) -> Fraction:
        """Tokens held by live sequences over token slots of the blocks in use
        (a shared block's tokens count once per sequence that reads them)."""
        used = self.blocks_in_use()
        total = sum(s["len"] for s in self.seqs.values())
        return Fraction(total, used * self.block_size) if used else Fraction(0)
