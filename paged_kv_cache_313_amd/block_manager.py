"""Python handle on the native KV block manager (include/pa_block_manager.h).

Argument marshalling only: every decision (which block, whether to copy,
what a table holds) is made by libpagedkv.  Arrays come back as NumPy host
arrays in the layouts the device calls take (int64 slots for kv_append,
int32 (src, dst) pairs for block_copy, int32 padded tables and lengths for
decode_attention).
"""

from __future__ import annotations

import ctypes
from fractions import Fraction

import numpy as np

from . import _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a.size else None


class BlockManager:
    """Owns blocks 0 .. num_blocks-1 of block_size tokens of one KV pool."""

    def __init__(self, num_blocks: int, block_size: int):
        self._lib = _lib.load()
        h = ctypes.c_void_p()
        _lib.check("pa_bm_create", self._lib.pa_bm_create(num_blocks, block_size, ctypes.byref(h)))
        self._h = h
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # -- sequences -----------------------------------------------------------
    def add_sequence(self) -> int:
        out = ctypes.c_int64()
        _lib.check("pa_bm_add_sequence", self._lib.pa_bm_add_sequence(self._h, ctypes.byref(out)))
        return out.value

    def fork(self, parent: int) -> int:
        out = ctypes.c_int64()
        _lib.check("pa_bm_fork", self._lib.pa_bm_fork(self._h, int(parent), ctypes.byref(out)))
        return out.value

    def free_sequence(self, seq_id: int) -> None:
        _lib.check("pa_bm_free_sequence", self._lib.pa_bm_free_sequence(self._h, int(seq_id)))

    def length(self, seq_id: int) -> int:
        out = ctypes.c_int64()
        _lib.check("pa_bm_sequence_length",
                   self._lib.pa_bm_sequence_length(self._h, int(seq_id), ctypes.byref(out)))
        return out.value

    # -- allocation ----------------------------------------------------------
    def append_slots(self, seq_ids, counts):
        """(slots int64 [sum(counts)], pairs int32 [n, 2]); raises
        PagedKVError (status PA_ERR_NO_BLOCKS ...) and changes nothing on failure."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        cnt = np.ascontiguousarray(counts, dtype=np.int32)
        if ids.shape != cnt.shape or ids.ndim != 1:
            raise ValueError("seq_ids and counts must be 1-D and of one length")
        total = int(cnt.astype(np.int64).sum()) if cnt.size else 0
        slots = np.empty(max(total, 0), dtype=np.int64)
        pairs = np.empty((ids.size, 2), dtype=np.int32)
        n = ctypes.c_int32()
        _lib.check("pa_bm_append_slots",
                   self._lib.pa_bm_append_slots(self._h, _ptr(ids), _ptr(cnt), ids.size, _ptr(slots),
                                                slots.size, _ptr(pairs), ids.size, ctypes.byref(n)))
        return slots, pairs[: n.value].copy()

    def append_prompt_large(self, seq_id: int, num_tokens: int, pages_per_large: int) -> np.ndarray:
        """Slots of an empty sequence's prompt, full large pages first."""
        slots = np.empty(max(int(num_tokens), 0), dtype=np.int64)
        _lib.check("pa_bm_append_prompt_large",
                   self._lib.pa_bm_append_prompt_large(self._h, int(seq_id), int(num_tokens), int(pages_per_large),
                                                       _ptr(slots), slots.size))
        return slots

    # -- preemption ------------------------------------------------------------
    def _ids_call(self, fn: str, seq_id: int) -> np.ndarray:
        cap = max(1, -(-self.length(seq_id) // self.block_size))
        ids = np.empty(cap, dtype=np.int32)
        n = ctypes.c_int32()
        _lib.check(fn, getattr(self._lib, fn)(self._h, int(seq_id), _ptr(ids), cap, ctypes.byref(n)))
        return ids[: n.value].copy()

    def swap_out(self, seq_id: int) -> np.ndarray:
        """Blocks of the sequence in table order (copy them out before reuse);
        the sequence becomes swapped out."""
        return self._ids_call("pa_bm_swap_out", seq_id)

    def swap_in(self, seq_id: int) -> np.ndarray:
        """Fresh blocks for a swapped-out sequence, in table order."""
        return self._ids_call("pa_bm_swap_in", seq_id)

    # -- read-outs -----------------------------------------------------------
    def block_tables(self, seq_ids, max_blocks_per_seq: int):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tables = np.empty((ids.size, max_blocks_per_seq), dtype=np.int32)
        lens = np.empty(ids.size, dtype=np.int32)
        _lib.check("pa_bm_block_tables",
                   self._lib.pa_bm_block_tables(self._h, _ptr(ids), ids.size, max_blocks_per_seq,
                                                _ptr(tables), _ptr(lens)))
        return tables, lens

    def block_tables_hier(self, seq_ids, pages_per_large: int, max_large_per_seq: int, max_small_per_seq: int):
        """(large_tables, num_large, small_tables, context_lens) for the
        two-level decode and prefill calls."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        large = np.empty((ids.size, max_large_per_seq), dtype=np.int32)
        nl = np.empty(ids.size, dtype=np.int32)
        small = np.empty((ids.size, max_small_per_seq), dtype=np.int32)
        lens = np.empty(ids.size, dtype=np.int32)
        _lib.check("pa_bm_block_tables_hier",
                   self._lib.pa_bm_block_tables_hier(self._h, _ptr(ids), ids.size, int(pages_per_large),
                                                     max_large_per_seq, max_small_per_seq, _ptr(large), _ptr(nl),
                                                     _ptr(small), _ptr(lens)))
        return large, nl, small, lens

    def num_free_blocks(self) -> int:
        return int(self._lib.pa_bm_num_free_blocks(self._h))

    def utilisation(self) -> Fraction:
        t, s = ctypes.c_int64(), ctypes.c_int64()
        _lib.check("pa_bm_utilisation", self._lib.pa_bm_utilisation(self._h, ctypes.byref(t), ctypes.byref(s)))
        return Fraction(t.value, s.value) if s.value else Fraction(0)

    def refcounts(self) -> np.ndarray:
        out = np.empty(self.num_blocks, dtype=np.int32)
        _lib.check("pa_bm_refcounts", self._lib.pa_bm_refcounts(self._h, _ptr(out), out.size))
        return out
