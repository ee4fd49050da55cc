"""The prefill grid's unit order, checked on the CPU: the index arithmetic of
prefill_kernel (pa_prefill_kernels.hip) maps the workgroups onto
(sequence x KV head, query block) pairs so that every block of every
sequence is taken exactly once and the other units exit, hands out the
query blocks in bands of 8 counted from each sequence's last block (so every
sequence's last blocks come first, whatever its number of new tokens), keeps
each (sequence, KV head)'s blocks of a band together (one run of 8 units on
an XCD), and reduces to the plain order (blocks of one pair together, last
first) when no sequence has more than 8 query blocks.  xcd_unit is mirrored
from pa_common.hpp."""

import pytest

BAND = 8


def xcd_unit(b, n):
    full = n & ~63
    if b >= full:
        return b
    x, k = b & 7, b >> 3
    return ((k >> 3) << 6) | (x << 3) | (k & 7)


def unit(u, SG, qblocks):
    """(blocks after this one in its sequence, sequence x KV head)"""
    band = u // (SG * BAND)
    bw = min(BAND, qblocks - band * BAND)
    rest = u - band * SG * BAND
    return band * BAND + rest % bw, rest // bw


def block(r, nblocks, qblocks):
    """The unit's query block, or None when its sequence has no block left."""
    qb = min(nblocks, qblocks) - 1 - r
    return qb if qb >= 0 else None


def run_grid(nblocks, Hkv, qblocks):
    """Walk the grid in dispatch order (u); nblocks[s] = ceil(n_s / QB)."""
    SG = len(nblocks) * Hkv
    n = SG * qblocks
    order = []
    for b in range(n):
        u = xcd_unit(b, n)
        r, sg = unit(u, SG, qblocks)
        qb = block(r, nblocks[sg // Hkv], qblocks)
        order.append((u, r, sg, qb))
    order.sort()
    return order


@pytest.mark.parametrize("SG", [1, 3, 8, 32, 128, 129])
@pytest.mark.parametrize("qblocks", [1, 2, 7, 8, 9, 16, 32, 33, 128])
def test_prefill_units_cover_each_block_once(SG, qblocks):
    n = SG * qblocks
    seen = {}
    order = []
    for b in range(n):
        u = xcd_unit(b, n)
        assert 0 <= u < n
        r, sg = unit(u, SG, qblocks)
        qb = block(r, qblocks, qblocks)
        assert 0 <= qb < qblocks and 0 <= sg < SG
        assert (qb, sg) not in seen
        seen[(qb, sg)] = b
        order.append((u, qb, sg))
    assert len(seen) == n
    order.sort()
    # bands in order, the last query blocks first
    bands = [(qblocks - 1 - qb) // BAND for _, qb, _ in order]
    assert bands == sorted(bands)
    # within a band: one pair's blocks together, last first
    for i in range(1, n):
        _, qb0, sg0 = order[i - 1]
        _, qb1, sg1 = order[i]
        if bands[i] == bands[i - 1] and sg0 == sg1:
            assert qb1 == qb0 - 1
        elif bands[i] == bands[i - 1]:
            assert sg1 == sg0 + 1
    if qblocks <= BAND:   # the plain order
        assert [(qb, sg) for _, qb, sg in order] == [(qblocks - 1 - r, s) for s in range(SG) for r in range(qblocks)]


def test_full_band_is_one_xcd_run():
    SG, qblocks = 16, 32
    n = SG * qblocks
    for b0 in range(0, n & ~63, 8):
        # workgroups b0 .. b0 + 7 of one XCD run: units 8 apart in b, consecutive in u
        us = [xcd_unit(b0 // 8 % 8 + 8 * (8 * (b0 // 64) + j), n) for j in range(8)]
        pairs = {unit(u, SG, qblocks)[1] for u in us}
        assert len(pairs) == 1


@pytest.mark.parametrize("nblocks", [[33, 11, 1, 2, 8], [1, 1, 40], [9, 0, 16], [5, 5, 5]])
def test_ragged_sequences_last_blocks_first(nblocks):
    Hkv = 2
    qblocks = max(nblocks)
    order = run_grid(nblocks, Hkv, qblocks)
    got = [(sg, qb) for _, _, sg, qb in order if qb is not None]
    want = {(s * Hkv + g, q) for s, nb in enumerate(nblocks) for g in range(Hkv) for q in range(nb)}
    assert len(got) == len(set(got)) and set(got) == want
    # every sequence's last block is in the first band, and a pair's blocks
    # come last first
    pos = {key: i for i, key in enumerate(got)}
    first_band = {(sg, qb) for _, r, sg, qb in order if qb is not None and r < BAND}
    for s, nb in enumerate(nblocks):
        for g in range(Hkv):
            if nb:
                assert (s * Hkv + g, nb - 1) in first_band
            for q in range(1, nb):
                assert pos[(s * Hkv + g, q)] < pos[(s * Hkv + g, q - 1)]


def test_blocks_past_the_grid_stay_unwritten():
    """A sequence with more blocks than the grid (more new tokens than
    max_query_len) gets its first qblocks blocks, as the rows past
    max_query_len are left alone."""
    order = run_grid([12, 3], 1, 8)
    got = {(sg, qb) for _, _, sg, qb in order if qb is not None}
    assert got == {(0, q) for q in range(8)} | {(1, q) for q in range(3)}
