"""The prefill grid's unit order, checked on the CPU: the index arithmetic of
prefill_kernel (pa_prefill_kernels.hip) maps the workgroups one to one onto
(sequence x KV head, query block) pairs, hands out the query blocks in bands
of 8 with the band nearest the context's end first, keeps each (sequence, KV
head)'s blocks of a band together (one run of 8 units on an XCD), and reduces
to the plain order (blocks of one pair together, last first) when a sequence
has at most 8 query blocks.  xcd_unit is mirrored from pa_common.hpp."""

import pytest

BAND = 8


def xcd_unit(b, n):
    full = n & ~63
    if b >= full:
        return b
    x, k = b & 7, b >> 3
    return ((k >> 3) << 6) | (x << 3) | (k & 7)


def unit(u, SG, qblocks):
    band = u // (SG * BAND)
    bw = min(BAND, qblocks - band * BAND)
    rest = u - band * SG * BAND
    return qblocks - 1 - (band * BAND + rest % bw), rest // bw


@pytest.mark.parametrize("SG", [1, 3, 8, 32, 128, 129])
@pytest.mark.parametrize("qblocks", [1, 2, 7, 8, 9, 16, 32, 33, 128])
def test_prefill_units_cover_each_block_once(SG, qblocks):
    n = SG * qblocks
    seen = {}
    order = []
    for b in range(n):
        u = xcd_unit(b, n)
        assert 0 <= u < n
        qb, sg = unit(u, SG, qblocks)
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
