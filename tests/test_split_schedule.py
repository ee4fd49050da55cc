"""The balanced split's bookkeeping, checked on the CPU: every tile of every
(sequence, head group) is processed by exactly one workgroup, every piece that
a workgroup writes to a partial slot is read back by the merge exactly once,
and the merge never reads a slot that no workgroup wrote.

The walk below mirrors the index arithmetic of decode_balanced_kernel and
decode_merge_balanced_kernel (tile prefix sums, range w*ntot/W, slot 2w or
2w+1, the merge's w_lo/w_hi and skip of empty ranges); it is a model of the
schedule, the kernels themselves are checked against the oracle on the GPU."""

import random

import pytest

TILE = 16


def walk(lens, C, W):
    S = len(lens)
    nts = [-(-L // TILE) for L in lens]
    cum = [0]
    for n in nts:
        cum.append(cum[-1] + n)
    ntot = C * cum[S]
    written, direct, seen = {}, set(), {}
    for w in range(W):
        f, fb = w * ntot // W, (w + 1) * ntot // W
        if f >= fb:
            continue
        lo, hi = 0, S - 1
        while lo < hi:
            mid = (lo + hi + 1) >> 1
            if C * cum[mid] <= f:
                lo = mid
            else:
                hi = mid - 1
        s = lo
        nt = cum[s + 1] - cum[s]
        rel = f - C * cum[s]
        c, t = rel // nt, rel % nt
        first = True
        while f < fb:
            n = min(nt - t, fb - f)
            for tt in range(t, t + n):
                assert (s, c, tt) not in seen
                seen[(s, c, tt)] = w
            if t == 0 and t + n == nt:
                direct.add((s, c))
            else:
                slot = 2 * w + (0 if first else 1)
                assert slot not in written
                written[slot] = (s, c, t, t + n)
            first = False
            f += n
            t += n
            if t == nt and f < fb:
                t, c = 0, c + 1
                if c == C:
                    c, s = 0, s + 1
                    while cum[s + 1] == cum[s]:
                        s += 1
                nt = cum[s + 1] - cum[s]
    assert len(seen) == ntot
    read = set()
    for s in range(S):
        for c in range(C):
            nt = nts[s]
            if nt == 0:
                continue
            A = C * cum[s] + c * nt
            B = A + nt
            w_lo, w_hi = ((A + 1) * W - 1) // ntot, (B * W - 1) // ntot
            if w_lo == w_hi:
                assert (s, c) in direct
                continue
            assert (s, c) not in direct
            covered = 0
            for w in range(w_lo, w_hi + 1):
                ws = w * ntot // W
                if ws == (w + 1) * ntot // W:
                    continue
                slot = 2 * w + (0 if ws >= A else 1)
                assert written.get(slot, (None, None))[:2] == (s, c)
                read.add(slot)
                covered += written[slot][3] - written[slot][2]
            assert covered == nt
    assert read == set(written)


def cases():
    out = [[1, 15, 16, 17, 300, 2100], [0, 40, 0, 3], [1, 1, 1], [700, 1500, 33], [5, 17, 33, 64],
           [0, 0, 5], [4096] * 7]
    rnd = random.Random(313)
    for _ in range(25):
        out.append([rnd.choice([0, 1, 7, 16, 17, rnd.randint(1, 9000)]) for _ in range(rnd.randint(1, 20))])
    return [c for c in out if sum(c) > 0]


@pytest.mark.parametrize("lens", cases())
def test_balanced_schedule_covers_each_tile_once(lens):
    for C in (1, 2, 8):
        for W in list(range(1, 70)) + [255, 256, 512, 768, 2048]:
            walk(lens, C, W)
