"""The balanced split's bookkeeping, checked on the CPU: every tile of every
(sequence, head group) is processed by exactly one wave, every piece that a
wave writes to a partial slot is read back by the merge exactly once, and the
merge never reads a slot that no wave wrote.

The walk below mirrors the index arithmetic of decode_balanced_kernel and
decode_merge_balanced_kernel: each (sequence, head group) with tiles costs X
virtual units (a segment start) followed by its nt tiles in the flattened
space, wave w of W takes [w ntot / W, (w+1) ntot / W), its first real segment
goes to slot 2w and its last to 2w+1, and the merge finds the waves w_lo..w_hi
that hold the real tiles and skips those with empty ranges.  It is a model of
the schedule; the kernels themselves are checked against the oracle on the
GPU."""

import random

import pytest

TILE = 16


def walk(lens, C, W, X=0):
    S = len(lens)
    nts = [-(-L // TILE) for L in lens]
    cum = [0]
    for n in nts:
        cum.append(cum[-1] + (n + X if n else 0))
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
        ntc = cum[s + 1] - cum[s]
        rel = f - C * cum[s]
        c, u = rel // ntc, rel % ntc
        first = True
        while f < fb:
            n = min(ntc - u, fb - f)
            nt = ntc - X
            t0, t1 = max(u - X, 0), min(u + n - X, nt)
            if t1 > t0:
                for tt in range(t0, t1):
                    assert (s, c, tt) not in seen
                    seen[(s, c, tt)] = w
                if t0 == 0 and t1 == nt:
                    direct.add((s, c))
                else:
                    slot = 2 * w + (0 if first else 1)
                    assert slot not in written
                    written[slot] = (s, c, t0, t1)
                first = False
            f += n
            u += n
            if u == ntc and f < fb:
                u, c = 0, c + 1
                if c == C:
                    c, s = 0, s + 1
                    while cum[s + 1] == cum[s]:
                        s += 1
                ntc = cum[s + 1] - cum[s]
    assert len(seen) == C * sum(nts)
    # the merge over wave boundaries: boundary w (1 <= w < W) merges the head
    # group whose tiles it is the first to split
    merged = {}
    for w in range(1, W):
        b = w * ntot // W
        if b == 0 or b >= ntot:
            continue
        lo, hi = 0, S - 1
        while lo < hi:
            mid = (lo + hi + 1) >> 1
            if C * cum[mid] <= b - 1:
                lo = mid
            else:
                hi = mid - 1
        s = lo
        ntc = cum[s + 1] - cum[s]
        c = (b - 1 - C * cum[s]) // ntc
        A = C * cum[s] + c * ntc + X
        B = A + ntc - X
        if A < b < B and (w - 1) * ntot // W <= A:
            assert (s, c) not in merged
            merged[(s, c)] = w
    split = {(s, c) for s in range(S) for c in range(C) if nts[s] and (s, c) not in direct}
    assert set(merged) == split
    read = set()
    for s in range(S):
        for c in range(C):
            nt = nts[s]
            if nt == 0:
                continue
            A0 = C * cum[s] + c * (nt + X)        # the unit's cost start
            A = A0 + X                             # its first real tile
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
                slot = 2 * w + (0 if ws >= A0 else 1)
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


@pytest.mark.parametrize("X", [0, 1, 3, 8])
@pytest.mark.parametrize("lens", cases())
def test_balanced_schedule_covers_each_tile_once(lens, X):
    for C in (1, 2, 8):
        for W in list(range(1, 70)) + [255, 256, 512, 768, 2048]:
            walk(lens, C, W, X)


def walk_parts(lens, C, W, P, X):
    """decode_parts_resident_kernel's schedule: units (s, c, p) of P tokens,
    unit (s, c, p) at C cum[s] + c cost(s) + p (X + P/16), cost(s) =
    ceil(L/16) + X ceil(L/P); wave w runs the units starting in
    [w ntot / W, (w+1) ntot / W), in order, as runs of one head group's
    consecutive partitions."""
    S, PT = len(lens), P // TILE
    nts = [-(-L // TILE) for L in lens]
    nps = [-(-L // P) for L in lens]
    cum = [0]
    for n, q in zip(nts, nps):
        cum.append(cum[-1] + (n + q * X if n else 0))
    ntot = C * cum[S]
    done = {}
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
        cost = cum[s + 1] - cum[s]
        assert cost > 0
        rel = f - C * cum[s]
        c = rel // cost
        r = rel - c * cost
        p = (r + X + PT - 1) // (X + PT)
        ustart = C * cum[s] + c * cost + p * (X + PT)
        np_ = nps[s]
        prev = None
        while True:
            if p >= np_:
                p = 0
                c += 1
                if c == C:
                    c = 0
                    s += 1
                    while s < S and cum[s + 1] == cum[s]:
                        s += 1
                    if s >= S:
                        break
                    cost = cum[s + 1] - cum[s]
                    np_ = nps[s]
                ustart = C * cum[s] + c * cost
            if ustart >= fb:
                break
            assert ustart >= f
            # the head group's partitions p .. pl that start before fb, one run
            sc0 = ustart - p * (X + PT)
            pl = min(np_ - 1, (fb - sc0 + X + PT - 1) // (X + PT) - 1)
            assert pl >= p
            for q in range(p, pl + 1):
                assert sc0 + q * (X + PT) < fb
                assert (s, c, q) not in done
                done[(s, c, q)] = w
                assert prev is None or prev < (s, c, q)      # in order
                prev = (s, c, q)
            ustart += (pl + 1 - p) * (X + PT)
            p = pl + 1
    want = {(s, c, p) for s in range(S) for c in range(C) for p in range(nps[s])}
    assert set(done) == want


@pytest.mark.parametrize("X", [0, 1, 3, 8])
@pytest.mark.parametrize("lens", cases())
def test_resident_partition_schedule_runs_each_unit_once(lens, X):
    for P in (16, 64, 512):
        for C in (1, 2, 8):
            for W in list(range(1, 40)) + [255, 1024]:
                walk_parts(lens, C, W, P, X)
