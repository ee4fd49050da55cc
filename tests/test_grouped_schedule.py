"""CPU model of the grouped decode's work units (decode_group_kernel): the
shared units (group, member chunk, head group, partition) and the private
units (sequence, head group, partition) together write every partial row
that the partition merge reads exactly once, write nothing else, give every
sequence that fits one partition its output directly, and read table
entries only inside the leader's valid blocks.  The model restates the
kernel's index arithmetic; group sizes, shared lengths and host bounds are
drawn at random, including the ones the call must correct."""

import numpy as np
import pytest


def shared_tokens(gs, gsh, lens, grp, first, end, P, shared_parts):
    sh = int(gsh[grp])
    sh = 0 if sh < 0 else sh - sh % P
    sh = min(sh, shared_parts * P)
    for s in range(max(first, 0), end):   # an empty member: (0 - 1) / P truncates to 0 in C
        sh = min(sh, max(int(lens[s]) - 1, 0) // P * P)
    return max(sh, 0)


def find_group(gs, s):
    G = len(gs) - 1
    if G <= 0 or s < gs[0] or s >= gs[G]:
        return None
    lo, hi = 0, G
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if gs[mid] <= s:
            lo = mid
        else:
            hi = mid
    return lo, int(gs[lo]), int(gs[lo + 1])


def run_grid(gs, gsh, lens, P, C, KM, max_group, max_shared):
    """Returns {(s, c, p): writer} for partial rows and the set of direct rows."""
    S = len(lens)
    NP = max(1, -(-int(lens.max(initial=0)) // P))
    G = len(gs) - 1
    shared_parts = min(-(-max_shared // P), NP)
    MC = -(-max_group // KM)
    nsh = MC * G * C * shared_parts
    partial, direct, reads = {}, set(), []
    for u in range(nsh + S * C * NP):
        if u < nsh:
            mc, rest = u % MC, u // MC
            grp, rest = rest % G, rest // G
            c, p = rest % C, rest // C
            first, end = int(gs[grp]), min(int(gs[grp + 1]), S)
            s0 = first + mc * KM
            km = min(KM, end - s0)
            if first < 0 or km <= 0:
                continue
            t0 = p * P
            if t0 >= shared_tokens(gs, gsh, lens, grp, first, end, P, shared_parts):
                continue
            reads.append((s0, t0, t0 + P))
            for i in range(km):
                key = (s0 + i, c, p)
                assert key not in partial, f"partial row {key} written twice"
                partial[key] = ("shared", u)
            continue
        v = u - nsh
        s, rest = v % S, v // S
        c, p = rest % C, rest // C
        L = int(lens[s])
        if L == 0:
            if p == 0:
                direct.add((s, c))
            continue
        t0 = p * P
        if t0 >= L:
            continue
        g = find_group(gs, s)
        if g is not None:
            grp, first, end = g
            if s - first < MC * KM and t0 < shared_tokens(gs, gsh, lens, grp, first, min(end, S), P, shared_parts):
                continue
        if L <= P:
            direct.add((s, c))
        else:
            key = (s, c, p)
            assert key not in partial, f"partial row {key} written twice"
            partial[key] = ("private", u)
        reads.append((s, t0, min(t0 + P, L)))
    return partial, direct, reads


@pytest.mark.parametrize("seed", range(40))
def test_every_merged_row_written_once(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.choice([16, 64, 256, 512]))
    KM = int(rng.choice([1, 2, 4]))
    C = int(rng.integers(1, 4))
    sizes = rng.integers(1, 10, size=int(rng.integers(1, 8)))
    S = int(sizes.sum()) + int(rng.integers(0, 4))          # some sequences outside every group
    lens = rng.integers(0, 6 * P, size=S)
    lens[rng.random(S) < 0.1] = 0
    gs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    gsh = rng.integers(-P, 5 * P, size=len(sizes))             # not whole partitions, too long, negative
    max_group = int(rng.integers(1, int(sizes.max()) + 2))      # may be below the true group size
    max_shared = int(rng.integers(0, 6 * P))
    partial, direct, reads = run_grid(gs, gsh, lens, P, C, KM, max_group, max_shared)
    for s in range(S):
        np_s = -(-int(lens[s]) // P)
        for c in range(C):
            if np_s <= 1:
                assert (s, c) in direct and not any((s, c, p) in partial for p in range(8 * P))
            else:
                assert (s, c) not in direct
                for p in range(np_s):
                    assert (s, c, p) in partial, f"merge reads unwritten row {(s, c, p)}"
    assert all(p < -(-int(lens[s]) // P) for (s, c, p) in partial)
    for s, t0, t1 in reads:   # the reader's own valid tokens, whole partitions of them when shared
        assert 0 <= t0 < t1 <= lens[s]


def test_shared_units_cover_the_prefix_shared_workload():
    """64 prompts x 8 samples sharing 1024 tokens of 1288, 512-token
    partitions, 4 samples per shared unit: the first two partitions of every
    sample come from shared units, 128 x 8 of them, the third from its own."""
    S, P, C = 512, 512, 8
    lens = np.full(S, 1288)
    gs = np.arange(0, S + 1, 8)
    gsh = np.full(64, 1024)
    partial, direct, reads = run_grid(gs, gsh, lens, P, C, 4, 8, 1024)
    kinds = {}
    for (s, c, p), (kind, _) in partial.items():
        kinds.setdefault(p, set()).add(kind)
    assert kinds == {0: {"shared"}, 1: {"shared"}, 2: {"private"}}
    assert len(partial) == S * C * 3 and not direct
    shared_units = {u for kind, u in partial.values() if kind == "shared"}
    assert len(shared_units) == 64 * 2 * C * 2
