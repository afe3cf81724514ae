"""The decode's work split, checked on the host.

The decode cuts each KV head's tiles (all sequences in order, ceil(ctx / 16)
per sequence) into K equal contiguous shares, share k = [k T / K, (k + 1) T / K)
with integer division; pa_split.h and the prep, decode and merge kernels use
the integer formulas restated below. A wave finds the row holding its share's
first tile either by its own scan of the context lengths (up to 256
sequences: the row whose tile range contains the tile) or, for larger
batches, from the prep kernel's table of share first rows; both are modelled
and must agree. These tests walk the shares the way the decode waves do and
check that every tile is visited exactly once, that each cut (sequence, KV
head) row leaves exactly one partial per share holding its tiles in a
distinct (share, slot) place, and that the merge's share range (first and
last share from the row's prefix sums) and slot rule find exactly those
partials -- including empty contexts and fewer tiles than shares. The GPU
parity tests then compare the kernels' outputs with the oracle for many share
counts.
"""

import random

import pytest


def first_share_at(x, T, K):  # least k with k T / K >= x
    return (x * K + T - 1) // T


def share_of(x, T, K):  # largest k with k T / K <= x, for 0 <= x < T
    return ((x + 1) * K - 1) // T


def share_empty(k, T, K):
    return (k + 1) * T // K == k * T // K


def walk(ctxs, K, max_blocks):
    S = len(ctxs)
    nblk = [(min(max(c, 0), max_blocks * 16) + 15) // 16 for c in ctxs]
    rows = [0]
    for b in nblk:
        rows.append(rows[-1] + b)
    T = rows[S]
    # prep (large batches): first row of every share
    first_row = [None] * K
    for s in range(S):
        r0, r1 = rows[s], rows[s + 1]
        if r0 == r1:
            continue
        for k in range(first_share_at(r0, T, K), min(first_share_at(r1, T, K), K)):
            assert first_row[k] is None
            first_row[k] = s
    if T:
        assert None not in first_row

    # a wave's own scan (small batches): the one row with rows[s] <= p0 < rows[s + 1]
    def scan_first_row(p0):
        hits = [s for s in range(S) if nblk[s] > 0 and rows[s] <= p0 < rows[s] + nblk[s]]
        assert len(hits) == (1 if p0 < T else 0)
        return hits[0] if hits else 0

    for k in range(K):
        p0 = k * T // K
        if p0 < (k + 1) * T // K:
            assert scan_first_row(p0) == first_row[k]
    # merge: first / last share of every row, from its prefix sums
    kf_kl = {s: (share_of(rows[s], T, K), share_of(rows[s + 1] - 1, T, K))
             for s in range(S) if rows[s + 1] > rows[s]}
    # decode waves: a share's later segments (each from a row's first block)
    # first, its first segment (which may start mid-row) last
    def next_row(r):
        r += 1
        while rows[r + 1] == rows[r]:
            r += 1
        return r

    owner, parts, finished = {}, {}, set()
    for k in range(K):
        p0, p1 = k * T // K, (k + 1) * T // K
        if p0 >= p1:
            continue
        s0 = first_row[k]
        j0 = p0 - rows[s0]
        assert 0 <= j0 < nblk[s0]
        nseg0 = min(nblk[s0] - j0, p1 - p0)
        segs = []
        pos, s, j = p0, s0, j0
        while pos < p1:
            nseg = min(rows[s + 1] - rows[s] - j, p1 - pos)
            segs.append((s, j, nseg))
            pos += nseg
            if pos < p1:
                s, j = next_row(s), 0
        if j0 > 0 and len(segs) > 1:
            segs = segs[1:] + segs[:1]
        assert segs[-1 if j0 > 0 and len(segs) > 1 else 0] == (s0, j0, nseg0)
        for s, j, nseg in segs:
            nb = rows[s + 1] - rows[s]
            for t in range(rows[s] + j, rows[s] + j + nseg):
                assert t not in owner
                owner[t] = k
            if j > 0 or j + nseg < nb:
                slot = 0 if (s, j) == (s0, j0) else 1
                assert (k, slot) not in parts
                parts[(k, slot)] = s
            else:
                assert s not in finished
                finished.add(s)
    assert len(owner) == T
    # merge
    for s in range(S):
        r0, r1 = rows[s], rows[s + 1]
        if r0 == r1:
            assert s not in finished
            continue
        kf, kl = kf_kl[s]
        if kf == kl:
            assert s in finished
            continue
        assert s not in finished
        merged = set()
        for k in range(kf, kl + 1):
            if share_empty(k, T, K):
                continue
            slot = 1 if (k == kf and k * T // K < r0) else 0
            assert parts[(k, slot)] == s
            merged.add(k)
        assert merged == {owner[t] for t in range(r0, r1)}


@pytest.mark.parametrize("K", [1, 2, 3, 5, 8, 13, 64, 300])
def test_random_batches(K):
    rng = random.Random(K)
    for _ in range(400):
        mb = rng.randint(1, 12)
        ctxs = [rng.choice([0, -2, rng.randint(1, mb * 16 + 30)]) for _ in range(rng.randint(1, 14))]
        walk(ctxs, K, mb)


def test_edge_batches():
    walk([0, 0, 0], 4, 8)          # nothing to do
    walk([5], 1, 1)                # one tile, one share
    walk([16 * 7], 64, 7)          # fewer tiles than shares
    walk([1] * 50, 7, 1)           # many one-tile rows per share
    walk([16 * 1000, 3, 0, 17], 128, 1000)
