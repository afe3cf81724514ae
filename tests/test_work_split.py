"""The decode's work split, checked on the host.

Every KV head's tiles (all sequences in order, ceil(ctx / 16) per sequence)
lie on a cost line: a row of nb > 0 tiles costs R = nb + c (c, the row cost,
is 3 tiles for fp16 and 8 for INT8 and FP8), spread over its tiles, so tile j
of the row covers [C + j R / nb, C + (j + 1) R / nb) with C the cost of the
rows before it (integer division); up to 256 sequences, rows that all have
the same length take c = 0, and so does every batch of at most 64 possible
blocks per KV head (the library passes it c = 0). The total cost Q is cut at
b_k = k Q / K into K shares; a tile belongs to the share holding the last
unit of its interval. pa_split.h and the prep, decode and merge kernels use
the integer formulas restated below. A wave finds its share's ends either by
its own scan of the context lengths (up to 256 sequences: the row whose cost
range holds b, then the tile whose interval holds it) or, for larger
batches, from the prep kernel's table of the row holding each share's first
tile; both are modelled and must agree. These tests walk the shares the way
the decode waves do and check that every tile is visited exactly once, that
c = 0 gives the plain split [k T / K, (k + 1) T / K), that equal rows give
the same shares for every row cost when the shares fall on row boundaries,
that each cut (sequence, KV head) row leaves exactly one partial per share
holding its tiles in a distinct (share, slot) place (slot 1: the share
holding the row's first tile; slot 0: any later share), and that the merge's
share range, its test of which shares hold tiles of the row and its slot
rule find exactly those partials -- including empty contexts, empty shares
and fewer tiles than shares. The GPU parity tests then compare the kernels'
outputs with the oracle for many share counts.
"""

import random

import pytest


def first_share_at(x, Q, K):  # least k with k Q / K >= x
    return (x * K + Q - 1) // Q


def share_of(x, Q, K):  # largest k with k Q / K <= x, for 0 <= x < Q
    return ((x + 1) * K - 1) // Q


def tile_at_cost(d, nb, R):  # largest j with j R / nb <= d, for 0 <= d < R
    return ((d + 1) * nb - 1) // R


def walk(ctxs, K, max_blocks, c):
    S = len(ctxs)
    nblk = [(min(max(x, 0), max_blocks * 16) + 15) // 16 for x in ctxs]
    # up to 256 sequences (the waves' own scan) rows of equal length take the
    # plain split; the prep kernel of larger batches always uses the row cost
    if S <= 256 and len({nb for nb in nblk if nb}) <= 1:
        c = 0
    rc = [nb + c if nb else 0 for nb in nblk]
    rows, costs = [0], [0]
    for s in range(S):
        rows.append(rows[-1] + nblk[s])
        costs.append(costs[-1] + rc[s])
    T, Q = rows[S], costs[S]
    b = [k * Q // K for k in range(K + 1)] if Q else [0] * (K + 1)

    # the definition: each tile's cost interval, and the share of its last unit
    tile_share = []
    for s in range(S):
        for j in range(nblk[s]):
            a, e = costs[s] + j * rc[s] // nblk[s], costs[s] + (j + 1) * rc[s] // nblk[s]
            assert e > a  # every tile covers at least one unit
            tile_share.append(share_of(e - 1, Q, K))
    assert tile_share == sorted(tile_share)
    if c == 0 and T:
        assert tile_share == [share_of(t, T, K) for t in range(T)]

    # prep kernel (large batches): the row whose cost range holds b_k (none
    # when no sequence has a tile)
    first_row = [None] * K
    for s in range(S if Q else 0):
        for k in range(first_share_at(costs[s], Q, K), min(first_share_at(costs[s + 1], Q, K), K)):
            assert first_row[k] is None
            first_row[k] = s
    if Q:
        assert None not in first_row

    def tile_at(row, x):  # through a known row
        return rows[row] + tile_at_cost(x - costs[row], nblk[row], rc[row])

    # a wave's own scan (small batches): the one row with costs[s] <= x < costs[s] + rc[s]
    def scan_tile_at(x):
        hits = [s for s in range(S) if rc[s] > 0 and costs[s] <= x < costs[s] + rc[s]]
        assert len(hits) == 1
        return tile_at(hits[0], x), hits[0]

    shares = []
    for k in range(K):
        p0 = scan_tile_at(b[k])[0] if b[k] < Q else T
        p1 = scan_tile_at(b[k + 1])[0] if b[k + 1] < Q else T
        # the prep path agrees
        if Q:
            assert p0 == (tile_at(first_row[k], b[k]) if b[k] < Q else T)
            assert p1 == (tile_at(first_row[k + 1], b[k + 1]) if k + 1 < K else T)
        assert p0 <= p1
        assert all(tile_share[t] == k for t in range(p0, p1))
        shares.append((p0, p1))
    if c == 0:
        assert shares == [(k * T // K, (k + 1) * T // K) for k in range(K)]

    # decode waves: a share's later segments (each from a row's first block)
    # first, its first segment (which may start mid-row) last
    def next_row(r):
        r += 1
        while rows[r + 1] == rows[r]:
            r += 1
        return r

    def row_of(t):
        return max(s for s in range(S) if rows[s] <= t and nblk[s] > 0)

    owner, parts, finished = {}, {}, set()
    for k, (p0, p1) in enumerate(shares):
        if p0 >= p1:
            continue
        s0 = row_of(p0)
        j0 = p0 - rows[s0]
        assert 0 <= j0 < nblk[s0]
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
        for s, j, nseg in segs:
            nb = nblk[s]
            for t in range(rows[s] + j, rows[s] + j + nseg):
                assert t not in owner
                owner[t] = k
            if j > 0 or j + nseg < nb:
                slot = 1 if j == 0 else 0
                assert (k, slot) not in parts
                parts[(k, slot)] = s
            else:
                assert s not in finished
                finished.add(s)
    assert len(owner) == T

    # merge
    for s in range(S):
        nb = nblk[s]
        if nb == 0:
            assert s not in finished
            continue
        c0, c1 = costs[s], costs[s + 1]
        R = c1 - c0
        kf, kl = share_of(c0 + R // nb - 1, Q, K), share_of(c1 - 1, Q, K)
        assert kf == tile_share[rows[s]] and kl == tile_share[rows[s + 1] - 1]
        if kf == kl:
            assert s in finished
            continue
        assert s not in finished
        merged = set()
        none_empty = Q >= K * (1 + c)  # every share spans the widest tile
        for k in range(kf, kl + 1):
            if k == kf or none_empty:
                live = True
                if none_empty:
                    assert shares[k][0] < shares[k][1]
            else:
                b1 = (k + 1) * Q // K
                live = b1 >= c1 or tile_at_cost(b1 - c0, nb, R) != tile_at_cost(k * Q // K - c0, nb, R)
            if not live:
                assert (k, 0) not in parts or parts[(k, 0)] != s
                continue
            slot = 1 if k == kf else 0
            assert parts[(k, slot)] == s
            merged.add(k)
        assert merged == {owner[t] for t in range(rows[s], rows[s + 1])}
    return shares


@pytest.mark.parametrize("c", [0, 3, 6, 8, 10])
@pytest.mark.parametrize("K", [1, 2, 3, 5, 8, 13, 64, 300])
def test_random_batches(K, c):
    rng = random.Random(K * 10 + c)
    for _ in range(300):
        mb = rng.randint(1, 12)
        ctxs = [rng.choice([0, -2, rng.randint(1, mb * 16 + 30)]) for _ in range(rng.randint(1, 14))]
        walk(ctxs, K, mb, c)


@pytest.mark.parametrize("c", [0, 3, 6, 8, 10])
def test_edge_batches(c):
    walk([0, 0, 0], 4, 8, c)          # nothing to do
    walk([5], 1, 1, c)                # one tile, one share
    walk([16 * 7], 64, 7, c)          # fewer tiles than shares
    walk([1] * 50, 7, 1, c)           # many one-tile rows per share
    walk([16 * 1000, 3, 0, 17], 128, 1000, c)
    walk([16 * 40] * 300, 1500, 40, c)  # every row cut into several shares
    rng = random.Random(7)
    walk([rng.randint(0, 80) for _ in range(300)], 97, 5, c)


def test_equal_rows_keep_the_plain_split():
    # shares that fall on row boundaries under the plain split stay there,
    # with the same tiles, whatever the row cost (the uniform batches:
    # 32 x 1,024 and 64 x 2,048 tokens over 128 shares per head; and past 256
    # sequences, where the prep kernel keeps the row cost for equal rows too)
    for S, nb, K in ((32, 64, 128), (64, 128, 128), (8, 32, 32), (4, 16, 16), (300, 8, 600)):
        plain = walk([16 * nb] * S, K, nb, 0)
        for c in (3, 4, 8):
            assert walk([16 * nb] * S, K, nb, c) == plain


def test_row_cost_moves_tiles_off_shares_that_start_many_rows():
    # short rows next to a long one: with a row cost, the shares over the
    # short rows hold fewer tiles than those inside the long row
    ctxs = [16 * 4] * 24 + [16 * 96]
    sh = walk(ctxs, 8, 96, 8)
    lengths = [p1 - p0 for p0, p1 in sh]
    assert lengths[0] < lengths[-1]
    assert walk(ctxs, 8, 96, 0) == [(k * 192 // 8, (k + 1) * 192 // 8) for k in range(8)]


def _div_floor_model(x, y, rel_err):
    """The split's integer division as the kernels do it: a reciprocal of y with
    relative error rel_err (the hardware's is 2^-23 or better), two Newton
    steps, the double-precision estimate of x / y truncated, then at most one
    exact integer correction either way; None if more would be needed."""
    yd = float(y)
    r = (1.0 / yd) * (1.0 + rel_err)
    for _ in range(2):
        r = r + r * (1.0 - yd * r)
    q = int(float(x) * r)
    if q * y > x:
        q -= 1
    elif (q + 1) * y <= x:
        q += 1
    return q if q * y <= x < (q + 1) * y else None


def test_div_floor_estimate_is_within_one():
    # every quotient of the split is below 2^31; numerators reach k * Q with
    # k < 2^16 shares per head; the reciprocal taken 2^10 times worse than the
    # hardware's promise still leaves the estimate within one
    rng = random.Random(5)
    cases = [(0, 1), (1, 1), (2**31 - 1, 1), (2**62, 2**31 + 5), (2**47 - 1, 2**16 - 1)]
    for _ in range(20000):
        y = rng.choice([rng.randint(1, 64), rng.randint(1, 2**16), rng.randint(1, 2**31 - 1)])
        q = rng.randint(0, 2**31 - 1)
        x = q * y + rng.choice([0, 1, y - 1, rng.randint(0, y - 1)])
        cases.append((x, y))
    for x, y in cases:
        for e in (0.0, 2.0**-13, -(2.0**-13)):
            assert _div_floor_model(x, y, e) == x // y, (x, y, e)
