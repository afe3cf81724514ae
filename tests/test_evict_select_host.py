"""The eviction kernel's selection method, run on the host and checked
against the oracle: integer keys 3 * age - 7 * refcount, 8-bit radix passes
over the key range to find the k-th largest key, then one pass in block
order taking the keys above it and the first (by id) of the keys equal to
it. This restates pa_evict.hip's steps in Python so that the arithmetic of
the passes (digit choice, remaining count, ties) is tested for many shapes
without a GPU; the GPU tests then compare the kernel itself with the oracle.
"""

import numpy as np
import pytest

from oracle import evict as E


def radix_select(ref, last, tick, k):
    cand = [b for b in range(len(ref)) if ref[b] > 0]
    keys = {b: 3 * (int(tick) - int(last[b])) - 7 * int(ref[b]) for b in cand}
    keff = min(k, len(cand))
    if keff == 0:
        return np.full(k, -1, np.int32)
    kmin, kmax = min(keys.values()), max(keys.values())
    prefix, rem = 0, keff
    nbits = (kmax - kmin).bit_length()
    shift = ((nbits + 7) // 8 - 1) * 8
    while shift >= 0:
        hist = [0] * 256
        for b in cand:
            u = keys[b] - kmin
            if (u >> (shift + 8)) != (prefix >> (shift + 8)):
                continue
            hist[(u >> shift) & 255] += 1
        above = 0
        for d in range(255, -1, -1):  # the digit holding the rem-th largest
            if above < rem <= above + hist[d]:
                break
            above += hist[d]
        rem -= above
        prefix |= d << shift
        shift -= 8
    out, equal = [], 0
    for b in cand:  # block order
        u = keys[b] - kmin
        if u > prefix:
            out.append(b)
        elif u == prefix:
            if equal < rem:
                out.append(b)
            equal += 1
    assert len(out) == keff
    return np.array(out + [-1] * (k - keff), np.int32)


@pytest.mark.parametrize("seed", range(8))
def test_radix_select_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    for _ in range(150):
        nb = int(rng.integers(1, 150))
        ref = rng.integers(0, int(rng.integers(1, 12)), size=nb)
        hi = int(rng.choice([1, 4, 300, 2**20, 2**31 - 1]))
        last = rng.integers(-hi if seed % 2 else 0, hi, size=nb)
        tick = int(rng.integers(0, hi))
        k = int(rng.integers(0, nb + 4))
        want = E.evict_select(ref, last, tick, k)
        want = np.concatenate([want, np.full(k - want.size, -1, np.int32)])
        assert np.array_equal(radix_select(ref, last, tick, k), want)
