"""Pins of the eviction oracle (oracle/evict.py).

The oracle scores blocks with exact rationals and sorts. These tests check it
against the README's printed eviction counts, against closed forms (equal
reference counts: the oldest blocks; equal ages: the least shared), and
against the defining property of a top-k computed on a separate route
(integer scores x 10): every chosen block outranks every candidate left out.
"""

import os

import numpy as np
import pytest

from oracle import evict as E

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_printed_eviction_counts():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "evict_counts.txt"))
            if l.strip() and not l.startswith("#")]
    assert rows
    for blocks, evicted in rows:
        assert E.evict_count(int(blocks)) == int(evicted)


def _outranks_everything_left_out(ref, last, tick, k, chosen):
    cand = np.flatnonzero(ref > 0)
    if cand.size == 0:
        return chosen.size == 0
    maxr = ref[cand].max()
    s10 = {int(b): 7 * (int(maxr) - int(ref[b])) + 3 * (tick - int(last[b])) for b in cand}
    chosen_set = set(int(b) for b in chosen)
    if len(chosen_set) != min(k, cand.size) or not chosen_set <= set(s10):
        return False
    if list(chosen) != sorted(chosen_set):
        return False
    for c in chosen_set:
        for u in set(s10) - chosen_set:
            if not (s10[c] > s10[u] or (s10[c] == s10[u] and c < u)):
                return False
    return True


@pytest.mark.parametrize("seed", range(12))
def test_top_k_property_on_random_blocks(seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(1, 60))
    ref = rng.integers(0, 5, size=nb).astype(np.int32)
    last = rng.integers(0, 40, size=nb).astype(np.int32)
    tick = 45
    for k in (0, 1, 3, nb // 2, nb, nb + 5):
        chosen = E.evict_select(ref, last, tick, k)
        assert _outranks_everything_left_out(ref, last, tick, k, chosen)


def test_equal_reference_counts_evict_the_oldest():
    rng = np.random.default_rng(5)
    nb, k = 300, 45
    ref = np.full(nb, 2, np.int32)
    last = rng.integers(0, 1000, size=nb).astype(np.int32)
    chosen = E.evict_select(ref, last, 1000, k)
    oldest = np.lexsort((np.arange(nb), last))[:k]  # by last use, then id
    assert np.array_equal(chosen, np.sort(oldest))


def test_equal_ages_evict_the_least_shared():
    rng = np.random.default_rng(6)
    nb, k = 200, 30
    ref = rng.integers(1, 9, size=nb).astype(np.int32)
    last = np.full(nb, 17, np.int32)
    chosen = E.evict_select(ref, last, 20, k)
    least = np.lexsort((np.arange(nb), ref))[:k]
    assert np.array_equal(chosen, np.sort(least))


def test_free_blocks_are_never_chosen_and_k_is_capped():
    ref = np.array([0, 1, 0, 3, 1], np.int32)
    last = np.array([0, 5, 0, 1, 9], np.int32)
    assert list(E.evict_select(ref, last, 10, 10)) == [1, 3, 4]
    assert E.evict_select(ref, last, 10, 0).size == 0
    assert E.evict_select(np.zeros(4, np.int32), np.zeros(4, np.int32), 3, 2).size == 0


def test_section_431_weights():
    # a reference weighs 0.7 and a tick of age 0.3. Block 0 has 3 fewer
    # references than the most shared block: 0.7 * 3 = 2.1; block 1 is that
    # most shared block, aged age1: 0.3 * age1. 7 ticks tie (smaller id wins).
    ref = np.array([1, 4], np.int32)
    for age1, expect in ((6, 0), (7, 0), (8, 1)):
        last = np.array([100, 100 - age1], np.int32)
        assert list(E.evict_select(ref, last, 100, 1)) == [expect]
