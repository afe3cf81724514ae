"""Pins of the block-manager oracle (oracle/blockmgr.py).

Checked against what the pages state (the summary's block manager items,
the glossary page's prefix-sharing allocator: a cached prefix hash returns
the same block with one more reference; the free list starts at block 0;
running out raises) and against invariants any run must keep: every block is
either free or referenced, the references add up to what the callers hold,
a hash maps to one live block, copy-on-write never writes a shared block.
"""

import random

import pytest

from oracle.blockmgr import BlockManager, internal_fragmentation


def test_free_list_order_and_exhaustion():
    m = BlockManager(4)
    assert [m.allocate()[0] for _ in range(4)] == [0, 1, 2, 3]
    with pytest.raises(MemoryError):
        m.allocate()
    m.release(2)
    m.release(0)
    assert m.allocate() == (0, False) and m.allocate() == (2, False)


def test_prefix_hash_hit_returns_the_same_block():
    m = BlockManager(8)
    b, hit = m.allocate(0xABC)
    assert not hit
    for k in range(3):
        assert m.allocate(0xABC) == (b, True)
    assert m.refcount[b] == 4 and m.num_free == 7
    for _ in range(4):
        m.release(b)
    assert m.num_free == 8
    assert m.allocate(0xABC) == (0, False)  # the hash was forgotten with the block


def test_copy_on_write():
    m = BlockManager(4)
    b, _ = m.allocate()
    assert m.copy_on_write(b) == (b, False)  # held once: write in place
    m.share(b)
    nb, copy = m.copy_on_write(b)
    assert copy and nb != b and m.refcount[b] == 1 and m.refcount[nb] == 1


def test_random_operations_keep_the_invariants():
    rng = random.Random(5)
    m = BlockManager(64)
    held = []  # one entry per reference a caller holds
    for step in range(20000):
        op = rng.random()
        try:
            if op < 0.4:
                h = rng.choice([None, None, rng.randint(0, 30)])
                b, hit = m.allocate(h)
                held.append(b)
            elif op < 0.55 and held:
                b = rng.choice(held)
                m.share(b)
                held.append(b)
            elif op < 0.9 and held:
                b = held.pop(rng.randrange(len(held)))
                m.release(b)
            elif held:
                i = rng.randrange(len(held))
                nb, copy = m.copy_on_write(held[i])
                assert copy == (nb != held[i])
                held[i] = nb
        except MemoryError:
            assert m.num_free == 0
        counts = {}
        for b in held:
            counts[b] = counts.get(b, 0) + 1
        assert all(m.refcount[b] == counts.get(b, 0) for b in range(64))
        assert sorted(m.free) == [b for b in range(64) if m.refcount[b] == 0]
        for h, b in m.cache.items():
            assert m.refcount[b] > 0 and m.hash_of[b] == h


def test_internal_fragmentation():
    assert internal_fragmentation([16, 32]) == 0.0
    assert internal_fragmentation([1]) == 15 / 16
    assert internal_fragmentation([17, 0]) == 1 - 17 / 32
    assert internal_fragmentation([]) == 0.0
