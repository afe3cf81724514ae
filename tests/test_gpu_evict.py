"""GPU parity of the eviction choice (pa_evict_select) against the oracle.

The chosen block ids must equal the oracle's exactly (ascending, -1 padded)
at the README's pool sizes (1,024 and 16,384 blocks), the mixed batch's
65,536-block pool with its reference counts, and the edge cases: k = 0, k
above the number of candidates, no candidates, every score equal, and ticks
spanning the whole int32 range.
"""

import numpy as np
import pytest

import oracle.evict as E
import paged_kv_cache_228_amd as pa
from paged_kv_cache_228_amd import workloads as W

from gpu_util import dev, say, sync

pytestmark = pytest.mark.gpu


def gpu_select(ref, last, tick, k):
    out = pa.pa_evict_select(dev(ref), dev(last), tick, k)
    sync()
    return out.cpu().numpy()


def expect(ref, last, tick, k):
    ids = E.evict_select(ref, last, tick, k)
    return np.concatenate([ids, np.full(k - ids.size, -1, np.int32)])


@pytest.mark.parametrize("nb", [1024, 16384])
@pytest.mark.parametrize("frac", [0.0, 0.15, 0.5, 1.0])
def test_readme_pool_sizes(nb, frac):
    ref, last = W.eviction_inputs(nb, 50 + nb)
    k = int(nb * frac)
    say(f"evict nb={nb} k={k}")
    assert np.array_equal(gpu_select(ref, last, 10_000, k), expect(ref, last, 10_000, k))


def test_mixed_batch_pool():
    w = W.mixed_prefix()
    ref, last = W.eviction_inputs(w.num_blocks, 51, refcount=w.refcount)
    k = E.evict_count(int((ref > 0).sum()))
    say(f"evict mixed pool nb={w.num_blocks} candidates={(ref > 0).sum()} k={k}")
    assert np.array_equal(gpu_select(ref, last, 10_000, k), expect(ref, last, 10_000, k))


def test_edge_cases():
    rng = np.random.default_rng(9)
    ref = np.array([0, 2, 0, 1, 1], np.int32)
    last = np.array([0, 3, 0, 9, 1], np.int32)
    for k in (1, 3, 4, 9):
        assert np.array_equal(gpu_select(ref, last, 10, k), expect(ref, last, 10, k))
    z = np.zeros(4000, np.int32)
    assert np.array_equal(gpu_select(z, z, 5, 7), np.full(7, -1, np.int32))
    flat = np.ones(5000, np.int32)  # every score equal: the smallest ids
    assert np.array_equal(gpu_select(flat, z[:1] + np.zeros(5000, np.int32), 3, 700),
                          np.arange(700, dtype=np.int32))
    big = rng.integers(1, 2**31 - 1, size=3000).astype(np.int32)
    ages = rng.integers(-2**31, 2**31 - 1, size=3000).astype(np.int32)
    for k in (1, 450, 2999):
        assert np.array_equal(gpu_select(big, ages, 2**31 - 1, k),
                              expect(big, ages, 2**31 - 1, k))
