"""CPU oracle for the eviction choice over physical KV blocks.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg are the only callers; the product library never imports it.

What it computes, from the pages:
  * PagedKV-Fusion README, "Overview" (component A: scoring plus a top-k over
    the paged KV blocks) and the "Architecture" sequence diagram (score all
    physical blocks, get back the bottom-k eviction ids, quantize the
    survivors); its demos evict 15 % of the blocks.
  * PagedAttention & KV-Cache Memory Management (monograph), section 4.3.1
    (least reference count plus age): every page keeps a reference count and
    the tick of its last use, and
        score = alpha (max_refcnt - refcnt) + beta (current_tick - last_used_tick)
    with alpha = 0.7, beta = 0.3; a higher score marks a better page to evict.

Readings (the pages leave these open):
  * The candidates are the allocated blocks (reference count > 0); a free
    block has nothing to evict. max_refcnt is the largest reference count
    among them.
  * The README's "bottom-k" is read as the k blocks least worth keeping, that
    is the k largest scores of section 4.3.1; equal scores go to the smaller
    block id first. With k above the number of candidates, all of them.
  * The result is the set of chosen block ids, returned in ascending order.

The scores are exact rationals (alpha and beta as 7/10 and 3/10), so no
rounding decides the order.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

ALPHA = Fraction(7, 10)
BETA = Fraction(3, 10)


def eviction_scores(refcount, last_used, current_tick):
    """{block id: exact score} over the allocated blocks."""
    refcount = np.asarray(refcount, np.int64)
    last_used = np.asarray(last_used, np.int64)
    cand = np.flatnonzero(refcount > 0)
    if cand.size == 0:
        return {}
    max_ref = int(refcount[cand].max())
    return {int(b): ALPHA * (max_ref - int(refcount[b])) + BETA * (int(current_tick) - int(last_used[b]))
            for b in cand}


def evict_select(refcount, last_used, current_tick, k):
    """Ascending int32 ids of the min(k, candidates) blocks with the largest
    scores (ties: smaller id first)."""
    scores = eviction_scores(refcount, last_used, current_tick)
    order = sorted(scores, key=lambda b: (-scores[b], b))
    return np.array(sorted(order[: max(int(k), 0)]), dtype=np.int32)


def evict_count(num_blocks: int, fraction: Fraction = Fraction(15, 100)) -> int:
    """Blocks a demo evicts: floor(fraction x blocks) (the README's 15 %)."""
    return int(Fraction(num_blocks) * fraction)
