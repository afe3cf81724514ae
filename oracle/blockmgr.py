"""CPU oracle for the KV block manager.

TEST INFRASTRUCTURE ONLY: the tests and the benchmark's CPU baseline leg are
the only callers; the product library never imports it.

What it models, from the pages:
  * paged-attention-runtime summary, "CORE CAPABILITIES" 1 (Block Manager):
    fixed 16-token blocks, a free-list allocator, reference counting, prefix
    sharing, copy-on-write, fragmentation metrics.
  * PagedAttention & KV-Cache Memory Management (glossary page): the
    prefix-sharing allocator keeps, per physical block, a reference count and
    an optional prefix (content) hash; allocating with a hash that is
    already cached hands out that block again with one more reference; the
    free list hands out the lowest free id first (its initial order is the
    ids in ascending order); running out raises.

Readings (the pages leave these open):
  * Releasing a reference that brings a block to zero returns it to the free
    list (it is handed out before higher free ids) and forgets its hash.
  * Copy-on-write of a block with more than one reference takes a fresh
    block (no hash), moves the caller's reference to it and reports that the
    contents must be copied; a block held once is written in place.
  * Internal fragmentation of a batch: the unused token slots of the
    sequences' blocks over all their slots, 1 - sum(ctx) / (16 sum(ceil(ctx/16))).
"""

from __future__ import annotations

import heapq


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int = 16):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("sizes must be positive")
        self.block_size = block_size
        self.refcount = [0] * num_blocks
        self.hash_of = [None] * num_blocks
        self.free = list(range(num_blocks))  # a heap: lowest id first
        self.cache: dict[int, int] = {}

    def allocate(self, prefix_hash=None):
        """(block id, cache hit)."""
        if prefix_hash is not None and prefix_hash in self.cache:
            b = self.cache[prefix_hash]
            self.refcount[b] += 1
            return b, True
        if not self.free:
            raise MemoryError("no free KV block")
        b = heapq.heappop(self.free)
        self.refcount[b] = 1
        self.hash_of[b] = prefix_hash
        if prefix_hash is not None:
            self.cache[prefix_hash] = b
        return b, False

    def share(self, b: int) -> None:
        if self.refcount[b] <= 0:
            raise ValueError("block is not allocated")
        self.refcount[b] += 1

    def release(self, b: int) -> None:
        if self.refcount[b] <= 0:
            raise ValueError("block is not allocated")
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            h = self.hash_of[b]
            if h is not None and self.cache.get(h) == b:
                del self.cache[h]
            self.hash_of[b] = None
            heapq.heappush(self.free, b)

    def copy_on_write(self, b: int):
        """(block to write, whether its contents must first be copied from b)."""
        if self.refcount[b] <= 0:
            raise ValueError("block is not allocated")
        if self.refcount[b] == 1:
            return b, False
        nb, _ = self.allocate(None)
        self.refcount[b] -= 1
        return nb, True

    @property
    def num_free(self) -> int:
        return len(self.free)


def internal_fragmentation(context_lens, block_size: int = 16) -> float:
    slots = sum(-(-int(n) // block_size) * block_size for n in context_lens if n > 0)
    used = sum(int(n) for n in context_lens if n > 0)
    return 0.0 if slots == 0 else 1.0 - used / slots
