"""Seeded synthetic inputs for paged single-token decode attention.

This module draws random numbers and lays them out in the paged format; it
does none of the attention or quantization arithmetic. Both the CPU oracle
(``oracle/``) and the HIP path are fed from it, so it must stay free of the
method's math.

Layout (shared by every consumer):

* K and V pools: fp16 ``[num_blocks][num_kv_heads][16][head_dim]``; slot ``o``
  of physical block ``b`` for KV head ``h`` is ``pool[b, h, o, :]``.
* Block table: int32 ``[num_seqs][max_blocks_per_seq]``; token ``t`` of
  sequence ``s`` lives in block ``table[s, t // 16]`` at slot ``t % 16``
  (PagedAttention & KV-Cache glossary page, section 2.1 "Logical Token Blocks
  & Page Tables"). Entries past a sequence's last block are ``-1``.
* ``context_lens``: int32 ``[num_seqs]``; queries: fp16 ``[num_seqs][H_q][d]``.

Physical blocks come from a small reference-counted allocator with a shuffled
free list, modelled on the block managers the pages describe (PagedKV-Fusion
README "Architecture", scheduler / block table; paged-attention-runtime
summary, "CORE CAPABILITIES" 1 "Block Manager": fixed 16-token blocks, free
list, reference counting, prefix sharing; glossary page "Implementation
Example", ``KVBlockAllocator``).

Values: fp32 draws from numpy's PCG64, rounded to fp16 (round-half-even).
Large pools are drawn in fixed chunks of blocks, each chunk from its own
``SeedSequence`` child keyed by (tensor, chunk index), so results do not
depend on the number of threads used.
"""

from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
_CHUNK_BLOCKS = 256


class BlockAllocator:
    """Free list of physical block ids with per-block reference counts.

    ``allocate`` pops a fresh block (refcount 1); ``share`` adds a reference to
    an already allocated block, the way a prefix-shared block is handed to a
    second sequence.
    """

    def __init__(self, num_blocks: int, rng: np.random.Generator, shuffle: bool = True):
        order = rng.permutation(num_blocks) if shuffle else np.arange(num_blocks)
        self._free = [int(b) for b in order[::-1]]  # pop() yields order[0] first
        self.refcount = np.zeros(num_blocks, dtype=np.int32)

    def allocate(self) -> int:
        if not self._free:
            raise MemoryError("KV block pool exhausted")
        bid = self._free.pop()
        self.refcount[bid] = 1
        return bid

    def share(self, bid: int) -> int:
        if self.refcount[bid] <= 0:
            raise ValueError(f"block {bid} is not allocated")
        self.refcount[bid] += 1
        return bid

    @property
    def num_free(self) -> int:
        return len(self._free)


@dataclass
class Workload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    context_lens: np.ndarray  # int32 [S]
    block_tables: np.ndarray  # int32 [S][MB], -1 past the last block
    q: np.ndarray  # fp16 [S][Hq][d]
    k_pool: np.ndarray  # fp16 [NB][Hkv][16][d], dead slots hold 0
    v_pool: np.ndarray  # fp16, same layout
    live: np.ndarray  # bool [NB][16]: slot holds a token some sequence attends to
    refcount: np.ndarray  # int32 [NB]
    block_size: int = BLOCK_SIZE
    notes: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(1.0) / np.sqrt(np.float32(self.head_dim)))

    def live_block_ids(self) -> np.ndarray:
        return np.flatnonzero(self.refcount > 0).astype(np.int32)

    def dead_slot_mask(self) -> np.ndarray:
        """bool [NB][16]: slots no sequence reads (tails and unused blocks)."""
        return ~self.live

    def poisoned(self, pool: np.ndarray) -> np.ndarray:
        """Copy of an fp16 pool with NaN in every dead slot (proves masking)."""
        out = pool.copy()
        out.transpose(0, 2, 1, 3)[self.dead_slot_mask()] = np.float16(np.nan)
        return out


def _table_from_lists(lists: list[list[int]]) -> np.ndarray:
    mb = max(1, max((len(x) for x in lists), default=1))
    table = np.full((len(lists), mb), -1, dtype=np.int32)
    for s, ids in enumerate(lists):
        table[s, : len(ids)] = ids
    return table


def _live_mask(num_blocks: int, context_lens: np.ndarray, table: np.ndarray) -> np.ndarray:
    live = np.zeros((num_blocks, BLOCK_SIZE), dtype=bool)
    for s, n in enumerate(context_lens):
        n = int(n)
        full, rem = divmod(n, BLOCK_SIZE)
        if full:
            live[table[s, :full]] = True
        if rem:
            live[table[s, full], :rem] = True
    return live


def _fill_normal_blocks(pool: np.ndarray, block_ids: np.ndarray, seed: int, tensor: int,
                        threads: int | None = None) -> None:
    """pool[block_ids] = fp16(N(0,1) fp32 draws), chunk by chunk."""
    per_block = int(np.prod(pool.shape[1:]))
    chunks = [block_ids[i : i + _CHUNK_BLOCKS] for i in range(0, len(block_ids), _CHUNK_BLOCKS)]

    def work(ci: int) -> None:
        ids = chunks[ci]
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tensor, ci)))
        vals = rng.standard_normal(len(ids) * per_block, dtype=np.float32)
        pool[ids] = vals.reshape((len(ids),) + pool.shape[1:]).astype(np.float16)

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if len(chunks) <= 1 or threads <= 1:
        for ci in range(len(chunks)):
            work(ci)
        return
    with _cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, range(len(chunks))))


def _fill_normal_blocks_with_outliers(pool: np.ndarray, block_ids: np.ndarray, live: np.ndarray,
                                      seed: int, tensor: int, frac: float, factor: float) -> int:
    """Like ``_fill_normal_blocks`` but multiplies ``round(frac * N)`` live entries by
    ``factor`` in fp32 before the fp16 rounding. Returns the number of outliers."""
    shape = pool.shape[1:]
    rng0 = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tensor, 0)))
    vals = rng0.standard_normal(len(block_ids) * int(np.prod(shape)), dtype=np.float32)
    vals = vals.reshape((len(block_ids),) + shape)  # [n][H][16][d]
    # live entries: slot live for every head and dim
    slot_live = live[block_ids]  # [n][16]
    entry_live = np.broadcast_to(slot_live[:, None, :, None], vals.shape)
    flat_idx = np.flatnonzero(entry_live.reshape(-1))
    n_out = int(round(frac * flat_idx.size))
    rng1 = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tensor, 1)))
    pick = flat_idx[rng1.choice(flat_idx.size, size=n_out, replace=False)]
    flat = vals.reshape(-1)
    flat[pick] *= np.float32(factor)
    pool[block_ids] = vals.astype(np.float16)
    return n_out


def build(name: str, seed: int, context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
          num_blocks: int | None = None, share_groups: int = 1, shared_blocks: int = 0,
          k_outlier_frac: float = 0.0, k_outlier_factor: float = 10.0,
          shuffle: bool = True, threads: int | None = None) -> Workload:
    """Generic seeded workload.

    ``share_groups`` consecutive sequences form a prefix-sharing group whose
    first ``shared_blocks`` table entries point at the same physical blocks
    (each with one reference per sequence that uses it). ``num_blocks``
    defaults to the exact number of blocks needed.
    """
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    ctx = np.asarray(context_lens, dtype=np.int32)
    nblk = [(int(n) + BLOCK_SIZE - 1) // BLOCK_SIZE for n in ctx]
    S = len(ctx)
    groups = [list(range(i, min(S, i + share_groups))) for i in range(0, S, share_groups)]
    need = 0
    for g in groups:
        sh = min(shared_blocks, max(nblk[s] for s in g)) if shared_blocks else 0
        need += sh + sum(max(0, nblk[s] - min(shared_blocks, nblk[s])) for s in g)
    if num_blocks is None:
        num_blocks = max(need, 1)
    if need > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {need}")

    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(0,)))
    alloc = BlockAllocator(num_blocks, rng, shuffle=shuffle)
    lists: list[list[int]] = [[] for _ in range(S)]
    for g in groups:
        sh = min(shared_blocks, max(nblk[s] for s in g)) if shared_blocks else 0
        prefix = [alloc.allocate() for _ in range(sh)]
        claimed = [False] * sh
        for s in g:
            use = min(sh, nblk[s])
            for i in range(use):
                if claimed[i]:
                    alloc.share(prefix[i])
                claimed[i] = True
                lists[s].append(prefix[i])
            for _ in range(nblk[s] - use):
                lists[s].append(alloc.allocate())
    table = _table_from_lists(lists)
    live = _live_mask(num_blocks, ctx, table)

    qrng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(1,)))
    q = qrng.standard_normal((S, num_q_heads, head_dim), dtype=np.float32).astype(np.float16)

    shape = (num_blocks, num_kv_heads, BLOCK_SIZE, head_dim)
    k_pool = np.zeros(shape, dtype=np.float16)
    v_pool = np.zeros(shape, dtype=np.float16)
    ids = np.flatnonzero(alloc.refcount > 0)
    notes: dict = {}
    if k_outlier_frac > 0:
        notes["k_outliers"] = _fill_normal_blocks_with_outliers(
            k_pool, ids, live, seed, 2, k_outlier_frac, k_outlier_factor)
    else:
        _fill_normal_blocks(k_pool, ids, seed, 2, threads)
    _fill_normal_blocks(v_pool, ids, seed, 3, threads)
    dead = ~live[ids]  # [n][16]
    partial = ids[dead.any(axis=1)]
    for pool in (k_pool, v_pool):
        for b in partial:
            pool[b][:, ~live[b], :] = 0
    return Workload(name=name, seed=seed, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, num_blocks=num_blocks, context_lens=ctx,
                    block_tables=table, q=q, k_pool=k_pool, v_pool=v_pool, live=live,
                    refcount=alloc.refcount.copy(), notes=notes)


def from_contiguous(name: str, q: np.ndarray, k_seqs: list, v_seqs: list, num_blocks: int,
                    seed: int = 0) -> Workload:
    """Scatter per-sequence contiguous K/V (``[ctx][Hkv][d]`` fp16 each) into a
    shuffled pool. Used by tests that compare against dense attention."""
    S = len(k_seqs)
    hkv, d = k_seqs[0].shape[1], k_seqs[0].shape[2]
    ctx = np.array([k.shape[0] for k in k_seqs], dtype=np.int32)
    nblk = [(int(n) + BLOCK_SIZE - 1) // BLOCK_SIZE for n in ctx]
    rng = np.random.default_rng(seed)
    alloc = BlockAllocator(num_blocks, rng)
    lists = [[alloc.allocate() for _ in range(n)] for n in nblk]
    table = _table_from_lists(lists)
    shape = (num_blocks, hkv, BLOCK_SIZE, d)
    k_pool = np.zeros(shape, dtype=np.float16)
    v_pool = np.zeros(shape, dtype=np.float16)
    for s in range(S):
        for t in range(int(ctx[s])):
            b, o = table[s, t // BLOCK_SIZE], t % BLOCK_SIZE
            k_pool[b, :, o, :] = k_seqs[s][t]
            v_pool[b, :, o, :] = v_seqs[s][t]
    live = _live_mask(num_blocks, ctx, table)
    return Workload(name=name, seed=seed, num_q_heads=q.shape[1], num_kv_heads=hkv, head_dim=d,
                    num_blocks=num_blocks, context_lens=ctx, block_tables=table,
                    q=q.astype(np.float16), k_pool=k_pool, v_pool=v_pool, live=live,
                    refcount=alloc.refcount.copy())


# ---------------------------------------------------------------------------
# The five workloads. Seeds are 228 + workload index.

def tiny(seed: int = 228) -> Workload:
    """2 seqs (ctx 37 and 70), H_q 4 / H_kv 2, d 64, pool of 16 shuffled blocks."""
    return build("tiny", seed, [37, 70], 4, 2, 64, num_blocks=16)


def qwen2_layer(num_seqs: int, seed: int = 229) -> Workload:
    """Qwen2-0.5B attention shapes: H_q 14 / H_kv 2, d 64, ctx 512, pool of exactly
    32 blocks per sequence (shuffled)."""
    return build(f"qwen2_s{num_seqs}", seed * 100 + num_seqs, [512] * num_seqs, 14, 2, 64,
                 num_blocks=32 * num_seqs)


def int8_gaussian(seed: int = 230) -> Workload:
    """32 seqs x ctx 1024, 8 heads (MHA), d 128, pool 2048 shuffled, K/V ~ N(0,1)."""
    return build("int8_gaussian", seed, [1024] * 32, 8, 8, 128, num_blocks=2048)


def int8_heavy_tailed(seed: int = 231) -> Workload:
    """64 seqs x ctx 2048, 8 heads, d 128; 0.1 % of K entries multiplied by 10."""
    return build("int8_heavy_tailed", seed, [2048] * 64, 8, 8, 128, num_blocks=8192,
                 k_outlier_frac=1e-3, k_outlier_factor=10.0)


def mixed_prefix(seed: int = 232, num_seqs: int = 64, num_blocks: int = 65536,
                 ctx_lo: int = 512, ctx_hi: int = 16384) -> Workload:
    """Pool of 65,536 blocks, 64 seqs with ctx ~ U[512, 16384], H_q 32 / H_kv 8,
    d 128; groups of 4 sequences share their first 64 physical blocks."""
    crng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(9,)))
    ctx = crng.integers(ctx_lo, ctx_hi + 1, size=num_seqs)
    return build("mixed_prefix", seed, ctx, 32, 8, 128, num_blocks=num_blocks,
                 share_groups=4, shared_blocks=64)


def by_index(idx: int, variant: int | None = None) -> Workload:
    """Workload ``idx`` (0..4) in the order tiny, qwen2, int8 gaussian,
    int8 heavy-tailed, mixed prefix. ``variant`` picks the qwen2 batch (1, 4, 8)."""
    if idx == 0:
        return tiny()
    if idx == 1:
        return qwen2_layer(variant or 8)
    if idx == 2:
        return int8_gaussian()
    if idx == 3:
        return int8_heavy_tailed()
    if idx == 4:
        return mixed_prefix()
    raise ValueError(idx)


@dataclass
class AppendInputs:
    """One decode step's new tokens: token ``positions[s]`` of sequence s, with
    K/V rows ``k_new[s]``/``v_new[s]`` ([H_kv][d] fp16 each), goes to block
    ``block_tables[s][positions[s] // 16]``. ``refcount`` counts the pool's
    references after the step's block allocations."""
    block_tables: np.ndarray  # int32 [S][MB'], MB' >= the workload's MB
    positions: np.ndarray  # int32 [S], -1: the sequence appends nothing
    k_new: np.ndarray  # fp16 [S][H_kv][d]
    v_new: np.ndarray
    refcount: np.ndarray  # int32 [NB]


def append_inputs(w: Workload, seed: int, block_tables=None, context_lens=None, refcount=None,
                  grow_frac: float = 0.0, grow_factor: float = 3.0) -> AppendInputs:
    """Seeded inputs for appending the next token of every sequence.

    The next token of sequence s is token ``context_lens[s]``. When it starts a
    new block, a free pool block (refcount 0, picked at random) is added to the
    sequence's table row, widening the table by a column if needed. A sequence
    whose next slot lies in a block other sequences also read (refcount > 1)
    would need a private copy first; it appends nothing (position -1). New rows
    are N(0, 1) in fp16; a ``grow_frac`` share of the (sequence, KV head) rows
    is multiplied by ``grow_factor`` (for an INT8 cache, rows that raise their
    tile's scale). Pass the previous step's tables, contexts and refcounts to
    chain steps."""
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(17,)))
    tables = np.array(w.block_tables if block_tables is None else block_tables, dtype=np.int32)
    ctx = np.array(w.context_lens if context_lens is None else context_lens, dtype=np.int64)
    ref = np.array(w.refcount if refcount is None else refcount, dtype=np.int32)
    S = tables.shape[0]
    positions = np.full(S, -1, dtype=np.int32)
    for s in range(S):
        t = int(ctx[s])
        j, o = divmod(t, BLOCK_SIZE)
        if j >= tables.shape[1]:
            tables = np.concatenate([tables, np.full((S, 1), -1, np.int32)], axis=1)
        if o == 0:
            free = np.flatnonzero(ref == 0)
            if free.size == 0:
                raise MemoryError("KV block pool exhausted")
            b = int(free[rng.integers(free.size)])
            ref[b] = 1
            tables[s, j] = b
        elif ref[tables[s, j]] > 1:
            continue
        positions[s] = t
    hkv, d = w.num_kv_heads, w.head_dim
    k_new = rng.standard_normal((S, hkv, d), dtype=np.float32)
    v_new = rng.standard_normal((S, hkv, d), dtype=np.float32)
    if grow_frac > 0:
        for x in (k_new, v_new):
            x[rng.random((S, hkv)) < grow_frac] *= np.float32(grow_factor)
    return AppendInputs(block_tables=tables, positions=positions,
                        k_new=k_new.astype(np.float16), v_new=v_new.astype(np.float16),
                        refcount=ref)


def eviction_inputs(num_blocks: int, seed: int, current_tick: int = 10_000,
                    free_frac: float = 0.2, refcount=None):
    """Seeded block metadata for the eviction choice: int32 reference counts
    (``free_frac`` of the blocks free, most of the rest held once, some
    shared by 2-4 sequences; or the given ``refcount``) and int32 ticks of
    last use, uniform over [0, current_tick] for allocated blocks, 0 for free
    ones."""
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(23,)))
    if refcount is None:
        ref = np.where(rng.random(num_blocks) < 0.85, 1, rng.integers(2, 5, size=num_blocks))
        ref[rng.random(num_blocks) < free_frac] = 0
    else:
        ref = np.asarray(refcount)
    ref = ref.astype(np.int32)
    last = rng.integers(0, current_tick + 1, size=num_blocks).astype(np.int32)
    last[ref == 0] = 0
    return ref, last


def algorithmic_bytes(w: Workload, kv_bytes_per_elem: int, with_scales: bool) -> int:
    """Bytes the decode step must move: each distinct live (block, head) slot's
    K and V once, INT8 scales once per distinct (block, head), one int32 per
    logical table entry, fp16 q, fp32 out and the int32 context lengths."""
    live_slots = int(w.live.sum())
    d, hkv = w.head_dim, w.num_kv_heads
    total = live_slots * hkv * d * kv_bytes_per_elem * 2
    if with_scales:
        total += int((w.refcount > 0).sum()) * hkv * 2 * 4
    total += 4 * sum((int(n) + BLOCK_SIZE - 1) // BLOCK_SIZE for n in w.context_lens)
    total += w.num_seqs * w.num_q_heads * d * (2 + 4) + 4 * w.num_seqs
    return total


def logical_kv_tokens(w: Workload) -> int:
    return int(w.context_lens.sum())


__all__ = [
    "BLOCK_SIZE", "BlockAllocator", "Workload", "build", "from_contiguous", "tiny",
    "qwen2_layer", "int8_gaussian", "int8_heavy_tailed", "mixed_prefix", "by_index",
    "algorithmic_bytes", "logical_kv_tokens", "AppendInputs", "append_inputs",
    "eviction_inputs",
]
