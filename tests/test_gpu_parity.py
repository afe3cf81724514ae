"""GPU parity: the HIP path, called through the C-ABI, against the CPU oracle
on the same seeded inputs.

Bars: INT8 codes and scales bit-exact; fp16-path outputs within max-abs 2e-3
of the oracle; INT8-path outputs within max-abs 1e-3 of the oracle's own
dequantized computation. Every workload is compared in full (every output
element), the full-size ones included.
"""

import functools

import numpy as np
import pytest

import oracle
from paged_kv_cache_228_amd import workloads as W

from gpu_util import decode_f16, decode_int8, poison_codes, quantize, say
from test_gpu_fp8 import gpu_decode as decode_fp8

pytestmark = pytest.mark.gpu

TOL_F16 = 2e-3
TOL_I8 = 1e-3


@functools.lru_cache(maxsize=None)
def workload(name: str) -> W.Workload:
    say(f"generating {name}")
    return {
        "tiny": W.tiny,
        "qwen2_s1": lambda: W.qwen2_layer(1),
        "qwen2_s4": lambda: W.qwen2_layer(4),
        "qwen2_s8": lambda: W.qwen2_layer(8),
        "int8_gaussian": W.int8_gaussian,
        "int8_heavy_tailed": W.int8_heavy_tailed,
        "mixed_prefix": W.mixed_prefix,
    }[name]()


@functools.lru_cache(maxsize=None)
def oracle_codes(name: str):
    w = workload(name)
    ids = w.live_block_ids() if name == "mixed_prefix" else None
    kc, ks = oracle.quantize_kv_int8(w.k_pool, ids)
    vc, vs = oracle.quantize_kv_int8(w.v_pool, ids)
    return ids, kc, vc, ks, vs


ALL = ["tiny", "qwen2_s1", "qwen2_s4", "qwen2_s8", "int8_gaussian", "int8_heavy_tailed",
       "mixed_prefix"]


@pytest.mark.parametrize("name", ALL)
def test_quantize_bit_exact(name):
    w = workload(name)
    ids, kc, vc, ks, vs = oracle_codes(name)
    say(f"quantize {name} blocks={w.num_blocks} ids={'all' if ids is None else len(ids)}")
    gkc, gvc, gks, gvs = quantize(w.k_pool, w.v_pool, ids)
    assert np.array_equal(gks.view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(gvs.view(np.uint32), vs.view(np.uint32))
    assert np.array_equal(gkc, kc)
    assert np.array_equal(gvc, vc)


def test_quantize_exhaustive_over_all_finite_fp16():
    """Every finite fp16 value x, quantized in tiles whose amax is one of several
    values (x kept only when |x| <= amax), matches the oracle bit for bit."""
    bits = np.arange(65536, dtype=np.uint16)
    vals = bits.view(np.float16)
    finite = vals[np.isfinite(vals)]
    assert finite.size == 63488
    tiles = []
    for amax in (65504.0, 1000.0, 127.0, 3.140625, 1.0, 0.0999, 6.1e-5, 5.96e-8):
        a = np.float16(amax)
        xs = finite[np.abs(finite.astype(np.float32)) <= np.float32(a)]
        per = 16 * 64 - 1
        for i in range(0, xs.size, per):
            t = np.zeros(16 * 64, np.float16)
            t[0] = a
            chunk = xs[i : i + per]
            t[1 : 1 + chunk.size] = chunk
            tiles.append(t.reshape(16, 64))
    pool = np.stack(tiles)[:, None]  # [n][1][16][64]
    say(f"exhaustive quantize sweep tiles={pool.shape[0]}")
    kc, ks = oracle.quantize_kv_int8(pool)
    gkc, gvc, gks, gvs = quantize(pool, pool[::-1].copy())
    assert np.array_equal(gks.view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(gkc, kc)
    assert np.array_equal(gvc, kc[::-1])


@pytest.mark.parametrize("name", ALL)
def test_decode_f16_matches_oracle(name):
    w = workload(name)
    kp, vp = w.poisoned(w.k_pool), w.poisoned(w.v_pool)
    say(f"decode f16 {name} S={w.num_seqs} ctx_sum={int(w.context_lens.sum())}")
    out = decode_f16(w, kp, vp)
    ref = oracle.decode_workload_f16(w)
    assert np.isfinite(out).all()
    err = float(np.max(np.abs(out - ref)))
    say(f"decode f16 {name} max_abs={err:.3e}")
    assert err <= TOL_F16


@pytest.mark.parametrize("name", ALL)
def test_decode_int8_matches_oracle(name):
    w = workload(name)
    ids, kc, vc, ks, vs = oracle_codes(name)
    kcp, vcp = poison_codes(w, kc), poison_codes(w, vc)
    say(f"decode int8 {name} S={w.num_seqs}")
    out = decode_int8(w, kcp, vcp, ks, vs)
    ref = oracle.decode_workload_int8(w, kc, vc, ks, vs)
    assert np.isfinite(out).all()
    err = float(np.max(np.abs(out - ref)))
    say(f"decode int8 {name} max_abs={err:.3e}")
    assert err <= TOL_I8


def _ragged():
    return W.build("ragged", 501, [1, 15, 16, 17, 100, 513, 2000, 4100, 0, 33], 8, 2, 128,
                   num_blocks=600)


@pytest.mark.parametrize("path", ["f16", "int8"])
def test_partition_size_invariance(path):
    # share lengths of 16..4096 tokens and the automatic one; the short ones
    # give more shares than the batch has tiles
    w = _ragged()
    if path == "int8":
        kc, ks = oracle.quantize_kv_int8(w.k_pool)
        vc, vs = oracle.quantize_kv_int8(w.v_pool)
        ref = oracle.decode_workload_int8(w, kc, vc, ks, vs)
        run = lambda p: decode_int8(w, kc, vc, ks, vs, partition_tokens=p)  # noqa: E731
        tol = TOL_I8
    else:
        ref = oracle.decode_workload_f16(w)
        run = lambda p: decode_f16(w, w.poisoned(w.k_pool), w.poisoned(w.v_pool),  # noqa: E731
                                   partition_tokens=p)
        tol = TOL_F16
    outs = {}
    for p in (16, 48, 64, 256, 512, 4096, 0):
        say(f"partition {path} tokens={p}")
        outs[p] = run(p)
        assert np.max(np.abs(outs[p] - ref)) <= tol
    # split-K invariance: outputs agree within 1e-6 whatever the share length
    # (measured: at most 2.4e-7, reduction order and the rounding of P's hi/lo
    # halves against a different running maximum)
    for p, o in outs.items():
        diff = float(np.max(np.abs(o - outs[4096])))
        say(f"  share length {p}: max |out - out(4096)| = {diff:.3e}")
        assert diff <= 1e-6, p
    assert not outs[0][8].any()  # the empty sequence


@pytest.mark.parametrize("path", ["f16", "int8"])
def test_block_permutation_invariance_is_bitwise(path):
    w = W.build("perm", 502, [70, 333, 16, 1000], 8, 2, 64, num_blocks=120)
    perm = np.random.default_rng(9).permutation(w.num_blocks).astype(np.int32)
    t2 = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    k2, v2 = np.empty_like(w.k_pool), np.empty_like(w.v_pool)
    k2[perm], v2[perm] = w.k_pool, w.v_pool
    say(f"permutation {path}")
    if path == "f16":
        a = decode_f16(w)
        b = decode_f16(w, k2, v2, tables=t2)
    else:
        kc, ks = oracle.quantize_kv_int8(w.k_pool)
        vc, vs = oracle.quantize_kv_int8(w.v_pool)
        kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
        ks2, vs2 = np.empty_like(ks), np.empty_like(vs)
        kc2[perm], vc2[perm], ks2[perm], vs2[perm] = kc, vc, ks, vs
        a = decode_int8(w, kc, vc, ks, vs)
        b = decode_int8(w, kc2, vc2, ks2, vs2, tables=t2)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 3, 4, 5, 6, 7, 8])
def test_every_group_size_and_head_dim(g, d):
    w = W.build(f"g{g}d{d}", 600 + 10 * g + d, [5, 77, 300, 16], 2 * g, 2, d, num_blocks=40)
    say(f"group {g} head_dim {d}")
    out = decode_f16(w, w.poisoned(w.k_pool), w.poisoned(w.v_pool))
    ref = oracle.decode_workload_f16(w)
    assert np.max(np.abs(out - ref)) <= TOL_F16
    kc, ks = oracle.quantize_kv_int8(w.k_pool)
    vc, vs = oracle.quantize_kv_int8(w.v_pool)
    out8 = decode_int8(w, poison_codes(w, kc), poison_codes(w, vc), ks, vs)
    ref8 = oracle.decode_workload_int8(w, kc, vc, ks, vs)
    assert np.max(np.abs(out8 - ref8)) <= TOL_I8


def test_edge_context_lengths():
    """ctx 0 gives zeros; negative counts as 0; lengths past the table are
    clamped to max_blocks_per_seq * 16."""
    w = W.build("edge", 700, [0, 1, 16, 17, 64], 4, 2, 64, num_blocks=12)
    ctx = w.context_lens.copy()
    ctx[0] = -5
    ctx[4] = 10_000  # clamps to 4 blocks = 64 tokens, the real length
    say("edge contexts")
    out = decode_f16(w, ctx=ctx)
    ref = oracle.decode_workload_f16(w)
    assert not out[0].any()
    assert np.max(np.abs(out - ref)) <= TOL_F16
    # ctx 1: exactly the single value row (softmax weight 1)
    b = w.block_tables[1, 0]
    assert np.max(np.abs(out[1] - np.repeat(w.v_pool[b, :, 0].astype(np.float32), 2, 0))) <= 1e-6


def test_out_of_range_block_ids_read_as_zero_tiles():
    w = W.build("oob", 701, [40, 20], 4, 2, 64, num_blocks=6)
    t = w.block_tables.copy()
    t[0, 1] = 6  # == num_blocks: outside the pool
    t[1, 0] = -7
    # oracle: a pool with an extra all-zero block 6, and -7 redirected to it
    kz = np.concatenate([w.k_pool, np.zeros_like(w.k_pool[:1])])
    vz = np.concatenate([w.v_pool, np.zeros_like(w.v_pool[:1])])
    tz = np.where(t < 0, 6, t).astype(np.int32)
    ref = oracle.paged_decode_f16(w.q, kz, vz, tz, w.context_lens, w.softmax_scale)
    say("out-of-range block ids")
    out = decode_f16(w, tables=t)
    assert np.max(np.abs(out - ref)) <= TOL_F16
    kc, ks = oracle.quantize_kv_int8(kz)
    vc, vs = oracle.quantize_kv_int8(vz)
    ref8 = oracle.paged_decode_int8(w.q, kc, vc, ks, vs, tz, w.context_lens, w.softmax_scale)
    out8 = decode_int8(w, kc, vc, ks, vs, tables=t, num_blocks=6)
    assert np.max(np.abs(out8 - ref8)) <= TOL_I8


@pytest.mark.parametrize("name", ["int8_gaussian", "int8_heavy_tailed"])
def test_int8_error_against_fp32_is_reported(name):
    """INT8-versus-fp32 quality on the GPU path (the fp32 reference is the
    oracle on the fp16-stored K/V), reported like the pages' quality table."""
    w = workload(name)
    ids, kc, vc, ks, vs = oracle_codes(name)
    ref = oracle.decode_workload_f16(w).astype(np.float64)
    out = decode_int8(w, kc, vc, ks, vs).astype(np.float64)
    rmse = float(np.sqrt(np.mean((out - ref) ** 2)))
    mx = float(np.max(np.abs(out - ref)))
    say(f"{name}: INT8 vs FP32 rmse={rmse:.5f} max_abs={mx:.4f} fp32_out_std={ref.std():.4f}")
    assert np.isfinite(rmse)
    if name == "int8_gaussian":
        assert rmse < 1e-2


@pytest.mark.parametrize("path", ["f16", "int8"])
@pytest.mark.parametrize("num_seqs", [256, 257, 1500])
def test_many_short_sequences(path, num_seqs):
    # up to 256 sequences every decode wave scans the context lengths itself;
    # from 257 the prep kernel does it once (1500: in several passes of its
    # 1024 threads); a tenth of the contexts empty (zero rows, written by the
    # merge kernel)
    rng = np.random.default_rng(703 + num_seqs)
    ctx = rng.integers(1, 200, size=num_seqs)
    ctx[rng.random(num_seqs) < 0.1] = 0
    w = W.build("many", 703, ctx, 4, 2, 64, num_blocks=int(((ctx + 15) // 16).sum()) + 8)
    say(f"many short sequences {path} S={num_seqs}")
    if path == "f16":
        out = decode_f16(w)
        ref = oracle.decode_workload_f16(w)
        tol = TOL_F16
    else:
        kc, ks = oracle.quantize_kv_int8(w.k_pool)
        vc, vs = oracle.quantize_kv_int8(w.v_pool)
        out = decode_int8(w, kc, vc, ks, vs)
        ref = oracle.decode_workload_int8(w, kc, vc, ks, vs)
        tol = TOL_I8
    assert np.max(np.abs(out - ref)) <= tol
    assert not out[ctx == 0].any()


@pytest.mark.parametrize("path", ["f16", "int8"])
@pytest.mark.parametrize("num_seqs", [8, 257])
def test_every_context_empty(path, num_seqs):
    # no tile at all: the work split is empty (with 257 sequences the prep
    # kernel finds no share a first row), every row is zeros
    ctx = np.zeros(num_seqs, dtype=np.int64)
    w = W.build("empty", 705, ctx, 4, 2, 64, num_blocks=4)
    say(f"every context empty {path} S={num_seqs}")
    if path == "f16":
        out = decode_f16(w)
    else:
        kc, ks = oracle.quantize_kv_int8(w.k_pool)
        vc, vs = oracle.quantize_kv_int8(w.v_pool)
        out = decode_int8(w, kc, vc, ks, vs)
    assert out.shape == (num_seqs, 4, 64) and not out.any()


def test_maximum_sequence_count():
    """The largest batch the calls accept (65,535 sequences; the merge grid's
    second dimension): contexts of 0 to 40 tokens, so most rows are short and
    a tenth are empty, through the prep kernel's path; fp16 and INT8 against
    the oracle element by element."""
    rng = np.random.default_rng(65535)
    ctx = rng.integers(0, 41, size=65535)
    ctx[rng.random(ctx.size) < 0.1] = 0
    w = W.build("max_seqs", 65535, ctx.tolist(), 2, 1, 64)
    say(f"max_seqs: {w.num_seqs} seqs, {int(w.context_lens.sum())} tokens, {w.num_blocks} blocks")
    out = decode_f16(w)
    assert np.max(np.abs(out - oracle.decode_workload_f16(w))) <= 2e-3
    assert not out[w.context_lens <= 0].any()
    kc, ks = oracle.quantize_kv_int8(w.k_pool)
    vc, vs = oracle.quantize_kv_int8(w.v_pool)
    out8 = decode_int8(w, kc, vc, ks, vs)
    assert np.max(np.abs(out8 - oracle.decode_workload_int8(w, kc, vc, ks, vs))) <= 1e-3
    assert not out8[w.context_lens <= 0].any()


def test_very_long_context():
    """One context of 1,048,576 tokens (65,536 blocks, cut into about 2,000
    shares whose partials the merge combines in rounds of 8) beside a short,
    an empty and a mid-length one; fp16 and INT8 against the oracle."""
    w = W.build("long_ctx", 1048576, [1 << 20, 100, 0, 5000], 4, 1, 64)
    say(f"long_ctx: {int(w.context_lens.sum())} tokens, {w.num_blocks} blocks")
    out = decode_f16(w)
    assert np.max(np.abs(out - oracle.decode_workload_f16(w))) <= 2e-3
    kc, ks = oracle.quantize_kv_int8(w.k_pool)
    vc, vs = oracle.quantize_kv_int8(w.v_pool)
    out8 = decode_int8(w, kc, vc, ks, vs)
    assert np.max(np.abs(out8 - oracle.decode_workload_int8(w, kc, vc, ks, vs))) <= 1e-3
    assert not out[2].any() and not out8[2].any()


@pytest.mark.parametrize("hkv,g,d", [(3, 5, 128), (64, 2, 64), (48, 1, 128)])
def test_kv_head_counts_beyond_eight(hkv, g, d):
    """KV head counts that are not a power of two or exceed the eight compute
    dies (the grid's heads-fastest order wraps over the dies unevenly), fp16,
    INT8 and FP8 against the oracle."""
    rng = np.random.default_rng(700 + hkv)
    ctx = rng.integers(0, 400, size=12)
    w = W.build(f"heads{hkv}", 700 + hkv, ctx.tolist(), g * hkv, hkv, d)
    say(f"heads: Hkv={hkv} G={g} d={d}")
    assert np.max(np.abs(decode_f16(w) - oracle.decode_workload_f16(w))) <= 2e-3
    kc, ks = oracle.quantize_kv_int8(w.k_pool)
    vc, vs = oracle.quantize_kv_int8(w.v_pool)
    assert np.max(np.abs(decode_int8(w, kc, vc, ks, vs) - oracle.decode_workload_int8(w, kc, vc, ks, vs))) <= 1e-3
    fk, fks = oracle.quantize_kv_fp8(w.k_pool)
    fv, fvs = oracle.quantize_kv_fp8(w.v_pool)
    ref = oracle.paged_decode_fp8(w.q, fk, fv, fks, fvs, w.block_tables, w.context_lens, w.softmax_scale)
    assert np.max(np.abs(decode_fp8(w, fk, fv, fks, fvs) - ref)) <= 1e-3


@pytest.mark.parametrize("scale", [8.0, 1e-3, -0.2])
def test_softmax_scale_extremes(scale):
    """A sharp softmax (scale 8: nearly one-hot, the lazy reference max moves
    often), a flat one (1e-3) and a negative scale, fp16, INT8 and FP8 against
    the oracle."""
    rng = np.random.default_rng(808)
    w = W.build("scales", 808, rng.integers(1, 900, size=24).tolist(), 16, 4, 128)
    say(f"softmax scale {scale}")
    ref = oracle.paged_decode_f16(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, scale)
    assert np.max(np.abs(decode_f16(w, scale=scale) - ref)) <= 2e-3
    kc, ks = oracle.quantize_kv_int8(w.k_pool)
    vc, vs = oracle.quantize_kv_int8(w.v_pool)
    ref8 = oracle.paged_decode_int8(w.q, kc, vc, ks, vs, w.block_tables, w.context_lens, scale)
    assert np.max(np.abs(decode_int8(w, kc, vc, ks, vs, scale=scale) - ref8)) <= 1e-3
    fk, fks = oracle.quantize_kv_fp8(w.k_pool)
    fv, fvs = oracle.quantize_kv_fp8(w.v_pool)
    reff = oracle.paged_decode_fp8(w.q, fk, fv, fks, fvs, w.block_tables, w.context_lens, scale)
    assert np.max(np.abs(decode_fp8(w, fk, fv, fks, fvs, scale=scale) - reff)) <= 1e-3


def _mixed_d64():
    """The mixed batch's lengths and prefix sharing at head dim 64 on a
    smaller pool: 16 sequences of 512 to 4,096 tokens, groups of 4 sharing
    their first 64 blocks."""
    crng = np.random.default_rng(np.random.SeedSequence(233, spawn_key=(9,)))
    ctx = crng.integers(512, 4097, size=16)
    return W.build("mixed_d64", 233, ctx, 32, 8, 64, num_blocks=8192, share_groups=4, shared_blocks=64)


def test_mixed_d64_matches_oracle():
    """The mixed batch's shape at head dim 64 (two waves per SIMD, shared
    prefixes read with their own cache policy): every output element of the
    fp16, INT8 and FP8 decodes against the oracle at the parity bars."""
    w = _mixed_d64()
    say(f"mixed_d64: {w.num_seqs} seqs, {int(w.context_lens.sum())} tokens")
    assert np.max(np.abs(decode_f16(w) - oracle.decode_workload_f16(w))) <= 2e-3
    kc, ks = oracle.quantize_kv_int8(w.k_pool)
    vc, vs = oracle.quantize_kv_int8(w.v_pool)
    assert np.max(np.abs(decode_int8(w, kc, vc, ks, vs) - oracle.decode_workload_int8(w, kc, vc, ks, vs))) <= 1e-3
    fk, fks = oracle.quantize_kv_fp8(w.k_pool)
    fv, fvs = oracle.quantize_kv_fp8(w.v_pool)
    ref = oracle.paged_decode_fp8(w.q, fk, fv, fks, fvs, w.block_tables, w.context_lens, w.softmax_scale)
    assert np.max(np.abs(decode_fp8(w, fk, fv, fks, fvs) - ref)) <= 1e-3


@pytest.mark.parametrize("name", ["mixed_prefix", "mixed_d64"])
def test_cache_policy_of_shared_blocks_never_changes_the_arithmetic(name):
    """The decodes (fp16, INT8, FP8) read blocks that a neighbouring row's
    table also names with another cache policy. Filling every row's table past its
    last block with its neighbours' ids (entries the decode never reads as
    tiles) makes the comparison find shared runs where there were none; the
    outputs must stay bit-identical, as must a shared prefix turned private."""
    if name == "mixed_prefix":
        w = workload(name)
        _, kc, vc, ks, vs = oracle_codes(name)
    else:
        w = _mixed_d64()
        kc, ks = oracle.quantize_kv_int8(w.k_pool)
        vc, vs = oracle.quantize_kv_int8(w.v_pool)
    fk, fks = oracle.quantize_kv_fp8(w.k_pool)
    fv, fvs = oracle.quantize_kv_fp8(w.v_pool)

    def all_three(k, v, kc_, vc_, ks_, vs_, fk_, fv_, fks_, fvs_, tables):
        return (decode_f16(w, k_pool=k, v_pool=v, tables=tables),
                decode_int8(w, kc_, vc_, ks_, vs_, tables=tables),
                decode_fp8(w, fk_, fv_, fks_, fvs_, tables=tables))

    def same(outs, base):
        return all(np.array_equal(o.view(np.uint32), b.view(np.uint32)) for o, b in zip(outs, base))

    base = all_three(w.k_pool, w.v_pool, kc, vc, ks, vs, fk, fv, fks, fvs, w.block_tables)
    t = w.block_tables.copy()
    nb = (w.context_lens + 15) // 16
    for s in range(w.num_seqs):
        src = t[s + 1] if s + 1 < w.num_seqs else t[s - 1]
        t[s, nb[s]:] = src[nb[s]:]
    say(f"shared-block policy ({name}): tables filled with the neighbours' ids")
    assert same(all_three(w.k_pool, w.v_pool, kc, vc, ks, vs, fk, fv, fks, fvs, t), base)
    # the second row of every sharing group reads its prefix from private
    # copies of the same blocks: no shared run left for it
    pools = [a.copy() for a in (w.k_pool, w.v_pool, kc, vc, ks, vs, fk, fv, fks, fvs)]
    t2 = w.block_tables.copy()
    free = np.setdiff1d(np.arange(w.num_blocks), w.block_tables[w.block_tables >= 0])
    used = 0
    for s in range(1, w.num_seqs, 4):
        for j in range(min(64, int(nb[s]))):
            b, f = t2[s, j], free[used]
            used += 1
            for a in pools:
                a[f] = a[b]
            t2[s, j] = f
    say(f"shared-block policy ({name}): {used} prefix blocks made private")
    assert same(all_three(*pools, t2), base)
