"""GPU parity of the FP8 (OCP E4M3) path against the oracle.

Bars as for INT8: codes and scales bit-exact (every workload, plus every
finite fp16 value in tiles of several scales); decode outputs within max-abs
1e-3 of the oracle's computation on the same codes, every output element,
the 65,536-block mixed batch included, with every dead slot holding a random
byte (E4M3 NaN codes included) to prove the masking.
"""

import functools

import numpy as np
import pytest

import oracle
import paged_kv_cache_228_amd as pa
from paged_kv_cache_228_amd import workloads as W

from gpu_util import dev, say, sync

pytestmark = pytest.mark.gpu

TOL = 1e-3


@functools.lru_cache(maxsize=None)
def workload(name: str) -> W.Workload:
    say(f"generating {name}")
    return {
        "tiny": W.tiny,
        "qwen2_s4": lambda: W.qwen2_layer(4),
        "int8_gaussian": W.int8_gaussian,
        "int8_heavy_tailed": W.int8_heavy_tailed,
        "mixed_prefix": W.mixed_prefix,
    }[name]()


@functools.lru_cache(maxsize=None)
def oracle_codes(name: str):
    w = workload(name)
    ids = w.live_block_ids() if name == "mixed_prefix" else None
    kc, ks = oracle.quantize_kv_fp8(w.k_pool, ids)
    vc, vs = oracle.quantize_kv_fp8(w.v_pool, ids)
    return ids, kc, vc, ks, vs


def gpu_quantize(k_pool, v_pool, block_ids=None):
    import torch

    k, v = dev(k_pool), dev(v_pool)
    kc = torch.zeros(k.shape, dtype=torch.uint8, device=k.device)
    vc = torch.zeros(v.shape, dtype=torch.uint8, device=v.device)
    ks = torch.zeros(k.shape[:2], dtype=torch.float32, device=k.device)
    vs = torch.zeros(v.shape[:2], dtype=torch.float32, device=v.device)
    ids = None if block_ids is None else dev(np.asarray(block_ids, np.int32))
    pa.pa_quantize_kv_fp8(k, v, kc, vc, ks, vs, ids)
    sync()
    return kc.cpu().numpy(), vc.cpu().numpy(), ks.cpu().numpy(), vs.cpu().numpy()


def gpu_decode(w, kc, vc, ks, vs, partition_tokens=0, tables=None, scale=None):
    import torch

    q = dev(w.q)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
    pa.pa_paged_decode_fp8(q, dev(kc), dev(vc), dev(ks), dev(vs), dev(w.block_tables if tables is None else tables),
                           dev(w.context_lens), out, w.softmax_scale if scale is None else scale,
                           partition_tokens)
    sync()
    return out.cpu().numpy()


def poison(w, codes, seed):
    out = codes.copy()
    view = out.transpose(0, 2, 1, 3)
    dead = w.dead_slot_mask()
    rng = np.random.default_rng(seed)
    view[dead] = rng.integers(0, 256, size=view[dead].shape, dtype=np.uint8)
    return out


ALL = ["tiny", "qwen2_s4", "int8_gaussian", "int8_heavy_tailed", "mixed_prefix"]


@pytest.mark.parametrize("name", ALL)
def test_fp8_quantize_bit_exact(name):
    w = workload(name)
    ids, kc, vc, ks, vs = oracle_codes(name)
    say(f"fp8 quantize {name}")
    gkc, gvc, gks, gvs = gpu_quantize(w.k_pool, w.v_pool, ids)
    assert np.array_equal(gks.view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(gvs.view(np.uint32), vs.view(np.uint32))
    assert np.array_equal(gkc, kc) and np.array_equal(gvc, vc)


def test_fp8_quantize_exhaustive_over_all_finite_fp16():
    bits = np.arange(65536, dtype=np.uint16)
    vals = bits.view(np.float16)
    finite = vals[np.isfinite(vals)]
    tiles = []
    for amax in (65504.0, 1000.0, 448.0, 3.140625, 1.0, 0.0999, 6.1e-5, 5.96e-8):
        a = np.float16(amax)
        xs = finite[np.abs(finite.astype(np.float32)) <= np.float32(a)]
        per = 16 * 64 - 1
        for i in range(0, xs.size, per):
            t = np.zeros(16 * 64, np.float16)
            t[0] = a
            chunk = xs[i : i + per]
            t[1 : 1 + chunk.size] = chunk
            tiles.append(t.reshape(16, 64))
    pool = np.stack(tiles)[:, None]
    say(f"fp8 exhaustive sweep tiles={pool.shape[0]}")
    kc, ks = oracle.quantize_kv_fp8(pool)
    gkc, gvc, gks, gvs = gpu_quantize(pool, pool[::-1].copy())
    assert np.array_equal(gks.view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(gkc, kc)
    assert np.array_equal(gvc, kc[::-1])


@pytest.mark.parametrize("name", ALL)
def test_fp8_decode_matches_oracle(name):
    w = workload(name)
    ids, kc, vc, ks, vs = oracle_codes(name)
    say(f"fp8 decode {name} S={w.num_seqs}")
    out = gpu_decode(w, poison(w, kc, 1), poison(w, vc, 2), ks, vs)
    ref = oracle.paged_decode_fp8(w.q, kc, vc, ks, vs, w.block_tables, w.context_lens,
                                  w.softmax_scale)
    assert np.isfinite(out).all()
    err = float(np.max(np.abs(out - ref)))
    say(f"fp8 decode {name} max_abs={err:.3e}")
    assert err <= TOL


def test_fp8_share_count_invariance_and_group_sizes():
    w = W.build("ragged8", 801, [1, 15, 16, 17, 100, 513, 2000, 0, 33], 8, 2, 128, num_blocks=400)
    kc, ks = oracle.quantize_kv_fp8(w.k_pool)
    vc, vs = oracle.quantize_kv_fp8(w.v_pool)
    ref = oracle.paged_decode_fp8(w.q, kc, vc, ks, vs, w.block_tables, w.context_lens,
                                  w.softmax_scale)
    for p in (16, 64, 512, 4096, 0):
        say(f"fp8 partition tokens={p}")
        assert np.max(np.abs(gpu_decode(w, kc, vc, ks, vs, p) - ref)) <= TOL
    for g in (1, 3, 8):
        for d in (64, 128):
            w2 = W.build(f"f8g{g}d{d}", 810 + g + d, [5, 77, 300], 2 * g, 2, d, num_blocks=30)
            kc2, ks2 = oracle.quantize_kv_fp8(w2.k_pool)
            vc2, vs2 = oracle.quantize_kv_fp8(w2.v_pool)
            r2 = oracle.paged_decode_fp8(w2.q, kc2, vc2, ks2, vs2, w2.block_tables,
                                         w2.context_lens, w2.softmax_scale)
            say(f"fp8 group {g} head_dim {d}")
            o2 = gpu_decode(w2, poison(w2, kc2, 3), poison(w2, vc2, 4), ks2, vs2)
            assert np.max(np.abs(o2 - r2)) <= TOL
