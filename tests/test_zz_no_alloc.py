"""pa_paged_decode_int8_noalloc: the INT8 decode with the library's static
per-GPU workspace instead of a caller's. Its outputs must equal those of
pa_paged_decode_int8 (the same kernels) bit for bit, on consecutive calls
whose second is smaller than the first (the static array keeps the first
call's contents), and stay within the INT8 tolerance of the oracle."""

import ctypes as C

import numpy as np
import pytest

import paged_kv_cache_228_amd as pa
from paged_kv_cache_228_amd import workloads as W

FAKE = 0x10000  # aligned, never dereferenced: the call fails validation first


def noalloc(S=2, hq=4, hkv=2, d=64, mb=5, nb=16, part=0, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, t=FAKE, c=FAKE, o=FAKE, scale=0.125)
    a.update(over)
    return pa.lib().pa_paged_decode_int8_noalloc(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["t"],
                                                 a["c"], a["o"], S, hq, hkv, d, 16, mb, nb,
                                                 a["scale"], part, None)


def test_noalloc_rejects_on_the_host():
    # a shape whose workspace exceeds the static array: refused before any HIP call
    need = pa.pa_decode_workspace_bytes(64, 32, 8, 128, 1024, 16, 16, pa.KV_INT8)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    assert noalloc(S=64, hq=32, hkv=8, d=128, mb=1024, nb=65536, part=16) == pa.PA_ERR_WORKSPACE
    assert noalloc(q=None) == pa.PA_ERR_NULL
    assert noalloc(vs=None) == pa.PA_ERR_NULL
    assert noalloc(hq=3) == pa.PA_ERR_SHAPE
    assert noalloc(d=96) == pa.PA_ERR_UNSUPPORTED
    assert noalloc(scale=float("inf")) == pa.PA_ERR_SHAPE
    assert noalloc(q=FAKE + 8) == pa.PA_ERR_UNSUPPORTED
    assert noalloc(S=0) == pa.PA_OK  # nothing to do, nothing launched


def test_largest_workload_fits_the_static_array():
    # the mixed batch's shape (64 sequences, 32/8 heads, d 128, 1,024-block rows)
    # at the automatic share count on a 256-CU device
    need = pa.pa_decode_workspace_bytes(64, 32, 8, 128, 1024, 16, 0, pa.KV_INT8)
    assert 0 < need <= pa.NOALLOC_SCRATCH_BYTES


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_call_on_consecutive_calls(oracle_lib):
    import torch

    import gpu_util as G

    oracle = oracle_lib
    # the second call is smaller than the first; the static array still holds
    # the first call's prefix sums and partials when it runs
    for name, w in (("int8_heavy_tailed", W.int8_heavy_tailed()),
                    ("qwen2_s4", W.qwen2_layer(4)),
                    ("tiny", W.tiny())):
        G.say(f"noalloc vs workspace decode: {name} S={w.num_seqs} Hq={w.num_q_heads} "
              f"Hkv={w.num_kv_heads} d={w.head_dim}")
        live = w.live_block_ids()
        kc, ks = oracle.quantize_kv_int8(w.k_pool, live)
        vc, vs = oracle.quantize_kv_int8(w.v_pool, live)
        dq, dt, dc = G.dev(w.q), G.dev(w.block_tables), G.dev(w.context_lens)
        dkc, dvc, dks, dvs = G.dev(kc), G.dev(vc), G.dev(ks), G.dev(vs)
        ref = torch.full(dq.shape, float("nan"), dtype=torch.float32, device=G.DEV)
        got = torch.full(dq.shape, float("nan"), dtype=torch.float32, device=G.DEV)
        pa.pa_paged_decode_int8(dq, dkc, dvc, dks, dvs, dt, dc, ref, w.softmax_scale)
        pa.pa_paged_decode_int8_noalloc(dq, dkc, dvc, dks, dvs, dt, dc, got, w.softmax_scale)
        G.sync()
        r, g = ref.cpu().numpy(), got.cpu().numpy()
        assert np.array_equal(r.view(np.uint32), g.view(np.uint32)), name
        want = oracle.paged_decode_int8(w.q, kc, vc, ks, vs, w.block_tables, w.context_lens,
                                        w.softmax_scale)
        err = float(np.max(np.abs(g - want)))
        G.say(f"  bit-identical; max|noalloc - oracle| = {err:.2e}")
        assert err <= 1e-3, name
