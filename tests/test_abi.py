"""The C-ABI library loads, exports every call include/pa.h declares, and
rejects bad arguments on the host before launching anything (no GPU needed:
none of these calls reaches a kernel launch)."""

import ctypes as C
import os
import re

import pytest

import paged_kv_cache_228_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_\w+)\s*\(", text)))


def test_library_exports_every_declared_call():
    names = declared_functions()
    assert set(names) == set(pa.EXPORTED)
    L = C.CDLL(pa.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_error_strings():
    for code in (0, -1, -2, -3, -4, -5, -99):
        assert pa.pa_error_string(code)


def decode_f16(**over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, t=FAKE, c=FAKE, o=FAKE, S=2, hq=4, hkv=2, d=64, bs=16,
                mb=5, nb=16, scale=0.125, part=0, ws=None, wsb=0, stream=None)
    args.update(over)
    a = args
    return pa.lib().pa_paged_decode_f16(a["q"], a["k"], a["v"], a["t"], a["c"], a["o"], a["S"],
                                        a["hq"], a["hkv"], a["d"], a["bs"], a["mb"], a["nb"],
                                        a["scale"], a["part"], a["ws"], a["wsb"], a["stream"])


def decode_i8(**over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, t=FAKE, c=FAKE, o=FAKE, S=2, hq=4,
                hkv=2, d=64, bs=16, mb=5, nb=16, scale=0.125, part=0, ws=None, wsb=0)
    args.update(over)
    a = args
    return pa.lib().pa_paged_decode_int8(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["t"], a["c"],
                                         a["o"], a["S"], a["hq"], a["hkv"], a["d"], a["bs"],
                                         a["mb"], a["nb"], a["scale"], a["part"], a["ws"],
                                         a["wsb"], None)


@pytest.mark.parametrize(
    "over,code",
    [
        (dict(q=None), pa.PA_ERR_NULL),
        (dict(t=None), pa.PA_ERR_NULL),
        (dict(o=None), pa.PA_ERR_NULL),
        (dict(hq=5), pa.PA_ERR_SHAPE),
        (dict(hq=0), pa.PA_ERR_SHAPE),
        (dict(S=-1), pa.PA_ERR_SHAPE),
        (dict(mb=0), pa.PA_ERR_SHAPE),
        (dict(nb=0), pa.PA_ERR_SHAPE),
        (dict(part=24), pa.PA_ERR_SHAPE),
        (dict(part=-16), pa.PA_ERR_SHAPE),
        (dict(scale=float("nan")), pa.PA_ERR_SHAPE),
        (dict(bs=8), pa.PA_ERR_UNSUPPORTED),
        (dict(d=96), pa.PA_ERR_UNSUPPORTED),
        (dict(hq=32, hkv=2), pa.PA_ERR_UNSUPPORTED),
        (dict(q=FAKE + 8), pa.PA_ERR_UNSUPPORTED),
        (dict(mb=64, part=16), pa.PA_ERR_WORKSPACE),
        (dict(mb=64, part=16, ws=FAKE, wsb=100), pa.PA_ERR_WORKSPACE),
        (dict(), pa.PA_ERR_WORKSPACE),
        (dict(ws=FAKE + 8, wsb=1 << 20), pa.PA_ERR_UNSUPPORTED),
        (dict(S=0), pa.PA_OK),
    ],
)
def test_decode_f16_rejects_bad_arguments_on_host(over, code):
    assert decode_f16(**over) == code


@pytest.mark.parametrize(
    "over,code",
    [
        (dict(ks=None), pa.PA_ERR_NULL),
        (dict(vs=None), pa.PA_ERR_NULL),
        (dict(d=32), pa.PA_ERR_UNSUPPORTED),
        (dict(mb=64, part=32), pa.PA_ERR_WORKSPACE),
        (dict(S=0), pa.PA_OK),
    ],
)
def test_decode_int8_rejects_bad_arguments_on_host(over, code):
    assert decode_i8(**over) == code


def test_quantize_rejects_bad_arguments_on_host():
    q = pa.lib().pa_quantize_kv_int8
    assert q(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 2, 16, 64, None) == pa.PA_ERR_NULL
    assert q(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 0, 2, 16, 64, None) == pa.PA_ERR_SHAPE
    assert q(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 2, 8, 64, None) == pa.PA_ERR_UNSUPPORTED
    assert q(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 2, 16, 80, None) == pa.PA_ERR_UNSUPPORTED
    assert q(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1, 4, 2, 16, 64, None) == pa.PA_ERR_SHAPE
    # an empty block list is valid and launches nothing
    assert q(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4, 2, 16, 64, None) == pa.PA_OK


def append_call(int8, **over):
    args = dict(kn=FAKE, vn=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, t=FAKE, p=FAKE, S=2, hkv=2,
                d=64, bs=16, mb=5, nb=16)
    args.update(over)
    a = args
    tail = (a["t"], a["p"], a["S"], a["hkv"], a["d"], a["bs"], a["mb"], a["nb"], None)
    if int8:
        return pa.lib().pa_append_kv_int8(a["kn"], a["vn"], a["k"], a["v"], a["ks"], a["vs"], *tail)
    return pa.lib().pa_append_kv_f16(a["kn"], a["vn"], a["k"], a["v"], *tail)


@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize(
    "over,code",
    [
        (dict(kn=None), pa.PA_ERR_NULL),
        (dict(v=None), pa.PA_ERR_NULL),
        (dict(t=None), pa.PA_ERR_NULL),
        (dict(p=None), pa.PA_ERR_NULL),
        (dict(S=-1), pa.PA_ERR_SHAPE),
        (dict(hkv=0), pa.PA_ERR_SHAPE),
        (dict(mb=0), pa.PA_ERR_SHAPE),
        (dict(nb=0), pa.PA_ERR_SHAPE),
        (dict(bs=8), pa.PA_ERR_UNSUPPORTED),
        (dict(d=96), pa.PA_ERR_UNSUPPORTED),
        (dict(S=70000), pa.PA_ERR_UNSUPPORTED),
        (dict(k=FAKE + 4), pa.PA_ERR_UNSUPPORTED),
        (dict(vn=FAKE + 2), pa.PA_ERR_UNSUPPORTED),
        (dict(S=0), pa.PA_OK),  # nothing to append, nothing launched
    ],
)
def test_append_rejects_bad_arguments_on_host(int8, over, code):
    assert append_call(int8, **over) == code


def test_int8_append_needs_scales():
    assert append_call(True, ks=None) == pa.PA_ERR_NULL
    assert append_call(False, ks=None, vs=None, S=0) == pa.PA_OK


@pytest.mark.parametrize(
    "args,code",
    [
        ((None, FAKE, 16, 5, 3, FAKE), pa.PA_ERR_NULL),
        ((FAKE, None, 16, 5, 3, FAKE), pa.PA_ERR_NULL),
        ((FAKE, FAKE, 16, 5, 3, None), pa.PA_ERR_NULL),
        ((FAKE, FAKE, 0, 5, 3, FAKE), pa.PA_ERR_SHAPE),
        ((FAKE, FAKE, 16, 5, -1, FAKE), pa.PA_ERR_SHAPE),
        ((FAKE, FAKE, 2**31, 5, 3, FAKE), pa.PA_ERR_UNSUPPORTED),
        ((FAKE + 2, FAKE, 16, 5, 3, FAKE), pa.PA_ERR_UNSUPPORTED),
        ((FAKE, FAKE + 4, 16, 5, 3, FAKE), pa.PA_ERR_UNSUPPORTED),
        ((FAKE, FAKE, 16, 5, 0, None), pa.PA_OK),  # k == 0: nothing launched
    ],
)
def test_evict_rejects_bad_arguments_on_host(args, code):
    assert pa.lib().pa_evict_select(*args, None) == code


def test_workspace_and_share_sizing():
    # Without a device to ask, the library sizes for 256 compute units.
    # A tiny batch: at most one share per 8 blocks of the 2 x 5-block bound.
    assert pa.pa_decode_shares(2, 2, 64, 5) == 10  # a tiny bound: one block per share
    # int32 tile and cost prefix sums [S + 1] each, share first rows [K],
    # padded to 256 B; then the partials: K x 2 slots x Hq x (D + 2) floats
    def ints(S, K, hkv):
        return ((2 * (S + 1) + K) * 4 + 255) // 256 * 256

    assert pa.pa_decode_workspace_bytes(2, 4, 2, 64, 5) == ints(2, 10, 2) + 10 * 2 * 4 * 66 * 4
    # the mixed batch's shape: one share per wave, one wave per SIMD (256 CUs x
    # 4 SIMDs) over 8 KV heads, whatever the cache format
    for fmt in (pa.KV_F16, pa.KV_INT8, pa.KV_FP8):
        assert pa.pa_decode_shares(64, 8, 128, 1024, kv_format=fmt) == 128
        assert (pa.pa_decode_workspace_bytes(64, 32, 8, 128, 1024, kv_format=fmt)
                == ints(64, 128, 8) + 128 * 2 * 32 * 130 * 4)
    # head dim 64: two waves per SIMD, twice the shares
    for fmt in (pa.KV_F16, pa.KV_INT8, pa.KV_FP8):
        assert pa.pa_decode_shares(64, 8, 64, 1024, kv_format=fmt) == 256
    # explicit share length: 1 x 1024 blocks x 16 tokens / 256 tokens
    assert pa.pa_decode_shares(1, 1, 64, 1024, 16, 256) == 64
    # never more shares than blocks in the bound
    assert pa.pa_decode_shares(1, 1, 64, 8, 16, 16) == 8
    # rejected shapes size nothing
    assert pa.pa_decode_workspace_bytes(1, 3, 2, 64, 8) == 0
    with pytest.raises(pa.PagedAttentionError):
        pa.pa_decode_shares(1, 1, 64, 8, 16, 20)
    with pytest.raises(pa.PagedAttentionError):
        pa.pa_decode_shares(1, 1, 96, 8)


def test_partition_tokens_counts_tokens_per_share_of_the_whole_batch():
    # A share is a run of one KV head's tiles across sequences, so
    # partition_tokens is tokens per share of the longest possible batch
    # (num_seqs x max_blocks_per_seq x 16 tokens), not of one sequence.
    for S, hkv, d, mb in ((2, 2, 64, 5), (64, 8, 128, 1024), (32, 8, 128, 64)):
        whole = S * mb * 16
        for fmt in (pa.KV_F16, pa.KV_INT8, pa.KV_FP8):
            # covering the whole batch: one share per KV head, no row is cut
            assert pa.pa_decode_shares(S, hkv, d, mb, 16, whole, fmt) == 1
            assert pa.pa_decode_shares(S, hkv, d, mb, 16, 4 * whole, fmt) == 1
            # the longest possible context: still one share per sequence's worth
            assert pa.pa_decode_shares(S, hkv, d, mb, 16, mb * 16, fmt) == S
            # the workspace follows the share count: ints + K x 2 x Hq x (d + 2) floats
            hq = 4 * hkv
            one = pa.pa_decode_workspace_bytes(S, hq, hkv, d, mb, 16, whole, fmt)
            ints = ((2 * (S + 1) + 1) * 4 + 255) // 256 * 256
            assert one == ints + 1 * 2 * hq * (d + 2) * 4
    # the sizing helpers take num_kv_heads: the automatic count spreads one wave
    # per SIMD (256 CUs x 4 without a device) over the KV heads
    assert pa.pa_decode_shares(64, 8, 128, 1024) == 128
    assert pa.pa_decode_shares(64, 4, 128, 1024) == 256


def test_bench_traffic_is_reported_only_for_unchanged_sources(tmp_path, monkeypatch):
    import hashlib
    import json

    import bench

    (tmp_path / "profiles").mkdir()
    src = tmp_path / "k.hip"
    src.write_text('int v = 1; // the kernel\nasm("s_nop 0  // x");\n')
    code = 'int v = 1; asm("s_nop 0  // x");'
    rec = {"calls": {"pa_paged_decode_f16": {
        "fetch_bytes": 1000, "write_bytes": 24,
        "sources": {"k.hip": hashlib.sha256(code.encode()).hexdigest()}}}}
    (tmp_path / "profiles" / "hbm_traffic_wl.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("pa_paged_decode_f16", "wl") == 1024
    assert bench.measured_traffic("pa_paged_decode_int8", "wl") is None
    assert bench.measured_traffic("pa_paged_decode_f16", "other") is None
    # comments and layout may change; code, string literals included, may not
    src.write_text('/* v1 */ int v = 1;\n\n  asm("s_nop 0  // x"); // done\n')
    assert bench.measured_traffic("pa_paged_decode_f16", "wl") == 1024
    src.write_text('int v = 1; asm("s_nop 0 // x");\n')
    assert bench.measured_traffic("pa_paged_decode_f16", "wl") is None
    src.write_text('int v = 2; // the kernel\nasm("s_nop 0  // x");\n')
    assert bench.measured_traffic("pa_paged_decode_f16", "wl") is None


@pytest.mark.parametrize(
    "args, code",
    [
        ((None, 1024, FAKE, 4), pa.PA_ERR_NULL),
        ((FAKE, 1024, None, 4), pa.PA_ERR_NULL),
        ((FAKE, 0, FAKE, 4), pa.PA_ERR_SHAPE),
        ((FAKE, 1024, FAKE, 0), pa.PA_ERR_SHAPE),
        ((FAKE, 1000, FAKE, 4), pa.PA_ERR_UNSUPPORTED),  # not a multiple of 16 bytes
        ((FAKE + 8, 1024, FAKE, 4), pa.PA_ERR_UNSUPPORTED),  # not 16-byte aligned
    ],
)
def test_read_probe_rejects_bad_arguments_on_host(args, code):
    assert pa.lib().pa_hbm_read_probe(*args, None) == code


@pytest.mark.parametrize(
    "args, code",
    [
        ((None, 1024, FAKE, 4), pa.PA_ERR_NULL),
        ((FAKE, 1024, None, 4), pa.PA_ERR_NULL),
        ((FAKE, 0, FAKE, 4), pa.PA_ERR_SHAPE),
        ((FAKE, 1024, FAKE, 0), pa.PA_ERR_SHAPE),
        ((FAKE, 1000, FAKE, 4), pa.PA_ERR_UNSUPPORTED),
        ((FAKE + 8, 1024, FAKE, 4), pa.PA_ERR_UNSUPPORTED),
        ((FAKE, 1024, FAKE + 4, 4), pa.PA_ERR_UNSUPPORTED),
    ],
)
def test_rw_probe_rejects_bad_arguments_on_host(args, code):
    assert pa.lib().pa_hbm_rw_probe(*args, None) == code
