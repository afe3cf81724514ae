"""The HBM read-bandwidth probe reads every byte once: the XOR of what its
workgroups report equals the XOR of all 32-bit words of the buffer, and one
workgroup reports exactly that XOR (a ragged last chunk included)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_228_amd as pa
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes, groups", [(16, 1), (32768 + 48, 1), (1 << 20, 7), ((1 << 24) + 4096, 1024)])
def test_read_probe_folds_every_word(nbytes, groups):
    say(f"read probe {nbytes} B, {groups} workgroups")
    rng = np.random.default_rng(nbytes + groups)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    sink = torch.full((groups,), -1, dtype=torch.int32, device=DEV)
    pa.pa_hbm_read_probe(src, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(host)
    assert np.bitwise_xor.reduce(got) == want
    if groups == 1:
        assert got[0] == want


@pytest.mark.parametrize("nbytes, groups", [(16, 1), (32768 + 48, 3), ((1 << 22) + 4096, 1024)])
def test_rw_probe_writes_every_word(nbytes, groups):
    say(f"read-write probe {nbytes} B, {groups} workgroups")
    rng = np.random.default_rng(nbytes * 7 + groups)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    dst = torch.full((nbytes // 8,), -1, dtype=torch.int32, device=DEV)
    pa.pa_hbm_rw_probe(src, dst, groups)
    torch.cuda.synchronize()
    w = host.reshape(-1, 4)
    want = np.stack([w[:, 0] ^ w[:, 2], w[:, 1] ^ w[:, 3]], 1).reshape(-1)
    assert np.array_equal(dst.cpu().numpy().view(np.uint32), want)
