"""Build ``libpa.so`` (the C-ABI library) in-tree with hipcc for gfx950.

    python -m paged_kv_cache_228_amd.build

Every HIP translation unit is compiled with packed fp32 instructions switched
off (the compiler's own ``v_pk_*_f32`` selection is disabled); the host
compiler pass warns that it does not know that target feature, which is
harmless. Objects go to ``_build/`` next to this file; the shared library
lands next to this file.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpa.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["pa_api.cpp", "pa_decode.hip", "pa_decode_mfma.hip", "pa_quantize.hip", "pa_append.hip",
           "pa_evict.hip", "pa_copy.hip", "pa_probe.hip", "pa_blockmgr.cpp"]
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
# Device code only: the first kernel arguments of a kernel that takes them as
# plain scalars or pointers arrive in registers when its waves start (the
# decode and merge kernels put what their first loads need there), instead
# of after a load of the argument block; the code object keeps a short entry
# that loads them for firmware without this.
HIP_FLAGS = ["-mllvm", "-amdgpu-kernarg-preload-count=8", "-mllvm", "-amdgpu-mfma-vgpr-form"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip", *HIP_FLAGS] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in ln and ln.strip() and "warning generated" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
