"""Exhaustive host check of the INT8 quantizer's division shortcut.

The quantizer's code is round_half_even(x / scale) clamped to +-127, with
scale = amax / 127 and x / scale an IEEE fp32 division (glossary monograph,
section 5.1: Q = round(K / S); PagedKV-Fusion README, "Overview": symmetric
INT8 per (block, head)). The GPU kernel forms that quotient with one
reciprocal per tile and a Markstein correction per element, then rounds by
the 1.5 * 2^23 shift. ``quotient_check.c`` restates that sequence in C and
compares it, for every finite fp16 amax and every fp16 x with |x| <= amax,
with the IEEE division and with nearbyintf: quotients bit for bit, codes
exactly. (The GPU parity tests sweep every finite fp16 x at several amax
values on the device itself.)
"""

import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_markstein_quotient_equals_ieee_division_for_every_fp16_pair(tmp_path):
    exe = str(tmp_path / "quotient_check")
    flags = ["-O2", "-ffp-contract=off", "-fopenmp"]
    cpu = open("/proc/cpuinfo").read() if os.path.exists("/proc/cpuinfo") else ""
    if re.search(r"\bfma\b", cpu):
        flags.append("-mfma")  # hardware fmaf; glibc's fmaf is exact either way
    subprocess.run(["gcc", *flags, os.path.join(HERE, "quotient_check.c"), "-o", exe, "-lm"],
                   check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=600).stdout
    m = re.search(r"pairs (\d+) quotient_mismatches (\d+) code_mismatches (\d+)", out)
    assert m, out
    pairs, bad_q, bad_c = map(int, m.groups())
    # 31,743 positive finite fp16 amax values; for each, the 2 (hx + 1) signed x
    # with |x| <= amax, hx the amax pattern
    assert pairs == sum(2 * (ha + 1) for ha in range(1, 0x7C00))
    assert bad_q == 0 and bad_c == 0, out
