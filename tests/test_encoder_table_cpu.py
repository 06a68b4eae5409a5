"""The row encoder's table path for block scales and crossing thresholds
against its direct construction, over the whole input domain of that step.

tests/encoder_table_check.cpp restates both ways the NVFP4 row encoder forms
a block's E4M3 scale and its seven bf16 crossing thresholds (one correctly
rounded FP64 division and exact FP64 products; or the per-row reciprocal with
an exact midpoint check and the per-row threshold table shifted by the
block's exponent) and runs them over every pair of finite bf16 magnitudes
(row maximum, block maximum <= row maximum): 532,701,120 pairs.  They must
agree on every scale byte and packed threshold, including the pairs whose
quotient rounds to a float32 that is an E4M3 rounding midpoint (exact ties,
and near-ties whose side only the exact quotient decides).  The GPU parity
tests then hold the kernel itself to the FP64 oracle.
"""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_table_path_matches_direct_construction_everywhere(tmp_path):
    exe = str(tmp_path / "encoder_table_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-pthread",
                    os.path.join(HERE, "encoder_table_check.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    m = re.search(r"pairs (\d+) mismatches (\d+) midpoint (\d+) near_ties (\d+)", r.stdout)
    assert m and r.returncode == 0, r.stdout + r.stderr
    pairs, bad, mids, near = map(int, m.groups())
    assert pairs == 532_701_120
    assert bad == 0
    # the midpoint branch is exercised both ways
    assert near > 100_000 and mids - near > 10_000
