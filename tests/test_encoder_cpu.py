"""The row encoder's fast arithmetic against the direct rounding, on the CPU.

tests/encoder_check.cpp restates how the NVFP4 row encoder forms a block's
E4M3 scale (a per-row reciprocal of 6 g with an exact check at E4M3
midpoints) and its elements' E2M1 codes (the hardware round-to-nearest-even
conversion of the quotient bracketed from below and above, and an exact FP64
check of the elements the bracket leaves open), and compares both with the
direct rounding of the exact quotients:
- the scale code over every pair (row maximum, block maximum <= row maximum)
  of finite bf16 magnitudes whose outer scale takes the fast route;
- the codes of the bf16 elements next to every E2M1 midpoint (where a
  rounding error could move a code) for sampled pairs, with the hardware
  reciprocal at the correctly rounded value and one float ulp either side.
Both must agree everywhere, with the midpoint branches exercised both ways.
The GPU parity tests then hold the kernel itself to the FP64 oracle.
"""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_fast_encoder_arithmetic_matches_direct_rounding(tmp_path):
    exe = str(tmp_path / "encoder_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-pthread",
                    os.path.join(HERE, "encoder_check.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    a = re.search(r"pairs (\d+) scale_mismatches (\d+) midpoint (\d+) near_ties (\d+)", r.stdout)
    b = re.search(r"elements (\d+) code_mismatches (\d+) open (\d+) exact_ties (\d+)", r.stdout)
    assert a and b and r.returncode == 0, r.stdout + r.stderr
    pairs, bad, mids, near = map(int, a.groups())
    elems, cbad, opened, ties = map(int, b.groups())
    assert pairs == 453_265_706          # every pair of a row with g in [2^-100, 2^100]
    assert bad == 0 and cbad == 0
    # the E4M3 midpoint branch is exercised both ways
    assert near > 100_000 and mids - near > 10_000
    # elements decided by the bracket, by the exact check, and exact ties
    assert elems > 20_000_000 and opened > 500_000 and ties > 50_000
