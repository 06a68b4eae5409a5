"""The benchmark's algorithmic work per launch (CPU only): the per-token and
per-row figures its roofline divides by, checked against the counts the
layer shape fixes (T tokens, k experts per token, H hidden, I FFN width):
6 k H I flop per token in the forward GEMMs, twice that in the backward,
13,440 bytes per token for quantize+permute at H = 2048, k = 8."""
import subprocess
import sys
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

pytestmark = pytest.mark.cpu

T, H, E, k, I = 16384, 2048, 128, 8, 768


def test_gemm_flops():
    fl, _ = bench.algorithmic_work(T, H, E, k, I)
    fwd = fl["gemm_fc1"] + fl["gemm_fc2"]
    bwd = sum(fl[n] for n in ("gemm_dgrad_fc2", "gemm_wgrad_fc2", "gemm_dgrad_fc1", "gemm_wgrad_fc1"))
    assert fwd == 6 * k * H * I * T                     # 75.5 MFLOP per token
    assert bwd == 2 * fwd                               # 151.0 MFLOP per token
    assert round((fwd + bwd) / 1e9, 1) == 3710.9        # GFLOP per learner step
    # the MX kernels do the same algorithmic work
    for n in ("fc1", "fc2"):
        assert fl["mx_gemm_" + n] == fl["gemm_" + n]
    for n in ("dgrad_fc2", "wgrad_fc2", "dgrad_fc1", "wgrad_fc1"):
        assert fl["mx8_" + n] == fl["gemm_" + n]


def test_hbm_bytes():
    _, by = bench.algorithmic_work(T, H, E, k, I)
    # read x (2H) + the token's k ids; k rows of codes (H/2), E4M3 scales
    # (H/16), FP32 outer (4); row_map and src_row entries (4 + 4 per row)
    assert by["quantize_scatter"] == T * 13440
    assert by["requant"] == T * k * 1972
    assert by["unpermute"] == T * 36928
    assert by["dx_gather_sum"] == T * 36896
    # MXFP4: one E8M0 byte per 32 elements instead of E4M3 per 16 and no outer scale
    assert by["quantize_scatter"] - by["mx_quantize_scatter"] == T * k * (H // 16 - H // 32 + 4)


def test_peaks_per_kernel():
    assert bench.KERNEL_PEAK.get("gemm_fc1", bench.PEAK_MFMA_TFLOPS) == 2500.0
    assert bench.KERNEL_PEAK["mx_gemm_fc1"] == 10100.0
    assert bench.KERNEL_PEAK["mx8_wgrad_fc1"] == 5000.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
