#!/usr/bin/env python3
"""Benchmark of the MI355X W4A4 MoE expert path: one learner step of a
Qwen3-30B-A3B-shaped MoE layer (T=16384 tokens, H=2048, E=128, top-8, I=768).

A step is the whole hot path over one batch of synthetic inputs resident in
HBM: quantize+permute (route, per-token amax, NVFP4 encode, scatter), the
grouped expert forward (FC1 + SwiGLU, requantise, FC2, unpermute; h and a
saved) and the straight-through BF16 backward (dX, dW1, dW2).  Weights are
quantised once before timing (offline, as on the pages).

Timing: W warm-up steps, then K reps, each preceded by a write of a 1 GiB
scratch buffer (evicting the L2s and the 256 MB MALL) and bracketed by HIP
events on the caller's stream; `value` = T / the median rep, with min, max
and mean beside it.  Per-kernel times come from a second pass of the same
flushed reps with the library's per-launch timing on (events attached to the
dispatches on the launch stream), so those events stay out of the measured
reps.

Prints ONE JSON line.  `value` is tokens/s of the learner step; `roofline`
reports the dominant kernel (by total time, among the kernels that do not
run beside another on the second stream) against its bound; `configs` holds
the other layer configurations timed the same way (quantize+permute alone on
Student-t activations, the forward at T=8192, the skewed routing at
T=32768 forward and forward + backward), each with its own roofline;
`cpu_baseline` times the FP64 oracle on a bounded sample on the host.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 MoE expert fwd+bwd tokens/s and % MFMA/HBM peak, Qwen3-30B-A3B layer"
WORKLOAD = "learner"
PEAK_MFMA_TFLOPS = 2500.0      # MI355X dense f16 / bf16 MFMA
PEAK_MFMA_FP4_TFLOPS = 10100.0  # MI355X dense MXFP4 (scaled FP4) MFMA
# kernels whose MFMA peak is not the f16 / bf16 one
PEAK_MFMA_FP8_TFLOPS = 5000.0   # MI355X dense FP8 (scaled FP8) MFMA
KERNEL_PEAK = {"mx_gemm_fc1": PEAK_MFMA_FP4_TFLOPS, "mx_gemm_fc2": PEAK_MFMA_FP4_TFLOPS,
               "mx8_dgrad_fc2": PEAK_MFMA_FP8_TFLOPS, "mx8_wgrad_fc2": PEAK_MFMA_FP8_TFLOPS,
               "mx8_dgrad_fc1": PEAK_MFMA_FP8_TFLOPS, "mx8_wgrad_fc1": PEAK_MFMA_FP8_TFLOPS}
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

# kernel name -> source file whose content decides whether stored counters still apply
KERNEL_SOURCES = {
    "gemm_fc1": "gemm_fwd.hip", "gemm_fc2": "gemm_fwd.hip",
    "gemm_dgrad_fc1": "gemm_bwd.hip", "gemm_dgrad_fc2": "gemm_bwd.hip",
    "gemm_wgrad_fc1": "gemm_bwd.hip", "gemm_wgrad_fc2": "gemm_bwd.hip",
    "quantize_scatter": "quantize.hip", "requant": "quantize.hip",
    "unpermute": "elementwise.hip", "dy_scatter": "elementwise.hip", "x_scatter": "elementwise.hip",
    "dx_gather_sum": "elementwise.hip",
    "gemm_linear": "gemm_fwd.hip", "gemm_linear_dgrad": "gemm_bwd.hip",
    "gemm_linear_wgrad": "gemm_bwd.hip",
    "mx_gemm_fc1": "gemm_fwd.hip", "mx_gemm_fc2": "gemm_fwd.hip",
    "mx_quantize_scatter": "quantize.hip", "mx_requant": "quantize.hip",
    "mx8_dgrad_fc2": "gemm_fwd.hip", "mx8_wgrad_fc2": "gemm_fwd.hip",
    "mx8_dgrad_fc1": "gemm_fwd.hip", "mx8_wgrad_fc1": "gemm_fwd.hip",
    "mx8_swiglu_quant_dual_dH": "mx8.hip",
}
for _n in ("dual_dO", "cols_a", "cols_w2", "cols_w1", "cols_xp"):
    KERNEL_SOURCES["mx8_quant_" + _n] = "mx8.hip"


def algorithmic_work(T, H, E, k, I):
    """Per-launch algorithmic flops (MFMA kernels) or bytes (HBM kernels).
    Rows M = T*k dispatched rows (padding excluded)."""
    M = T * k
    fl = {
        "gemm_fc1": 2.0 * M * H * 2 * I,
        "gemm_fc2": 2.0 * M * I * H,
        "gemm_dgrad_fc2": 2.0 * M * H * I,
        "gemm_wgrad_fc2": 2.0 * M * H * I,
        "gemm_dgrad_fc1": 2.0 * M * 2 * I * H,
        "gemm_wgrad_fc1": 2.0 * M * 2 * I * H,
    }
    by = {
        # read x and topk_idx; write k copies of codes/scales/outer, row_map, src_row
        "quantize_scatter": T * (H * 2 + k * 4) + M * (H // 2 + H // 16 + 4) + T * k * 4 + M * 4,
        "requant": M * (I * 2 + I // 2 + I // 16 + 4),
        "unpermute": T * (k * H * 2 + k * 8 + H * 2),
        # read dY[t] and the token's k maps / weights; write k rows of dO
        "dy_scatter": T * (H * 2 + k * 8) + M * H * 2,
        # read x[t] and the token's k maps; write k rows of xp
        "x_scatter": T * (H * 2 + k * 4) + M * H * 2,
        "dx_gather_sum": T * (k * H * 2 + k * 4 + H * 2),
        # MXFP4 recipe: one E8M0 byte per 32 elements, no outer scales
        "mx_quantize_scatter": T * (H * 2 + k * 4) + M * (H // 2 + H // 32) + T * k * 4 + M * 4,
        "mx_requant": M * (I * 2 + I // 2 + I // 32),
    }
    fl["mx_gemm_fc1"] = fl["gemm_fc1"]
    fl["mx_gemm_fc2"] = fl["gemm_fc2"]
    for n in ("dgrad_fc2", "wgrad_fc2", "dgrad_fc1", "wgrad_fc1"):
        fl["mx8_" + n] = fl["gemm_" + n]
    # MXFP8 quantisers: read bf16, write one E4M3 byte per element and one E8M0 byte per 32
    q8 = lambda n: n * (2 + 1) + n // 32
    by.update({"mx8_quant_dual_dO": M * H * 2 + 2 * (M * H + M * H // 32),
               # the SwiGLU backward's inputs dA and h; both forms of dH out
               "mx8_swiglu_quant_dual_dH": M * I * 2 + M * 2 * I * 2 + 2 * (M * 2 * I + M * 2 * I // 32),
               "mx8_quant_cols_a": q8(M * I), "mx8_quant_cols_xp": q8(M * H),
               "mx8_quant_cols_w2": q8(E * H * I), "mx8_quant_cols_w1": q8(E * 2 * I * H)})
    return fl, by


# Kernels the library runs concurrently with another one (second stream).
CONCURRENT = {"wgrad_schedule": "dy_scatter, gemm_dgrad_fc2",
              "x_scatter": "gemm_wgrad_fc2, gemm_dgrad_fc1"}


def source_hash(name):
    path = os.path.join(ROOT, "precision_rl_amd", "csrc", KERNEL_SOURCES[name])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic(name):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, or None
    when none exist or the kernel source changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(name)
    if not rec or rec.get("source_sha256_16") != source_hash(name):
        return None
    return rec.get("hbm_bytes_per_launch")


# Dense linear workload: a Qwen3-30B-A3B query projection (hidden 2048 -> 32
# heads x 128) at the learner batch.
LINEAR = dict(T=16384, K=2048, N=4096)
LINEAR_METRIC = "W4A4 dense per-token NVFP4 linear fwd+bwd tokens/s, Qwen3-30B-A3B q projection"


def linear_work(T, K, N):
    """Per-launch algorithmic flops / bytes of the dense linear step."""
    fl = {n: 2.0 * T * K * N for n in ("gemm_linear", "gemm_linear_dgrad", "gemm_linear_wgrad")}
    # read x; write codes, scales, outer, row_map, src_row (identity routing)
    by = {"quantize_scatter": T * (K * 2 + K // 2 + K // 16 + 12)}
    # the K split of the weight gradient (2 pieces at this shape on 256 CUs):
    # read the FP32 sums of the pieces, write bf16 dW
    by["splitk_reduce"] = N * K * (2 * 4 + 2)
    return fl, by


def host_info():
    """The host CPUs the oracle may use and their model name (from /proc/cpuinfo)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return {"host_cpus": len(os.sched_getaffinity(0)), "cpu_model": model}


def cpu_baseline_linear(x, w, dy, tokens):
    """The FP64 oracle's linear forward + backward on the first `tokens` tokens
    (the weight's quantisation inside the oracle call is included)."""
    from oracle import linear, nvfp4 as q
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    xf, wf, dyf = (q.bf16_bits_to_f64(v) for v in (x[:tokens], w, dy[:tokens]))
    t0 = time.perf_counter()
    linear.forward(xf, wf)
    linear.backward(dyf, xf, wf)
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{tokens} tokens of the linear workload (K={w.shape[1]}, N={w.shape[0]}), "
                      f"FP64 numpy, quantize (x and W) + forward + backward, {dt:.1f} s",
            "seconds": dt, **host_info()}


def main_linear(args):
    import torch
    from precision_rl_amd import binding as b, synth

    T, K, N = LINEAR["T"], LINEAR["K"], LINEAR["N"]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(1005)))
    xb = synth.normal_bf16(rng, (T, K))
    wb = synth.normal_bf16(rng, (N, K), synth.W_STD)
    dyb = synth.normal_bf16(rng, (T, N))
    dev = torch.device("cuda:0")

    def bf(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x, W, dy = bf(xb), bf(wb), bf(dyb)
    wq = b.w4a4_quantize_permute(W, None, 1)      # offline, untimed
    xq = dict(codes=torch.empty(T, K // 2, dtype=torch.uint8, device=dev),
              scales=torch.empty(T, K // 16, dtype=torch.uint8, device=dev),
              outer=torch.empty(T, dtype=torch.float32, device=dev),
              offsets=torch.empty(2, dtype=torch.int32, device=dev),
              row_map=torch.empty(T, 1, dtype=torch.int32, device=dev),
              src_row=torch.empty(T, dtype=torch.int32, device=dev))
    ws_qp = torch.empty(b.workspace_size(b.WS_QUANTIZE_PERMUTE, T, K, 0, 1, 1, 1) + 256,
                        dtype=torch.uint8, device=dev)
    ws_b = torch.empty(b.workspace_size(b.WS_LINEAR_BACKWARD, 0, K, N, 1, 1, 1),
                       dtype=torch.uint8, device=dev)
    y = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    grads = dict(dx=torch.empty(T, K, dtype=torch.bfloat16, device=dev),
                 dw=torch.empty(N, K, dtype=torch.bfloat16, device=dev))

    calibration_copy(torch, dev)

    def step():
        b.w4a4_quantize_permute(x, None, 1, out=xq, workspace=ws_qp)
        b.w4a4_linear_fwd(xq, wq, T, K, N, y=y)
        b.w4a4_linear_bwd(dy, x, W, xq, T, K, N, out=grads, workspace=ws_b)

    flush = Flusher(torch, dev)
    st, kern = time_steps(b, torch, step, args, flush, "linear step")
    ms = st["median"]
    fl, by = linear_work(T, K, N)
    per_kernel, roof = summarize(kern, ms, args.steps, fl, by, concurrent={})
    out = {
        "metric": LINEAR_METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "timing": time_fields(st, args.steps),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4->f16 MFMA fwd, bf16 MFMA bwd, fp32 accumulate",
        "data": "synthetic (seeded; random-init weight of the layer's shape)",
        "config": {"workload": "linear: quantize + NVFP4 linear fwd + BF16 STE bwd",
                   "T": T, "K": K, "N": N},
        "roofline": roof,
        "step_mfma_tflops": round(sum(fl.values()) / (ms * 1e-3) / 1e12, 1),
        "kernels": per_kernel,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the FP64 oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_linear(xb, wb, dyb, tokens=T)
    print(json.dumps(out), flush=True)


QP_METRIC = "W4A4 quantize+permute tokens/s and % HBM peak (route + per-row amax + NVFP4 encode + scatter)"


def qp_work(T, H, k, outer, recipe="nvfp4"):
    """Per-launch algorithmic bytes of quantize+permute (c2 shape)."""
    M = T * k
    by = {"quantize_scatter": T * (H * 2 + k * 4) + M * (H // 2 + H // 16 + 4) + T * k * 4 + M * 4,
          # MXFP4: one E8M0 byte per 32 elements, no outer scale
          "mx_quantize_scatter": T * (H * 2 + k * 4) + M * (H // 2 + H // 32) + T * k * 4 + M * 4}
    by = {n: v for n, v in by.items() if n.startswith("mx_") == (recipe == "mxfp4")}
    if outer == "tensor":
        by["group_amax"] = T * H * 2     # one extra read of x
    return {}, by


def cpu_baseline_qp(d, tokens, group_rows, recipe="nvfp4"):
    from oracle import moe, nvfp4 as q
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    x = q.bf16_bits_to_f64(d["x"][:tokens])
    idx = d["topk_idx"][:tokens]
    E = int(d["topk_idx"].max()) + 1
    t0 = time.perf_counter()
    if recipe == "mxfp4":
        moe.quantize_permute_mx(x, idx, E, 1)
    else:
        moe.quantize_permute(x, idx, E, 1, group_rows=min(group_rows, tokens))
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{tokens} tokens of the quantize+permute workload"
                      f"{' (MXFP4)' if recipe == 'mxfp4' else ''}, FP64 numpy, {dt:.1f} s",
            "seconds": dt, **host_info()}


def main_qp(args):
    import torch
    from precision_rl_amd import binding as b, synth

    w = synth.WORKLOADS["qp"]
    T, H, E, k = w.T, w.H, w.E, w.k
    d = synth.workload_inputs("qp")
    dev = torch.device("cuda:0")
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    idx = torch.from_numpy(d["topk_idx"]).to(dev)
    cap = b.rows_capacity(T, k, E, 1)
    mx = args.recipe == "mxfp4"
    if mx and args.outer != "token":
        print("bench.py: the MXFP4 recipe has no outer scale (--outer applies to nvfp4)", file=sys.stderr)
        sys.exit(2)
    xq = dict(codes=torch.empty(cap, H // 2, dtype=torch.uint8, device=dev),
              scales=torch.empty(cap, H // (32 if mx else 16), dtype=torch.uint8, device=dev),
              offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
              row_map=torch.empty(T, k, dtype=torch.int32, device=dev),
              src_row=torch.empty(cap, dtype=torch.int32, device=dev))
    if not mx:
        xq["outer"] = torch.empty(cap, dtype=torch.float32, device=dev)
    per_tensor = args.outer == "tensor"
    kind = b.WS_QUANTIZE_PERMUTE_DOMAIN if per_tensor else b.WS_QUANTIZE_PERMUTE
    ws = torch.empty(b.workspace_size(kind, T, H, 0, E, k, 1) + 256, dtype=torch.uint8, device=dev)
    calibration_copy(torch, dev)

    def step():
        if mx:
            b.w4a4_mx_quantize_permute(x, idx, E, 1, out=xq, workspace=ws)
        elif per_tensor:
            b.w4a4_quantize_permute_domain(x, idx, E, 1, group_rows=T, out=xq, workspace=ws)
        else:
            b.w4a4_quantize_permute(x, idx, E, 1, out=xq, workspace=ws)

    flush = Flusher(torch, dev)
    st, kern = time_steps(b, torch, step, args, flush, "quantize+permute")
    ms = st["median"]
    fl, by = qp_work(T, H, k, args.outer, args.recipe)
    per_kernel, roof = summarize(kern, ms, args.steps, fl, by, concurrent={})
    alg = sum(by.values()) - by.get("group_amax", 0)
    out = {
        "metric": QP_METRIC.replace("NVFP4", "MXFP4") if mx else QP_METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "timing": time_fields(st, args.steps),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 -> mxfp4 (u8 codes, e8m0 scales)" if mx else "bf16 -> nvfp4 (u8 codes, e4m3 scales, f32 outer)",
        "data": "synthetic (seeded; Student-t x)",
        "config": {"workload": "qp: route + quantize+permute, MXFP4" if mx else
                               f"qp: route + quantize+permute, outer scale per {args.outer}",
                   "T": T, "H": H, "E": E, "top_k": k},
        "roofline": roof,
        "call_hbm_frac": round(alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "kernels": per_kernel,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the FP64 oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_qp(d, 8192, T if per_tensor else 1, args.recipe)
    print(json.dumps(out), flush=True)


def cpu_baseline(d, w, tokens=512, experts=8, recipe="nvfp4", bwd="bf16"):
    """The FP64 oracle on a bounded sample of the learner workload: the first
    `tokens` tokens, each routed to all `experts` experts (k = 8 per token as
    in the workload, so the per-token work is the same), expert weights
    quantised before timing.  Times quantize+permute + forward + backward
    (the forward of the given recipe)."""
    from oracle import moe, nvfp4 as q
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    k = w.k
    assert experts == k
    x = q.bf16_bits_to_f64(d["x"][:tokens])
    dy = q.bf16_bits_to_f64(d["dy"][:tokens])
    w1 = q.bf16_bits_to_f64(d["w1"][:experts])
    w2 = q.bf16_bits_to_f64(d["w2"][:experts])
    idx = np.tile(np.arange(k, dtype=np.int32), (tokens, 1))
    p = d["topk_w"][:tokens]
    mx = recipe == "mxfp4"
    quant = moe.quantize_weights_mx if mx else moe.quantize_weights
    w1q, w2q = quant(w1), quant(w2)
    t0 = time.perf_counter()
    f = (moe.forward_mx if mx else moe.forward)(x, idx, p, w1q, w2q, experts)
    xq = f["xq"]
    (moe.backward_mx8 if bwd == "mxfp8" else moe.backward)(
        dy, x, w1, w2, f["h"], f["a"], p, xq["offsets"], xq["row_map"], xq["src_row"])
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{tokens} tokens of the learner workload (H={w.H}, I={w.I}, k={k}) routed "
                      f"to {experts} experts, FP64 numpy, quantize+permute+forward+backward"
                      f"{' (MXFP4 recipe)' if mx else ''}{' (MXFP8 backward)' if bwd == 'mxfp8' else ''}, "
                      f"{dt:.1f} s", "seconds": dt, **host_info()}


def calibration_copy(torch, dev):
    """A plain elementwise copy of known size (reads 256 MiB, writes 256 MiB),
    run once before timing, for scaling the HBM counters of --pmc runs."""
    calib = torch.ones(128 << 20, dtype=torch.bfloat16, device=dev)
    calib_out = torch.empty_like(calib)
    torch.cuda.synchronize()
    torch.neg(calib, out=calib_out)
    del calib, calib_out


FLUSH_BYTES = 1 << 30   # > the 256 MB MALL plus every XCD's 4 MB L2


class Flusher:
    """Writes a 1 GiB scratch buffer on the current stream, which evicts the
    L2s and the MALL, so that every timed rep starts with cold caches."""

    def __init__(self, torch, dev):
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(self.n)


def measure(torch, step, reps, warmup, flush):
    """`warmup` untimed steps, then `reps` timed steps, each after a cache
    flush and between two HIP events on the current stream (the library
    launches on it and joins its second stream back into it).  The loop is
    bracketed by device synchronisations.  Returns the per-rep times (ms)."""
    for _ in range(warmup):
        flush()
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for s, e in ev:
        flush()
        s.record()
        step()
        e.record()
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in ev]


def stats(times):
    t = sorted(times)
    n = len(t)
    med = t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2])
    return {"median": med, "min": t[0], "max": t[-1], "mean": sum(t) / n}


def profile(b, torch, step, reps, flush):
    """The same flushed reps with the library's per-launch timing on (a
    separate pass: its events stay out of the measured reps).  Returns the
    per-kernel record {name: {count, total_ms}}."""
    b.w4a4_profiler_enable(True)
    measure(torch, step, reps, 0, flush)
    kern = b.w4a4_profiler_report()
    b.w4a4_profiler_enable(False)
    return kern


def time_steps(b, torch, step, args, flush, label="step"):
    """Flushed, event-timed reps (the value) and a profiled pass (per-kernel
    times).  Returns (stats in ms, per-kernel record)."""
    times = measure(torch, step, args.steps, args.warmup, flush)
    st = stats(times)
    print(f"[bench] {label}: {args.steps} flushed reps, median {st['median']:.3f} ms "
          f"(min {st['min']:.3f}, max {st['max']:.3f})", file=sys.stderr, flush=True)
    kern = profile(b, torch, step, args.steps, flush)
    return st, kern


def time_fields(st, steps):
    return {"ms_median": round(st["median"], 4), "ms_min": round(st["min"], 4),
            "ms_max": round(st["max"], 4), "ms_mean": round(st["mean"], 4), "reps": steps}


def summarize(kern, ms, steps, fl, by, concurrent=None):
    """Per-kernel table and the roofline object of the dominant kernel.
    `concurrent`: kernels that run on the library's second stream."""
    concurrent = CONCURRENT if concurrent is None else concurrent
    per_kernel = {}
    for name, rec in sorted(kern.items(), key=lambda kv: -kv[1]["total_ms"]):
        avg_ms = rec["total_ms"] / rec["count"]
        entry = {"avg_ms": round(avg_ms, 4), "launches": rec["count"],
                 "share": round(rec["total_ms"] / (ms * steps), 4)}
        if name in fl:
            entry["tflops"] = round(fl[name] / (avg_ms * 1e-3) / 1e12, 1)
            entry["frac_mfma"] = round(entry["tflops"] / KERNEL_PEAK.get(name, PEAK_MFMA_TFLOPS), 4)
        elif name in by:
            entry["gbs"] = round(by[name] / (avg_ms * 1e-3) / 1e9, 1)
            entry["frac_hbm"] = round(entry["gbs"] / PEAK_HBM_GBS, 4)
        if name in concurrent:
            # launched on a second stream beside another kernel: its duration is
            # time shared with that kernel, not its standalone rate
            entry["runs_beside"] = concurrent[name]
        per_kernel[name] = entry
    # the dominant kernel is taken among those that own the GPU while they run:
    # a second-stream kernel's duration includes the time it shares with the
    # kernel beside it, so it states no rate of its own
    alone = [n for n in kern if n not in concurrent and (n in fl or n in by)] or list(kern)
    dom = max(alone, key=lambda n: kern[n]["total_ms"])
    dom_avg_s = kern[dom]["total_ms"] / kern[dom]["count"] * 1e-3
    if dom not in fl and dom not in by:
        roof = {"bound": None, "achieved": None, "peak": None, "unit": None, "frac": None}
    elif dom in fl:
        ach = fl[dom] / dom_avg_s / 1e12
        peak = KERNEL_PEAK.get(dom, PEAK_MFMA_TFLOPS)
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4)}
    else:
        ach = by[dom] / dom_avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4)}
    roof["kernel"] = dom
    roof["avg_ms"] = round(dom_avg_s * 1e3, 4)
    roof["traffic"] = stored_traffic(dom)

    return per_kernel, roof


def moe_buffers(torch, dev, b, T, H, E, k, I, A, mx, mx8):
    """Preallocated outputs and workspaces of one quantize+permute + forward
    (+ backward) of a MoE layer."""
    cap = b.rows_capacity(T, k, E, A)
    xq = dict(codes=torch.empty(cap, H // 2, dtype=torch.uint8, device=dev),
              scales=torch.empty(cap, H // (32 if mx else 16), dtype=torch.uint8, device=dev),
              offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
              row_map=torch.empty(T, k, dtype=torch.int32, device=dev),
              src_row=torch.empty(cap, dtype=torch.int32, device=dev))
    if not mx:
        xq["outer"] = torch.empty(cap, dtype=torch.float32, device=dev)
    return dict(
        xq=xq,
        ws_qp=torch.empty(b.workspace_size(b.WS_QUANTIZE_PERMUTE, T, H, I, E, k, A) + 256,
                          dtype=torch.uint8, device=dev),
        ws_f=torch.empty(b.workspace_size(b.WS_FORWARD, T, H, I, E, k, A), dtype=torch.uint8, device=dev),
        ws_b=torch.empty(b.workspace_size(b.WS_MX8_BACKWARD if mx8 else b.WS_BACKWARD, T, H, I, E, k, A),
                         dtype=torch.uint8, device=dev),
        y=torch.empty(T, H, dtype=torch.bfloat16, device=dev),
        saved=dict(h=torch.empty(cap, 2 * I, dtype=torch.bfloat16, device=dev),
                   a=torch.empty(cap, I, dtype=torch.bfloat16, device=dev)),
        grads=dict(dx=torch.empty(T, H, dtype=torch.bfloat16, device=dev),
                   dw1=torch.empty(E, 2 * I, H, dtype=torch.bfloat16, device=dev),
                   dw2=torch.empty(E, H, I, dtype=torch.bfloat16, device=dev)))


def moe_step(b, bufs, x, idx, p, w1q, w2q, w1, w2, dy, T, H, E, k, I, A, mx=False, mx8=False,
             backward=True):
    """One pass of the hot path: quantize+permute, the grouped expert forward
    (saving h and a) and, with `backward`, the straight-through backward."""
    xq, saved, grads = bufs["xq"], bufs["saved"], bufs["grads"]

    def step():
        if mx:
            b.w4a4_mx_quantize_permute(x, idx, E, A, out=xq, workspace=bufs["ws_qp"])
            b.w4a4_mx_grouped_expert_fwd(xq, p, w1q, w2q, T, H, I, E, k, A, save=backward, y=bufs["y"],
                                         workspace=bufs["ws_f"], saved=saved if backward else None)
        else:
            b.w4a4_quantize_permute(x, idx, E, A, out=xq, workspace=bufs["ws_qp"])
            b.w4a4_grouped_expert_fwd(xq, p, w1q, w2q, T, H, I, E, k, A, save=backward, y=bufs["y"],
                                      workspace=bufs["ws_f"], saved=saved if backward else None)
        if backward:
            bwd = b.w4a4_mx8_expert_bwd if mx8 else b.w4a4_expert_bwd
            bwd(dy, x, w1, w2, saved["h"], saved["a"], p, xq, T, H, I, E, k, A, out=grads,
                workspace=bufs["ws_b"])
    return step


def gemm_fracs(per_kernel):
    return {n: e["frac_mfma"] for n, e in per_kernel.items() if "frac_mfma" in e}


def sub_config(name, workload, timed, st, kern, steps, T, fl, by, concurrent, extra=None):
    """One secondary configuration's record for the JSON line."""
    per_kernel, roof = summarize(kern, st["median"], steps, fl, by, concurrent=concurrent)
    rec = {"workload": workload, "timed": timed, "T": T,
           "tokens_per_s": round(T / (st["median"] * 1e-3), 1)}
    rec.update(time_fields(st, steps))
    rec["roofline"] = roof
    rec["gemm_frac_mfma"] = gemm_fracs(per_kernel)
    rec["kernels"] = {n: {k2: v for k2, v in e.items() if k2 in ("avg_ms", "frac_mfma", "frac_hbm", "runs_beside")}
                      for n, e in per_kernel.items()}
    if extra:
        rec.update(extra)
    print(f"[bench] {name}: {rec['tokens_per_s']:.4g} tokens/s", file=sys.stderr, flush=True)
    return rec


def secondary_configs(b, torch, dev, args, flush, weights):
    """The other layer configurations, each timed like the main step (flushed
    reps, median) with its own per-kernel pass: quantize+permute alone on
    Student-t activations (T=16384), the forward at T=8192 (near-uniform
    routing), and the skewed routing at T=32768 (Zipf 1.2, 10 experts
    without tokens), forward and forward + backward.  The expert weights are
    the main workload's (same shapes and distribution)."""
    from precision_rl_amd import synth
    w1q, w2q, w1, w2 = weights
    out = {}

    # c2: quantize+permute alone
    wq = synth.WORKLOADS["qp"]
    d = synth.workload_inputs("qp")
    T, H, E, k = wq.T, wq.H, wq.E, wq.k
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    idx = torch.from_numpy(d["topk_idx"]).to(dev)
    bufs = moe_buffers(torch, dev, b, T, H, E, k, 0, 1, False, False)

    def qp_step():
        b.w4a4_quantize_permute(x, idx, E, 1, out=bufs["xq"], workspace=bufs["ws_qp"])
    st, kern = time_steps(b, torch, qp_step, args, flush, "c2 quantize+permute")
    _, by = qp_work(T, H, k, "token")
    alg = sum(by.values())
    out["c2_quantize_permute"] = sub_config(
        "c2", "qp: route + quantize+permute, Student-t x (T=16384, H=2048, E=128, top-8)",
        "w4a4_quantize_permute (routing included)", st, kern, args.steps, T, {}, by, {},
        extra={"call_bytes": alg, "call_gbs": round(alg / (st["median"] * 1e-3) / 1e9, 1),
               "call_hbm_frac": round(alg / (st["median"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)})
    del x, idx, bufs, d

    for key, wl, backward in (("c3_forward", "fwd", False), ("c4_skew_forward", "skew", False),
                              ("c4_skew_forward_backward", "skew", True)):
        w = synth.WORKLOADS[wl]
        T, H, E, k, I = w.T, w.H, w.E, w.k, w.I
        d = synth.make_inputs(T, H, E, k, I, w.routing, w.x_dist, backward=backward,
                              seed=1000 + w.index, weights=False)
        bf = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        x = bf(d["x"])
        dy = bf(d["dy"]) if backward else None
        idx = torch.from_numpy(d["topk_idx"]).to(dev)
        p = torch.from_numpy(d["topk_w"]).to(dev)
        bufs = moe_buffers(torch, dev, b, T, H, E, k, I, 1, False, False)
        step = moe_step(b, bufs, x, idx, p, w1q, w2q, w1, w2, dy, T, H, E, k, I, 1, backward=backward)
        st, kern = time_steps(b, torch, step, args, flush, key)
        fl, by = algorithmic_work(T, H, E, k, I)
        if not backward:
            fl = {n: v for n, v in fl.items() if n in ("gemm_fc1", "gemm_fc2")}
        out[key] = sub_config(
            key, f"{wl}: quantize+permute + grouped expert fwd" + (" + BF16 STE bwd" if backward else "")
            + f" (T={T}, H={H}, E={E}, top-{k}, I={I}, {w.routing} routing)",
            "quantize_permute + fwd" + (" + bwd" if backward else ""), st, kern, args.steps, T, fl, by,
            None if backward else {})
        del x, dy, idx, p, bufs, d, step
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="learner: skip the other layer configurations (quantize+permute alone, "
                         "forward at T=8192, skewed routing at T=32768)")
    ap.add_argument("--cpu-tokens", type=int, default=6144)
    ap.add_argument("--workload", choices=["learner", "linear", "qp"], default="learner",
                    help="learner: the MoE expert step (default); linear: the dense projection; "
                         "qp: quantize+permute alone")
    ap.add_argument("--outer", choices=["token", "tensor"], default="token",
                    help="qp: outer-scale domain of the activations")
    ap.add_argument("--bwd", choices=["bf16", "mxfp8"], default="bf16",
                    help="learner: the straight-through backward's GEMM operands -- bf16 (the "
                         "default) or mxfp8 (E4M3 + E8M0 per 32 along each GEMM's reduction axis, "
                         "scaled FP8 MFMA; routes with row_align 128)")
    ap.add_argument("--recipe", choices=["nvfp4", "mxfp4"], default="nvfp4",
                    help="learner and qp: the forward's format -- nvfp4 (E4M3 per 16 + FP32 outer "
                         "scales, exact f16 decode, the default) or mxfp4 (E8M0 per 32, scaled "
                         "FP4 MFMA)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "the library's expert path is single-GPU (sharding is described in the design notes).",
              file=sys.stderr)
        sys.exit(2)

    if args.workload == "linear":
        return main_linear(args)
    if args.workload == "qp":
        return main_qp(args)

    import torch
    from precision_rl_amd import binding as b, synth

    w = synth.WORKLOADS[WORKLOAD]
    mx8 = args.bwd == "mxfp8"
    T, H, E, k, I, A = w.T, w.H, w.E, w.k, w.I, (128 if mx8 else 1)
    d = synth.workload_inputs(WORKLOAD)
    dev = torch.device("cuda:0")

    def bf(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x, w1, w2, dy = bf(d["x"]), bf(d["w1"]), bf(d["w2"]), bf(d["dy"])
    idx = torch.from_numpy(d["topk_idx"]).to(dev)
    p = torch.from_numpy(d["topk_w"]).to(dev)
    mx = args.recipe == "mxfp4"
    if mx:
        w1q, w2q = b.quantize_weights_mx(w1), b.quantize_weights_mx(w2)   # offline, untimed
    else:
        w1q, w2q = b.quantize_weights(w1), b.quantize_weights(w2)         # offline, untimed

    bufs = moe_buffers(torch, dev, b, T, H, E, k, I, A, mx, mx8)
    step = moe_step(b, bufs, x, idx, p, w1q, w2q, w1, w2, dy, T, H, E, k, I, A, mx=mx, mx8=mx8)
    calibration_copy(torch, dev)
    flush = Flusher(torch, dev)

    st, kern = time_steps(b, torch, step, args, flush, "learner step")
    ms = st["median"]
    fl, by = algorithmic_work(T, H, E, k, I)
    # the MXFP8 backward runs on the caller's stream alone
    per_kernel, roof = summarize(kern, ms, args.steps, fl, by, concurrent={} if mx8 else None)

    gemm_ms = sum(kern[n]["total_ms"] for n in kern if n in fl) / args.steps
    total_flop = sum(v for n, v in fl.items() if n.startswith("gemm_"))
    out = {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp4 scaled-FP4 MFMA fwd" if mx else "nvfp4->f16 MFMA fwd")
                 + (", mxfp8 scaled-FP8 MFMA bwd" if mx8 else ", bf16 MFMA bwd") + ", fp32 accumulate",
        "data": "synthetic (seeded; random-init weights of the layer's shape)",
        "config": {"workload": f"{WORKLOAD}: quantize+permute + grouped expert fwd + "
                               + ("MXFP8" if mx8 else "BF16") + " STE bwd"
                               + (" (MXFP4 recipe: E2M1 + E8M0 per 32)" if mx else ""),
                   "T": T, "H": H, "E": E, "top_k": k, "I": I, "row_align": A,
                   "routing": w.routing},
        "timing": dict(time_fields(st, args.steps), flush_bytes=FLUSH_BYTES,
                       method="HIP events around each rep on the caller's stream, L2 + MALL flushed "
                              "before each rep; value from the median; per-kernel times from a "
                              "separate profiled pass"),
        "roofline": roof,
        "step_mfma_tflops": round(total_flop / (ms * 1e-3) / 1e12, 1),
        "gemm_ms_per_step": round(gemm_ms, 4),
        "gemm_frac_mfma": gemm_fracs(per_kernel),
        "kernels": per_kernel,
    }
    if not args.no_secondary and not mx and not mx8:
        out["configs"] = secondary_configs(b, torch, dev, args, flush, (w1q, w2q, w1, w2))
    if not args.no_cpu_baseline:
        print("[bench] timing the FP64 oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(d, w, tokens=args.cpu_tokens, recipe=args.recipe, bwd=args.bwd)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
