"""Whole-tensor GPU parity at the layer's full sizes, and the context swap
of the path's outputs.

Full sizes (Qwen3-30B-A3B expert layer: H=2048, E=128, top-8, I=768):
the forward at T=8192 (near-uniform routing), the skewed routing at
T=32768 (Zipf 1.2, 10 experts without tokens, experts of ~31k rows whose
weight-gradient tiles the device schedule cuts into chunks) and the learner
step at T=16384, forward + backward.  Every token's y and dX and every
expert's dW1 and dW2 are compared with the FP64 oracle, which runs expert by
expert (tests/oracle_by_expert.py).  Bars: the routing bit-exact; FC1
pre-cast values rel-L2 <= 1e-5 (whole tensor and every expert); <= 0.1% of
the FC2-input codes differ; y rel-L2 <= 2e-3; dX rel-L2 <= 1e-2; dW1, dW2
rel-L2 <= 1e-2 for the whole tensors and for every live expert; the dW of
an empty expert exactly zero.

Context swap (AI summary, "Methodology in Plain English": with per-token
scaling a token's codes and outputs must not depend on the rest of the
batch, and a per-tensor reference is the negative control): two batches
share some target tokens (same activations, routing, router weights and
output gradients) and differ in every other token, including the expert
loads, so that the targets' rows land at other offsets and tile positions.
The targets' encoded rows, FC1 pre-cast values, h, a, FC2-input encoding, y
and dX must be bitwise identical; with one outer scale per tensor their y
changes.
"""
import numpy as np
import pytest

from oracle import moe, nvfp4 as q
from precision_rl_amd import synth
from gpu_util import bf16_dev, bf16_host, u8, f32_bits, rel_l2, print_case

import oracle_by_expert as obe

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

FC1_TOL = 1e-5
Y_TOL = 2e-3
CODE_FLIP_BUDGET = 1e-3
BWD_TOL = 1e-2


def _b():
    from precision_rl_amd import binding
    return binding


def _gpu(d, T, H, E, k, I, backward, domain_rows=None):
    """Quantize+permute, forward (h, a, FC1 pre-cast values and the FC2-input
    encoding saved) and optionally the backward, through the C ABI."""
    b = _b()
    x = bf16_dev(d["x"], torch)
    idx = torch.from_numpy(d["topk_idx"]).cuda()
    p = torch.from_numpy(d["topk_w"]).cuda()
    w1, w2 = bf16_dev(d["w1"], torch), bf16_dev(d["w2"], torch)
    w1q, w2q = b.quantize_weights(w1), b.quantize_weights(w2)
    if domain_rows is None:
        xq = b.w4a4_quantize_permute(x, idx, E, 1)
    else:
        xq = b.w4a4_quantize_permute_domain(x, idx, E, 1, group_rows=domain_rows)
    f = b.w4a4_grouped_expert_fwd(xq, p, w1q, w2q, T, H, I, E, k, 1, save=True, debug=True)
    g = None
    if backward:
        dy = bf16_dev(d["dy"], torch)
        g = b.w4a4_expert_bwd(dy, x, w1, w2, f["h"], f["a"], p, xq, T, H, I, E, k, 1)
    torch.cuda.synchronize()
    return xq, f, g


def _check_full(name, d, T, H, E, k, I, backward):
    print_case(name, T=T, H=H, E=E, k=k, I=I, backward=backward)
    xq, f, g = _gpu(d, T, H, E, k, I, backward)
    offsets, row_map, src_row = moe.route_fast(d["topk_idx"], E, 1)
    assert np.array_equal(xq["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(xq["row_map"].cpu().numpy(), row_map)
    assert np.array_equal(xq["src_row"].cpu().numpy()[:offsets[-1]], src_row)
    # GPU results to the host before the oracle's pool starts
    fc1 = f["fc1_f32"].cpu().numpy()
    a_codes = q.unpack_codes(u8(f["a_codes"]))
    y = bf16_host(f["y"])
    if backward:
        dx, dw1, dw2 = bf16_host(g["dx"]), bf16_host(g["dw1"]), bf16_host(g["dw2"])
    del xq, f, g
    torch.cuda.empty_cache()
    print(f"[case] {name}: oracle expert by expert ({obe.workers()} workers)", flush=True)
    ref = obe.layer(d, E, backward=backward, want_rows=True)
    # FC1 pre-cast values and FC2-input codes, row by row of every expert
    num = den = 0.0
    worst_fc1 = 0.0
    flips = rows = 0
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        h64 = ref["h64"][e]
        diff = fc1[r0:r1].astype(np.float64) - h64
        num += float(np.sum(diff * diff))
        den += float(np.sum(h64 * h64))
        worst_fc1 = max(worst_fc1, rel_l2(fc1[r0:r1], h64))
        flips += int(np.count_nonzero(a_codes[r0:r1] != ref["a_codes"][e]))
        rows += r1 - r0
    e_fc1 = (num / den) ** 0.5
    flip_rate = flips / (rows * I)
    e_y = rel_l2(y, ref["y"])
    print(f"[case] {name}: FC1 rel-L2 {e_fc1:.2e} (worst expert {worst_fc1:.2e}), "
          f"FC2-input code flips {flip_rate:.2e}, y rel-L2 {e_y:.2e}", flush=True)
    assert e_fc1 <= FC1_TOL and worst_fc1 <= FC1_TOL
    assert flip_rate <= CODE_FLIP_BUDGET
    assert e_y <= Y_TOL
    if backward:
        counts = np.diff(offsets)
        e_dx = rel_l2(dx, ref["dX"])
        e_dw1, e_dw2 = rel_l2(dw1, ref["dW1"]), rel_l2(dw2, ref["dW2"])
        per = [(rel_l2(dw1[e], ref["dW1"][e]), rel_l2(dw2[e], ref["dW2"][e])) for e in range(E) if counts[e]]
        w1_worst, w2_worst = max(p[0] for p in per), max(p[1] for p in per)
        print(f"[case] {name}: dX {e_dx:.2e}, dW1 {e_dw1:.2e} (worst expert {w1_worst:.2e}), "
              f"dW2 {e_dw2:.2e} (worst expert {w2_worst:.2e})", flush=True)
        assert e_dx <= BWD_TOL and e_dw1 <= BWD_TOL and e_dw2 <= BWD_TOL
        assert w1_worst <= BWD_TOL and w2_worst <= BWD_TOL
        for e in np.nonzero(counts == 0)[0]:
            assert not dw1[e].any() and not dw2[e].any()
    return offsets


def test_full_forward_workload_whole_tensors():
    """T=8192, near-uniform routing: every row's FC1 value and FC2-input
    codes, every token's y."""
    w = synth.WORKLOADS["fwd"]
    d = synth.workload_inputs("fwd")
    _check_full("full_forward", d, w.T, w.H, w.E, w.k, w.I, backward=False)


def test_full_skew_workload_whole_tensors():
    """T=32768, Zipf(1.2) routing with 10 empty experts, forward and
    backward, every tensor whole (including the largest experts, whose
    wgrad tiles the schedule deals out in chunks)."""
    w = synth.WORKLOADS["skew"]
    d = synth.make_inputs(w.T, w.H, w.E, w.k, w.I, w.routing, w.x_dist, backward=True,
                          seed=1000 + w.index)
    offsets = _check_full("full_skew", d, w.T, w.H, w.E, w.k, w.I, backward=True)
    counts = np.diff(offsets)
    assert np.count_nonzero(counts == 0) == 10
    # the most popular expert holds ~31k rows: ~3x the mean work of a
    # workgroup's share, so the wgrad schedule cuts its tiles into chunks
    assert counts.max() > 25000


def test_full_learner_workload_whole_tensors():
    """T=16384, the learner step: forward and backward, every tensor whole."""
    w = synth.WORKLOADS["learner"]
    d = synth.workload_inputs("learner")
    _check_full("full_learner", d, w.T, w.H, w.E, w.k, w.I, backward=True)


# ------------------------------------------------------------ context swap
def _swap_batches():
    T, H, E, k, I = 2048, 512, 16, 4, 256
    a = synth.make_inputs(T, H, E, k, I, backward=True, seed=501)
    bb = synth.make_inputs(T, H, E, k, I, routing="zipf", backward=True, seed=502, n_empty=3)
    targets = np.array([0, 17, 1000, 1555, T - 1])
    for n in ("x", "topk_idx", "topk_w", "dy"):
        bb[n] = bb[n].copy()
        bb[n][targets] = a[n][targets]
    bb["w1"], bb["w2"] = a["w1"], a["w2"]
    # a non-target token of the second batch gets the largest magnitude of
    # both batches (3x the first batch's maximum; the per-tensor outer
    # scale then differs by a non-power-of-two factor)
    big = q.bf16_bits_to_f64(a["x"])
    row = q.bf16_bits_to_f64(bb["x"][5])
    row[np.argmax(np.abs(row))] = 3.0 * np.abs(big).max()
    bb["x"][5] = q.f64_to_bf16_bits(row)
    return (T, H, E, k, I), a, bb, targets


def test_context_swap_of_the_outputs():
    (T, H, E, k, I), da, db, tg = _swap_batches()
    print_case("context_swap_outputs", T=T, H=H, E=E, k=k, I=I, targets=tg.tolist())
    ra, rb = _gpu(da, T, H, E, k, I, True), _gpu(db, T, H, E, k, I, True)
    ma, mb = ra[0]["row_map"].cpu().numpy()[tg], rb[0]["row_map"].cpu().numpy()[tg]
    # the targets' rows moved (other offsets / tile positions)
    assert not np.array_equal(ma, mb)
    for key in ("codes", "scales"):
        assert np.array_equal(u8(ra[0][key])[ma.reshape(-1)], u8(rb[0][key])[mb.reshape(-1)]), key
    assert np.array_equal(f32_bits(ra[0]["outer"])[ma.reshape(-1)], f32_bits(rb[0]["outer"])[mb.reshape(-1)])
    fa, fb = ra[1], rb[1]
    rows_a, rows_b = torch.from_numpy(ma.reshape(-1)).long().cuda(), torch.from_numpy(mb.reshape(-1)).long().cuda()
    for key in ("fc1_f32", "h", "a", "a_codes", "a_scales", "a_outer"):
        assert torch.equal(fa[key][rows_a], fb[key][rows_b]), key
    ti = torch.from_numpy(tg).long().cuda()
    assert torch.equal(fa["y"][ti], fb["y"][ti])
    assert torch.equal(ra[2]["dx"][ti], rb[2]["dx"][ti])
    # negative control: one outer scale per tensor
    na = _gpu(da, T, H, E, k, I, False, domain_rows=T)
    nb = _gpu(db, T, H, E, k, I, False, domain_rows=T)
    changed = [not torch.equal(na[1]["y"][int(t)], nb[1]["y"][int(t)]) for t in tg]
    print(f"[case] per-tensor control: y of {sum(changed)} of {len(tg)} targets changed", flush=True)
    assert all(changed)
