"""GPU parity of the grouped expert forward and the straight-through
BF16 backward against the FP64 oracle.

Bars: FC1 pre-cast values rel-L2 <= 1e-5 (bit-exact on lossless inputs);
<= 0.1 % of the requantised FC2-input codes differ; y rel-L2 <= 2e-3;
dX, dW1, dW2 rel-L2 <= 1e-2 each; codes, scales, outer scales and the
permutation bit-exact.
"""
import numpy as np
import pytest

from oracle import moe, nvfp4 as q
from precision_rl_amd import synth
from gpu_util import bf16_dev, bf16_host, u8, f32_bits, rel_l2, print_case

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

FC1_TOL = 1e-5
Y_TOL = 2e-3
CODE_FLIP_BUDGET = 1e-3
BWD_TOL = 1e-2


def _binding():
    from precision_rl_amd import binding
    return binding


class Run:
    """One GPU forward (+ optional backward) of a workload through the C ABI."""

    def __init__(self, d, T, H, E, k, I, A=1, backward=False):
        b = _binding()
        self.d, self.T, self.H, self.E, self.k, self.I, self.A = d, T, H, E, k, I, A
        self.x = bf16_dev(d["x"], torch)
        self.idx = torch.from_numpy(d["topk_idx"]).cuda()
        self.p = torch.from_numpy(d["topk_w"]).cuda()
        self.w1 = bf16_dev(d["w1"], torch)
        self.w2 = bf16_dev(d["w2"], torch)
        self.w1q = b.quantize_weights(self.w1)
        self.w2q = b.quantize_weights(self.w2)
        self.xq = b.w4a4_quantize_permute(self.x, self.idx, E, A)
        self.f = b.w4a4_grouped_expert_fwd(self.xq, self.p, self.w1q, self.w2q, T, H, I, E, k, A,
                                           save=True, debug=True)
        if backward:
            self.dy = bf16_dev(d["dy"], torch)
            self.g = b.w4a4_expert_bwd(self.dy, self.x, self.w1, self.w2, self.f["h"], self.f["a"],
                                       self.p, self.xq, T, H, I, E, k, A)
        torch.cuda.synchronize()
        self.rows = int(self.xq["offsets"][-1].item())


def _oracle_fwd(d, E, A):
    x = q.bf16_bits_to_f64(d["x"])
    w1q = moe.quantize_weights(q.bf16_bits_to_f64(d["w1"]))
    w2q = moe.quantize_weights(q.bf16_bits_to_f64(d["w2"]))
    return moe.forward(x, d["topk_idx"], d["topk_w"], w1q, w2q, E, A), w1q, w2q


def _check_forward(run, ref):
    rows = run.rows
    live = ref["xq"]["src_row"] >= 0
    # permutation and activation encoding: bit-exact
    assert np.array_equal(run.xq["row_map"].cpu().numpy(), ref["xq"]["row_map"])
    assert np.array_equal(u8(run.xq["codes"])[:rows], ref["xq"]["packed"])
    # FC1 pre-cast values
    fc1 = run.f["fc1_f32"].cpu().numpy()[:rows]
    e1 = rel_l2(fc1[live], ref["h64"][live])
    assert e1 <= FC1_TOL, e1
    # pad rows are zeros
    assert not fc1[~live].any()
    # FC2-input codes
    gc = q.unpack_codes(u8(run.f["a_codes"])[:rows])[live]
    flips = np.mean(gc != ref["a_codes"][live])
    assert flips <= CODE_FLIP_BUDGET, flips
    # final output
    y = bf16_host(run.f["y"])
    ey = rel_l2(y, ref["y"])
    assert ey <= Y_TOL, ey
    return e1, flips, ey


@pytest.mark.parametrize("A", [1, 16])
def test_forward_tiny(A):
    w = synth.WORKLOADS["tiny"]
    d = synth.workload_inputs("tiny")
    print_case("forward_tiny", T=w.T, H=w.H, E=w.E, k=w.k, I=w.I, A=A)
    run = Run(d, w.T, w.H, w.E, w.k, w.I, A)
    ref, _, _ = _oracle_fwd(d, w.E, A)
    print(_check_forward(run, ref))


def test_forward_ragged_empty_multi_tile():
    """Skewed routing, empty experts, groups spanning several 256-row tiles
    with ragged tails, several N tiles, row_align 32."""
    T, H, E, k, I = 1200, 512, 12, 4, 256
    d = synth.make_inputs(T, H, E, k, I, routing="zipf", seed=91, n_empty=3)
    empty = set(range(E)) - set(np.unique(d["topk_idx"]))
    print_case("forward_ragged", T=T, H=H, E=E, k=k, I=I, empty=len(empty))
    run = Run(d, T, H, E, k, I, A=32)
    ref, _, _ = _oracle_fwd(d, E, 32)
    print(_check_forward(run, ref))


def test_forward_lossless_fc1_bit_exact():
    """Inputs NVFP4 encodes exactly (g = 2^j, elements g d c): the FC1 sums
    are exact in FP32 in any order, so the GPU's pre-cast FC1 values must equal
    the oracle's bit for bit."""
    rng = np.random.default_rng(17)
    T, H, E, k, I = 96, 256, 4, 2, 128

    def lossless(R, K, gexp):
        out = np.zeros((R, K))
        for r in range(R):
            g = 2.0 ** gexp[r]
            for bk in range(K // 16):
                dd = 448.0 * 2.0 ** -int(rng.integers(0, 3)) if bk else 448.0
                c = rng.choice(q.E2M1_MAGNITUDES, 16) * rng.choice([-1, 1], 16)
                c[0] = 6.0
                out[r, bk * 16:(bk + 1) * 16] = g * dd * c
        return out

    x = lossless(T, H, rng.integers(-14, -10, T))
    w1 = lossless(E * 2 * I, H, rng.integers(-14, -10, E * 2 * I)).reshape(E, 2 * I, H)
    d = synth.make_inputs(T, H, E, k, I, seed=3)
    d["x"] = q.f64_to_bf16_bits(x)
    d["w1"] = q.f64_to_bf16_bits(w1)
    assert np.array_equal(q.bf16_bits_to_f64(d["x"]), x)
    print_case("forward_lossless", T=T, H=H, E=E, k=k, I=I)
    run = Run(d, T, H, E, k, I)
    ref, _, _ = _oracle_fwd(d, E, 1)
    rows = run.rows
    fc1 = run.f["fc1_f32"].cpu().numpy()[:rows].astype(np.float64)
    assert np.array_equal(fc1, ref["h64"]), np.abs(fc1 - ref["h64"]).max()


def test_forward_deterministic():
    T, H, E, k, I = 256, 512, 8, 2, 256
    d = synth.make_inputs(T, H, E, k, I, seed=8)
    print_case("forward_determinism", T=T, H=H, E=E, k=k, I=I)
    r1 = Run(d, T, H, E, k, I)
    r2 = Run(d, T, H, E, k, I)
    for key in ("y", "h", "a", "fc1_f32", "a_codes"):
        assert torch.equal(r1.f[key], r2.f[key]), key


# ------------------------------------------------------------------ backward
def _oracle_bwd(d, E, A, ref_fwd):
    x = q.bf16_bits_to_f64(d["x"])
    w1 = q.bf16_bits_to_f64(d["w1"])
    w2 = q.bf16_bits_to_f64(d["w2"])
    dy = q.bf16_bits_to_f64(d["dy"])
    xq = ref_fwd["xq"]
    return moe.backward(dy, x, w1, w2, ref_fwd["h"], ref_fwd["a"], d["topk_w"], xq["offsets"],
                        xq["row_map"], xq["src_row"])


def _check_backward(run, ref_b):
    dx = bf16_host(run.g["dx"])
    dw1 = bf16_host(run.g["dw1"])
    dw2 = bf16_host(run.g["dw2"])
    errs = (rel_l2(dx, ref_b["dX"]), rel_l2(dw1, ref_b["dW1"]), rel_l2(dw2, ref_b["dW2"]))
    assert max(errs) <= BWD_TOL, errs
    return errs


@pytest.mark.parametrize("A", [1, 16])
def test_backward_tiny(A):
    w = synth.WORKLOADS["tiny"]
    d = synth.make_inputs(w.T, w.H, w.E, w.k, w.I, backward=True, seed=1000)
    print_case("backward_tiny", T=w.T, H=w.H, E=w.E, k=w.k, I=w.I, A=A)
    run = Run(d, w.T, w.H, w.E, w.k, w.I, A, backward=True)
    ref, _, _ = _oracle_fwd(d, w.E, A)
    print(_check_backward(run, _oracle_bwd(d, w.E, A, ref)))


def test_backward_ragged_empty():
    T, H, E, k, I = 900, 512, 10, 3, 256
    d = synth.make_inputs(T, H, E, k, I, routing="zipf", backward=True, seed=55, n_empty=2)
    print_case("backward_ragged", T=T, H=H, E=E, k=k, I=I)
    run = Run(d, T, H, E, k, I, A=16, backward=True)
    ref, _, _ = _oracle_fwd(d, E, 16)
    rb = _oracle_bwd(d, E, 16, ref)
    print(_check_backward(run, rb))
    counts = np.bincount(d["topk_idx"].reshape(-1), minlength=E)
    for e in np.nonzero(counts == 0)[0]:
        assert not run.g["dw1"][e].any() and not run.g["dw2"][e].any()


def test_forward_backward_ungrouped_scales_odd_pairs():
    """I = 384: FC2's K (384) is not a multiple of 256, so its block scales
    arrive per stage with the codes (not grouped by four stages), over an odd
    number (3) of two-stage code copies; FC1 (K = 512) groups them.  The
    backward's K-contiguous operands arrive in two-stage copies as well
    (K = 512 and 768).  Forward and backward against the oracle."""
    T, H, E, k, I = 600, 512, 6, 2, 384
    d = synth.make_inputs(T, H, E, k, I, routing="zipf", backward=True, seed=384, n_empty=1)
    print_case("ungrouped_scales", T=T, H=H, E=E, k=k, I=I)
    run = Run(d, T, H, E, k, I, A=16, backward=True)
    ref, _, _ = _oracle_fwd(d, E, 16)
    print(_check_forward(run, ref))
    print(_check_backward(run, _oracle_bwd(d, E, 16, ref)))


def test_backward_skewed_split_experts():
    """Few experts of very different sizes: the wgrad schedule deals the
    tiles of the costly experts in chunks (their tiles, run whole on one
    XCD's workgroups in rounds, would take longer than an even share) and
    those of the cheapest expert whole.  Every expert's dW1 and dW2, and dX,
    against the oracle."""
    T, H, E, k, I = 4096, 1024, 4, 1, 512
    d = synth.make_inputs(T, H, E, k, I, routing="zipf", backward=True, seed=303, n_empty=0)
    counts = np.bincount(d["topk_idx"].reshape(-1), minlength=E)
    # wgrad FC1: 4 x 4 tiles per expert and a grid of 64 workgroups (8 per
    # XCD), so an expert runs whole in two rounds or in two chunks of 8;
    # wgrad FC2: 4 x 2 tiles, 32 workgroups, the same split
    cost = (counts + 31) // 32 + 2
    split = 2 * cost > 16 * cost.sum() // 64
    assert split.any() and not split.all(), (counts, cost)
    print_case("backward_split", T=T, H=H, E=E, k=k, I=I, counts=counts.tolist())
    run = Run(d, T, H, E, k, I, backward=True)
    ref, _, _ = _oracle_fwd(d, E, 1)
    rb = _oracle_bwd(d, E, 1, ref)
    print(_check_backward(run, rb))
    dw1, dw2 = bf16_host(run.g["dw1"]), bf16_host(run.g["dw2"])
    for e in range(E):
        assert rel_l2(dw1[e], rb["dW1"][e]) <= BWD_TOL, e
        assert rel_l2(dw2[e], rb["dW2"][e]) <= BWD_TOL, e


def test_backward_concurrent_calls_on_two_streams():
    """Two host threads run the backward at the same time on two streams with
    their own workspaces (the library's second stream is shared; each thread
    forks and joins with events of its own, with no common lock around the
    enqueue).  Each result equals the sequential one
    bit for bit; the second thread's dy is 2 dy, so its results are exactly
    twice the first's (a power-of-two scale commutes with every rounding)."""
    import threading
    b = _binding()
    T, H, E, k, I = 1500, 512, 12, 4, 256
    d = synth.make_inputs(T, H, E, k, I, routing="zipf", backward=True, seed=77, n_empty=2)
    print_case("backward_two_streams", T=T, H=H, E=E, k=k, I=I)
    run = Run(d, T, H, E, k, I, A=16, backward=True)
    ref = {n: v.clone() for n, v in run.g.items()}
    dys = [run.dy, run.dy * 2]
    torch.cuda.synchronize()   # inputs and the reference complete before the side streams start
    outs = [[], []]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    outs[i].append(b.w4a4_expert_bwd(dys[i], run.x, run.w1, run.w2, run.f["h"], run.f["a"],
                                                     run.p, run.xq, T, H, I, E, k, 16))
            s.synchronize()
        except Exception as e:   # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, scale in ((0, 1.0), (1, 2.0)):
        for g in outs[i]:
            for n in ("dx", "dw1", "dw2"):
                assert torch.equal(g[n], ref[n] * scale), (i, n)


def test_graph_capture_of_a_learner_step():
    """quantize+permute, forward and backward captured in one HIP graph (the
    backward's second stream joins the capture through its fork / join
    events) and replayed three times with eager work between the replays:
    every replay equals the eager step bit for bit."""
    b = _binding()
    T, H, E, k, I = 700, 512, 8, 2, 256
    d = synth.make_inputs(T, H, E, k, I, routing="zipf", backward=True, seed=91, n_empty=1)
    print_case("graph_capture_step", T=T, H=H, E=E, k=k, I=I)
    x, dy = bf16_dev(d["x"], torch), bf16_dev(d["dy"], torch)
    idx, p = torch.from_numpy(d["topk_idx"]).cuda(), torch.from_numpy(d["topk_w"]).cuda()
    w1, w2 = bf16_dev(d["w1"], torch), bf16_dev(d["w2"], torch)
    w1q, w2q = b.quantize_weights(w1), b.quantize_weights(w2)

    def step():
        xq = b.w4a4_quantize_permute(x, idx, E, 16)
        f = b.w4a4_grouped_expert_fwd(xq, p, w1q, w2q, T, H, I, E, k, 16, save=True)
        g = b.w4a4_expert_bwd(dy, x, w1, w2, f["h"], f["a"], p, xq, T, H, I, E, k, 16)
        return [f["y"], g["dx"], g["dw1"], g["dw2"]]

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step()
    for i in range(3):
        noise = torch.randn(1 << 20, device="cuda") * 3.0   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        del noise
        for j, (a, e) in enumerate(zip(out, eager)):
            assert torch.equal(a, e), (i, j)


@pytest.mark.parametrize("T,H,E,k,seed", [(512, 512, 8, 4, 31), (16500, 256, 16, 8, 32)])
def test_requant_bit_exact_on_the_gpus_own_a(T, H, E, k, seed):
    """The FC2-input requantisation equals the oracle quantiser applied to
    the bf16 a the GPU itself saved, bit for bit: codes, E4M3 scales and
    FP32 outer scales of every dispatched row (the tolerance-checked
    comparison with the FP64 forward allows flips only where a itself
    differs by an ulp).  The second case has more rows (132000 plus
    padding, 32 per workgroup) than 16 workgroups per CU take in one pass,
    so the encoder's waves stride over a second row group."""
    I = 768
    d = synth.make_inputs(T, H, E, k, I, seed=seed)
    print_case("requant_bit_exact", T=T, H=H, E=E, k=k, I=I)
    run = Run(d, T, H, E, k, I, A=16)
    rows = run.rows
    a = bf16_host(run.f["a"][:rows])
    c, s, g = q.quantize_rows(a)
    assert np.array_equal(u8(run.f["a_codes"])[:rows], q.pack_codes(c))
    assert np.array_equal(u8(run.f["a_scales"])[:rows], s)
    assert np.array_equal(f32_bits(run.f["a_outer"])[:rows], g.view(np.uint32))
