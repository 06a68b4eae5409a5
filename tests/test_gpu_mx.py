"""GPU parity of the MXFP4 recipe (E2M1 + E8M0 per 32, scaled FP4 MFMA)
against the FP64 oracle, through the C ABI.

Bars (the NVFP4 path's, applied to this recipe): codes, E8M0 scales and the
permutation bit-exact; FC1 pre-cast values rel-L2 <= 1e-5 (bit-exact on
lossless inputs); <= 0.1 % of the requantised FC2-input codes differ; y
rel-L2 <= 2e-3; the straight-through backward on the MXFP4 forward's saved
h and a within rel-L2 1e-2.
"""
import numpy as np
import pytest

from oracle import moe, mxfp4 as mx, nvfp4 as q
from precision_rl_amd import synth
from gpu_util import bf16_dev, bf16_host, u8, rel_l2, print_case

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

FC1_TOL = 1e-5
Y_TOL = 2e-3
CODE_FLIP_BUDGET = 1e-3
BWD_TOL = 1e-2


def _b():
    from precision_rl_amd import binding
    return binding


class MxRun:
    def __init__(self, d, T, H, E, k, I, A=1, backward=False):
        b = _b()
        self.x = bf16_dev(d["x"], torch)
        self.idx = torch.from_numpy(d["topk_idx"]).cuda()
        self.p = torch.from_numpy(d["topk_w"]).cuda()
        self.w1 = bf16_dev(d["w1"], torch)
        self.w2 = bf16_dev(d["w2"], torch)
        self.w1q = b.quantize_weights_mx(self.w1)
        self.w2q = b.quantize_weights_mx(self.w2)
        self.xq = b.w4a4_mx_quantize_permute(self.x, self.idx, E, A)
        self.f = b.w4a4_mx_grouped_expert_fwd(self.xq, self.p, self.w1q, self.w2q, T, H, I, E, k, A,
                                              save=True, debug=True)
        if backward:
            self.dy = bf16_dev(d["dy"], torch)
            # the NVFP4 call's straight-through backward: it reads only the saved bf16 operands
            self.g = b.w4a4_expert_bwd(self.dy, self.x, self.w1, self.w2, self.f["h"], self.f["a"],
                                       self.p, self.xq, T, H, I, E, k, A)
        torch.cuda.synchronize()
        self.rows = int(self.xq["offsets"][-1].item())


def _oracle(d, E, A):
    x = q.bf16_bits_to_f64(d["x"])
    w1q = moe.quantize_weights_mx(q.bf16_bits_to_f64(d["w1"]))
    w2q = moe.quantize_weights_mx(q.bf16_bits_to_f64(d["w2"]))
    return moe.forward_mx(x, d["topk_idx"], d["topk_w"], w1q, w2q, E, A), w1q, w2q


def _check(run, ref, w1q=None, w2q=None):
    rows = run.rows
    xr = ref["xq"]
    live = xr["src_row"] >= 0
    assert np.array_equal(run.xq["offsets"].cpu().numpy(), xr["offsets"])
    assert np.array_equal(run.xq["row_map"].cpu().numpy(), xr["row_map"])
    assert np.array_equal(run.xq["src_row"].cpu().numpy()[:rows], xr["src_row"])
    assert np.array_equal(u8(run.xq["codes"])[:rows], xr["packed"])
    assert np.array_equal(u8(run.xq["scales"])[:rows], xr["scales"])
    if w1q is not None:
        assert np.array_equal(u8(run.w1q["codes"]), w1q["packed"])
        assert np.array_equal(u8(run.w1q["scales"]), w1q["scales"])
        assert np.array_equal(u8(run.w2q["codes"]), w2q["packed"])
        assert np.array_equal(u8(run.w2q["scales"]), w2q["scales"])
    fc1 = run.f["fc1_f32"].cpu().numpy()[:rows]
    e1 = rel_l2(fc1[live], ref["h64"][live])
    assert e1 <= FC1_TOL, e1
    assert not fc1[~live].any()
    gc = q.unpack_codes(u8(run.f["a_codes"])[:rows])[live]
    flips = float(np.mean(gc != ref["a_codes"][live]))
    assert flips <= CODE_FLIP_BUDGET, flips
    sflips = float(np.mean(u8(run.f["a_scales"])[:rows][live] != ref["a_scales"][live]))
    assert sflips <= CODE_FLIP_BUDGET, sflips
    ey = rel_l2(bf16_host(run.f["y"]), ref["y"])
    assert ey <= Y_TOL, ey
    return e1, flips, ey


@pytest.mark.parametrize("A", [1, 16])
def test_mx_quantize_permute_student_t(A):
    """Heavy-tailed tokens (Student-t, nu = 3) at a reduced quantize+permute
    shape with several routing chunks and a ragged last chunk."""
    T, H, E, k = 1000, 2048, 32, 8
    d = synth.make_inputs(T, H, E, k, 0, x_dist="t3", seed=77, weights=False)
    print_case("mx_quantize_permute", T=T, H=H, E=E, k=k, A=A)
    x = bf16_dev(d["x"], torch)
    got = _b().w4a4_mx_quantize_permute(x, torch.from_numpy(d["topk_idx"]).cuda(), E, A)
    torch.cuda.synchronize()
    ref = moe.quantize_permute_mx(q.bf16_bits_to_f64(d["x"]), d["topk_idx"], E, A)
    rows = int(ref["offsets"][-1])
    assert np.array_equal(got["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(got["row_map"].cpu().numpy(), ref["row_map"])
    assert np.array_equal(got["src_row"].cpu().numpy()[:rows], ref["src_row"])
    assert np.array_equal(u8(got["codes"])[:rows], ref["packed"])
    assert np.array_equal(u8(got["scales"])[:rows], ref["scales"])


def test_mx_quantize_edge_rows():
    """Zero rows, -0, subnormal and huge blocks (scale bytes 0 and 252), and
    blocks of E2M1 midpoints times 2^X with their bf16 neighbours (exact ties
    of x / 2^X) for X from the subnormal clamp to the top of the range;
    identity routing."""
    rng = np.random.default_rng(5)
    v = rng.standard_normal((12, 256))
    v[0] = 0.0
    v[1, :] = -0.0
    v[2, :32] = 2.0 ** -133
    v[3, 32:64] *= 2.0 ** 126
    v[4, 64:96] *= 2.0 ** -120
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    xs = [-127, -126, -125, -100, -9, -2, 0, 3, 50, 100, 124, 125, -60, 7, -1, 1,
          20, -20, 64, -64, 110, -110, 90, -90, 30, -30, 11, -11, 2, -3, 5, -5]
    for blk, X in enumerate(xs):
        r, c0 = 5 + blk // 8, 32 * (blk % 8)
        t = mids * 2.0 ** X
        b = q.f64_to_bf16_bits(t).astype(np.int64)
        nb = np.concatenate([b - 1, b, b + 1])
        vals = q.bf16_bits_to_f64(nb[(nb > 0) & (nb < 0x7F80)].astype(np.uint16))
        vals = vals[np.abs(vals) < 6.0 * 2.0 ** X][:31]
        row = np.zeros(32)
        row[:len(vals)] = vals * rng.choice([-1.0, 1.0], len(vals))
        row[31] = 4.0 * 2.0 ** X * rng.choice([-1.0, 1.0])   # block max: 2^(X+2) sets the scale to 2^X
        v[r, c0:c0 + 32] = rng.permutation(row)
    bits = q.f64_to_bf16_bits(v)
    x = bf16_dev(bits, torch)
    print_case("mx_quantize_edges", rows=v.shape[0], K=256)
    got = _b().w4a4_mx_quantize_permute(x, None, 1)
    torch.cuda.synchronize()
    c, s = mx.quantize_rows_mx(q.bf16_bits_to_f64(bits))
    assert np.array_equal(u8(got["codes"]), q.pack_codes(c))
    assert np.array_equal(u8(got["scales"]), s)


@pytest.mark.parametrize("A", [1, 16])
def test_mx_forward_tiny(A):
    w = synth.WORKLOADS["tiny"]
    d = synth.workload_inputs("tiny")
    print_case("mx_forward_tiny", T=w.T, H=w.H, E=w.E, k=w.k, I=w.I, A=A)
    run = MxRun(d, w.T, w.H, w.E, w.k, w.I, A)
    ref, w1q, w2q = _oracle(d, w.E, A)
    print(_check(run, ref, w1q, w2q))


def test_mx_forward_ragged_empty_multi_tile():
    """Skewed routing, empty experts, groups spanning several 128-row tiles
    with ragged tails, several N tiles, row_align 32."""
    T, H, E, k, I = 1200, 512, 12, 4, 256
    d = synth.make_inputs(T, H, E, k, I, routing="zipf", seed=91, n_empty=3)
    print_case("mx_forward_ragged", T=T, H=H, E=E, k=k, I=I)
    run = MxRun(d, T, H, E, k, I, A=32)
    ref, w1q, w2q = _oracle(d, E, 32)
    print(_check(run, ref, w1q, w2q))


def test_mx_forward_lossless_fc1_bit_exact():
    """Inputs MXFP4 encodes exactly (each block: E2M1 magnitudes times 2^X,
    X in [-2, 0], one element at 6 * 2^X), so every FC1 sum is exact in FP32
    in any order: the GPU's pre-cast FC1 equals the oracle bit for bit."""
    rng = np.random.default_rng(23)
    T, H, E, k, I = 96, 256, 4, 2, 128

    def lossless(R, K):
        c = rng.choice(q.E2M1_MAGNITUDES, (R, K // 32, 32)) * rng.choice([-1.0, 1.0], (R, K // 32, 32))
        c[:, :, 0] = 6.0
        X = rng.integers(-2, 1, (R, K // 32, 1))
        return np.ldexp(c, X).reshape(R, K)

    d = synth.make_inputs(T, H, E, k, I, seed=23)
    d["x"] = q.f64_to_bf16_bits(lossless(T, H))
    d["w1"] = q.f64_to_bf16_bits(lossless(E * 2 * I, H).reshape(E, 2 * I, H))
    print_case("mx_forward_lossless", T=T, H=H, E=E, k=k, I=I)
    run = MxRun(d, T, H, E, k, I)
    ref, _, _ = _oracle(d, E, 1)
    rows = run.rows
    fc1 = run.f["fc1_f32"].cpu().numpy()[:rows].astype(np.float64)
    assert np.array_equal(fc1, ref["h64"])


def test_mx_learner_step_tiny_backward():
    """MXFP4 forward with h and a saved, then the straight-through BF16
    backward on them (the backward is the recipe-independent call)."""
    w = synth.WORKLOADS["tiny"]
    d = synth.make_inputs(w.T, w.H, w.E, w.k, w.I, backward=True, seed=1000)
    print_case("mx_learner_tiny", T=w.T, H=w.H, E=w.E, k=w.k, I=w.I)
    run = MxRun(d, w.T, w.H, w.E, w.k, w.I, backward=True)
    ref, _, _ = _oracle(d, w.E, 1)
    _check(run, ref)
    xr = ref["xq"]
    rb = moe.backward(q.bf16_bits_to_f64(d["dy"]), q.bf16_bits_to_f64(d["x"]),
                      q.bf16_bits_to_f64(d["w1"]), q.bf16_bits_to_f64(d["w2"]), ref["h"], ref["a"],
                      d["topk_w"], xr["offsets"], xr["row_map"], xr["src_row"])
    errs = (rel_l2(bf16_host(run.g["dx"]), rb["dX"]), rel_l2(bf16_host(run.g["dw1"]), rb["dW1"]),
            rel_l2(bf16_host(run.g["dw2"]), rb["dW2"]))
    assert max(errs) <= BWD_TOL, errs


def test_mx_forward_deterministic():
    T, H, E, k, I = 256, 512, 8, 2, 256
    d = synth.make_inputs(T, H, E, k, I, seed=8)
    print_case("mx_forward_determinism", T=T, H=H, E=E, k=k, I=I)
    r1 = MxRun(d, T, H, E, k, I)
    r2 = MxRun(d, T, H, E, k, I)
    for key in ("y", "h", "a", "fc1_f32", "a_codes", "a_scales"):
        assert torch.equal(r1.f[key], r2.f[key]), key


def test_mx_forward_full_workload_sampled():
    """The forward workload at full size (T=8192, H=2048, E=128, k=8, I=768):
    sampled tokens against the oracle run on those tokens alone (a token's
    outputs depend on its own row only)."""
    w = synth.WORKLOADS["fwd"]
    d = synth.workload_inputs("fwd")
    print_case("mx_forward_full_sampled", T=w.T, H=w.H, E=w.E, k=w.k, I=w.I)
    run = MxRun(d, w.T, w.H, w.E, w.k, w.I)
    sample = np.array([0, 1, 4097, w.T - 1])
    experts = np.unique(d["topk_idx"][sample])
    remap = -np.ones(w.E, dtype=np.int64)
    remap[experts] = np.arange(experts.size)
    sub = dict(x=d["x"][sample], topk_idx=remap[d["topk_idx"][sample]].astype(np.int32),
               topk_w=d["topk_w"][sample], w1=d["w1"][experts], w2=d["w2"][experts])
    ref, w1q, w2q = _oracle(sub, experts.size, 1)
    assert np.array_equal(u8(run.w1q["codes"])[experts], w1q["packed"])
    assert np.array_equal(u8(run.w1q["scales"])[experts], w1q["scales"])
    assert np.array_equal(u8(run.w2q["scales"])[experts], w2q["scales"])
    rows_gpu = run.xq["row_map"].cpu().numpy()[sample].reshape(-1)
    rows_ref = ref["xq"]["row_map"].reshape(-1)
    assert np.array_equal(u8(run.xq["codes"])[rows_gpu], ref["xq"]["packed"][rows_ref])
    fc1 = run.f["fc1_f32"].cpu().numpy()[rows_gpu]
    assert rel_l2(fc1, ref["h64"][rows_ref]) <= FC1_TOL
    gc = q.unpack_codes(u8(run.f["a_codes"])[rows_gpu])
    assert np.mean(gc != ref["a_codes"][rows_ref]) <= CODE_FLIP_BUDGET
    y = bf16_host(run.f["y"])[sample]
    assert rel_l2(y, ref["y"]) <= Y_TOL


def test_mx_forward_full_skew_sampled():
    """Skewed workload at full size (T=32768, H=2048, E=128, k=8, I=768;
    Zipf(1.2) popularity, 10 experts without tokens) in the MXFP4 recipe:
    the permutation bit-exact against the oracle's routing of all tokens;
    the encodings and forward outputs of sampled tokens (the first and last
    rows of the most and least popular experts) against the oracle on those
    tokens alone."""
    w = synth.WORKLOADS["skew"]
    d = synth.make_inputs(w.T, w.H, w.E, w.k, w.I, w.routing, w.x_dist, seed=1000 + w.index)
    print_case("mx_skew_full_sampled", T=w.T, H=w.H, E=w.E, k=w.k, I=w.I)
    run = MxRun(d, w.T, w.H, w.E, w.k, w.I)
    offsets, row_map, src_row = moe.route_fast(d["topk_idx"], w.E, 1)
    assert np.array_equal(run.xq["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(run.xq["row_map"].cpu().numpy(), row_map)
    counts = np.diff(offsets)
    assert (counts == 0).sum() == 10
    big = int(np.argmax(counts))
    small = int(np.argmin(np.where(counts > 0, counts, counts.max() + 1)))
    picks = [src_row[offsets[big]], src_row[offsets[big + 1] - 1], src_row[offsets[small]],
             src_row[offsets[small + 1] - 1], 0, w.T - 1]
    sample = np.unique(np.array(picks))
    experts = np.unique(d["topk_idx"][sample])
    remap = -np.ones(w.E, dtype=np.int64)
    remap[experts] = np.arange(experts.size)
    sub = dict(x=d["x"][sample], topk_idx=remap[d["topk_idx"][sample]].astype(np.int32),
               topk_w=d["topk_w"][sample], w1=d["w1"][experts], w2=d["w2"][experts])
    ref, _, _ = _oracle(sub, experts.size, 1)
    rows_gpu = row_map[sample].reshape(-1)
    rows_ref = ref["xq"]["row_map"].reshape(-1)
    assert np.array_equal(u8(run.xq["codes"])[rows_gpu], ref["xq"]["packed"][rows_ref])
    assert np.array_equal(u8(run.xq["scales"])[rows_gpu], ref["xq"]["scales"][rows_ref])
    fc1 = run.f["fc1_f32"].cpu().numpy()[rows_gpu]
    assert rel_l2(fc1, ref["h64"][rows_ref]) <= FC1_TOL
    gc = q.unpack_codes(u8(run.f["a_codes"])[rows_gpu])
    assert np.mean(gc != ref["a_codes"][rows_ref]) <= CODE_FLIP_BUDGET
    assert rel_l2(bf16_host(run.f["y"])[sample], ref["y"]) <= Y_TOL


@pytest.mark.parametrize("T,H,E,k,seed", [(512, 512, 8, 4, 31), (16500, 256, 16, 8, 32)])
def test_mx_requant_bit_exact_on_the_gpus_own_a(T, H, E, k, seed):
    """The MXFP4 FC2-input requantisation equals the oracle's MXFP4 of the
    bf16 a the GPU saved, bit for bit (codes and E8M0 scales).  The second
    case has more rows than 16 workgroups per CU take in one pass, so the
    encoder's waves stride over a second row group."""
    I = 768
    d = synth.make_inputs(T, H, E, k, I, seed=seed)
    print_case("mx_requant_bit_exact", T=T, H=H, E=E, k=k, I=I)
    run = MxRun(d, T, H, E, k, I, A=16)
    rows = run.rows
    a = bf16_host(run.f["a"][:rows])
    c, s = mx.quantize_rows_mx(a)
    assert np.array_equal(u8(run.f["a_codes"])[:rows], q.pack_codes(c))
    assert np.array_equal(u8(run.f["a_scales"])[:rows], s)
