"""GPU parity of the outer-scale domains wider than a token (per group of
rows, per tensor, per expert weight tensor) against the FP64 oracle.

Bars: codes, scales, outer scales and the permutation bit-exact; with these
operands the forward's FC1 pre-cast values rel-L2 <= 1e-5, FC2-input code
flips <= 0.1%, y rel-L2 <= 2e-3 (the per-token path's bars).
"""
import numpy as np
import pytest

from oracle import moe, nvfp4 as q
from precision_rl_amd import synth
from gpu_util import bf16_dev, bf16_host, u8, rel_l2, print_case

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _b():
    from precision_rl_amd import binding
    return binding


def _check_qp(got, ref, rows):
    assert np.array_equal(got["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(got["row_map"].cpu().numpy(), ref["row_map"])
    assert np.array_equal(u8(got["codes"])[:rows], ref["packed"])
    assert np.array_equal(u8(got["scales"])[:rows], ref["scales"])
    assert np.array_equal(got["outer"].cpu().numpy()[:rows].view(np.uint32), ref["outer"].view(np.uint32))


@pytest.mark.parametrize("G", ["T", 1, 100])
def test_quantize_permute_grouped_outer_scales(G):
    T, H, E, k = 2048, 2048, 128, 8
    d = synth.make_inputs(T, H, E, k, 0, x_dist="t3", seed=1001)
    G = T if G == "T" else G
    print_case("qp_domain", T=T, H=H, E=E, k=k, group_rows=G)
    x = bf16_dev(d["x"], torch)
    idx = torch.from_numpy(d["topk_idx"]).cuda()
    got = _b().w4a4_quantize_permute_domain(x, idx, E, 1, group_rows=G)
    torch.cuda.synchronize()
    ref = moe.quantize_permute(q.bf16_bits_to_f64(d["x"]), d["topk_idx"], E, 1, group_rows=G)
    _check_qp(got, ref, int(ref["offsets"][-1]))
    if G == 1:   # the per-token entry point gives the same bytes
        base = _b().w4a4_quantize_permute(x, idx, E, 1)
        torch.cuda.synchronize()
        for key in ("codes", "scales", "outer", "offsets", "row_map", "src_row"):
            assert torch.equal(got[key], base[key]), key


def test_per_expert_weight_scales():
    E, N, K = 8, 512, 768
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(61)))
    w = synth.normal_bf16(rng, (E, N, K), synth.W_STD)
    w[3] = synth.f32_to_bf16_bits(q.bf16_bits_to_f64(w[3]).astype(np.float32) * 16.0)
    print_case("per_expert_weights", E=E, N=N, K=K)
    got = _b().quantize_weights(bf16_dev(w, torch), per_expert=True)
    torch.cuda.synchronize()
    ref = moe.quantize_weights(q.bf16_bits_to_f64(w), per_expert=True)
    assert np.array_equal(u8(got["codes"]), ref["packed"])
    assert np.array_equal(u8(got["scales"]), ref["scales"])
    assert np.array_equal(got["outer"].cpu().numpy().view(np.uint32), ref["outer"].view(np.uint32))


def test_context_swap_negative_control_on_the_gpu():
    """Per-token scales: a token's codes do not change when the other tokens
    do; per-tensor scales: they do (the pages' context-swap check and its
    negative control), on the GPU's own outputs."""
    T, H, E, k = 512, 1024, 16, 4
    d = synth.make_inputs(T, H, E, k, 0, seed=1002)
    x = bf16_dev(d["x"], torch)
    x2 = x.clone()
    x2[1:] *= 64.0
    idx = torch.from_numpy(d["topk_idx"]).cuda()
    print_case("context_swap", T=T, H=H, E=E, k=k)
    rows0 = idx.new_tensor(0)
    out = {}
    for G in (1, T):
        a = _b().w4a4_quantize_permute_domain(x, idx, E, 1, group_rows=G)
        b = _b().w4a4_quantize_permute_domain(x2, idx, E, 1, group_rows=G)
        torch.cuda.synchronize()
        r = a["row_map"][rows0].long()
        out[G] = torch.equal(a["codes"][r], b["codes"][r]) and torch.equal(a["outer"][r], b["outer"][r])
    assert out[1] and not out[T]


def test_forward_with_per_tensor_activations_and_per_expert_weights():
    T, H, E, k, I = 600, 512, 10, 3, 256
    d = synth.make_inputs(T, H, E, k, I, routing="zipf", seed=1003, n_empty=2)
    print_case("fwd_domains", T=T, H=H, E=E, k=k, I=I)
    b = _b()
    x = bf16_dev(d["x"], torch)
    idx = torch.from_numpy(d["topk_idx"]).cuda()
    p = torch.from_numpy(d["topk_w"]).cuda()
    w1q = b.quantize_weights(bf16_dev(d["w1"], torch), per_expert=True)
    w2q = b.quantize_weights(bf16_dev(d["w2"], torch), per_expert=True)
    xq = b.w4a4_quantize_permute_domain(x, idx, E, 1, group_rows=T)
    f = b.w4a4_grouped_expert_fwd(xq, p, w1q, w2q, T, H, I, E, k, 1, save=True, debug=True)
    torch.cuda.synchronize()
    W1 = moe.quantize_weights(q.bf16_bits_to_f64(d["w1"]), per_expert=True)
    W2 = moe.quantize_weights(q.bf16_bits_to_f64(d["w2"]), per_expert=True)
    ref = moe.forward(q.bf16_bits_to_f64(d["x"]), d["topk_idx"], d["topk_w"], W1, W2, E, 1,
                      act_group_rows=T)
    rows = int(ref["xq"]["offsets"][-1])
    live = ref["xq"]["src_row"] >= 0
    assert np.array_equal(u8(xq["codes"])[:rows], ref["xq"]["packed"])
    fc1 = f["fc1_f32"].cpu().numpy()[:rows]
    assert rel_l2(fc1[live], ref["h64"][live]) <= 1e-5
    gc = q.unpack_codes(u8(f["a_codes"])[:rows])[live]
    assert np.mean(gc != ref["a_codes"][live]) <= 1e-3
    assert rel_l2(bf16_host(f["y"]), ref["y"]) <= 2e-3
