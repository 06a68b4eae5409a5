"""GPU parity of the dense per-token NVFP4 linear layer (forward and
straight-through BF16 backward) against the FP64 oracle.

Bars: codes, scales and outer scales bit-exact; y rel-L2 <= 2e-3 (the MoE
output bar) with at least 99.9% of the BF16 outputs bit-identical (the rest
differ by FP32 versus FP64 accumulation order at a rounding boundary);
dX, dW rel-L2 <= 1e-2 each.
"""
import numpy as np
import pytest

from oracle import linear, nvfp4 as q
from gpu_util import bf16_dev, bf16_host, u8, rel_l2, print_case

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

Y_TOL = 2e-3
Y_SAME = 0.999
BWD_TOL = 1e-2


def _inputs(T, K, N, seed):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    x = q.f64_to_bf16_bits(rng.standard_normal((T, K)))
    w = q.f64_to_bf16_bits(0.02 * rng.standard_normal((N, K)))
    dy = q.f64_to_bf16_bits(rng.standard_normal((T, N)))
    return x, w, dy


def _run(x, w, dy, T, K, N, backward=True):
    from precision_rl_amd import binding as b
    X, W = bf16_dev(x, torch), bf16_dev(w, torch)
    xq = b.w4a4_quantize_permute(X, None, 1)
    wq = b.w4a4_quantize_permute(W, None, 1)
    y = b.w4a4_linear_fwd(xq, wq, T, K, N)
    g = b.w4a4_linear_bwd(bf16_dev(dy, torch), X, W, xq, T, K, N) if backward else None
    torch.cuda.synchronize()
    return xq, wq, y, g


def _check_y(y, ref_y):
    same = np.mean(y == ref_y)
    e = rel_l2(y, ref_y)
    assert e <= Y_TOL and same >= Y_SAME, (e, same)
    return e, same


# (4096, 256, 256) and (2500, 512, 512): one group with fewer weight-gradient
# tiles than CUs, split over K (4 and 2 pieces, the last one ragged)
@pytest.mark.parametrize("T,K,N", [(300, 512, 768), (1, 256, 256), (1000, 1024, 512),
                                   (4096, 256, 256), (2500, 512, 512)])
def test_linear_small(T, K, N):
    x, w, dy = _inputs(T, K, N, 500 + T)
    print_case("linear_small", T=T, K=K, N=N)
    xq, wq, y, g = _run(x, w, dy, T, K, N)
    xf, wf, dyf = (q.bf16_bits_to_f64(v) for v in (x, w, dy))
    ref = linear.forward(xf, wf)
    assert np.array_equal(u8(xq["codes"]), q.pack_codes(ref["xq"][0]))
    assert np.array_equal(u8(xq["scales"]), ref["xq"][1])
    assert np.array_equal(xq["outer"].cpu().numpy(), ref["xq"][2])
    assert np.array_equal(u8(wq["codes"]), q.pack_codes(ref["wq"][0]))
    print("y", _check_y(bf16_host(y), ref["y"]))
    rb = linear.backward(dyf, xf, wf)
    dx, dw = bf16_host(g["dx"]), bf16_host(g["dw"])
    errs = (rel_l2(dx, rb["dX"]), rel_l2(dw, rb["dW"]))
    assert max(errs) <= BWD_TOL, errs
    print("bwd", errs)


@pytest.mark.parametrize("T,K,N", [(700, 512, 512), (4096, 256, 256)])
def test_linear_backward_deterministic_and_empty(T, K, N):
    """Two backward calls give bit-identical results (the weight-gradient
    tiles are taken dynamically; with a K split, the pieces are summed in a
    fixed order); with T = 0 dW is all zeros."""
    from precision_rl_amd import binding as b
    x, w, dy = _inputs(T, K, N, 77)
    print_case("linear_determinism", T=T, K=K, N=N)
    _, _, _, g1 = _run(x, w, dy, T, K, N)
    _, _, _, g2 = _run(x, w, dy, T, K, N)
    assert torch.equal(g1["dx"], g2["dx"]) and torch.equal(g1["dw"], g2["dw"])
    W = bf16_dev(w, torch)
    X0 = torch.empty(0, K, dtype=torch.bfloat16, device="cuda")
    xq0 = b.w4a4_quantize_permute(X0, None, 1)
    dw = torch.full((N, K), 7.0, dtype=torch.bfloat16, device="cuda")
    out = dict(dx=torch.empty(0, K, dtype=torch.bfloat16, device="cuda"), dw=dw)
    b.w4a4_linear_bwd(torch.empty(0, N, dtype=torch.bfloat16, device="cuda"), X0, W, xq0, 0, K, N,
                      out=out)
    torch.cuda.synchronize()
    assert not dw.float().any()


def test_linear_full_projection_sampled():
    """A Qwen3-30B-A3B query projection at the learner batch (T=16384,
    K=2048, N=4096): y and dX of sampled tokens against the oracle on those
    rows (rows are independent), dW of sampled entries against float64 dot
    products over all tokens."""
    T, K, N = 16384, 2048, 4096
    x, w, dy = _inputs(T, K, N, 4242)
    print_case("linear_full_sampled", T=T, K=K, N=N)
    _, _, y, g = _run(x, w, dy, T, K, N)
    sample = np.array([0, 1, 5000, 12345, T - 1])
    xf, wf, dyf = (q.bf16_bits_to_f64(v) for v in (x, w, dy))
    ref = linear.forward(xf[sample], wf)
    print("y", _check_y(bf16_host(y)[sample], ref["y"]))
    rb = linear.backward(dyf[sample], xf[sample], wf)
    assert rel_l2(bf16_host(g["dx"])[sample], rb["dX"]) <= BWD_TOL
    dw = bf16_host(g["dw"])
    rng = np.random.default_rng(1)
    ns, ks = rng.integers(0, N, 64), rng.integers(0, K, 64)
    ref_dw = q.round_bf16(np.einsum("tn,tn->n", dyf[:, ns], xf[:, ks]))
    assert rel_l2(dw[ns, ks], ref_dw) <= BWD_TOL
