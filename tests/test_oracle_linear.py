"""Pins for the oracle's dense linear layer (CPU only)."""
import numpy as np
import pytest

from oracle import linear, moe, nvfp4 as q
from test_oracle_moe import lossless_operands

pytestmark = pytest.mark.cpu


def test_lossless_operands_give_the_exact_product():
    """Operands that NVFP4 encodes exactly: the pre-cast output is the exact
    product x W^T (a dropped outer factor, a wrong block scale or a
    transposed operand would change it)."""
    rng = np.random.default_rng(21)
    T, N, K = 12, 6, 96
    x, w = lossless_operands(rng, T, N, K, rng.integers(-8, 8, T), rng.integers(-14, -4, N))
    f = linear.forward(x, w)
    assert np.array_equal(f["pre"], x @ w.T)
    assert np.array_equal(f["y"], q.round_bf16(x @ w.T))


def test_forward_is_the_one_group_grouped_product():
    """One expert holding every row: the linear forward is the grouped
    product of the MoE oracle (pinned there by brute force)."""
    rng = np.random.default_rng(22)
    T, N, K = 9, 5, 64
    x = q.round_bf16(rng.standard_normal((T, K)))
    w = q.round_bf16(0.05 * rng.standard_normal((N, K)))
    f = linear.forward(x, w)
    xc, xs, xg = f["xq"]
    wc, ws, wg = f["wq"]
    ref = moe.grouped_gemm_nvfp4(xc, xs, xg, np.array([0, T]), wc[None], ws[None], wg[None])
    assert np.array_equal(f["pre"], ref)


def test_forward_rows_are_independent():
    """Per-token scale domain: a row's output does not depend on the other
    rows of the batch (the pages' context-swap property)."""
    rng = np.random.default_rng(23)
    x = q.round_bf16(rng.standard_normal((8, 64)))
    w = q.round_bf16(0.05 * rng.standard_normal((4, 64)))
    x2 = x.copy()
    x2[1:] = q.round_bf16(100.0 * rng.standard_normal((7, 64)))
    assert np.array_equal(linear.forward(x, w)["y"][0], linear.forward(x2, w)["y"][0])


def test_backward_against_autograd():
    """Without bf16 roundings the backward equals float64 autograd of the
    dense product (the straight-through estimator treats the quantisers as
    identity)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(24)
    T, N, K = 7, 5, 32
    x, w, dy = rng.standard_normal((T, K)), rng.standard_normal((N, K)), rng.standard_normal((T, N))
    X = torch.tensor(x, requires_grad=True)
    W = torch.tensor(w, requires_grad=True)
    ((X @ W.T) * torch.tensor(dy)).sum().backward()
    g = linear.backward(dy, x, w, rnd=False)
    assert np.allclose(g["dX"], X.grad.numpy(), rtol=1e-13, atol=1e-13)
    assert np.allclose(g["dW"], W.grad.numpy(), rtol=1e-13, atol=1e-13)
