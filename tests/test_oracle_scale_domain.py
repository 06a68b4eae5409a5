"""Pins for the oracle's outer-scale domains wider than a row: per group of
rows, per tensor, per expert weight tensor (CPU only)."""
import numpy as np
import pytest

from oracle import moe, nvfp4 as q
from test_oracle_quantize import exact_quantize_row

pytestmark = pytest.mark.cpu


def _rows(rng, shape, scale=1.0):
    return q.round_bf16(scale * rng.standard_normal(shape))


def test_group_of_one_row_is_the_row_domain():
    x = _rows(np.random.default_rng(1), (20, 96))
    for a, b in zip(q.quantize_rows_grouped(x, 1), q.quantize_rows(x)):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("G", [2, 5, 20])
def test_group_equals_one_long_row(G):
    """A group's rows quantised together equal the per-row quantiser on the
    concatenated row (blocks never straddle rows, K % 16 == 0)."""
    x = _rows(np.random.default_rng(2), (20, 64))
    x[3] *= 50.0
    c, s, g = q.quantize_rows_grouped(x, G)
    lc, ls, lg = q.quantize_rows(x.reshape(20 // G, G * 64))
    assert np.array_equal(c, lc.reshape(20, 64))
    assert np.array_equal(s, ls.reshape(20, 4))
    assert np.array_equal(g, np.repeat(lg, G))


def test_groups_match_exact_rationals():
    """Against the exact-rational quantiser run on each group's elements,
    including a ragged last group."""
    rng = np.random.default_rng(3)
    x = _rows(rng, (7, 32), scale=3.0)
    x[5, 7] = -2688.0 * 2.0 ** -9          # a group max with g a power of two
    c, s, g = q.quantize_rows_grouped(x, 3)
    for g0 in range(0, 7, 3):
        rows = x[g0:g0 + 3]
        ec, es, eg = exact_quantize_row(rows.reshape(-1))
        n = rows.shape[0]
        assert list(c[g0:g0 + n].reshape(-1)) == ec
        assert list(s[g0:g0 + n].reshape(-1)) == es
        assert all(v.view(np.uint32) == eg.view(np.uint32) for v in g[g0:g0 + n])


def test_row_holding_the_group_max_is_encoded_as_alone():
    rng = np.random.default_rng(4)
    x = _rows(rng, (16, 128))
    x[9] *= 8.0
    c, s, g = q.quantize_rows_grouped(x, 16)
    rc, rs, rg = q.quantize_rows(x[9:10])
    assert np.array_equal(c[9], rc[0]) and np.array_equal(s[9], rs[0]) and g[9] == rg[0]
    # every other row's g is at least its own per-row g (a wider domain)
    assert np.all(g >= q.quantize_rows(x)[2])


def test_per_tensor_domain_breaks_the_context_swap():
    """Negative control of the pages' context-swap check: with one outer
    scale per tensor, a token's codes change when other tokens change; per
    token they do not."""
    rng = np.random.default_rng(5)
    x = _rows(rng, (32, 256))
    x2 = x.copy()
    x2[1:] = _rows(rng, (31, 256), scale=1000.0)
    assert not np.array_equal(q.quantize_rows_grouped(x, 32)[0][0], q.quantize_rows_grouped(x2, 32)[0][0])
    assert np.array_equal(q.quantize_rows_grouped(x, 1)[0][0], q.quantize_rows_grouped(x2, 1)[0][0])


def test_per_expert_weight_scale():
    rng = np.random.default_rng(6)
    E, N, K = 3, 8, 64
    w = _rows(rng, (E, N, K), scale=0.02)
    w[1] *= 10.0
    wq = moe.quantize_weights(w, per_expert=True)
    for e in range(E):
        assert np.all(wq["outer"][e] == q.round_f32(np.abs(w[e]).max() / q.OUTER_DIVISOR))
    c, s, g = q.quantize_rows(w.reshape(E, N * K))
    assert np.array_equal(wq["codes"], c.reshape(E, N, K))
