"""Pins for the oracle's per-row NVFP4 quantiser (CPU only).

Independent derivation: ``exact_quantize_row`` below recomputes the
two-level encoding with exact rational arithmetic (``fractions.Fraction``)
and a nearest-value search over the finite codebooks, straight from the
block-scale equation of the miniTE Technical Report, section 5.1, and the
outer scale g = max|X| / (6 * 448) of the rainbus review's method step 4.
It shares nothing with the oracle's float64 ``rint`` implementation, so a
wrong constant, a dropped factor, a wrong tie rule or a transposed block
index in either one fails the comparison.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import nvfp4 as q
from golden_io import load

pytestmark = pytest.mark.cpu

E2M1 = [Fraction(v) for v in ("0", "1/2", "1", "3/2", "2", "3", "4", "6")]
E4M3 = []
for b in range(0x7F):
    e, m = b >> 3, b & 7
    E4M3.append(Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7))


def _nearest(v, table):
    """Index of the nearest table entry; ties to the even index (= even code)."""
    best = None
    for i, t in enumerate(table):
        d = abs(t - v)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def _rn_f32(v):
    """Exact round-to-nearest-even of a non-negative Fraction to float32."""
    f = np.float32(float(v))
    cands = {f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(0))}
    best = None
    for c in sorted(cands):
        d = abs(Fraction(float(c)) - v)
        even = (np.float32(c).view(np.uint32) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, c)
    return np.float32(best[1])


def exact_quantize_row(x):
    """Exact-rational reference: (codes list, scale bytes, g float32)."""
    xs = [Fraction(float(v)) for v in x]
    a = max(abs(v) for v in xs)
    g = _rn_f32(a / 2688)
    G = Fraction(float(g))
    codes, scales = [], []
    for b0 in range(0, len(xs), 16):
        blk = xs[b0:b0 + 16]
        if G == 0:
            d_idx = 0
        else:
            d_idx = _nearest(max(abs(v) for v in blk) / (6 * G), E4M3)
        scales.append(d_idx)
        D = E4M3[d_idx]
        for v, raw in zip(blk, x[b0:b0 + 16]):
            sign = 8 if np.signbit(raw) else 0
            if D == 0 or G == 0:
                codes.append(sign)
            else:
                codes.append(sign | _nearest(abs(v) / (G * D), E2M1))
    return codes, scales, g


def _bf16_row(vals):
    return q.round_bf16(np.asarray(vals, dtype=np.float64))


def _check_against_exact(rows):
    c, s, g = q.quantize_rows(rows)
    for r in range(rows.shape[0]):
        ec, es, eg = exact_quantize_row(rows[r])
        assert list(c[r]) == ec, r
        assert list(s[r]) == es, r
        assert g[r].view(np.uint32) == eg.view(np.uint32), r


@pytest.mark.parametrize("name", ["w1_g_exactly_one.txt", "w2_g_rounds_up.txt", "p6_e4m3_edges.txt"])
def test_golden_worked_examples(name):
    fx = load(name)
    x = np.array([float(v) for v in fx["x"]])
    assert np.array_equal(q.round_bf16(x), x), "fixture values must be bf16"
    c, s, g = q.quantize_rows(x[None, :])
    assert int(g[0].view(np.uint32)) == int(fx["g_bits"][0], 16)
    assert list(s[0]) == [int(v, 16) for v in fx["scales"]]
    assert list(c[0]) == [int(v, 16) for v in fx["codes"]]
    if "packed" in fx:
        assert list(q.pack_codes(c)[0]) == [int(v, 16) for v in fx["packed"]]
    # the independent exact-rational derivation agrees with the fixture too
    ec, es, eg = exact_quantize_row(x)
    assert ec == [int(v, 16) for v in fx["codes"]]
    assert es == [int(v, 16) for v in fx["scales"]]


def test_random_rows_match_exact_rationals():
    rng = np.random.default_rng(11)
    rows = [rng.standard_normal(64),
            rng.standard_t(3, 64) * 50,
            rng.standard_normal(64) * 1e-30,
            rng.standard_normal(64) * np.repeat(10.0 ** rng.integers(-8, 8, 4), 16),
            np.r_[rng.standard_normal(48) * 1e-4, rng.standard_normal(16) * 1e4],
            rng.integers(-8, 9, 64).astype(np.float64),
            np.zeros(64),
            -np.zeros(64)]
    _check_against_exact(_bf16_row(rows))


def test_constructed_ties_match_exact_rationals():
    """Rows whose elements sit exactly on E2M1 midpoints for several (g, d)."""
    rng = np.random.default_rng(12)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    rows = []
    for amax in [2688.0, 1344.0, 6.0, 96.0, 3.0 * 2 ** -5, 1000.0, 7.0]:
        row = np.zeros(64)
        row[0] = amax
        for b in range(4):
            dd = q.E4M3_MAX * 2.0 ** -rng.integers(0, 5)
            gd = (amax / 2688.0) * dd
            blk = rng.choice(mids, 16) * gd * rng.choice([-1, 1], 16)
            row[b * 16 + 1:b * 16 + 16] = blk[1:]
            if b:
                row[b * 16] = 6 * gd
        rows.append(row)
    _check_against_exact(_bf16_row(rows))


def test_zero_row_and_signed_zeros():
    x = np.array([[0.0] * 8 + [-0.0] * 8])
    c, s, g = q.quantize_rows(x)
    assert g[0] == 0 and s[0, 0] == 0
    assert list(c[0]) == [0] * 8 + [8] * 8


def _random_bf16(rng, shape, scale=1.0):
    return q.round_bf16(rng.standard_normal(shape) * scale)


def test_invariant_amax_element_is_max_code():
    rng = np.random.default_rng(3)
    x = _random_bf16(rng, (200, 256))
    c, s, g = q.quantize_rows(x)
    for r in range(x.shape[0]):
        j = np.argmax(np.abs(x[r]))
        assert s[r, j // 16] == 0x7E
        assert c[r, j] & 7 == 7


def test_invariant_power_of_two_scaling():
    rng = np.random.default_rng(4)
    x = _random_bf16(rng, (50, 128))
    c0, s0, g0 = q.quantize_rows(x)
    for j in (-5, 3, 17):
        c, s, g = q.quantize_rows(x * 2.0 ** j)
        assert np.array_equal(c, c0) and np.array_equal(s, s0)
        assert np.array_equal(g.astype(np.float64), g0.astype(np.float64) * 2.0 ** j)


def test_invariant_negation_flips_sign_bit():
    rng = np.random.default_rng(5)
    x = _random_bf16(rng, (50, 128))
    c0, s0, g0 = q.quantize_rows(x)
    c, s, g = q.quantize_rows(-x)
    assert np.array_equal(c, c0 ^ 8)
    assert np.array_equal(s, s0) and np.array_equal(g, g0)


def test_invariant_context_swap_rows_independent():
    """Per-token scale domain: a row's encoding ignores the other rows
    (AI summary, "Methodology in Plain English": context-swap test)."""
    rng = np.random.default_rng(6)
    x = _random_bf16(rng, (64, 256))
    c0, s0, g0 = q.quantize_rows(x)
    x2 = x.copy()
    x2[1:] = _random_bf16(rng, (63, 256), scale=1000.0)
    c, s, g = q.quantize_rows(x2)
    assert np.array_equal(c[0], c0[0]) and np.array_equal(s[0], s0[0]) and g[0] == g0[0]


def test_negative_control_per_tensor_scale_breaks_context_swap():
    """A per-tensor outer scale (one g for the whole tensor) makes row 0's
    codes depend on the other rows: the negative control of the context-swap
    test.  Implemented here in the test by quantising the flattened tensor."""
    rng = np.random.default_rng(6)
    x = _random_bf16(rng, (64, 256))
    c0, _, _ = q.quantize_rows(x.reshape(1, -1))
    x2 = x.copy()
    x2[1:] *= 1000.0
    c, _, _ = q.quantize_rows(x2.reshape(1, -1))
    assert not np.array_equal(c[0, :256], c0[0, :256])


def test_invariant_reencode_decoded_values():
    rng = np.random.default_rng(8)
    x = _random_bf16(rng, (40, 128))
    c, s, g = q.quantize_rows(x)
    xh = q.dequantize_rows(c, s, g)
    c2, s2, g2 = q.quantize_rows(xh)
    # re-encoding under the same (g, d) returns the same codes; the amax of
    # x_hat may differ from that of x, so compare through the fixed scales
    d = q.e4m3_decode(s)
    gg = g.astype(np.float64)
    vals = np.abs(xh).reshape(40, 8, 16) / (gg[:, None, None] * d[:, :, None])
    assert np.array_equal(q.e2m1_magnitude_code(q.e2m1_round(vals)).reshape(40, 128), c & 7)


def test_sanity_band_quantization_error():
    """NVFP4 on N(0,1) rows: relative L2 about 0.10 (SNR about 20 dB), the
    band of the Technical Report's section 2.3 format sweep (E2M1 with E4M3
    scales).  A sanity band, not a pin."""
    rng = np.random.default_rng(9)
    x = _random_bf16(rng, (256, 2048))
    c, s, g = q.quantize_rows(x)
    xh = q.dequantize_rows(c, s, g)
    rel = np.linalg.norm(xh - x) / np.linalg.norm(x)
    assert 0.08 < rel < 0.12
