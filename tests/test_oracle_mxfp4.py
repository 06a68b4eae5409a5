"""Pins for the oracle's MXFP4 recipe (CPU only).

Independent derivation: ``exact_mx_row`` recomputes the encoding with exact
rational arithmetic (``fractions.Fraction``): the shared exponent by
doubling / halving until 2^e <= amax < 2^(e+1), the element by a
nearest-value search over the 8 E2M1 magnitudes times 2^X with the tie going
to the even code (OCP Microscaling Formats (MX) Specification v1.0, section
6.3; "E2M1 + E8M0" of the miniTE Technical Report's appendix D1 sweep).  It
shares nothing with the oracle's float64 ``frexp`` / ``rint`` route.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import moe, mxfp4 as mx, nvfp4 as q
from golden_io import load

pytestmark = pytest.mark.cpu

E2M1 = [Fraction(v) for v in ("0", "1/2", "1", "3/2", "2", "3", "4", "6")]


def _floor_log2(a):
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    return e


def exact_mx_row(row):
    """Exact MXFP4 of one row of float values: (codes list, scale bytes list)."""
    codes, scales = [], []
    for b0 in range(0, len(row), 32):
        blk = [Fraction(float(v)) for v in row[b0:b0 + 32]]
        neg = [bool(np.signbit(v)) for v in row[b0:b0 + 32]]
        amax = max(abs(v) for v in blk)
        X = -127 if amax == 0 else min(127, max(-127, _floor_log2(amax) - 2))
        scales.append(X + 127)
        unit = Fraction(2) ** X
        for v, n in zip(blk, neg):
            best = None
            for i, t in enumerate(E2M1):
                d = abs(abs(v) - t * unit)
                if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
                    best = (d, i)
            codes.append(best[1] | (8 if n else 0))
    return codes, scales


def _bf16_values(v):
    return q.bf16_bits_to_f64(q.f64_to_bf16_bits(v))


def test_e8m0_table():
    assert mx.e8m0_decode(127) == 1.0
    assert mx.e8m0_decode(0) == 2.0 ** -127
    assert mx.e8m0_decode(254) == 2.0 ** 127
    assert mx.e8m0_decode(130) == 8.0
    with pytest.raises(ValueError):
        mx.e8m0_decode(0xFF)


def test_worked_row_fixture():
    g = load("mx_worked_row.txt")
    x = np.array([[float(v) for k in "ABCD" for v in g["x" + k]]])
    codes, scales = mx.quantize_rows_mx(x)
    want = [int(c, 16) for k in "ABCD" for c in g["codes" + k]]
    assert codes[0].tolist() == want
    assert scales[0].tolist() == [int(v) for v in g["scales"]]
    packed = [int(c, 16) for k in "ABCD" for c in g["packed" + k]]
    assert q.pack_codes(codes)[0].tolist() == packed
    # the fixture itself agrees with the exact rational derivation
    ec, es = exact_mx_row(x[0])
    assert ec == want and es == [int(v) for v in g["scales"]]


@pytest.mark.parametrize("dist", ["normal", "student_t", "wide"])
def test_oracle_equals_exact_search(dist):
    rng = np.random.default_rng(7)
    if dist == "normal":
        v = rng.standard_normal((6, 96))
    elif dist == "student_t":
        v = rng.standard_t(3, (6, 96))
    else:   # block maxima spread over many binades, incl. tiny ones
        v = rng.standard_normal((6, 96)) * np.ldexp(1.0, rng.integers(-60, 60, (6, 1)))
    x = _bf16_values(v)
    codes, scales = mx.quantize_rows_mx(x)
    for r in range(x.shape[0]):
        ec, es = exact_mx_row(x[r])
        assert codes[r].tolist() == ec
        assert scales[r].tolist() == es


def test_midpoints_and_neighbours():
    """Every E2M1 midpoint times 2^X, and the bf16 neighbours on both sides,
    in blocks whose amax fixes X = 3."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = []
    for m in mids:
        t = m * 8.0
        b = int(q.f64_to_bf16_bits(np.array([t]))[0])
        vals += [t, float(q.bf16_bits_to_f64(np.array([b + 1], np.uint16))[0]),
                 float(q.bf16_bits_to_f64(np.array([b - 1], np.uint16))[0])]
    x = np.zeros((1, 32))
    x[0, 0] = 32.0                      # floor(log2 32) - 2 = 3
    x[0, 1:1 + len(vals)] = vals
    codes, scales = mx.quantize_rows_mx(x)
    assert scales[0, 0] == 130
    ec, _ = exact_mx_row(x[0])
    assert codes[0].tolist() == ec


def test_invariants():
    rng = np.random.default_rng(11)
    x = _bf16_values(rng.standard_normal((8, 128)))
    c, s = mx.quantize_rows_mx(x)
    # power-of-two scaling moves only the scale byte
    for j in (-5, 3, 40):
        c2, s2 = mx.quantize_rows_mx(np.ldexp(x, j))
        assert np.array_equal(c2, c) and np.array_equal(s2.astype(int), s.astype(int) + j)
    # negation flips the sign bit of every code
    cn, sn = mx.quantize_rows_mx(-x)
    assert np.array_equal(cn, c ^ 8) and np.array_equal(sn, s)
    # each block's amax element lands on magnitude 4 or 6 (codes 6, 7): amax / 2^X in [4, 8)
    blocks = np.abs(x).reshape(8, 4, 32)
    arg = blocks.argmax(axis=2)
    cb = c.reshape(8, 4, 32)
    top = np.take_along_axis(cb, arg[:, :, None], axis=2)[:, :, 0] & 7
    assert np.all((top == 6) | (top == 7))
    # re-encoding the reconstruction returns the same codes and scales
    c3, s3 = mx.quantize_rows_mx(mx.block_values_mx(c, s))
    assert np.array_equal(s3, s)
    assert np.array_equal(mx.block_values_mx(c3, s3), mx.block_values_mx(c, s))


def test_zero_and_clamped_blocks():
    x = np.zeros((1, 64))
    x[0, 5] = -0.0
    x[0, 32] = 2.0 ** -133            # smallest bf16 subnormal: X clamps to -127
    c, s = mx.quantize_rows_mx(x)
    assert s[0].tolist() == [0, 0]
    assert c[0, 5] == 8 and c[0].sum() == 8   # 2^-133 / 2^-127 = 1/64 -> code 0


def test_error_band_against_the_pages_ordering():
    """Not a pin: the pages measure E2M1 + E8M0 as the less accurate scale
    format (Technical Report appendix D1: rel-L2 0.13950 against 0.10140 on
    real QKV; SNR 17.97 against 20.17 dB on a simulated batch).  N(0,1)
    rows here show the same ordering and a comparable size."""
    rng = np.random.default_rng(3)
    x = _bf16_values(rng.standard_normal((256, 512)))
    c, s = mx.quantize_rows_mx(x)
    e_mx = np.linalg.norm(mx.block_values_mx(c, s) - x) / np.linalg.norm(x)
    cn, sn, gn = q.quantize_rows(x)
    e_nv = np.linalg.norm(q.dequantize_rows(cn, sn, gn) - x) / np.linalg.norm(x)
    assert e_nv < e_mx < 0.16
    assert e_mx > 0.10


def test_grouped_gemm_brute_force_and_empty_expert():
    rng = np.random.default_rng(5)
    T, H, E, k, I = 12, 64, 4, 2, 32
    x = _bf16_values(rng.standard_normal((T, H)))
    idx = np.array([[0, 2]] * 6 + [[2, 3]] * 6)   # expert 1 receives nothing
    w1 = _bf16_values(rng.standard_normal((E, 2 * I, H)) * 0.02)
    xq = moe.quantize_permute_mx(x, idx, E, row_align=4)
    wq = moe.quantize_weights_mx(w1)
    out = moe.grouped_gemm_mx(xq["codes"], xq["scales"], xq["offsets"], wq["codes"], wq["scales"])
    off = xq["offsets"]
    assert off[2] - off[1] == 0
    # brute force: exact rational triple loop on a few entries per expert
    for e in (0, 2, 3):
        for r in (int(off[e]), int(off[e + 1]) - 1):
            t = int(xq["src_row"][r])
            if t < 0:
                assert np.all(out[r] == 0)
                continue
            xc, xs = exact_mx_row(x[t])
            for n in (0, 2 * I - 1):
                wc, ws = exact_mx_row(w1[e, n])
                acc = Fraction(0)
                for kk in range(H):
                    xv = E2M1[xc[kk] & 7] * Fraction(2) ** (xs[kk // 32] - 127) * (-1 if xc[kk] & 8 else 1)
                    wv = E2M1[wc[kk] & 7] * Fraction(2) ** (ws[kk // 32] - 127) * (-1 if wc[kk] & 8 else 1)
                    acc += xv * wv
                assert out[r, n] == float(acc)


def test_forward_closed_forms():
    rng = np.random.default_rng(9)
    T, H, E, I = 16, 64, 4, 32
    w1q = moe.quantize_weights_mx(_bf16_values(rng.standard_normal((E, 2 * I, H)) * 0.02))
    w2q = moe.quantize_weights_mx(_bf16_values(rng.standard_normal((E, H, I)) * 0.02))
    idx = rng.integers(0, E, (T, 1))
    # zero input -> zero output
    f0 = moe.forward_mx(np.zeros((T, H)), idx, np.ones((T, 1)), w1q, w2q, E)
    assert np.all(f0["y"] == 0)
    # k = 1 with p = 1: y is the expert output row itself
    x = _bf16_values(rng.standard_normal((T, H)))
    f = moe.forward_mx(x, idx, np.ones((T, 1)), w1q, w2q, E)
    assert np.array_equal(f["y"], f["o"][f["xq"]["row_map"][:, 0]])
    # the FC2 input codes are the MXFP4 of the bf16 SwiGLU output
    c, s = mx.quantize_rows_mx(f["a"])
    assert np.array_equal(c, f["a_codes"]) and np.array_equal(s, f["a_scales"])
