"""Pins for the oracle's E2M1 / E4M3 / BF16 codecs (CPU only).

The E2M1 value set and the E4M3 range are fixed by the pages (miniTE
Technical Report, sections 2.2 and 5.1; the 448 maximum from the rainbus
review's method step 4).  The round-to-nearest-even encoders are pinned by an
independent nearest-value search over the finite codebooks at every rounding
midpoint and one float64 ulp either side of it.
"""
import numpy as np
import pytest

from oracle import nvfp4 as q

pytestmark = pytest.mark.cpu


def test_e2m1_value_set():
    vals = q.e2m1_decode(np.arange(16))
    expect = [0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    assert list(vals) == expect
    assert np.signbit(vals[8])


def test_e4m3_landmarks():
    assert q.e4m3_decode(0x7E) == 448.0
    assert q.e4m3_decode(0x08) == 2.0 ** -6          # smallest normal
    assert q.e4m3_decode(0x01) == 2.0 ** -9          # smallest subnormal
    assert q.e4m3_decode(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert q.e4m3_decode(0x38) == 1.0
    assert q.e4m3_decode(0x3C) == 1.5
    assert q.e4m3_decode(0x58) == 16.0
    assert q.e4m3_decode(0x5A) == 20.0
    with pytest.raises(ValueError):
        q.e4m3_decode(0x7F)
    finite = q.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(finite) > 0)               # monotone in the byte value
    assert finite.max() == 448.0


def test_e4m3_encode_roundtrip():
    b = np.arange(0x7F, dtype=np.uint8)
    assert np.array_equal(q.e4m3_encode_exact(q.e4m3_decode(b)), b)


def _nearest_even(v, table, codes):
    """Nearest table value to v; ties to the even code; above the max saturates."""
    d = np.abs(table - v)
    best = d.min()
    cand = np.nonzero(d == best)[0]
    if cand.size > 1:
        cand = [c for c in cand if codes[c] % 2 == 0]
    return table[cand[0]]


def _probe_points(table, vmax):
    mids = (table[1:] + table[:-1]) / 2
    pts = list(table) + list(mids) + [vmax * 1.03, vmax * 1.1, vmax * 4]
    out = []
    for p in pts:
        out += [p, np.nextafter(p, np.inf), np.nextafter(p, -np.inf)]
    return np.array([p for p in out if p >= 0])


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_rne_encoder_matches_nearest_search(fmt):
    if fmt == "e2m1":
        table = q.E2M1_MAGNITUDES
        codes = np.arange(8)
        enc = q.e2m1_round
        vmax = 6.0
    else:
        codes = np.arange(0x7F)
        table = q.e4m3_decode(codes)
        enc = q.e4m3_round
        vmax = 448.0
    pts = _probe_points(table, vmax)
    got = enc(pts)
    want = np.array([_nearest_even(p, table, codes) for p in pts])
    assert np.array_equal(got, want)


def test_bf16_round_against_torch_and_ties():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 2 ** -133, 2 ** -134]])
    v32 = v.astype(np.float32)
    mine = q.f64_to_bf16_bits(v32.astype(np.float64))
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    # float64 inputs that a float32 detour would double-round:
    # 1 + 2^-8 + 2^-30 is just above the bf16 midpoint 1 + 2^-8, so it rounds up.
    assert q.round_bf16(1.0 + 2 ** -8 + 2 ** -30) == 1.0 + 2 ** -7
    assert q.round_bf16(1.0 + 2 ** -8) == 1.0                      # tie -> even
    assert q.round_bf16(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6        # tie -> even (up)


def test_pack_unpack():
    c = np.arange(32, dtype=np.uint8).reshape(2, 16) % 16
    p = q.pack_codes(c)
    assert p[0, 0] == (0 | (1 << 4))
    assert np.array_equal(q.unpack_codes(p), c)
