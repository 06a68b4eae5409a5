"""NVFP4 codecs and the per-row two-level quantiser, in float64 (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Formats (miniTE Technical Report, section 2.2 and section 5.1; rainbus review,
"prerequisites: the NVFP4 format"):

* E2M1 element code: 1 sign bit, 2 exponent bits, 1 mantissa bit.  Magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}; codes 8..15 are the negatives of codes 0..7.
* E4M3 block scale, one per 16 consecutive elements of a row.  The 448 maximum
  used by the pages' outer-scale constant (6 * 448) fixes the E4M3FN flavour:
  bias 7, subnormals m * 2^-9, 0x7E = 448, 0x7F is NaN and never produced.
* FP32 outer scale, one per row (per dispatched token for activations, per
  output feature for weights).

Rounding: round-to-nearest, ties to the even code, saturating at the largest
finite magnitude (the "finite E2M1/E4M3 codebook with round-to-nearest-even"
of the Technical Report, section 2.3; stochastic rounding off per the AI
summary's methodology).  Readings the pages leave open are listed in the
repository design notes and repeated at each function.
"""

import numpy as np

# The eight E2M1 magnitudes, indexed by the 3 low bits of the code.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

E2M1_MAX = 6.0
E4M3_MAX = 448.0
# Outer-scale divisor: the largest E2M1 magnitude times the largest E4M3 scale
# (rainbus review, method step 4: g = max|X| / (6 * 448)).
OUTER_DIVISOR = E2M1_MAX * E4M3_MAX  # 2688
BLOCK = 16


# ---------------------------------------------------------------------------
# Generic round-to-nearest-even onto a small binary floating-point grid.
# ---------------------------------------------------------------------------
def round_minifloat(v, e_min, mbits, vmax):
    """Round |v| >= 0 to the nearest value of a binary format, ties to even.

    The format has ``mbits`` explicit mantissa bits, minimum exponent
    ``e_min`` (below it the spacing stays 2^(e_min - mbits): subnormals) and
    saturates at ``vmax``.  Inside a binade [2^e, 2^(e+1)) the spacing is
    q = 2^(e - mbits); v / q is then an exact float64 (scaling by a power of
    two) and numpy's ``rint`` rounds half to even, which is the tie rule
    because an even multiple of q has an even last mantissa bit.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    nz = v > 0
    _, ex = np.frexp(v[nz])           # v = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, e_min)     # floor(log2 v), clamped to the subnormal binade
    q = np.ldexp(1.0, e - mbits)
    out[nz] = np.minimum(np.rint(v[nz] / q) * q, vmax)
    return out


def e2m1_round(v):
    """RNE of |v| onto the E2M1 magnitudes, saturating at 6."""
    return round_minifloat(v, e_min=0, mbits=1, vmax=E2M1_MAX)


def e4m3_round(v):
    """RNE of |v| onto the E4M3FN magnitudes (subnormals kept), saturating at 448."""
    return round_minifloat(v, e_min=-6, mbits=3, vmax=E4M3_MAX)


# ---------------------------------------------------------------------------
# Value <-> bit-pattern tables.
# ---------------------------------------------------------------------------
def e2m1_decode(codes):
    """E2M1 code (0..15, sign in bit 3) -> float64 value."""
    codes = np.asarray(codes, dtype=np.int64)
    mag = E2M1_MAGNITUDES[codes & 7]
    return np.where(codes & 8, -mag, mag)


def e2m1_magnitude_code(mag):
    """Exact E2M1 magnitude (one of the eight values) -> its 3-bit code."""
    mag = np.asarray(mag, dtype=np.float64)
    idx = np.searchsorted(E2M1_MAGNITUDES, mag)
    if not np.all(E2M1_MAGNITUDES[np.minimum(idx, 7)] == mag):
        raise ValueError("not an E2M1 magnitude")
    return idx.astype(np.uint8)


def e4m3_decode(bits):
    """E4M3FN byte -> float64 value.  0x7F / 0xFF (NaN) are rejected."""
    bits = np.asarray(bits, dtype=np.int64)
    if np.any((bits & 0x7F) == 0x7F):
        raise ValueError("E4M3 NaN pattern")
    e = (bits >> 3) & 0xF
    m = bits & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    return np.where(bits & 0x80, -mag, mag)


def e4m3_encode_exact(v):
    """Non-negative E4M3-representable float64 value -> E4M3FN byte."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint8)
    nz = v > 0
    _, ex = np.frexp(v[nz])
    e = ex - 1
    sub = e < -6
    bits = np.where(sub,
                    np.ldexp(v[nz], 9),                                   # m * 2^-9
                    (e + 7) * 8 + (np.ldexp(v[nz], -e) - 1.0) * 8.0)      # (E << 3) | M
    if not np.all(bits == np.rint(bits)):
        raise ValueError("not an E4M3 value")
    out[nz] = bits.astype(np.uint8)
    if np.any(e4m3_decode(out) != v):
        raise ValueError("not an E4M3 value")
    return out


# ---------------------------------------------------------------------------
# BF16 <-> float64.
# ---------------------------------------------------------------------------
def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(v):
    """Round float64 values to the nearest bf16 value, ties to even (one rounding).

    bf16 keeps 7 explicit mantissa bits and float32's exponent range
    (subnormals down to 2^-133).  Results overflowing bf16 become +-inf.
    Rounding straight from float64 avoids the double rounding a detour
    through float32 would add.
    """
    v = np.asarray(v, dtype=np.float64)
    mag = round_minifloat(np.abs(v), e_min=-126, mbits=7, vmax=np.inf)
    bf16_max = np.ldexp(2.0 - 2.0 ** -7, 127)
    mag = np.where(mag > bf16_max, np.inf, mag)
    return np.copysign(mag, v)


def f64_to_bf16_bits(v):
    """float64 -> bf16 bit patterns (uint16), RNE, sign of zero kept."""
    r = round_bf16(v).astype(np.float32)      # exact: a bf16 value is a float32 value
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def round_f32(v):
    """float64 -> nearest float32 (numpy's cast rounds to nearest even)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)


# ---------------------------------------------------------------------------
# Row quantiser.
# ---------------------------------------------------------------------------
def quantize_rows(x, scale_amax=None):
    """Two-level NVFP4 quantisation of each row of ``x`` (float64, bf16 values).

    Follows the block-scale equation of the miniTE Technical Report, section
    5.1, with the outer scale of the rainbus review's method step 4:

      1. a   = max_k |x[k]| over the whole row (per-token / per-row domain)
      2. g   = RN_f32(a / (6 * 448))                 FP32 outer scale
      3. d_b = Q_E4M3(amax(block b) / (6 g))         one E4M3 scale per 16
      4. c   = Q_E2M1(x / (g d_b))                    E2M1 code per element

    Readings where the pages are silent: every Q(.) acts on the exact real
    quotient of the stored g, d (evaluated here as one correctly rounded
    float64 division, which keeps the side of every rounding midpoint because
    the operands have at most 8 + 31 significant bits); ties go to the even
    code; E2M1 saturates at 6 (needed whenever d_b rounds down); a zero row
    (g = 0) or an underflowed block (d_b = 0) encodes every element as a zero
    code carrying the sign bit of x.

    ``scale_amax`` (float64 [R]), when given, replaces the row's own max in
    step 1: the outer scale of a wider scale domain (quantize_rows_grouped).

    Returns (codes uint8 [R, K] unpacked 0..15, scales uint8 [R, K/16] E4M3
    bytes, outer float32 [R]).
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] % BLOCK:
        raise ValueError("rows of a multiple of 16 elements expected")
    R, K = x.shape
    ax = np.abs(x)

    # 1-2: per-row outer scale, stored as float32.
    if scale_amax is not None:
        a = np.asarray(scale_amax, dtype=np.float64)
    else:
        a = ax.max(axis=1) if K else np.zeros(R)
    g32 = round_f32(a / OUTER_DIVISOR)
    g = g32.astype(np.float64)

    # 3: block scales from the block amax.
    blocks = ax.reshape(R, K // BLOCK, BLOCK)
    a_b = blocks.max(axis=2)
    d = np.zeros_like(a_b)
    has_g = g > 0
    d[has_g] = e4m3_round(a_b[has_g] / (6.0 * g[has_g, None]))
    scales = e4m3_encode_exact(d)

    # 4: element codes.
    denom = (g[:, None] * d)[:, :, None]                 # exact: 24 x 4 bits
    live = np.broadcast_to(denom > 0, blocks.shape)
    mag = np.zeros_like(blocks)
    mag[live] = e2m1_round(blocks[live] / np.broadcast_to(denom, blocks.shape)[live])
    codes = e2m1_magnitude_code(mag).reshape(R, K)
    codes |= (np.signbit(x).astype(np.uint8) << 3)
    return codes, scales, g32


def quantize_rows_grouped(x, group_rows):
    """quantize_rows with one outer scale per group of ``group_rows``
    consecutive rows (the last group may be shorter): step 1 takes the max
    over the whole group.  group_rows = 1 is the per-row domain; R the
    per-tensor domain; the rows of one expert's weight the per-expert domain
    (miniTE Technical Report, section 2.2: the recipe decides whether the
    outer scale is per tensor, per expert or per row; section 4.3 table:
    miniTE CUTLASS keeps one outer scale per expert weight tensor).  Block
    scales and codes are per row as before, against the group's g.
    """
    x = np.asarray(x, dtype=np.float64)
    R = x.shape[0]
    if group_rows < 1:
        raise ValueError("group_rows >= 1")
    row_max = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(R)
    grp = np.arange(R) // group_rows
    gmax = np.zeros(grp.max() + 1 if R else 0)
    np.maximum.at(gmax, grp, row_max)
    return quantize_rows(x, scale_amax=gmax[grp])


def pack_codes(codes):
    """Pack 4-bit codes two per byte: element 2j in the low nibble of byte j."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed):
    """Inverse of ``pack_codes``."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def block_values(codes, scales):
    """d_b * c per element (float64), without the outer scale g."""
    codes = np.asarray(codes)
    R, K = codes.shape
    d = e4m3_decode(scales)
    return (e2m1_decode(codes).reshape(R, K // BLOCK, BLOCK) * d[:, :, None]).reshape(R, K)


def dequantize_rows(codes, scales, outer):
    """x_hat = g * d_b * c (float64), the reconstruction of section 5.1."""
    return block_values(codes, scales) * np.asarray(outer, dtype=np.float64)[:, None]
