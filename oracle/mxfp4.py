"""MXFP4 recipe: E2M1 elements with one E8M0 scale per 32, in float64 (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The miniTE Technical Report's format sweep (appendix D1, "Exponent and
Mantissa Sweeps", tables 2-1 and 2-3 and the complete format summary) sets
E2M1 elements with E8M0 (power-of-two) block scales beside the NVFP4 recipe's
E4M3 block scales: the E8M0 variant loses about 2.8 dB of SNR on real QKV
inputs (E2M1 + E4M3 19.88 dB against E2M1 + E8M0 17.11 dB) and about 2 dB on
the simulated batches.  This module is that variant as a format of its own,
the OCP Microscaling (MX) FP4 format, whose block of 32 elements and E8M0
scale are what gfx950's scaled FP4 matrix instructions consume.  It is a
different recipe from NVFP4, not an encoding of it.

Format (OCP Microscaling Formats (MX) Specification v1.0, sections 5.1-5.3
and 6.3, restated):

* E8M0 scale byte s: the value 2^(s - 127); 0xFF (NaN) is never produced.
* Block: 32 consecutive elements of a row share one scale.
* Shared exponent of a block with amax a > 0: X = floor(log2 a) - 2, where 2
  is the exponent of E2M1's largest magnitude (6 = 1.5 * 2^2); X is clamped
  to the E8M0 range [-127, 127].
* Element code: c = Q_E2M1(x / 2^X), round to nearest, ties to the even
  code, saturating at 6 (a / 2^X lies in [4, 8), so the block max can exceed
  6 and clamps to it, as the specification directs).

READINGS where neither source fixes the point:
* There is no per-token or per-row FP32 outer scale: the MX format has none,
  and E8M0 already spans the whole bf16 range, which the outer scale of the
  NVFP4 recipe exists to reach.
* An all-zero block (a = 0) takes X = -127 (scale byte 0); its codes are
  zero codes carrying the sign bit of x, as in the NVFP4 quantiser.
* The pages do not state the block length of their E8M0 simulation; 32 is
  the MX format's and the hardware's.
"""

import numpy as np

from . import nvfp4 as q

MX_BLOCK = 32
E8M0_BIAS = 127
E8M0_MIN_EXP = -127
E8M0_MAX_EXP = 127
# Exponent of E2M1's largest magnitude: 6 = 1.5 * 2^2.
E2M1_EMAX = 2


def e8m0_decode(bits):
    """E8M0 byte -> float64 value 2^(bits - 127).  0xFF (NaN) is rejected."""
    bits = np.asarray(bits, dtype=np.int64)
    if np.any(bits == 0xFF):
        raise ValueError("E8M0 NaN pattern")
    return np.ldexp(1.0, bits - E8M0_BIAS)


def shared_exponent(amax):
    """X = floor(log2 amax) - 2 clamped to [-127, 127]; amax = 0 gives -127.

    floor(log2 a) is read off the binary exponent of the float64 value
    (frexp: a = m 2^e with m in [0.5, 1), so floor(log2 a) = e - 1), which is
    exact for every finite a > 0.
    """
    a = np.asarray(amax, dtype=np.float64)
    X = np.full(a.shape, E8M0_MIN_EXP, dtype=np.int64)
    nz = a > 0
    _, ex = np.frexp(a[nz])
    X[nz] = np.clip(ex.astype(np.int64) - 1 - E2M1_EMAX, E8M0_MIN_EXP, E8M0_MAX_EXP)
    return X


def quantize_rows_mx(x):
    """MXFP4 quantisation of each row of ``x`` (float64 holding bf16 values).

    Per block b of 32 consecutive elements: X_b = shared_exponent(amax_b),
    scale byte X_b + 127, element code sign<<3 | Q_E2M1sat(|x| / 2^X_b).
    Dividing by a power of two is exact in float64, so the rounding acts on
    the exact quotient.

    Returns (codes uint8 [R, K] unpacked 0..15, scales uint8 [R, K/32] E8M0).
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] % MX_BLOCK:
        raise ValueError("rows of a multiple of 32 elements expected")
    R, K = x.shape
    blocks = np.abs(x).reshape(R, K // MX_BLOCK, MX_BLOCK)
    X = shared_exponent(blocks.max(axis=2) if K else np.zeros((R, 0)))
    mag = q.e2m1_round(np.ldexp(blocks, -X[:, :, None]))
    codes = q.e2m1_magnitude_code(mag).reshape(R, K)
    codes |= (np.signbit(x).astype(np.uint8) << 3)
    return codes, (X + E8M0_BIAS).astype(np.uint8)


def block_values_mx(codes, scales):
    """c * 2^X per element (float64): the MXFP4 reconstruction."""
    codes = np.asarray(codes)
    R, K = codes.shape
    s = e8m0_decode(scales)
    return (q.e2m1_decode(codes).reshape(R, K // MX_BLOCK, MX_BLOCK) * s[:, :, None]).reshape(R, K)


# ---------------------------------------------------------------------------
# MXFP8 (E4M3 elements, one E8M0 scale per 32): the backward's format in the
# MXFP8-backward variant the pages compare against their BF16 backward.
# ---------------------------------------------------------------------------
# Exponent of E4M3's largest magnitude: 448 = 1.75 * 2^8.
E4M3_EMAX = 8


def shared_exponent_e4m3(amax):
    """X = floor(log2 amax) - 8 clamped to [-127, 127]; amax = 0 gives -127
    (OCP Microscaling v1.0, section 6.3, with E4M3's emax = 8)."""
    a = np.asarray(amax, dtype=np.float64)
    X = np.full(a.shape, E8M0_MIN_EXP, dtype=np.int64)
    nz = a > 0
    _, ex = np.frexp(a[nz])
    X[nz] = np.clip(ex.astype(np.int64) - 1 - E4M3_EMAX, E8M0_MIN_EXP, E8M0_MAX_EXP)
    return X


def quantize_rows_mx8(x):
    """MXFP8 (E4M3) of each row of ``x`` along the row, blocks of 32.

    Per block: X = shared_exponent_e4m3(amax), scale byte X + 127, element
    Q_E4M3(x / 2^X): round to nearest, ties to even, subnormals kept,
    saturating at 448 (amax / 2^X lies in [256, 512), so the block max can
    exceed 448 and clamps to it).  Returns (values float64 [R, K]: the
    E4M3 values (sign included) without the scale, scales uint8 [R, K/32]).
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] % MX_BLOCK:
        raise ValueError("rows of a multiple of 32 elements expected")
    R, K = x.shape
    blocks = x.reshape(R, K // MX_BLOCK, MX_BLOCK)
    X = shared_exponent_e4m3(np.abs(blocks).max(axis=2) if K else np.zeros((R, 0)))
    mag = q.e4m3_round(np.ldexp(np.abs(blocks), -X[:, :, None]))
    vals = np.where(np.signbit(blocks), -mag, mag).reshape(R, K)
    return vals, (X + E8M0_BIAS).astype(np.uint8)


def e4m3_bytes(vals):
    """Signed E4M3 values (float64) -> E4M3FN bytes (sign in bit 7; -0 -> 0x80)."""
    vals = np.asarray(vals, dtype=np.float64)
    return (q.e4m3_encode_exact(np.abs(vals)) | (np.signbit(vals).astype(np.uint8) << 7)).astype(np.uint8)


def mx8_values(vals, scales):
    """E4M3 value times 2^X per element (float64)."""
    vals = np.asarray(vals, dtype=np.float64)
    R, K = vals.shape
    s = e8m0_decode(scales)
    return (vals.reshape(R, K // MX_BLOCK, MX_BLOCK) * s[:, :, None]).reshape(R, K)


def mx8_along_rows(x):
    """The MXFP8 reconstruction of x quantised along its rows (axis 1)."""
    v, s = quantize_rows_mx8(x)
    return mx8_values(v, s)


def mx8_along_columns(x):
    """The MXFP8 reconstruction of x quantised along its columns (axis 0):
    blocks of 32 consecutive rows of one column share a scale."""
    return mx8_along_rows(np.asarray(x, dtype=np.float64).T).T
