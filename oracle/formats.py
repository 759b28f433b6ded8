"""NVFP4 number formats for the oracle, written from their bit-level definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The model card "FastWAM UR3 3-task -- 4-bit quantisations" (method table at the
top of the page) fixes the format as NVFP4: E2M1 elements, block 16, E4M3 block
scales, for both weights and activations.  The pages give no more than that;
the readings this oracle takes where they are silent are:

* E2M1: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit, no inf/NaN.
  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* E4M3 is the OCP "E4M3FN" variant: bias 7, max 448, S.1111.111 is NaN, no inf,
  subnormals m * 2^-9.
* Blocks are 16 consecutive elements along a row (the reduction dimension K).
* Block scale S = E4M3(amax / 6), rounded to nearest, ties to even mantissa,
  saturating to 448; no second-level per-tensor scale.
* Element code = E2M1(|v| / decode(S)), rounded to nearest, ties to the even
  code, saturating to 6; sign bit copied from v (so -0.0 and small negatives
  give code 0x8).  A block whose scale decodes to 0 gets magnitude 0 everywhere.
* Packing: byte j of a row holds element 2j in bits [3:0] and 2j+1 in [7:4];
  scales are one byte per block, row-major [rows][cols/16].

Arithmetic note: the quotients amax/6 and |v|/sd are formed in float64.  For
float32 inputs this cannot change a rounding decision: a tie point of either
grid has at most 5 significant bits, so the exact quotient is either exactly a
tie (and float64 represents it exactly) or lies at least ~2^-24 relative away
from it, while float64 division errs by at most 2^-53 relative.
"""

import numpy as np

# ----------------------------------------------------------------------------
# Decoders: value of every code, straight from sign / exponent / mantissa.
# ----------------------------------------------------------------------------


def e2m1_decode(code: int) -> float:
    """Value of a 4-bit E2M1 code (sign | 2-bit exponent, bias 1 | 1-bit mantissa)."""
    sign = (code >> 3) & 1
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:  # subnormal: 0.m * 2^(1 - bias) = m * 0.5
        mag = man * 0.5
    else:
        mag = 2.0 ** (exp - 1) * (1.0 + man / 2.0)
    return -mag if sign else mag


def e4m3_decode(code: int) -> float:
    """Value of an 8-bit E4M3FN code (bias 7; S.1111.111 is NaN; no infinities)."""
    sign = (code >> 7) & 1
    exp = (code >> 3) & 15
    man = code & 7
    if exp == 15 and man == 7:
        return float("nan")
    if exp == 0:  # subnormal: 0.mmm * 2^(1 - 7)
        mag = man * 2.0 ** -9
    else:
        mag = 2.0 ** (exp - 7) * (1.0 + man / 8.0)
    return -mag if sign else mag


E2M1_VALUES = np.array([e2m1_decode(c) for c in range(16)], dtype=np.float64)
E4M3_VALUES = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)

E2M1_MAX = 6.0
E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_QUANTUM = 2.0 ** -9

# ----------------------------------------------------------------------------
# Encoders of non-negative magnitudes: IEEE-style round to nearest, ties to an
# even significand, computed as rint(q / quantum) * quantum with the quantum of
# q's binade.  rint() rounds half to even.  Results saturate at the format max.
# ----------------------------------------------------------------------------


def e2m1_round_magnitude(q):
    """Round q >= 0 onto the E2M1 magnitude grid {0,.5,1,1.5,2,3,4,6} (RNE, saturating)."""
    q = np.asarray(q, dtype=np.float64)
    # binades: [0,2) has quantum 0.5 (the subnormal 0.5 step continues through
    # the first normal binade), [2,4) quantum 1, [4,inf) quantum 2.
    quantum = np.where(q < 2.0, 0.5, np.where(q < 4.0, 1.0, 2.0))
    v = np.rint(q / quantum) * quantum
    return np.minimum(v, E2M1_MAX)


def e4m3_round_magnitude(q):
    """Round q >= 0 to the nearest E4M3FN value (RNE, saturating to 448)."""
    q = np.asarray(q, dtype=np.float64)
    _, e = np.frexp(q)  # q = f * 2^e, 0.5 <= f < 1, so the leading bit is 2^(e-1)
    lead = e - 1
    quantum = np.where(q < E4M3_MIN_NORMAL, E4M3_SUBNORMAL_QUANTUM,
                       np.ldexp(1.0, lead - 3))
    v = np.rint(q / quantum) * quantum
    return np.minimum(v, E4M3_MAX)


_E2M1_MAGNITUDES = E2M1_VALUES[:8]          # ascending: codes 0..7
_E4M3_POSITIVES = E4M3_VALUES[:0x7F]        # ascending: codes 0x00..0x7E


def _code_of(grid, v):
    """Index of each value of v in the ascending grid; every v must be on it."""
    idx = np.searchsorted(grid, v)
    idx = np.minimum(idx, len(grid) - 1)
    if not np.array_equal(grid[idx], v):
        raise AssertionError("rounded value not on the grid")
    return idx.astype(np.uint8)


def e2m1_encode_magnitude(q):
    """Magnitude code (0..7) of RNE(q) on the E2M1 grid."""
    return _code_of(_E2M1_MAGNITUDES, e2m1_round_magnitude(q))


def e4m3_encode(q):
    """Code (0x00..0x7E) of RNE(q) in E4M3FN, q >= 0, saturating."""
    return _code_of(_E4M3_POSITIVES, e4m3_round_magnitude(q))


# ----------------------------------------------------------------------------
# NVFP4 block quantiser / dequantiser on rows.
# ----------------------------------------------------------------------------

BLOCK = 16


def quantize_nvfp4(a):
    """NVFP4-quantise each row of a float32 matrix along its columns.

    a: (rows, cols) float32, cols % 16 == 0, finite values.
    Returns (codes, scales): codes (rows, cols // 2) uint8 with element 2j in the
    low nibble of byte j; scales (rows, cols // 16) uint8 E4M3FN codes.
    """
    a = np.asarray(a)
    if a.dtype != np.float32:
        raise TypeError("the NVFP4 quantiser is defined on float32 input")
    rows, cols = a.shape
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 16")
    v = a.astype(np.float64).reshape(rows, cols // BLOCK, BLOCK)
    amax = np.abs(v).max(axis=2) if cols else np.zeros((rows, 0))
    scales = e4m3_encode(amax / 6.0).reshape(rows, cols // BLOCK)
    sd = E4M3_VALUES[scales][..., None]
    q = np.divide(np.abs(v), sd, out=np.zeros_like(v), where=sd > 0)
    mag = e2m1_encode_magnitude(q).reshape(v.shape)
    codes = mag | (np.signbit(v).astype(np.uint8) << 3)
    codes = codes.reshape(rows, cols)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales.astype(np.uint8)


def unpack_codes(packed):
    """(rows, cols//2) packed bytes -> (rows, cols) 4-bit codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    codes = np.empty((rows, 2 * half), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    return codes


def dequantize_nvfp4(packed, scales):
    """Value of every element: E2M1(code) * E4M3(scale of its block), float64."""
    codes = unpack_codes(packed)
    rows, cols = codes.shape
    vals = E2M1_VALUES[codes].reshape(rows, cols // BLOCK, BLOCK)
    sd = E4M3_VALUES[np.asarray(scales, dtype=np.uint8)][..., None]
    return (vals * sd).reshape(rows, cols)
