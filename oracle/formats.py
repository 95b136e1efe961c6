"""Number formats used by NVFP4, written out from their definitions.

Test infrastructure only (see the package docstring).

The pages ([P1] section "NVFP4量化") fix the structure -- 16-element blocks,
one FP32 per-tensor scale -- but never spell out the bit formats.  The formats
below are the NVFP4 ones: E2M1 elements and E4M3 block scales.

* E2M1 (reading R-1): a 4-bit code, bit 3 = sign, bits 2..1 = exponent with
  bias 1, bit 0 = mantissa.  Exponent 0 is subnormal (value = m * 0.5).  The
  magnitudes of codes 0..7 are therefore 0, 0.5, 1, 1.5, 2, 3, 4, 6; codes
  8..15 are their negatives (code 8 is -0).
* E4M3 (reading R-2): the OCP FP8 "fn" byte -- sign bit 7, 4 exponent bits with
  bias 7, 3 mantissa bits, no infinities, 0x7F / 0xFF are NaN, largest finite
  value 448 (0x7E), exponent 0 is subnormal (value = m * 2^-9).
* bf16: the top 16 bits of an IEEE binary32.

Rounding everywhere is "to nearest, ties to the even code" (R-6, R-8), with
saturation to the largest finite value, which is what "nearest representable
value" gives when infinities are not representable.
"""

from fractions import Fraction

import numpy as np

# ----------------------------------------------------------------------------
# E2M1
# ----------------------------------------------------------------------------


def e2m1_value(code):
    """Exact value of a 4-bit E2M1 code (R-1), as a Fraction.

    Decoded from the bit fields, not from a table: exponent field e = bits 2..1,
    mantissa m = bit 0; e == 0 -> m/2, else 2^(e-1) * (1 + m/2).
    """
    code = int(code)
    if not 0 <= code <= 15:
        raise ValueError("E2M1 code must be a nibble")
    sign = -1 if code & 8 else 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = Fraction(m, 2)
    else:
        mag = Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return sign * mag


#: magnitudes of codes 0..7, in code order (increasing)
E2M1_MAGNITUDES = np.array([float(e2m1_value(c)) for c in range(8)],
                           dtype=np.float32)
# Midpoints between consecutive magnitudes: exact in binary32.
_E2M1_MIDPOINTS = ((E2M1_MAGNITUDES[:-1].astype(np.float64)
                    + E2M1_MAGNITUDES[1:].astype(np.float64)) / 2.0)


def e2m1_encode_magnitude(v):
    """Round non-negative binary32 values to the nearest E2M1 magnitude code.

    Nearest of the eight magnitudes; a value exactly half-way between two
    neighbours goes to the even code (R-8); values above 6 saturate to code 7
    (6 is the nearest representable value).  Returns uint8 codes 0..7.

    Written as: count the midpoints strictly below v; on an exact tie the two
    candidates are i and i+1 and the even one wins.
    """
    v = np.asarray(v, dtype=np.float32)
    if np.any(np.isnan(v)) or np.any(v < 0):
        raise ValueError("e2m1_encode_magnitude takes finite non-negative input")
    vd = v.astype(np.float64)              # exact widening
    i = np.searchsorted(_E2M1_MIDPOINTS, vd, side="left")
    at_tie = np.zeros(vd.shape, dtype=bool)
    inside = i < len(_E2M1_MIDPOINTS)
    at_tie[inside] = vd[inside] == _E2M1_MIDPOINTS[i[inside]]
    code = np.where(at_tie & (i % 2 == 1), i + 1, i)
    return code.astype(np.uint8)


# ----------------------------------------------------------------------------
# E4M3 (OCP fp8 "fn")
# ----------------------------------------------------------------------------


def _e4m3_fraction(byte):
    byte = int(byte)
    sign = -1 if byte & 0x80 else 1
    e = (byte >> 3) & 0xF
    m = byte & 7
    if e == 15 and m == 7:
        raise ValueError("0x7F / 0xFF are NaN in E4M3")
    if e == 0:
        mag = Fraction(m, 8) * Fraction(1, 2 ** 6)
    else:
        mag = (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return sign * mag


#: the 127 finite non-negative E4M3 values, indexed by byte 0x00..0x7E
E4M3_VALUES = np.array([float(_e4m3_fraction(b)) for b in range(0x7F)],
                       dtype=np.float64)
_E4M3_MIDPOINTS = (E4M3_VALUES[:-1] + E4M3_VALUES[1:]) / 2.0   # exact in fp64


def e4m3_value(byte):
    """binary32 value of E4M3 bytes (R-2).  NaN bytes raise."""
    b = np.asarray(byte, dtype=np.uint8)
    if np.any((b & 0x7F) == 0x7F):
        raise ValueError("E4M3 NaN byte")
    mag = E4M3_VALUES[(b & 0x7F).astype(np.int64)]
    out = np.where(b & 0x80, -mag, mag)
    return out.astype(np.float32)


def e4m3_encode_nonneg(t):
    """Round non-negative binary32 values to an E4M3 byte (R-6).

    Nearest of the 127 finite non-negative values, ties to the even byte,
    saturating at 448 (0x7E) since E4M3 "fn" has no infinity.  Values at or
    below 2^-10 (half the smallest subnormal) give 0x00.
    """
    t = np.asarray(t, dtype=np.float32)
    if np.any(np.isnan(t)) or np.any(t < 0):
        raise ValueError("e4m3_encode_nonneg takes finite non-negative input")
    td = t.astype(np.float64)
    i = np.searchsorted(_E4M3_MIDPOINTS, td, side="left")
    at_tie = np.zeros(td.shape, dtype=bool)
    inside = i < len(_E4M3_MIDPOINTS)
    at_tie[inside] = td[inside] == _E4M3_MIDPOINTS[i[inside]]
    byte = np.where(at_tie & (i % 2 == 1), i + 1, i)
    return byte.astype(np.uint8)


# ----------------------------------------------------------------------------
# bf16
# ----------------------------------------------------------------------------


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> binary32, exactly (bf16 is the top half)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_bits_to_f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


_BF16_MAX = float(Fraction(2) ** 127 * (2 - Fraction(1, 2 ** 7)))


def round_to_bf16_bits(y):
    """Round real values (given as float32 or float64) to bf16, nearest-even.

    Done in one rounding from the given value: a bf16 keeps 8 significant bits,
    so y is scaled by a power of two so that its quantum becomes 1 and rounded
    to an integer half-to-even (``numpy.rint``), all exact in float64.  The
    quantum is 2^(e-8) for a value in [2^(e-1), 2^e), and never below 2^-133
    (bf16 subnormals).  Results above the largest finite bf16 become infinity.
    Returns uint16 bit patterns; the sign of zero is kept.
    """
    y = np.asarray(y, dtype=np.float64)
    if np.any(np.isnan(y)):
        raise ValueError("NaN has no bf16 rounding in this oracle")
    _, e = np.frexp(y)                      # |y| in [2^(e-1), 2^e)
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(y, -q)), q)
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, y), r)
    r = np.where(np.isinf(y), y, r)
    r = np.copysign(r, y)                   # keep -0.0
    f32 = r.astype(np.float32)              # exact: r is a bf16 value
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
