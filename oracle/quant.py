"""Two-level NVFP4 quantize and dequantize, step by step.

Test infrastructure only (see the package docstring).

What the pages fix ([P1] section "NVFP4量化"): a tensor is scaled twice -- one
per-tensor scale stored in FP32 ("static or dynamic"; dynamic here, R-19) and a
per-block scale computed dynamically, in real time, for every block of 16
elements.  Everything else is a reading, named where it is used:

  Q0  cols % 16 == 0; any Inf / NaN input is an error (R-17, R-18).
  Q1  amax = max |x| over the tensor (exact).
  Q2  s_enc = 2688 / amax, s_dec = 1 / s_enc, binary32 round-to-nearest
      (2688 = 6 * 448 = largest E2M1 magnitude * largest E4M3 value, R-3);
      the stored FP32 per-tensor scale is s_dec.  amax < 2^-96 (including an
      all-zero tensor) is degenerate: s_enc = s_dec = 1 (R-5).
  Q3  a_b = max |x| over each block of 16 consecutive elements of a row (R-4).
  Q4  t_b = (a_b / 6) * s_enc, then S_b = E4M3 nearest-even, saturating (R-6).
  Q5  S_b == 0: every code of the block is its input's sign bit only (R-7).
      Otherwise e_b = 1 / (S_b * s_dec), v = |x| * e_b, and
      code = sign(x) << 3 | E2M1(v) (R-7, R-8).
  Q6  two codes per byte, element 2j in the low nibble (R-10).
  Q7  scales stored row-major [rows, cols/16] (R-11).

  D1  dequantize: bf16( (value(code) * S_b) * s_dec ), binary32 products and
      one rounding to bf16 (R-13).

All binary32 steps are explicit ``numpy.float32`` scalar/array operations,
which are IEEE-754 round-to-nearest-even with gradual underflow.
"""

from dataclasses import dataclass

import numpy as np

from .formats import (E2M1_MAGNITUDES, bf16_bits_to_f32, e2m1_encode_magnitude,
                      e4m3_encode_nonneg, e4m3_value, round_to_bf16_bits)

BLOCK = 16                      # [P1] "NVFP4量化": blocks of 16 elements
F32 = np.float32
_TINY_AMAX = F32(2.0 ** -96)    # R-5


class NonFiniteInput(ValueError):
    """Raised for an input tensor holding +-Inf or NaN (R-17)."""


@dataclass
class Quantized:
    codes: np.ndarray         # uint8 [rows, cols/2]
    scales: np.ndarray        # uint8 [rows, cols/16], E4M3 bytes
    tensor_scale: np.float32  # s_dec, the stored FP32 per-tensor scale
    amax: np.float32          # the amax the scales were derived from
    s_enc: np.float32
    degenerate: bool


def unpack_codes(codes, cols):
    """uint8 [rows, cols/2] -> uint8 nibble codes [rows, cols] (R-10)."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty((codes.shape[0], cols), dtype=np.uint8)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out


def _pack(nibbles):
    return (nibbles[:, 0::2] | (nibbles[:, 1::2] << 4)).astype(np.uint8)


def tensor_scales(amax):
    """Q2: (s_enc, s_dec, degenerate) from a binary32 amax."""
    amax = F32(amax)
    if amax < _TINY_AMAX:
        return F32(1.0), F32(1.0), True
    s_enc = F32(2688.0) / amax
    s_dec = F32(1.0) / s_enc
    return s_enc, s_dec, False


def quantize(x_bits, amax=None):
    """Quantize a bf16 tensor [rows, cols] to NVFP4.

    x_bits: uint16 bf16 bit patterns, 2-D.  amax: optional binary32 amax
    supplied by the producer of x (the GEMM epilogue in an MLP); when None it is
    computed here (Q1).  Returns a ``Quantized``.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2:
        raise ValueError("quantize takes a 2-D tensor")
    rows, cols = x_bits.shape
    if cols % BLOCK != 0 or cols == 0:
        raise ValueError("cols must be a positive multiple of 16 (R-18)")
    x = bf16_bits_to_f32(x_bits)
    if not np.all(np.isfinite(x)):                           # Q0
        raise NonFiniteInput("non-finite value in the input tensor")
    mag = np.abs(x)
    sign = (x_bits >> np.uint16(15)).astype(np.uint8)       # 1 for negative, -0.0 included

    if amax is None:                                          # Q1
        amax = mag.max() if mag.size else F32(0.0)
    amax = F32(amax)
    s_enc, s_dec, degenerate = tensor_scales(amax)            # Q2

    nblk = cols // BLOCK
    blocks = mag.reshape(rows, nblk, BLOCK)
    a_b = blocks.max(axis=2) if rows else np.zeros((0, nblk), F32)   # Q3

    if degenerate:
        S = np.zeros((rows, nblk), dtype=np.uint8)
    else:
        t_b = (a_b / F32(6.0)) * s_enc                         # Q4, binary32
        S = e4m3_encode_nonneg(t_b)

    nib = np.zeros((rows, nblk, BLOCK), dtype=np.uint8)
    live = S != 0
    if np.any(live):
        S_val = e4m3_value(S)                                  # exact binary32
        with np.errstate(divide="ignore"):
            e_b = F32(1.0) / (S_val * s_dec)                   # Q5, binary32
        v = blocks[live] * e_b[live][:, None]                 # binary32 products
        nib[live] = e2m1_encode_magnitude(v)
    nib |= sign.reshape(rows, nblk, BLOCK) << 3               # R-7: sign always kept

    codes = _pack(nib.reshape(rows, cols))                    # Q6
    return Quantized(codes=codes, scales=S, tensor_scale=s_dec, amax=amax,
                     s_enc=s_enc, degenerate=degenerate)      # Q7


def dequantize(codes, scales, tensor_scale, cols):
    """D1: NVFP4 -> bf16 bit patterns [rows, cols] (R-13)."""
    nib = unpack_codes(codes, cols)
    rows = nib.shape[0]
    mag = E2M1_MAGNITUDES[(nib & 7).astype(np.int64)]
    val = np.where(nib & 8, -mag, mag).astype(F32)            # code 8 -> -0.0
    S = e4m3_value(np.asarray(scales, dtype=np.uint8))
    S_el = np.repeat(S, BLOCK, axis=1).reshape(rows, cols)
    p = val * S_el                                            # exact in binary32
    q = p * F32(tensor_scale)                                 # one binary32 rounding
    return round_to_bf16_bits(q)
