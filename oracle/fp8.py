"""FP8 row-wise quantize, dequantize and W8A8 GEMM (the "fp8r" variant).

Test infrastructure only (see the package docstring).

Besides NVFP4, the pages select an FP8 variant of the same model with
``--variant fp8r`` ([P3], the paragraph on running the pipeline) and give no
recipe for it.  Reading R-22: "fp8r" is FP8 with row-wise scales -- one FP32
scale per row of the activation (per token, computed dynamically on every
call) and one per row of the weight (per output channel, computed when the
weights are loaded), E4M3 elements (R-2), and a GEMM that sums the products of
the E4M3 values and applies the two row scales in the epilogue:

  F0  cols % 16 == 0; any Inf / NaN input is an error (as R-17, R-18).
  F1  amax_r = max |x| over row r (exact).
  F2  s_r = 448 / amax_r, d_r = 1 / s_r, binary32 round-to-nearest-even; d_r
      is the stored scale.  amax_r < 2^-96 (an all-zero row included) is
      degenerate: s_r = d_r = 1 (as R-5).
  F3  q = sign(x) << 7 | E4M3(|x| * s_r), the product in binary32, then
      nearest-even, saturating at 448; the sign of zero is kept (as R-7).
  F4  dequantize: bf16( value(q) * d_r ), one binary32 product, one rounding.
  G   Y[m,n] = bf16( epi( (sum_k value(qa[m,k]) * value(qw[n,k]))
                          * (dA[m] * dW[n]) + bias[n] ) )
      with the sum exact, dA[m] * dW[n] one binary32 product, and the rest as
      the NVFP4 epilogue (gemm.epilogue_to_bf16).
"""

from dataclasses import dataclass

import numpy as np

from .formats import bf16_bits_to_f32, e4m3_encode_nonneg, e4m3_value, round_to_bf16_bits
from .gemm import epilogue_to_bf16
from .quant import NonFiniteInput

F32 = np.float32
_TINY_AMAX = F32(2.0 ** -96)


@dataclass
class Fp8Rowwise:
    codes: np.ndarray    # uint8 [rows, cols], E4M3 bytes (sign in bit 7)
    scales: np.ndarray   # float32 [rows], d_r
    amax: np.ndarray     # float32 [rows]


def quantize_fp8_rowwise(x_bits):
    """F0-F3 on bf16 bit patterns [rows, cols]."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2 or x_bits.shape[1] % 16 != 0 or x_bits.shape[1] == 0:
        raise ValueError("cols must be a positive multiple of 16")
    x = bf16_bits_to_f32(x_bits)
    if not np.all(np.isfinite(x)):
        raise NonFiniteInput("Inf or NaN in the input")
    amax = np.abs(x).max(axis=1).astype(F32)
    degenerate = amax < _TINY_AMAX
    safe = np.where(degenerate, F32(1), amax).astype(F32)
    s = np.where(degenerate, F32(1), F32(448) / safe).astype(F32)
    d = np.where(degenerate, F32(1), F32(1) / s).astype(F32)
    v = (np.abs(x) * s[:, None]).astype(F32)
    mag = e4m3_encode_nonneg(v)
    sign = ((x_bits >> 15) & 1).astype(np.uint8) << 7
    return Fp8Rowwise(codes=(mag | sign).astype(np.uint8), scales=d, amax=amax)


def dequantize_fp8_rowwise(codes, scales):
    """F4: bf16 bit patterns [rows, cols]."""
    val = e4m3_value(np.asarray(codes, dtype=np.uint8))
    return round_to_bf16_bits((val * np.asarray(scales, dtype=F32)[:, None]).astype(F32))


def _scaled_ints(codes):
    """value(q) * 2^9 as exact int64 (E4M3 values are multiples of 2^-9)."""
    v = e4m3_value(np.asarray(codes, dtype=np.uint8)).astype(np.float64) * 512.0
    iv = v.astype(np.int64)
    assert np.array_equal(iv.astype(np.float64), v)
    return iv


def _row_col_scale(qa, qw, rows):
    da = np.asarray(qa.scales, dtype=F32)[rows]
    dw = np.asarray(qw.scales, dtype=F32)
    return (da[:, None] * dw[None, :]).astype(F32).astype(np.float64)   # one binary32 product


def gemm_fp8_exact_rows(qa, qw, rows, bias_bits=None, gelu=False):
    """G on selected rows of A with int64 sums: |value * 2^9| <= 229376, so
    each product is below 2^36 and any K below 2^27 sums exactly."""
    rows = np.asarray(rows)
    ia = _scaled_ints(qa.codes[rows])
    iw = _scaled_ints(qw.codes)
    if ia.shape[1] >= 1 << 27:
        raise ValueError("the int64 bound holds for K < 2^27")
    isum = np.zeros((len(rows), iw.shape[0]), dtype=np.int64)
    for k0 in range(0, ia.shape[1], 256):
        isum += ia[:, k0:k0 + 256] @ iw[:, k0:k0 + 256].T
    pre = isum.astype(np.float64) * 2.0 ** -18 * _row_col_scale(qa, qw, rows)
    return epilogue_to_bf16(pre, bias_bits, gelu), isum


def gemm_fp8_fp64(qa, qw, bias_bits=None, gelu=False, rows=None):
    """G with a float64 BLAS sum of the exact E4M3 values (error about
    K * 2^-53 of sum |terms|); returns (y_bits, pre-rounding values)."""
    rows = np.arange(qa.codes.shape[0]) if rows is None else np.asarray(rows)
    a = e4m3_value(qa.codes[rows]).astype(np.float64)
    w = e4m3_value(qw.codes).astype(np.float64)
    pre = (a @ w.T) * _row_col_scale(qa, qw, rows)
    return epilogue_to_bf16(pre, bias_bits, gelu), pre
