"""Block-scaled W4A4 GEMM, its epilogue, and the bf16 passthrough linear.

Test infrastructure only (see the package docstring).

The pages ([P2] time-breakdown paragraph; [P3] section "Квантование NVFP4 и
оптимизация вычислительных ядер") say only that the DiT linear layers run an
NVFP4 GEMM on NVFP4 weights.  The definition used here (G1, readings R-14,
R-16, R-19):

    Y[m, n] = bf16( epi( (sum_k A[m,k] * W[n,k]) * sA * sW + bias[n] ) )

where A[m,k] = value(codeA) * S_A[m, k//16] and W[n,k] = value(codeW) *
S_W[n, k//16] are the block-dequantized operands *without* the per-tensor
scales, sA / sW are the stored FP32 per-tensor scales (s_dec) applied once
after the sum, epi is the identity or erf-GELU, and bf16() is one
round-to-nearest-even.  The sum is the exact real value.

Two ways of computing it:
  G2 ``gemm_exact_rows``: every A[m,k] * 2^10 is an integer below 2^22 (E2M1
     values are multiples of 1/2, E4M3 values multiples of 2^-9), so each
     product is below 2^44 and any K <= 16384 sum is exact in int64.
  G3 ``gemm_fp64``: float64 BLAS on the exactly dequantized operands; its
     error is at most about K * 2^-53 of sum |terms|.
Both then apply the same float64 epilogue and one bf16 rounding.
"""

import numpy as np
from scipy.special import erfc

from .formats import (E2M1_MAGNITUDES, bf16_bits_to_f64, e4m3_value,
                      round_to_bf16_bits)
from .quant import BLOCK, unpack_codes


def block_values_f64(codes, scales, cols):
    """value(code) * S for every element, exactly, as float64 [rows, cols]."""
    nib = unpack_codes(codes, cols)
    mag = E2M1_MAGNITUDES[(nib & 7).astype(np.int64)].astype(np.float64)
    val = np.where(nib & 8, -mag, mag)
    S = e4m3_value(np.asarray(scales, dtype=np.uint8)).astype(np.float64)
    return val * np.repeat(S, BLOCK, axis=1)


def _block_values_int(codes, scales, cols):
    """value(code) * S * 2^10 as exact int64 [rows, cols] (G2)."""
    v = block_values_f64(codes, scales, cols) * 1024.0     # exact
    iv = v.astype(np.int64)
    assert np.array_equal(iv.astype(np.float64), v)
    return iv


def gelu_f64(z):
    """erf-form GELU, g(z) = z/2 * (1 + erf(z / sqrt 2)) (R-16), float64.

    Evaluated as z/2 * erfc(-z / sqrt 2), the same function: 1 + erf(u) and
    erfc(-u) are equal, but the erfc form keeps full relative accuracy in the
    negative tail, where 1 + erf(u) cancels (it is wrong by 100% near z = -12).
    """
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * erfc(-z / np.sqrt(2.0))


def epilogue_to_bf16(scaled, bias_bits=None, gelu=False):
    """bias add, optional GELU, one bf16 rounding; float64 in, bf16 bits out."""
    y = np.asarray(scaled, dtype=np.float64)
    if bias_bits is not None:
        y = y + bf16_bits_to_f64(bias_bits)[None, :]
    if gelu:
        y = gelu_f64(y)
    return round_to_bf16_bits(y)


def gemm_fp64(qa, qw, K, bias_bits=None, gelu=False, rows=None):
    """G3.  qa / qw are ``Quantized`` results for A [M,K] and W [N,K].

    rows: optional index array of the rows of A to compute.  Returns
    (y_bits uint16 [len(rows) or M, N], pre_rounding float64 values).
    """
    a_codes, a_scales = qa.codes, qa.scales
    if rows is not None:
        a_codes, a_scales = a_codes[rows], a_scales[rows]
    A = block_values_f64(a_codes, a_scales, K)
    W = block_values_f64(qw.codes, qw.scales, K)
    acc = A @ W.T
    pre = acc * np.float64(qa.tensor_scale) * np.float64(qw.tensor_scale)
    if bias_bits is not None:
        pre = pre + bf16_bits_to_f64(bias_bits)[None, :]
    if gelu:
        pre = gelu_f64(pre)
    return round_to_bf16_bits(pre), pre


def gemm_exact_rows(qa, qw, K, rows, bias_bits=None, gelu=False):
    """G2 on selected rows of A: exact int64 sums, then the float64 epilogue.

    Returns (y_bits [len(rows), N], exact integer sums int64 [len(rows), N]).
    """
    rows = np.asarray(rows)
    IA = _block_values_int(qa.codes[rows], qa.scales[rows], K)
    IW = _block_values_int(qw.codes, qw.scales, K)
    if K > 16384:
        raise ValueError("the int64 bound holds for K <= 16384")
    isum = np.zeros((len(rows), IW.shape[0]), dtype=np.int64)
    for k0 in range(0, K, 256):           # plain int64 products, chunked for memory
        isum += IA[:, k0:k0 + 256] @ IW[:, k0:k0 + 256].T
    scaled = (isum.astype(np.float64) * 2.0 ** -20 * np.float64(qa.tensor_scale)
              * np.float64(qw.tensor_scale))
    return epilogue_to_bf16(scaled, bias_bits, gelu), isum


def linear_bf16_fp64(x_bits, w_bits, bias_bits=None, gelu=False):
    """bf16 passthrough: bf16( epi( sum_k x[m,k] * w[n,k] + bias[n] ) ), float64 sum."""
    X = bf16_bits_to_f64(x_bits)
    Wt = bf16_bits_to_f64(w_bits)
    return epilogue_to_bf16(X @ Wt.T, bias_bits, gelu)
