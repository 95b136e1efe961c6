"""Pins for the oracle's block-scaled GEMM, GELU epilogue and bf16 linear.

  * G2 (exact int64) equals an exact-rational evaluation of the definition on
    tiny shapes, including the bf16 rounding, except at exact-rational ties;
  * G3 (float64 BLAS) equals G2 bit for bit on sampled rows of a DiT-width
    problem, except where the value sits within float64 noise of a bf16 tie;
  * closed forms: constant operands give Y = K * x * w; W = Q(identity) turns
    the GEMM into dequantize(A) within one bf16 ulp;
  * GELU against z * Phi(z) from scipy's normal CDF (a different routine),
    g(0) = 0, odd-part identity g(z) - g(-z) = z, and Phi(1);
  * the bf16 passthrough against an exact-rational dot product.
"""

from fractions import Fraction

import numpy as np
import pytest
from scipy.stats import norm

from oracle.formats import bf16_bits_to_f32, round_to_bf16_bits
from oracle.gemm import (block_values_f64, gelu_f64, gemm_exact_rows, gemm_fp64,
                         linear_bf16_fp64)
from oracle.quant import dequantize, quantize
from nvfp4_block_scaled_05_amd.inputs import f32_to_bf16_bits, random_matrix


def _frac_to_bf16(y):
    """Exact-rational nearest-even rounding to bf16 (normal range), as float."""
    if y == 0:
        return 0.0
    s = -1 if y < 0 else 1
    a = abs(y)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (e - 7)             # 8 significant bits
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return s * float(fl * q)


def _is_tie(y):
    """True when y lies exactly half-way between two bf16 values (normal range)."""
    a = abs(y)
    if a == 0:
        return False
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    n = a / Fraction(2) ** (e - 7)
    return n - n.numerator // n.denominator == Fraction(1, 2)


@pytest.mark.parametrize("K", [16, 32, 64])
def test_G2_equals_exact_rationals(K):
    ties = 0
    for seed in range(4):
        a = random_matrix(30 + seed, (3, K), "t3")
        w = random_matrix(40 + seed, (5, K), "normal", 0.02)
        qa, qw = quantize(a), quantize(w)
        y, isum = gemm_exact_rows(qa, qw, K, np.arange(3))
        A = block_values_f64(qa.codes, qa.scales, K)
        W = block_values_f64(qw.codes, qw.scales, K)
        sa, sw = Fraction(float(qa.tensor_scale)), Fraction(float(qw.tensor_scale))
        yf = bf16_bits_to_f32(y)
        for m in range(3):
            for n in range(5):
                exact = sum(Fraction(float(A[m, k])) * Fraction(float(W[n, k])) for k in range(K))
                assert isum[m, n] == exact * 1024 * 1024
                val = exact * sa * sw
                if _frac_to_bf16(val) != float(yf[m, n]):
                    ties += 1
                    assert _is_tie(val)               # only a rational tie may differ
    assert ties <= 1


def test_G3_equals_G2_on_sampled_rows():
    K = 3072
    a = random_matrix(50, (64, K), "t3")
    w = random_matrix(51, (384, K), "normal", 0.02)
    qa, qw = quantize(a), quantize(w)
    rows = np.arange(0, 64, 4)
    y3, pre = gemm_fp64(qa, qw, K, rows=rows)
    y2, _ = gemm_exact_rows(qa, qw, K, rows)
    diff = y3 != y2
    assert diff.sum() <= 2
    if diff.any():          # a difference must come from a float64-level near tie
        lo = bf16_bits_to_f32(y2[diff]).astype(np.float64)
        hi = bf16_bits_to_f32(y3[diff]).astype(np.float64)
        mid = (lo + hi) / 2
        assert np.all(np.abs(pre[diff] - mid) <= np.abs(mid) * 2.0 ** -40)


def test_closed_form_constant_operands():
    K = 1024
    a = f32_to_bf16_bits(np.ones((8, K), np.float32))
    w = f32_to_bf16_bits(np.full((16, K), 0.5, np.float32))
    qa, qw = quantize(a), quantize(w)
    y, _ = gemm_fp64(qa, qw, K)
    assert np.all(bf16_bits_to_f32(y) == np.float32(K * 0.5))
    # with a bias: K/2 + 12 (a bf16 value: 524 has quantum 4)
    bias = f32_to_bf16_bits(np.full(16, 12.0, np.float32))
    y, _ = gemm_fp64(qa, qw, K, bias_bits=bias)
    assert np.all(bf16_bits_to_f32(y) == np.float32(K * 0.5 + 12))


def test_identity_weight_gives_dequantize():
    K = 256
    a = random_matrix(52, (32, K), "outliers")
    qa = quantize(a)
    qi = quantize(f32_to_bf16_bits(np.eye(K, dtype=np.float32)))
    y, _ = gemm_fp64(qa, qi, K)
    d = dequantize(qa.codes, qa.scales, qa.tensor_scale, K)
    # compare values: a sum of zeros is +0 where dequantize keeps -0
    y, d = y & np.uint16(0xFFFF), np.where(d == 0x8000, np.uint16(0), d)
    ulp = np.abs(y.astype(np.int32) - d.astype(np.int32))
    assert ulp.max() <= 1
    assert (ulp == 0).mean() > 0.99


def test_gelu_pins():
    z = np.linspace(-8, 8, 4001)
    assert gelu_f64(np.array([0.0]))[0] == 0.0
    assert np.allclose(gelu_f64(z) - gelu_f64(-z), z, rtol=0, atol=1e-14)
    assert np.allclose(gelu_f64(z), z * norm.cdf(z), rtol=1e-13, atol=1e-15)
    # the negative tail keeps relative accuracy (no cancellation)
    zt = np.linspace(-30, -5, 1001)
    assert np.allclose(gelu_f64(zt), zt * norm.cdf(zt), rtol=1e-12, atol=0)
    assert abs(gelu_f64(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15


def test_gelu_epilogue_rounds_once():
    K = 64
    a = random_matrix(53, (4, K), "normal")
    w = random_matrix(54, (8, K), "normal", 0.2)
    qa, qw = quantize(a), quantize(w)
    y, pre = gemm_fp64(qa, qw, K, gelu=True)
    _, lin = gemm_fp64(qa, qw, K)
    assert np.array_equal(pre, gelu_f64(lin))
    assert np.array_equal(y, round_to_bf16_bits(gelu_f64(lin)))


def test_bf16_linear_exact_rationals():
    x = random_matrix(55, (3, 48), "normal")
    w = random_matrix(56, (4, 48), "normal", 0.02)
    bias = random_matrix(57, (1, 4), "normal")[0]
    y = bf16_bits_to_f32(linear_bf16_fp64(x, w, bias))
    xf, wf, bf = bf16_bits_to_f32(x), bf16_bits_to_f32(w), bf16_bits_to_f32(bias)
    for m in range(3):
        for n in range(4):
            exact = sum(Fraction(float(xf[m, k])) * Fraction(float(wf[n, k])) for k in range(48))
            exact += Fraction(float(bf[n]))
            assert _frac_to_bf16(exact) == float(y[m, n])
