"""Pins of the FP8 row-wise oracle (oracle/fp8.py) against exact rationals,
an independent FP8 cast (torch.float8_e4m3fn), invariants and closed forms."""

from fractions import Fraction

import numpy as np
import pytest

from nvfp4_block_scaled_05_amd import inputs as W
from oracle import (NonFiniteInput, bf16_bits_to_f32, dequantize_fp8_rowwise,
                    gemm_fp8_exact_rows, gemm_fp8_fp64, quantize_fp8_rowwise)
from oracle.formats import E4M3_VALUES
from oracle.fp8 import Fp8Rowwise

E4M3_FRACTIONS = [Fraction(float(v)) for v in E4M3_VALUES]   # exact (dyadic)


def _nearest_e4m3(v):
    """Brute force: nearest of the 127 values to the exact v >= 0, ties to the
    even byte, saturating; returns (byte, distance to the nearest midpoint)."""
    best = min(range(127), key=lambda b: (abs(E4M3_FRACTIONS[b] - v), b % 2))
    mids = [(E4M3_FRACTIONS[b] + E4M3_FRACTIONS[b + 1]) / 2 for b in range(126)]
    return best, min(abs(v - m) for m in mids)


@pytest.mark.parametrize("shape,seed", [((3, 16), 1), ((2, 32), 2), ((4, 48), 3)])
def test_codes_are_nearest_e4m3_of_exact_product(shape, seed):
    bits = W.random_matrix(seed, shape, "outliers")
    q = quantize_fp8_rowwise(bits)
    x = bf16_bits_to_f32(bits)
    near_ties = 0
    for r in range(shape[0]):
        s = Fraction(float(np.float32(448) / q.amax[r]))
        for c in range(shape[1]):
            v = abs(Fraction(float(x[r, c]))) * s
            want, gap = _nearest_e4m3(v)
            got = int(q.codes[r, c]) & 0x7F
            if got != want:
                # only where the binary32 product lands on the other side of a tie
                assert gap <= v * Fraction(1, 2 ** 23), (r, c, got, want)
                near_ties += 1
            assert (int(q.codes[r, c]) >> 7) == (int(bits[r, c]) >> 15)
    assert near_ties <= 2


def test_codes_match_torch_float8_cast():
    torch = pytest.importorskip("torch")
    bits = W.random_matrix(4, (64, 256), "t3")
    q = quantize_fp8_rowwise(bits)
    x = bf16_bits_to_f32(bits)
    s = (np.float32(448) / q.amax).astype(np.float32)
    v = (np.abs(x) * s[:, None]).astype(np.float32)       # <= 448 (up to one ulp)
    ref = torch.from_numpy(np.minimum(v, np.float32(448))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q.codes & 0x7F, ref)


def test_row_max_maps_to_448_and_scale_is_reciprocal():
    bits = W.random_matrix(5, (32, 512), "outliers")
    q = quantize_fp8_rowwise(bits)
    x = np.abs(bf16_bits_to_f32(bits))
    for r in range(32):
        j = int(np.argmax(x[r]))
        assert int(q.codes[r, j]) & 0x7F == 0x7E           # 448
    assert np.array_equal(q.scales, (np.float32(1) / (np.float32(448) / q.amax)).astype(np.float32))


def test_power_of_two_covariance_and_sign_symmetry():
    x = bf16_bits_to_f32(W.random_matrix(6, (8, 128), "normal"))
    base = quantize_fp8_rowwise(W.f32_to_bf16_bits(x))
    for k in (-12, -3, 5, 17):
        q = quantize_fp8_rowwise(W.f32_to_bf16_bits(x * np.float32(2.0 ** k)))
        assert np.array_equal(q.codes, base.codes)
        assert np.array_equal(q.scales, (base.scales * np.float32(2.0 ** k)).astype(np.float32))
    neg = quantize_fp8_rowwise(W.f32_to_bf16_bits(-x))
    assert np.array_equal(neg.codes, base.codes ^ 0x80)
    assert np.array_equal(neg.scales, base.scales)


def test_round_trip_is_stable():
    bits = W.random_matrix(7, (16, 256), "normal")
    q = quantize_fp8_rowwise(bits)
    again = quantize_fp8_rowwise(dequantize_fp8_rowwise(q.codes, q.scales))
    assert np.array_equal(again.codes, q.codes)


def test_degenerate_rows_and_errors():
    x = np.zeros((3, 32), np.float32)
    x[1, :] = -0.0
    x[2, 5] = 1e-38                     # below 2^-96: degenerate, codes flush to +-0
    q = quantize_fp8_rowwise(W.f32_to_bf16_bits(x))
    assert np.all(q.scales == 1.0)
    assert np.all(q.codes[0] == 0) and np.all(q.codes[1] == 0x80) and np.all(q.codes[2] == 0)
    bad = np.ones((2, 16), np.float32)
    bad[1, 3] = np.inf
    with pytest.raises(NonFiniteInput):
        quantize_fp8_rowwise(W.f32_to_bf16_bits(bad))
    with pytest.raises(ValueError):
        quantize_fp8_rowwise(np.zeros((2, 24), np.uint16))


def test_gemm_exact_equals_fp64_and_closed_forms():
    a_bits = W.random_matrix(8, (40, 512), "t3")
    w_bits = W.random_matrix(9, (24, 512), "normal", 0.02)
    qa, qw = quantize_fp8_rowwise(a_bits), quantize_fp8_rowwise(w_bits)
    rows = np.arange(40)
    exact, _ = gemm_fp8_exact_rows(qa, qw, rows)
    fp64, _ = gemm_fp8_fp64(qa, qw)
    assert np.array_equal(exact, fp64)
    # constant operands: value 1.0 (0x38) and 2.0 (0x40): Y = K * 2 * dA * dW
    K = 64
    da, dw = np.float32(0.375), np.float32(3.0)
    ca = Fp8Rowwise(np.full((2, K), 0x38, np.uint8), np.full(2, da, np.float32), None)
    cw = Fp8Rowwise(np.full((3, K), 0x40, np.uint8), np.full(3, dw, np.float32), None)
    y, _ = gemm_fp8_exact_rows(ca, cw, [0, 1])
    assert np.all(bf16_bits_to_f32(y) == np.float32(K * 2 * 0.375 * 3.0))
    # identity weight: Y = dequantize(A) within one bf16 ulp
    eye = W.f32_to_bf16_bits(np.eye(512, dtype=np.float32))
    y, _ = gemm_fp8_fp64(qa, quantize_fp8_rowwise(eye))
    deq = bf16_bits_to_f32(dequantize_fp8_rowwise(qa.codes, qa.scales))
    got = bf16_bits_to_f32(y)
    assert np.all(np.abs(got - deq) <= np.abs(deq) * 2.0 ** -7 + 1e-30)
