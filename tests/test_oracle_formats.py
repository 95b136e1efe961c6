"""Pins for the oracle's number formats (E2M1, E4M3, bf16 rounding).

Each converter is checked against something other than itself:
  * E2M1: brute-force nearest search in exact rationals around every midpoint
    and representable value, plus monotonicity over a dense sweep, plus the
    representable set of the NVFP4 element format {0, .5, 1, 1.5, 2, 3, 4, 6}.
  * E4M3: torch's float8_e4m3fn cast (an independent library conversion,
    round-to-nearest-even) on [0, 464], brute-force rationals, special values.
  * bf16: torch's float32 -> bfloat16 cast, and exact rationals from float64.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.formats import (E2M1_MAGNITUDES, E4M3_VALUES, bf16_bits_to_f32,
                            e2m1_encode_magnitude, e2m1_value,
                            e4m3_encode_nonneg, e4m3_value, round_to_bf16_bits)


def _f32_neighbourhood(center, radius):
    c = np.array([center], dtype=np.float32).view(np.int32)[0]
    lo = max(int(c) - radius, 0)
    bits = np.arange(lo, int(c) + radius + 1, dtype=np.int64).astype(np.int32)
    return bits.view(np.float32)


def _nearest_even(value, table):
    """Brute force: index of the nearest table entry, exact rationals, ties -> even index."""
    v = Fraction(float(value))
    best, best_d = None, None
    for i, t in enumerate(table):
        d = abs(v - t)
        if best_d is None or d < best_d or (d == best_d and i % 2 == 0):
            best, best_d = i, d
    return best


# ---------------------------------------------------------------- E2M1 -----

def test_e2m1_representable_set():
    # The NVFP4 element values: {0, 0.5, 1, 1.5, 2, 3, 4, 6}, codes 0..7 in order.
    assert [float(e2m1_value(c)) for c in range(8)] == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(E2M1_MAGNITUDES) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    # codes 8..15 are the negatives, code 8 is negative zero
    for c in range(8):
        assert e2m1_value(c + 8) == -e2m1_value(c)


def test_e2m1_bit_layout():
    # sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0
    assert e2m1_value(0b0011) == Fraction(3, 2)      # e=1, m=1 -> 1.5
    assert e2m1_value(0b0111) == 6                   # e=3, m=1 -> 4 * 1.5
    assert e2m1_value(0b0001) == Fraction(1, 2)      # subnormal
    assert e2m1_value(0b1101) == -3


def test_e2m1_encode_brute_force_near_every_boundary():
    mags = [Fraction(float(m)) for m in E2M1_MAGNITUDES]
    pts = [0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0, 7.0]
    vals = np.concatenate([_f32_neighbourhood(p, 160) for p in pts])
    got = e2m1_encode_magnitude(vals)
    for v, g in zip(vals, got):
        assert g == _nearest_even(v, mags), (float(v), int(g))


def test_e2m1_encode_brute_force_random_and_large():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.uniform(0, 8, 4000).astype(np.float32),
        np.exp(rng.uniform(-100, 80, 2000)).astype(np.float32),
        np.array([np.finfo(np.float32).max, 1e-45, 6.0, 100.0], dtype=np.float32)])
    mags = [Fraction(float(m)) for m in E2M1_MAGNITUDES]
    got = e2m1_encode_magnitude(vals)
    for v, g in zip(vals, got):
        assert g == _nearest_even(v, mags), (float(v), int(g))


def test_e2m1_exact_ties_go_to_even_code():
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    assert list(e2m1_encode_magnitude(ties)) == [0, 2, 2, 4, 4, 6, 6]


def test_e2m1_encode_monotone_dense_sweep():
    # every 97th binary32 pattern from 0 to 16.0: the code never decreases
    bits = np.arange(0, 0x41800000, 97, dtype=np.int64).astype(np.int32)
    codes = e2m1_encode_magnitude(bits.view(np.float32))
    assert np.all(np.diff(codes.astype(np.int16)) >= 0)
    assert codes[0] == 0 and codes[-1] == 7


# ---------------------------------------------------------------- E4M3 -----

def test_e4m3_decode_matches_torch():
    b = np.arange(0, 256, dtype=np.uint8)
    finite = (b & 0x7F) != 0x7F
    ref = torch.from_numpy(b[finite]).view(torch.float8_e4m3fn).float().numpy()
    ours = e4m3_value(b[finite])
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_e4m3_special_values():
    assert float(e4m3_value(np.uint8(0x7E))) == 448.0
    assert float(e4m3_value(np.uint8(0x08))) == 2.0 ** -6
    assert float(e4m3_value(np.uint8(0x01))) == 2.0 ** -9
    t = np.array([2.0 ** -10, 1.5 * 2.0 ** -10, 448.0, 460.0, 1e9, 0.0], dtype=np.float32)
    assert list(e4m3_encode_nonneg(t)) == [0x00, 0x01, 0x7E, 0x7E, 0x7E, 0x00]
    assert len(E4M3_VALUES) == 127 and np.all(np.diff(E4M3_VALUES) > 0)


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(2)
    parts = [rng.uniform(0, 464, 1_000_000).astype(np.float32),
             np.exp2(rng.uniform(-20, np.log2(463.9), 1_000_000)).astype(np.float32)]
    mids = (E4M3_VALUES[:-1] + E4M3_VALUES[1:]) / 2
    for c in np.concatenate([mids, E4M3_VALUES]):
        if c < 464:
            parts.append(_f32_neighbourhood(c, 64))
    t = np.concatenate(parts)
    t = t[(t >= 0) & (t < 464)]
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode_nonneg(t), ref)


def test_e4m3_encode_brute_force_rationals():
    table = [Fraction(float(v)) for v in E4M3_VALUES]
    rng = np.random.default_rng(3)
    mids = (E4M3_VALUES[:-1] + E4M3_VALUES[1:]) / 2
    t = np.concatenate([mids.astype(np.float32), rng.uniform(0, 600, 600).astype(np.float32),
                        np.exp2(rng.uniform(-14, 9, 600)).astype(np.float32)])
    got = e4m3_encode_nonneg(t)
    for v, g in zip(t, got):
        assert g == _nearest_even(v, table), (float(v), int(g))


# ---------------------------------------------------------------- bf16 -----

def test_bf16_round_matches_torch_from_f32():
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        (rng.standard_normal(20000) * 1e-39).astype(np.float32),
                        np.exp(rng.uniform(-80, 80, 20000)).astype(np.float32)])
    # exact ties: bf16 value + half its quantum
    base = rng.standard_normal(5000).astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    x = np.concatenate([x, (base | np.uint32(0x8000)).view(np.float32), np.array([-0.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(round_to_bf16_bits(x), ref)


def test_bf16_round_from_f64_is_nearest():
    rng = np.random.default_rng(5)
    y = rng.standard_normal(30000) * np.exp(rng.uniform(-30, 30, 30000))
    got = round_to_bf16_bits(y)
    back = bf16_bits_to_f32(got).astype(np.float64)
    bits = got.astype(np.int32)
    for delta in (-1, 1):           # neither bf16 neighbour is closer
        nb = bf16_bits_to_f32((bits + delta).astype(np.uint16)).astype(np.float64)
        assert np.all(np.abs(y - back) <= np.abs(y - nb))
    # exact float64 ties between two bf16 values go to the even pattern
    lo = bf16_bits_to_f32(np.array([0x3F80, 0x3F81], np.uint16)).astype(np.float64)
    assert round_to_bf16_bits(np.array([(lo[0] + lo[1]) / 2]))[0] == 0x3F80
    lo = bf16_bits_to_f32(np.array([0x3F81, 0x3F82], np.uint16)).astype(np.float64)
    assert round_to_bf16_bits(np.array([(lo[0] + lo[1]) / 2]))[0] == 0x3F82
