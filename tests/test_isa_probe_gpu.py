"""The gfx950 conversions the kernels rely on, against the CPU oracle, on every
input the kernels can give them (through lib/libnvfp4_probes.so, which
calls the kernels' own device helpers).

  * E2M1 encode: monotone in the binary32 pattern, so the exact list of
    patterns where the code changes, over all 2^31 - 2^23 non-NaN patterns of
    each sign, plus one anchor value per range, determines it completely.
  * E4M3 encode (block scale, non-negative inputs): same scan over [0, +Inf].
  * E2M1 decode to fp16 and fp32, and E4M3 decode to fp16 (hardware pair
    conversion) and fp32 (integer decoder): every byte value in every byte
    position of a word.
  * The single-pass quantizer's block-scale path: a / 6 against IEEE binary32
    division, the scale byte against the oracle's E4M3 encode, and the codes
    of a zero-scale block, on every bf16 pattern.
"""

import ctypes
import os

import numpy as np
import pytest

from oracle.formats import (E2M1_MAGNITUDES, e2m1_encode_magnitude, e4m3_encode_nonneg,
                            e4m3_value, round_to_bf16_bits)
from oracle.gemm import gelu_f64

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE_LIB = os.path.join(ROOT, "nvfp4_block_scaled_05_amd", "lib", "libnvfp4_probes.so")
CAP = 4096


@pytest.fixture(scope="module")
def probe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = ctypes.CDLL(PROBE_LIB)
    P, U, I = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int
    lib.nvfp4_probe_transitions.argtypes = [I, U, U, P, U, P, P, P]
    lib.nvfp4_probe_encode.argtypes = [I, P, I, P, P]
    lib.nvfp4_probe_decode.argtypes = [P, P, I, P, P, P, P, P]
    lib.nvfp4_probe_bf16_gelu.argtypes = [P, I, P, P, P]
    lib.nvfp4_probe_gelu16.argtypes = [P, I, P, P]
    lib.nvfp4_probe_block_scale.argtypes = [P, I, ctypes.c_float, P, P, P, P]
    return lib


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _scan(lib, which, lo, hi):
    import torch
    lst = torch.zeros(3 * CAP, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    mm = torch.zeros(1, dtype=torch.int32, device="cuda")
    rc = lib.nvfp4_probe_transitions(which, lo, (hi - lo) // 256, lst.data_ptr(), CAP,
                                     cnt.data_ptr(), mm.data_ptr(), _stream())
    assert rc == 0
    torch.cuda.synchronize()
    n = int(cnt.item())
    assert n <= CAP
    t = lst.cpu().numpy().view(np.uint32)[: 3 * n].reshape(n, 3)
    return sorted(map(tuple, t.tolist())), int(mm.item())


def _encode(lib, which, bits):
    import torch
    b = torch.from_numpy(np.asarray(bits, np.uint32).view(np.int32)).cuda()
    out = torch.zeros_like(b)
    assert lib.nvfp4_probe_encode(which, b.data_ptr(), b.numel(), out.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32)


def _e2m1_code(bits):
    bits = np.atleast_1d(np.asarray(bits, np.uint32))
    v = bits.view(np.float32)
    return (e2m1_encode_magnitude(np.abs(v)) | ((bits >> 31) << 3)).astype(np.uint32)


def _e4m3_code(bits):
    return e4m3_encode_nonneg(np.atleast_1d(np.asarray(bits, np.uint32)).view(np.float32)).astype(np.uint32)


def _expected_transitions(code_fn, lo, hi):
    """Patterns p in (lo, hi] where the oracle's code differs from p - 1 (bisection;
    the oracle is monotone over the range)."""
    out = []
    c_lo, c_hi = int(code_fn(lo)[0]), int(code_fn(hi)[0])
    start = lo
    while start < hi and int(code_fn(start)[0]) != c_hi:
        c0 = int(code_fn(start)[0])
        a, b = start, hi          # code(a) == c0, code(b) != c0
        while b - a > 1:
            mid = (a + b) // 2
            if int(code_fn(mid)[0]) == c0:
                a = mid
            else:
                b = mid
        out.append((b, c0, int(code_fn(b)[0])))
        start = b
    assert out or c_lo == c_hi
    return out


@pytest.mark.parametrize("lo,hi", [(0x00000000, 0x7F800000), (0x80000000, 0xFF800000)])
def test_e2m1_encode_every_binary32_pattern(probe, lo, hi):
    got, mismatch = _scan(probe, 0, lo, hi)
    assert mismatch == 0, "byte positions / nibbles of the packed conversion disagree"
    want = _expected_transitions(_e2m1_code, lo, hi)
    assert len(want) == 7
    assert got == want
    anchors = np.array([lo, lo + 1, hi], np.uint32)
    codes = _encode(probe, 0, anchors) & 0xF
    assert list(codes) == list(_e2m1_code(anchors))


def test_e2m1_encode_spot_values(probe):
    vals = np.array([0.0, -0.0, 0.25, 0.2500001, -0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.0000005,
                     6.0, 7.0, 1e30, -1e-40, 1e-45], np.float32)
    bits = vals.view(np.uint32)
    codes = _encode(probe, 0, bits)
    assert np.all(codes == (codes & 0xF) * 0x11111111)
    assert list(codes & 0xF) == list(_e2m1_code(bits))


def test_e4m3_encode_every_nonnegative_pattern(probe):
    lo, hi = 0x00000000, 0x7F800000
    got, mismatch = _scan(probe, 1, lo, hi)
    assert mismatch == 0
    want = _expected_transitions(_e4m3_code, lo, hi)
    assert len(want) == 126
    assert got == want
    anchors = np.array([lo, 0x3A800000, 0x43E00000, hi], np.uint32)   # 0, 2^-10, 448, +Inf
    assert list(_encode(probe, 1, anchors)) == list(_e4m3_code(anchors))


def test_fp8_row_encode_every_nonnegative_pattern(probe):
    # the FP8 row quantizer's element encode (clamp to 448, hardware packed
    # conversion) has exactly the transitions of the oracle's E4M3 encoder
    lo, hi = 0x00000000, 0x7F800000
    got, mismatch = _scan(probe, 2, lo, hi)
    assert mismatch == 0, "byte positions of the packed conversion disagree"
    want = _expected_transitions(_e4m3_code, lo, hi)
    assert got == want
    anchors = np.array([lo, 0x3A800000, 0x3A800001, 0x43E00000, 0x43E80000, hi], np.uint32)
    assert list(_encode(probe, 2, anchors) & 0xFF) == list(_e4m3_code(anchors))


def test_decodes_every_byte_and_scale(probe):
    import torch
    # every byte value in every byte position, times every finite E4M3 scale
    byte = np.repeat(np.arange(256, dtype=np.uint32), 127)
    sbyte = np.tile(np.arange(127, dtype=np.uint32), 256)
    words = byte * np.uint32(0x01010101)
    n = len(words)
    w = torch.from_numpy(words.view(np.int32)).cuda()
    sb = torch.from_numpy(sbyte.view(np.int32)).cuda()
    f16 = torch.zeros(n * 8, dtype=torch.int16, device="cuda")
    f32 = torch.zeros(n * 8, dtype=torch.float32, device="cuda")
    s16 = torch.zeros(n * 4, dtype=torch.int16, device="cuda")
    s32 = torch.zeros(n * 4, dtype=torch.float32, device="cuda")
    assert probe.nvfp4_probe_decode(w.data_ptr(), sb.data_ptr(), n, f16.data_ptr(), f32.data_ptr(),
                                    s16.data_ptr(), s32.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    f16 = f16.cpu().numpy().view(np.uint16).reshape(n, 8)
    f32 = f32.cpu().numpy().reshape(n, 8)
    s16 = s16.cpu().numpy().view(np.uint16).reshape(n, 4)
    s32 = s32.cpu().numpy().reshape(n, 4)
    S = e4m3_value(sbyte.astype(np.uint8)).astype(np.float64)
    for j in range(8):
        code = (byte & 0xF) if j % 2 == 0 else (byte >> 4)
        val = np.copysign(E2M1_MAGNITUDES[code & 7].astype(np.float64), np.where(code & 8, -1.0, 1.0))
        assert np.array_equal(f32[:, j].view(np.uint32), val.astype(np.float32).view(np.uint32)), j
        prod = val * S                        # exact; representable in fp16
        want = prod.astype(np.float16)
        assert np.array_equal(want.astype(np.float64), prod)
        bad = np.nonzero(f16[:, j] != want.view(np.uint16))[0]
        assert len(bad) == 0, (j, [(int(byte[k]), int(sbyte[k]), hex(f16[k, j])) for k in bad[:8]])
    # hardware pair conversion: every finite E4M3 byte, both signs
    finite = (byte & 0x7F) != 0x7F
    want = e4m3_value(byte[finite].astype(np.uint8))
    for j in range(4):
        assert np.array_equal(s16[finite, j], want.astype(np.float16).view(np.uint16))
    # integer decoder: its domain is the scale bytes a quantizer writes, 0x00..0x7E
    scale_bytes = byte <= 0x7E
    want = e4m3_value(byte[scale_bytes].astype(np.uint8))
    for j in range(4):
        assert np.array_equal(s32[scale_bytes, j].view(np.uint32), want.view(np.uint32))


def _bf16_gelu(lib, x):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    b = torch.zeros(len(x), dtype=torch.int16, device="cuda")
    g = torch.zeros(len(x), dtype=torch.float32, device="cuda")
    assert lib.nvfp4_probe_bf16_gelu(t.data_ptr(), len(x), b.data_ptr(), g.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    return b.cpu().numpy().view(np.uint16), g.cpu().numpy()


def test_bf16_conversion_rounds_to_nearest_even(probe):
    rng = np.random.default_rng(7)
    parts = [rng.standard_normal(1 << 20).astype(np.float32),
             np.exp(rng.uniform(-87, 88, 1 << 20)).astype(np.float32) * rng.choice([-1, 1], 1 << 20),
             (rng.standard_normal(1 << 16) * 1e-39).astype(np.float32)]
    # exact ties and their neighbours for every exponent: bf16 value + half its quantum
    hi = (np.arange(1 << 16, dtype=np.uint32) << 16)
    hi = hi[((hi >> 23) & 0xFF) != 0xFF]
    ties = hi | np.uint32(0x8000)
    parts += [ties.view(np.float32), (ties + 1).view(np.float32), (ties - 1).view(np.float32)]
    x = np.concatenate(parts)
    if len(x) % 2:
        x = x[:-1]
    got, _ = _bf16_gelu(probe, x)
    assert np.array_equal(got, round_to_bf16_bits(x))


def test_gelu_matches_oracle(probe):
    z = np.concatenate([np.linspace(-40, 40, 400002), np.random.default_rng(8).standard_normal(100000) * 3])
    z = z.astype(np.float32)
    _, g = _bf16_gelu(probe, z)
    ref = gelu_f64(z.astype(np.float64))
    # relative error far below a bf16 ulp (2^-8 = 3.9e-3; the epilogues round
    # GELU to bf16): the degree-5 fit of erfc is good to 8e-6, plus a few
    # binary32 ulps of the reciprocal, the Horner steps and exp2; in the far
    # tail binary32 rounding of x^2 and of the exponent argument (|arg| up to
    # 800 at |z| = 40) adds a few 1e-6
    big = np.abs(ref) > 1e-30
    rel = np.abs(g - ref) / np.where(big, np.abs(ref), 1.0)
    near = np.abs(z) <= 4
    assert rel[near & big].max() < 2e-5, rel[near & big].max()
    assert rel[big].max() < 5e-5, rel[big].max()
    assert np.all(np.abs(g[~big]) <= 1e-30)


def test_gelu16_equals_scalar_gelu_bitwise(probe):
    # the epilogues' 16-wide GELU against the scalar one, bit for bit, on
    # signed zeros, subnormals, infinities, NaN, huge values and a wide sweep
    import torch
    special = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-39, -1e-39, np.inf, -np.inf, np.nan,
                        3.4e38, -3.4e38, 1e30, -1e30, 0.5, -0.5, -0.75, 6.0, -6.0], np.float32)
    rng = np.random.default_rng(9)
    z = np.concatenate([special, np.linspace(-40, 40, 200014, dtype=np.float32),
                        (rng.standard_normal(100000) * 5).astype(np.float32),
                        rng.integers(0, 1 << 32, 100000, dtype=np.uint64).astype(np.uint32).view(np.float32)])
    z = z[: len(z) // 16 * 16]
    _, g1 = _bf16_gelu(probe, z)
    t = torch.from_numpy(np.ascontiguousarray(z)).cuda()
    o = torch.empty_like(t)
    assert probe.nvfp4_probe_gelu16(t.data_ptr(), len(z), o.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    g16 = o.cpu().numpy()
    nan1, nan16 = np.isnan(g1), np.isnan(g16)
    assert np.array_equal(nan1, nan16)
    assert np.array_equal(g1[~nan1].view(np.uint32), g16[~nan16].view(np.uint32))


@pytest.mark.parametrize("s_enc", [1.0, 2688.0 / 3.0, 2688.0 / 0.0123, 2688.0 / 6e4, 2688.0 / 3e-30, 1e30])
def test_block_scale_path_every_bf16(probe, s_enc):
    import torch
    h = np.arange(1 << 16, dtype=np.uint32)
    b = torch.from_numpy(h.view(np.int32)).cuda()
    quot = torch.zeros(h.size, dtype=torch.float32, device="cuda")
    scale = torch.zeros(h.size, dtype=torch.int32, device="cuda")
    zc = torch.zeros(h.size, dtype=torch.int32, device="cuda")
    s = np.float32(s_enc)
    assert probe.nvfp4_probe_block_scale(b.data_ptr(), h.size, float(s), quot.data_ptr(),
                                         scale.data_ptr(), zc.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    a = ((h & 0x7FFF) << 16).view(np.float32)
    finite = (h & 0x7FFF) < 0x7F80
    with np.errstate(invalid="ignore"):
        want_q = a / np.float32(6.0)                  # IEEE binary32 division
    got_q = quot.cpu().numpy()
    assert np.array_equal(got_q[finite].view(np.uint32), want_q[finite].view(np.uint32))
    with np.errstate(over="ignore"):
        t = (want_q * s).astype(np.float32)
    want_s = e4m3_encode_nonneg(t[finite])
    assert np.array_equal(scale.cpu().numpy().view(np.uint32)[finite], want_s.astype(np.uint32))
    want_z = np.where(h >> 15, 0x88888888, 0).astype(np.uint32)   # sign-only codes
    assert np.array_equal(zc.cpu().numpy().view(np.uint32)[finite], want_z[finite])
