"""C-ABI checks that need no GPU: the library loads, exports every function
include/nvfp4.h declares (and the test-only probe library every function of
its headers beside the sources), and reports argument errors synchronously before
touching a device.  Fake device pointers are plain integers that are never
dereferenced: every call here fails validation first (or fails the device
check on a machine without a gfx950)."""

import ctypes
import os
import re

import pytest

from nvfp4_block_scaled_05_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

OK, NULL, SHAPE, ALIGN, WORKSPACE, DEVICE, ARG = 0, -1, -2, -3, -4, -5, -6


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_binding.LIB_PATH):
        from nvfp4_block_scaled_05_amd import build
        build.build()
    return _binding.load()


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_\w+)\s*\(", text)))


def test_probe_library_exports_every_declared_symbol(lib):
    # the test-only library of conversion probes (built beside the main one)
    from nvfp4_block_scaled_05_amd import build
    probe = ctypes.CDLL(build.PROBE_LIB)
    names = declared_functions(os.path.join(build.CSRC, "isa_probe.h"))
    calib = declared_functions(os.path.join(build.CSRC, "calib.h"))
    assert len(names) >= 6 and len(calib) == 4, (names, calib)
    for n in names + calib:
        assert hasattr(probe, n), n


def test_public_include_holds_only_the_library_header():
    # test-only headers live beside their sources, not in the public include/
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["nvfp4.h"]


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 18
    for n in names:
        assert hasattr(lib, n), n
        assert n in _binding.SIGNATURES, n


def test_version_and_status_strings(lib):
    assert lib.nvfp4_abi_version() == 6
    for code in range(-8, 1):
        assert lib.nvfp4_status_string(code)
    assert lib.nvfp4_status_string(-99) == b"unknown status"


def test_workspace_bytes(lib):
    assert lib.nvfp4_quantize_workspace_bytes(0, 16) == 0
    assert lib.nvfp4_quantize_workspace_bytes(-1, 16) == 0
    small = lib.nvfp4_quantize_workspace_bytes(1, 16)
    big = lib.nvfp4_quantize_workspace_bytes(16896, 3072)
    assert small == big == 8192


A = 1 << 20        # fake, 16-byte aligned, never dereferenced
S = 64


def q(lib, x=A, rows=4, cols=32, codes=A, scales=A, ts=A, amax=None, ws=A, wsb=8192, st=None):
    return lib.nvfp4_quantize(x, rows, cols, codes, scales, ts, amax, ws, wsb, st, None)


def test_quantize_argument_errors(lib):
    assert q(lib, x=None) == NULL
    assert q(lib, ts=None) == NULL
    assert q(lib, ws=None) == NULL                  # computing amax needs the workspace
    assert q(lib, rows=-1) == SHAPE
    assert q(lib, cols=24) == SHAPE
    assert q(lib, cols=0) == SHAPE
    assert q(lib, x=A + 8) == ALIGN
    assert q(lib, codes=A + 4) == ALIGN
    assert q(lib, ts=A + 2) == ALIGN
    assert q(lib, ws=A + 4) == ALIGN                # 64-bit arrival counters
    assert q(lib, wsb=0) == WORKSPACE
    assert q(lib, wsb=4096) == WORKSPACE
    # workspace not needed when the producer's amax is given
    assert q(lib, ws=None, wsb=0, amax=A) in (OK, DEVICE)


def test_quantize_no_alloc_argument_errors(lib):
    def qn(x=A, rows=4, cols=32, codes=A, scales=A, ts=A, st=None):
        return lib.nvfp4_quantize_no_alloc(x, rows, cols, codes, scales, ts, st, None)
    assert qn(x=None) == NULL
    assert qn(ts=None) == NULL
    assert qn(rows=-1) == SHAPE
    assert qn(cols=24) == SHAPE
    assert qn(x=A + 8) == ALIGN
    assert qn(codes=A + 4) == ALIGN
    assert qn(st=A + 2) == ALIGN
    assert qn() in (OK, DEVICE)
    assert qn(rows=0, x=None, codes=None, scales=None) in (OK, DEVICE)


def test_quantize_valid_args_reach_device_check(lib):
    r = q(lib)
    assert r in (DEVICE, OK)
    if not _has_gfx950():
        assert r == DEVICE


def test_dequantize_argument_errors(lib):
    d = lib.nvfp4_dequantize
    assert d(None, A, A, 4, 32, A, None) == NULL
    assert d(A, A, A, 4, 20, A, None) == SHAPE
    assert d(A, A, A, 4, 32, A + 8, None) == ALIGN
    assert d(A + 4, A, A, 4, 32, A, None) == ALIGN


def g(lib, M=64, N=64, K=64, epi=0, y=A, bias=None, amax=None, ac=A, wc=A, ws=None, wsb=0):
    return lib.nvfp4_gemm(ac, A, A, wc, A, A, bias, M, N, K, epi, y, amax, ws, wsb, None)


def test_gemm_workspace_bytes(lib):
    wb = lib.nvfp4_gemm_workspace_bytes
    # invalid shapes and small problems (128x128 tiles) never split
    assert wb(0, 64, 64) == wb(-1, 64, 64) == wb(64, 64, 40) == 0
    assert wb(128, 1024, 1024) == 0
    # DiT MLP projections at 2048^2 with a CFG pair: the tiles past the last
    # whole round over the compute units are split over K
    # 792 tiles: 24 past 3 rounds over 256 compute units, split 8 ways (the
    # direct-to-LDS kernel's cap; 96 stages of 128 would allow more)
    assert wb(16896, 3072, 12288) == 24 * 8 * 256 * 256 * 4
    # K % 128 != 0 runs the register-staged kernel, whose stages are 64 wide:
    # 24 tail tiles, 10 ways
    assert wb(16896, 3072, 12288 + 64) == 24 * 10 * 256 * 256 * 4
    # 3168 tiles: 96 past 12 rounds would split only 2 ways, not worth it
    assert wb(16896, 12288, 3072) == 0
    # a whole number of rounds: nothing to split
    assert wb(256 * 16, 256 * 16, 4096) == 0


def test_gemm_argument_errors(lib):
    assert g(lib, y=None) == NULL
    assert g(lib, K=40) == SHAPE
    assert g(lib, K=0) == SHAPE
    assert g(lib, M=-3) == SHAPE
    assert g(lib, ac=A + 4) == ALIGN
    assert g(lib, y=A + 1) == ALIGN
    assert g(lib, amax=A + 2) == ALIGN
    assert g(lib, ws=A + 16, wsb=1 << 20) == ALIGN
    assert g(lib, epi=7) == ARG
    b = lib.nvfp4_gemm_bf16
    assert b(None, A, None, 8, 8, 64, 0, A, None) == NULL
    assert b(A, A, None, 8, 8, 12, 0, A, None) == SHAPE
    assert b(A + 8, A, None, 8, 8, 64, 0, A, None) == ALIGN
    assert b(A, A, None, 8, 8, 64, 3, A, None) == ARG


def test_gemm_quantized_argument_errors(lib):
    def gq(M=64, N=64, K=64, amax=A, yc=A, ys=A, yt=A, epi=0):
        return lib.nvfp4_gemm_quantized(A, A, A, A, A, A, None, M, N, K, epi, amax, yc, ys, yt, None)
    assert gq(amax=None) == NULL
    assert gq(yc=None) == NULL
    assert gq(N=40) == SHAPE            # output blocks of 16 along N
    assert gq(K=24) == SHAPE
    assert gq(yc=A + 4) == ALIGN
    assert gq(yt=A + 2) == ALIGN
    assert gq(epi=5) == ARG
    assert gq(M=0, amax=None, yc=None, ys=None, yt=None) in (OK, DEVICE)


def test_fp8_argument_errors(lib):
    fq = lib.nvfp4_fp8_quantize_rowwise
    assert fq(None, 4, 32, A, A, None, None) == NULL
    assert fq(A, 4, 24, A, A, None, None) == SHAPE
    assert fq(A + 8, 4, 32, A, A, None, None) == ALIGN
    assert fq(A, 4, 32, A + 4, A, None, None) == ALIGN
    fg = lib.nvfp4_fp8_gemm

    def f(M=8, N=8, K=64, epi=0, y=A, ac=A, ws=None, wsb=0):
        return fg(ac, A, A, A, None, M, N, K, epi, y, ws, wsb, None)
    assert f(y=None) == NULL
    assert f(K=40) == SHAPE
    assert f(ac=A + 8) == ALIGN
    assert f(ws=A + 64, wsb=1 << 20) == ALIGN
    assert f(epi=9) == ARG
    assert f() in (OK, DEVICE)


def test_fp8_gemm_workspace_bytes(lib):
    wb = lib.nvfp4_fp8_gemm_workspace_bytes
    assert wb(0, 64, 128) == wb(-1, 64, 128) == wb(64, 64, 48) == 0
    # K % 128 != 0 runs the register-staged kernel, which never splits
    assert wb(16896, 3072, 12288 + 64) == 0
    # MLP down at 2048^2 with a CFG pair: 792 tiles of 256x256, 24 past three
    # rounds over 256 compute units, split 8 ways (at most 8; 10 would fit)
    assert wb(16896, 3072, 12288) == 24 * 8 * 256 * 256 * 4
    # MLP up: 96 tiles past 12 rounds would split only 2 ways: whole
    assert wb(16896, 12288, 3072) == 0
    assert wb(256 * 16, 256 * 16, 4096) == 0        # whole rounds only


def test_graph_argument_errors(lib):
    import ctypes
    h = ctypes.c_void_p()
    assert lib.nvfp4_graph_begin(None) == NULL          # the null stream cannot be captured
    assert lib.nvfp4_graph_end(None, ctypes.byref(h)) == NULL
    assert lib.nvfp4_graph_end(A, None) == NULL
    assert lib.nvfp4_graph_launch(None, None) == NULL
    assert lib.nvfp4_graph_destroy(None) == NULL
    if not _has_gfx950():
        assert lib.nvfp4_graph_begin(A) == DEVICE


def test_layer_predicate_matches_python_re(lib):
    from tests.test_oracle_layers import load_golden   # hand-written list
    for name, want in load_golden():
        assert lib.nvfp4_layer_is_quantized(name.encode(), None) == int(want), name
    assert lib.nvfp4_layer_is_quantized(None, None) == NULL
    assert lib.nvfp4_layer_is_quantized(b"abc", b"(unclosed") == ARG
    assert lib.nvfp4_layer_is_quantized(b"blocks.1.ff", b"blocks") == 1
    assert lib.nvfp4_layer_is_quantized(b"x.blocks", b"blocks") == 0   # match at the start only


PAGE_PATTERN = b"^(?!.*(embedder|norm_out|proj_out|to_add_out|to_added_qkv|stream)).*"


def test_layer_predicate_default_is_the_page_regex(lib):
    # the default pattern is evaluated as a substring search; the same names
    # through the regex engine with the page's pattern spelled out must agree,
    # including the line-terminator edge (the pattern's `.` stops at \n, \r)
    from tests.test_oracle_layers import load_golden
    names = [n.encode() for n, _ in load_golden()] + [
        b"", b"norm_out", b"a.norm_out.b", b"norm_ou", b"to_add_outx", b"to_added_qk",
        b"to_added_qkv", b"x_embedder", b"upstream", b"proj_out.0", b"a\nnorm_out",
        b"a\rstream", b"stream\nx", b"a\n\rembedder", b"ab\xe2\x80\xa8proj_out",
        b"\xff\xfe.to_add_out", b"st\nream",
    ]
    for n in names:
        want = lib.nvfp4_layer_is_quantized(n, PAGE_PATTERN)
        assert want in (0, 1), n
        assert lib.nvfp4_layer_is_quantized(n, None) == want, n


def test_layer_predicate_long_names(lib):
    # the default pattern takes names of any length (one linear scan); a
    # caller's pattern is applied to names up to 1024 bytes
    f = lib.nvfp4_layer_is_quantized
    assert f(b"a" * 200_000, None) == 1
    assert f(b"a" * 200_000 + b".norm_out", None) == 0
    assert f(b"b" * 1024, b"b*") == 1
    assert f(b"b" * 1025, b"b*") == ARG
    assert f(b"b" * 1025, b"(unclosed") == ARG


def _has_gfx950():
    try:
        import torch
        return torch.cuda.is_available() and "gfx950" in torch.cuda.get_device_properties(0).gcnArchName
    except Exception:
        return False
