"""GPU parity of the FP8 row-wise variant against oracle/fp8.py: the quantizer
bit for bit, the W8A8 GEMM within the GEMM tolerance."""

import numpy as np
import pytest

import nvfp4_block_scaled_05_amd as nv
from nvfp4_block_scaled_05_amd import inputs as W
from oracle import (dequantize_fp8_rowwise, gemm_fp8_exact_rows, gemm_fp8_fp64,
                    quantize_fp8_rowwise)
from tests.gpu_util import bits_of, rel_frobenius, stratified_rows, to_dev, ulp_diff

pytestmark = pytest.mark.gpu

GEMM_TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load()


def _sync():
    import torch
    torch.cuda.synchronize()


def check_fp8_quantize(bits, label=""):
    q = nv.fp8_quantize(to_dev(bits))
    _sync()
    ref = quantize_fp8_rowwise(bits)
    codes, scales = q.codes.cpu().numpy(), q.scales.cpu().numpy()
    bad = np.argwhere(codes != ref.codes)
    assert len(bad) == 0, f"{label}: {len(bad)} code mismatches, first {bad[:3]}"
    assert np.array_equal(scales.view(np.uint32), ref.scales.view(np.uint32)), label
    return q, ref


# rows up to 4096 and up to 12288 columns are held in registers; longer rows
# take the wave-per-row path
SHAPES = [(1, 16), (3, 48), (37, 1040), (257, 3072), (9, 4112), (5, 12288), (3, 12304), (2, 20000)]
KINDS = ["normal", "t3", "outliers"]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("kind", KINDS)
def test_fp8_quantize_ragged(shape, kind):
    seed = 500 + 10 * SHAPES.index(shape) + KINDS.index(kind)
    check_fp8_quantize(W.random_matrix(seed, shape, kind), f"{shape} {kind}")


def test_fp8_quantize_full_size_and_round_trip():
    bits = W.quantize_act()["x"]
    q, ref = check_fp8_quantize(bits, "act [16896,3072]")
    back = dequantize_fp8_rowwise(ref.codes, ref.scales)
    assert np.array_equal(quantize_fp8_rowwise(back).codes, ref.codes)


def test_fp8_quantize_degenerate_and_nonfinite():
    import torch
    x = np.zeros((4, 64), np.float32)
    x[1, :] = -0.0
    x[2, 7] = 1e-38
    x[3, :] = np.linspace(-3, 3, 64, dtype=np.float32)
    check_fp8_quantize(W.f32_to_bf16_bits(x), "degenerate rows")
    x[3, 9] = np.nan
    status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    q = nv.fp8_quantize(to_dev(W.f32_to_bf16_bits(x)), dev_status=status)
    _sync()
    assert int(status.item()) == -8 and np.isnan(q.scales[3].item())
    status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    nv.fp8_quantize(to_dev(W.random_matrix(2, (8, 64))), dev_status=status)
    _sync()
    assert int(status.item()) == 0


def _close(y, ref, label):
    err = rel_frobenius(y, ref)
    assert err <= GEMM_TOL, f"{label}: rel Frobenius {err:.3e}"
    assert float((ulp_diff(y, ref) > 1).mean()) <= 1e-2, label


# K % 128 == 0 runs the direct-to-LDS kernel (1, 2, 3, 4, 9, 10 stages of 128,
# ragged M and N); other K the register-staged one.  "reg" pins the latter.
# These grids have fewer tiles than compute units: one tile per workgroup.
GEMM_SHAPES = [(64, 64, 64), (130, 70, 48), (300, 257, 1088), (200, 300, 3088), (1, 129, 16),
               (513, 256, 512), (1, 1, 128), (256, 256, 256), (257, 513, 384),
               (300, 257, 1152), (70, 600, 1280)]


@pytest.mark.parametrize("kernel", ["default", "reg"])
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_fp8_gemm_small_and_ragged(M, N, K, kernel, monkeypatch):
    if kernel == "reg":
        monkeypatch.setenv("NVFP4_FP8_GEMM_KERNEL", "reg")
    a_bits = W.random_matrix(M + K, (M, K), "t3")
    w_bits = W.random_matrix(N + K, (N, K), "normal", 0.02)
    b_bits = W.random_matrix(M + N, (1, N), "normal", 0.1)[0]
    qa, ra = check_fp8_quantize(a_bits, "A")
    qw, rw = check_fp8_quantize(w_bits, "W")
    for epi in ("none", "gelu"):
        y = bits_of(nv.fp8_gemm(qa, qw, bias=to_dev(b_bits), epilogue=epi))
        ref, _ = gemm_fp8_fp64(ra, rw, bias_bits=b_bits, gelu=epi == "gelu")
        _close(y, ref, f"fp8 {M}x{N}x{K} {epi}")


def test_fp8_gemm_mlp_up_sampled_rows():
    # the MLP up projection at 2048^2: X [16896,3072] t(3), W_up [12288,3072]
    d = W.mlp_2048()
    qx, rx = check_fp8_quantize(d["x"], "X")
    qw, rw = check_fp8_quantize(d["w_up"], "W_up")
    y = bits_of(nv.fp8_gemm(qx, qw, epilogue="gelu"))
    # a row in every 256-row tile band (each row covers all 48 column tiles of
    # its band, so every tile of the persistent grid is checked)
    rows = np.unique(np.concatenate([stratified_rows(16896), [16895],
                                     np.random.default_rng(0).choice(16896, 16, replace=False)]))
    ref, _ = gemm_fp8_exact_rows(rx, rw, rows, gelu=True)
    _close(y[rows], ref, "fp8 up sampled rows")


def test_fp8_gemm_mlp_down_sampled_rows():
    # the MLP down projection at 2048^2: W_down [3072,12288] against a seeded
    # N(0, 0.5) stand-in for the hidden activation H [16896,12288]
    d = W.mlp_2048()
    rng = np.random.default_rng(1)
    h_bits = W.random_matrix(77, (16896, 12288), "normal", 0.5)
    qh, rh = check_fp8_quantize(h_bits, "H")
    qw, rw = check_fp8_quantize(d["w_down"], "W_down")
    b_bits = W.random_matrix(78, (1, 3072), "normal", 0.1)[0]
    y = bits_of(nv.fp8_gemm(qh, qw, bias=to_dev(b_bits)))
    rows = np.unique(np.concatenate([stratified_rows(16896), [16895], rng.choice(16896, 8, replace=False)]))
    ref, _ = gemm_fp8_exact_rows(rh, rw, rows, bias_bits=b_bits)
    _close(y[rows], ref, "fp8 down sampled rows")


@pytest.mark.parametrize("ways", [2, 3, 7, 11])
@pytest.mark.parametrize("M,N,K", [(600, 520, 1280), (257, 300, 2048)])
def test_fp8_gemm_split_k(M, N, K, ways, monkeypatch):
    # the tail tiles split over K (forced), partial sums added in split order
    # (more than 8 ways: the reduce kernel loads the slices in groups of 8)
    monkeypatch.setenv("NVFP4_FP8_GEMM_SPLIT", str(ways))
    a_bits = W.random_matrix(M * 3 + K, (M, K), "t3")
    w_bits = W.random_matrix(N * 3 + K, (N, K), "normal", 0.02)
    b_bits = W.random_matrix(M + N + 5, (1, N), "normal", 0.1)[0]
    qa, ra = check_fp8_quantize(a_bits, "A")
    qw, rw = check_fp8_quantize(w_bits, "W")
    ws = nv.fp8_gemm_workspace(M, N, K)
    assert ws is not None
    for epi in ("none", "gelu"):
        y1 = bits_of(nv.fp8_gemm(qa, qw, bias=to_dev(b_bits), epilogue=epi, workspace=ws))
        y2 = bits_of(nv.fp8_gemm(qa, qw, bias=to_dev(b_bits), epilogue=epi, workspace=ws))
        assert np.array_equal(y1, y2), "split result depends on timing"
        ref, _ = gemm_fp8_fp64(ra, rw, bias_bits=b_bits, gelu=epi == "gelu")
        _close(y1, ref, f"fp8 split {ways} {M}x{N}x{K} {epi}")
        y0 = bits_of(nv.fp8_gemm(qa, qw, bias=to_dev(b_bits), epilogue=epi, workspace=None))
        _close(y0, ref, f"fp8 whole tiles {M}x{N}x{K} {epi}")


@pytest.mark.parametrize("M,N,K", [(4352, 4096, 384), (4352, 4096, 2048)])
def test_fp8_gemm_persistent_grid(M, N, K, monkeypatch):
    # 272 tiles, more than the compute units: the persistent grid, each
    # workgroup looping over tiles (and, at K = 2048, over the K ranges of the
    # 16 split tail tiles), the next tile's first stage loaded under the
    # epilogue.  K = 384 gives an odd number of stages.  The whole output
    # against the oracle; then one item per workgroup and no split give the
    # same bytes.
    a_bits = W.random_matrix(M + 7 * K, (M, K), "t3")
    w_bits = W.random_matrix(N + 7 * K, (N, K), "normal", 0.02)
    b_bits = W.random_matrix(M + N + 9, (1, N), "normal", 0.1)[0]
    qa, ra = check_fp8_quantize(a_bits, "A")
    qw, rw = check_fp8_quantize(w_bits, "W")
    ws = nv.fp8_gemm_workspace(M, N, K)
    bias = to_dev(b_bits)
    y = bits_of(nv.fp8_gemm(qa, qw, bias=bias, epilogue="gelu", workspace=ws))
    ref, _ = gemm_fp8_fp64(ra, rw, bias_bits=b_bits, gelu=True)
    _close(y, ref, f"fp8 persistent {M}x{N}x{K}")
    monkeypatch.setenv("NVFP4_GEMM_PERSISTENT", "0")
    y1 = bits_of(nv.fp8_gemm(qa, qw, bias=bias, epilogue="gelu", workspace=ws))
    assert np.array_equal(y, y1), "persistent and one-item grids differ"
    monkeypatch.delenv("NVFP4_GEMM_PERSISTENT")
    y2 = bits_of(nv.fp8_gemm(qa, qw, bias=bias, epilogue="gelu", workspace=None))
    _close(y2, ref, f"fp8 persistent, no split {M}x{N}x{K}")
