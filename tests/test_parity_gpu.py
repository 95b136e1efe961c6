"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

  * quantize: codes, scales and the FP32 tensor scale bit-exact, on the DiT
    workload shapes at full size, ragged shapes, and adversarial tensors;
  * dequantize: bf16 output bit-exact;
  * block-scaled GEMM: relative Frobenius error <= 2e-3 against the oracle's
    exact sum rounded to bf16 (the acceptance bar), with the share of outputs
    more than one bf16 ulp away reported and bounded;
  * epilogues (bias, GELU, output amax), the MLP chain stage by stage, and the
    bf16 passthrough.
Inputs are the seeded generators of nvfp4_block_scaled_05_amd.inputs; the
oracle always quantizes its own copy of the inputs.
"""

import functools

import numpy as np
import pytest

import nvfp4_block_scaled_05_amd as nv
from nvfp4_block_scaled_05_amd import inputs as W
from oracle import (bf16_bits_to_f32, dequantize as o_dequantize, gemm_fp64,
                    gemm_exact_rows, linear_bf16_fp64, quantize as o_quantize)
from tests.gpu_util import bits_of, f32_dev, rel_frobenius, stratified_rows, to_dev, ulp_diff

pytestmark = pytest.mark.gpu

GEMM_TOL = 2e-3          # relative Frobenius error bound of the block-scaled GEMM


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load()
    yield
    torch.cuda.synchronize()


def _sync():
    import torch
    torch.cuda.synchronize()


def gpu_quantize(bits, amax=None):
    q = nv.quantize(to_dev(bits), amax=None if amax is None else f32_dev(amax))
    _sync()
    return q


def assert_quant_equal(q, ref, label=""):
    codes = q.codes.cpu().numpy()
    scales = q.scales.cpu().numpy()
    ts = q.tensor_scale.cpu().numpy()
    bad_s = np.argwhere(scales != ref.scales)
    assert len(bad_s) == 0, f"{label}: {len(bad_s)} scale mismatches, first {bad_s[:3]}"
    bad_c = np.argwhere(codes != ref.codes)
    assert len(bad_c) == 0, f"{label}: {len(bad_c)} code mismatches, first {bad_c[:3]}"
    assert ts.view(np.uint32)[0] == np.float32(ref.tensor_scale).view(np.uint32), label


def check_quantize(bits, amax=None, label=""):
    q = gpu_quantize(bits, amax)
    ref = o_quantize(bits, amax=amax)
    assert_quant_equal(q, ref, label)
    return q, ref


# ----------------------------------------------------------------- quantize --

SHAPES = [(1, 16), (3, 48), (37, 1040), (257, 3072), (5, 12288)]


KINDS = ["normal", "t3", "outliers"]


# The dynamic-amax quantizer has three implementations: the one-launch
# kernel for small tensors (every workgroup folds the whole amax itself), the
# single-pass kernel that holds the tensor on chip (large tensors that fit),
# and the two-pass amax + encode kernels (everything else).  The fixture runs
# each case through the default choice and through each kernel forced.
@pytest.fixture(params=["default", "small", "resident", "twopass"])
def quant_kernel(request, monkeypatch):
    if request.param != "default":
        monkeypatch.setenv("NVFP4_QUANT_KERNEL", request.param)
    return request.param


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("kind", KINDS)
def test_quantize_ragged_shapes(shape, kind, quant_kernel):
    bits = W.random_matrix(1000 * SHAPES.index(shape) + KINDS.index(kind), shape, kind)
    q, ref = check_quantize(bits, label=f"{shape} {kind}")
    y = nv.dequantize(q)
    _sync()
    assert np.array_equal(bits_of(y), o_dequantize(ref.codes, ref.scales, ref.tensor_scale, shape[1]))


def test_quantize_linear_small_workload():
    d = W.linear_small()
    check_quantize(d["x"], label="X [128,1024]")
    check_quantize(d["w"], label="W [1024,1024]")


def test_quantize_activation_full_size():
    # 16896 x 3072, N(0,1) with 0.1% outliers x50: full tensor bit-exact, and
    # the bf16 round trip bit-exact
    bits = W.quantize_act()["x"]
    q, ref = check_quantize(bits, label="act [16896,3072]")
    y = nv.dequantize(q)
    _sync()
    assert np.array_equal(bits_of(y), o_dequantize(ref.codes, ref.scales, ref.tensor_scale, 3072))


def test_quantize_activation_full_size_two_pass(monkeypatch):
    # the same tensor through the two-pass kernels (the default there is the
    # single-pass one): the same bytes
    monkeypatch.setenv("NVFP4_QUANT_KERNEL", "twopass")
    bits = W.quantize_act()["x"]
    check_quantize(bits, label="act [16896,3072] two-pass")


@pytest.mark.parametrize("extra_rows", [0, 1])
def test_quantize_single_pass_capacity_edge(extra_rows):
    # the largest tensor of 3072 columns the single-pass kernel holds on chip
    # (units * 13 * 1024 blocks of 16), and one row more, which goes through
    # the two-pass kernels; sampled rows against the oracle given the exact
    # tensor amax, including the rows where one workgroup's range ends
    import torch
    units = torch.cuda.get_device_properties(0).multi_processor_count
    cap_blocks = units * 13 * 1024
    rows = cap_blocks * 16 // 3072 + extra_rows
    bits = W.random_matrix(31 + extra_rows, (rows, 3072), "outliers")
    q = gpu_quantize(bits)
    amax = np.float32(np.abs(bf16_bits_to_f32(bits)).max())
    nblocks = rows * 3072 // 16
    chunk = -(-nblocks // units)
    edges = [min(rows - 1, (g * chunk * 16) // 3072 + d) for g in (1, units // 2, units - 1) for d in (-1, 0)]
    rng = np.random.default_rng(extra_rows)
    sample = np.unique(np.concatenate([stratified_rows(rows), edges, rng.choice(rows, 40, replace=False)]))
    ref = o_quantize(bits[sample], amax=amax)
    assert np.array_equal(q.scales.cpu().numpy()[sample], ref.scales), "scales"
    assert np.array_equal(q.codes.cpu().numpy()[sample], ref.codes), "codes"
    assert q.tensor_scale.cpu().numpy().view(np.uint32)[0] == np.float32(ref.tensor_scale).view(np.uint32)


@pytest.mark.parametrize("blocks_per_thread,extra", [(2, 0), (2, 1), (4, 0), (4, 1)])
def test_quantize_single_pass_footprint_edges(blocks_per_thread, extra):
    # the single-pass kernel comes in three footprints (2, 4 and 13 blocks of
    # 16 per thread); a call takes the smallest whose 1024 threads hold its
    # workgroup's range.  At each edge, and one row past it (the next
    # footprint), the whole tensor against the oracle
    import torch
    units = torch.cuda.get_device_properties(0).multi_processor_count
    cols = 3072
    rows = blocks_per_thread * 1024 * units * 16 // cols + extra
    chunk = -(-(rows * cols // 16) // units)
    assert (chunk <= blocks_per_thread * 1024) == (extra == 0)
    bits = W.random_matrix(40 + 2 * blocks_per_thread + extra, (rows, cols), "outliers")
    check_quantize(bits, label=f"[{rows},{cols}] chunk {chunk}")


@functools.lru_cache(maxsize=None)
def _mlp():
    return W.mlp_2048()


def test_quantize_student_t_full_size():
    bits = _mlp()["x"]
    check_quantize(bits, label="mlp X t(3)")


def _adversarial(seed=0):
    rng = np.random.default_rng(seed)
    rows, cols = 64, 256
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[0, :16] = 0.0                                  # all-zero block
    x[0, 16:32] = -0.0                               # negative zeros
    x[1, :16] = 3.0                                  # constant block
    x[2, :16] = x[2, :16] / np.abs(x[2, :16]).max() * np.float32(0.05)   # subnormal E4M3 scale
    x[3, :16] = x[3, :16] * 3e-8                     # scale rounds to 0
    x[4, :] = np.float32(1e-39) * np.sign(x[4, :])   # bf16 subnormals
    x[5, 7] = 3000.0                                 # one huge outlier (the tensor max)
    for j in range(16):                              # tensor max in every block position
        x[6 + j, 16 * (j % 16) + j] = -2999.0
    return W.f32_to_bf16_bits(x)


def test_quantize_adversarial(quant_kernel):
    bits = _adversarial()
    q, ref = check_quantize(bits, label="adversarial")
    y = nv.dequantize(q)
    _sync()
    assert np.array_equal(bits_of(y), o_dequantize(ref.codes, ref.scales, ref.tensor_scale, 256))
    assert (ref.scales == 0).any() and ((ref.scales > 0) & (ref.scales < 8)).any()


def test_quantize_exact_e2m1_ties(quant_kernel):
    # amax = 2688 makes s_enc = s_dec = 1; a block with max 6 gets scale 1.0, so
    # the elements reach the E2M1 encoder unscaled and sit exactly on its ties
    x = np.zeros((4, 32), np.float32)
    x[0, 0] = 2688.0
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    x[1, :8], x[1, 8:16] = ties, -ties
    x[2, :16] = np.array([6.0, 0.2, 0.3, 0.7, 0.8, 1.2, 1.3, 1.7, 1.8, 2.4, 2.6, 3.4, 3.6, 4.9, 5.1, 7.0],
                         np.float32)
    bits = W.f32_to_bf16_bits(x)
    q, ref = check_quantize(bits, label="ties")
    assert ref.tensor_scale == np.float32(1.0) and ref.scales[1, 0] == 0x38   # 1.0


def test_quantize_degenerate(quant_kernel):
    for fill in (0.0, -0.0, 1e-38):
        bits = W.f32_to_bf16_bits(np.full((4, 32), fill, np.float32))
        check_quantize(bits, label=f"fill {fill}")


def test_quantize_with_producer_amax():
    bits = W.random_matrix(3, (96, 640), "t3")
    amax = np.abs(bf16_bits_to_f32(bits)).max()
    check_quantize(bits, amax=amax, label="amax given")
    check_quantize(bits, amax=np.float32(amax * 3.0), label="amax larger")


def test_quantize_nonfinite_reports_status(quant_kernel):
    import torch
    for bad in (np.inf, -np.inf, np.nan):
        x = np.ones((8, 64), np.float32)
        x[5, 9] = bad
        status = torch.full((1,), 123, dtype=torch.int32, device="cuda")
        q = nv.quantize(to_dev(W.f32_to_bf16_bits(x)), dev_status=status)
        _sync()
        assert int(status.item()) == -8
        assert np.isnan(q.tensor_scale.item())
    status = torch.full((1,), 123, dtype=torch.int32, device="cuda")
    nv.quantize(to_dev(W.random_matrix(1, (8, 64))), dev_status=status)
    _sync()
    assert int(status.item()) == 0


def test_quantize_empty_rows():
    import torch
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q = nv.quantize(x)
    _sync()
    assert q.codes.shape == (0, 32)


def test_binding_stream_is_torch_current_stream():
    # the binding enqueues on the stream torch.cuda.current_stream() names,
    # on the default stream and inside a side-stream context, and work
    # enqueued there is ordered with torch's own work on that stream
    import torch
    from nvfp4_block_scaled_05_amd import _stream
    assert _stream() == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    bits = W.random_matrix(23, (64, 256), "normal")
    ref = o_quantize(bits)
    with torch.cuda.stream(side):
        assert _stream() == side.cuda_stream != torch.cuda.default_stream().cuda_stream
        x = to_dev(bits)
        q = nv.quantize(x)
    side.synchronize()
    assert_quant_equal(q, ref, "side stream")


@pytest.mark.parametrize("which", ["a", "w"])
def test_gemm_empty_operand(which):
    # an operand with no rows: an empty output, no kernel reads the other
    # operand, and the output amax (the max over no values) is written as 0,
    # for the bf16 and the NVFP4-output GEMMs alike
    import torch
    K = 1024
    empty = nv.quantize(torch.empty((0, K), dtype=torch.bfloat16, device="cuda"))
    full, _ = check_quantize(W.random_matrix(17, (96, K), "t3"), label="operand")
    a, w = (empty, full) if which == "a" else (full, empty)
    amax = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    y = nv.gemm(a, w, epilogue="gelu", y_amax=amax)
    _sync()
    assert tuple(y.shape) == ((0, 96) if which == "a" else (96, 0))
    assert amax.item() == 0.0
    if which == "a":
        q = nv.gemm_quantized(a, w, torch.ones((1,), dtype=torch.float32, device="cuda"))
        _sync()
        assert tuple(q.codes.shape) == (0, 48)


def test_quantize_deterministic(quant_kernel):
    bits = W.random_matrix(9, (1000, 3072), "outliers")
    x = to_dev(bits)
    a = nv.quantize(x)
    b = nv.quantize(x)
    _sync()
    assert np.array_equal(a.codes.cpu().numpy(), b.codes.cpu().numpy())
    assert np.array_equal(a.scales.cpu().numpy(), b.scales.cpu().numpy())


# --------------------------------------------------------------------- GEMM --

def _gemm_case(M, N, K, seed, kind_a="t3", bias=False, epilogue="none"):
    a_bits = W.random_matrix(seed, (M, K), kind_a)
    w_bits = W.random_matrix(seed + 1, (N, K), "normal", 0.02)
    b_bits = W.random_matrix(seed + 2, (1, N), "normal", 0.1)[0] if bias else None
    qa, ra = check_quantize(a_bits, label="A")
    qw, rw = check_quantize(w_bits, label="W")
    y = nv.gemm(qa, qw, bias=None if b_bits is None else to_dev(b_bits), epilogue=epilogue)
    _sync()
    ref, _ = gemm_fp64(ra, rw, K, bias_bits=b_bits, gelu=epilogue == "gelu")
    return bits_of(y), ref


def assert_gemm_close(y, ref, label=""):
    err = rel_frobenius(y, ref)
    ulps = ulp_diff(y, ref)
    far = float((ulps > 1).mean())
    assert err <= GEMM_TOL, f"{label}: rel Frobenius {err:.3e}"
    assert far <= 1e-2, f"{label}: {far:.2e} of outputs more than 1 ulp away"
    return err


@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (130, 70, 48), (256, 384, 1024),
                                   (200, 300, 3088), (1, 129, 16), (129, 1, 256)])
def test_gemm_small_and_ragged(M, N, K):
    y, ref = _gemm_case(M, N, K, seed=M * 7 + N + K)
    assert_gemm_close(y, ref, f"{M}x{N}x{K}")


def test_gemm_bias_and_gelu():
    y, ref = _gemm_case(192, 256, 512, seed=5, bias=True, epilogue="gelu")
    assert_gemm_close(y, ref, "bias+gelu")
    y, ref = _gemm_case(192, 256, 512, seed=6, bias=True)
    assert_gemm_close(y, ref, "bias")


def test_gemm_linear_small_workload():
    # X [128,1024], W [1024,1024]: both dynamically quantized, full comparison
    d = W.linear_small()
    qa, ra = check_quantize(d["x"])
    qw, rw = check_quantize(d["w"])
    y = nv.gemm(qa, qw)
    _sync()
    ref, _ = gemm_fp64(ra, rw, 1024)
    assert_gemm_close(bits_of(y), ref, "linear 128x1024x1024")


def test_gemm_exact_sum_sampled_rows():
    # the float64 oracle agrees with the exact int64 form on these rows too
    M, N, K = 300, 512, 3072
    a_bits = W.random_matrix(41, (M, K), "t3")
    w_bits = W.random_matrix(42, (N, K), "normal", 0.02)
    qa, ra = check_quantize(a_bits)
    qw, rw = check_quantize(w_bits)
    y = bits_of(nv.gemm(qa, qw))
    rows = np.arange(0, M, 7)
    ref, _ = gemm_exact_rows(ra, rw, K, rows)
    assert_gemm_close(y[rows], ref, "exact rows")


@functools.lru_cache(maxsize=None)
def _oracle_weight(name, seed=0):
    bits = W.qkv_1024(seed)["w"] if name == "qkv" else _mlp()[name]
    return bits, o_quantize(bits)


def _sampled_rows(M, n=96, seed=0):
    """Rows compared at full size: one in every 256-row tile band (MFMA block
    and row inside it rotating; stratified_rows), plus n random ones."""
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([stratified_rows(M), rng.choice(M, min(n, M), replace=False)]))


def test_gemm_qkv_1024_sampled_rows():
    # X [4608,3072] quantized per call, W [9216,3072] pre-quantized
    x_bits = W.qkv_1024()["x"]
    w_bits, rw = _oracle_weight("qkv")
    qx = gpu_quantize(x_bits)
    qw = gpu_quantize(w_bits)
    y = bits_of(nv.gemm(qx, qw))
    rows = _sampled_rows(4608)
    amax = np.abs(bf16_bits_to_f32(x_bits)).max()
    rx = o_quantize(x_bits[rows], amax=amax)          # the rows of the full-tensor quantization
    assert_quant_equal(qw, rw, "W qkv")
    ref, _ = gemm_fp64(rx, rw, 3072)
    assert_gemm_close(y[rows], ref, "qkv sampled rows")


def test_mlp_2048_chain_stage_by_stage():
    import torch
    x_bits = _mlp()["x"]
    wu_bits, rwu = _oracle_weight("w_up")
    wd_bits, rwd = _oracle_weight("w_down")
    qwu, qwd = gpu_quantize(wu_bits), gpu_quantize(wd_bits)
    assert_quant_equal(qwu, rwu, "W_up")
    assert_quant_equal(qwd, rwd, "W_down")
    qx = gpu_quantize(x_bits)
    amax = torch.empty((1,), dtype=torch.float32, device="cuda")
    h = nv.gemm(qx, qwu, epilogue="gelu", y_amax=amax)
    qh = nv.quantize(h, amax=amax)
    y = nv.gemm(qh, qwd)
    _sync()
    rows = _sampled_rows(16896, n=48)
    # stage 1: H = GELU(Xq @ Wup^T) on sampled rows
    x_amax = np.abs(bf16_bits_to_f32(x_bits)).max()
    rx = o_quantize(x_bits[rows], amax=x_amax)
    h_ref, _ = gemm_fp64(rx, rwu, 3072, gelu=True)
    h_bits = bits_of(h)
    assert_gemm_close(h_bits[rows], h_ref, "up+gelu")
    # stage 2: the epilogue amax is max |H_gpu| exactly
    h_amax = np.abs(bf16_bits_to_f32(h_bits)).max()
    assert np.float32(amax.item()) == np.float32(h_amax)
    # stage 3: quantize(H_gpu) bit-exact on the sampled rows (amax is global)
    rh = o_quantize(h_bits[rows], amax=h_amax)
    assert np.array_equal(qh.codes.cpu().numpy()[rows], rh.codes)
    assert np.array_equal(qh.scales.cpu().numpy()[rows], rh.scales)
    assert np.float32(qh.tensor_scale.item()) == rh.tensor_scale
    # stage 4: Y = Hq @ Wdown^T on the sampled rows
    y_ref, _ = gemm_fp64(rh, rwd, 12288)
    assert_gemm_close(bits_of(y)[rows], y_ref, "down")


def test_gemm_amax_epilogue_exact():
    import torch
    a_bits = W.random_matrix(61, (333, 512), "t3")
    w_bits = W.random_matrix(62, (250, 512), "normal", 0.02)
    qa, qw = gpu_quantize(a_bits), gpu_quantize(w_bits)
    amax = torch.full((1,), 1e30, dtype=torch.float32, device="cuda")   # zeroed by the call
    y = nv.gemm(qa, qw, y_amax=amax)
    _sync()
    assert np.float32(amax.item()) == np.abs(bf16_bits_to_f32(bits_of(y))).max()


def test_gemm_deterministic():
    a_bits = W.random_matrix(71, (512, 1024), "t3")
    w_bits = W.random_matrix(72, (768, 1024), "normal", 0.02)
    qa, qw = gpu_quantize(a_bits), gpu_quantize(w_bits)
    y1, y2 = bits_of(nv.gemm(qa, qw)), bits_of(nv.gemm(qa, qw))
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("M,N,K", [(300, 520, 1088), (257, 300, 1040), (64, 33, 3072)])
@pytest.mark.parametrize("kernel,split", [("tiny", None), ("small", None), ("pipe", None),
                                          ("pipe", "3"), ("pipe", "7")])
def test_gemm_kernels_and_k_split(monkeypatch, M, N, K, kernel, split):
    # every kernel path on ragged tiles: 64x64 and 128x128 tiles, 256x256
    # tiles whole, and 256x256 tiles with their K range split over 3 or 7
    # workgroups
    monkeypatch.setenv("NVFP4_GEMM_KERNEL", kernel)
    if split:
        monkeypatch.setenv("NVFP4_GEMM_SPLIT", split)
        assert nv.gemm_workspace(M, N, K) is not None
    y, ref = _gemm_case(M, N, K, seed=M + 3 * N + K, epilogue="gelu" if split == "7" else "none")
    assert_gemm_close(y, ref, f"{kernel}/{split} {M}x{N}x{K}")


def test_gemm_large_odd_stage_count_default_kernel():
    # a problem the 256x256 kernels take (M*N above 8.4M) whose K is an odd
    # number of 128-wide stages: the paired scale loads of v5 need K % 256
    # == 0, so the default choice runs v3 here; the result is the same GEMM
    y, ref = _gemm_case(1024, 8448, 1152, seed=4242, bias=True, epilogue="gelu")
    assert_gemm_close(y, ref, "1024x8448x1152 gelu")


_V5_SHAPES = [(300, 520, 1280), (257, 300, 1024), (64, 33, 3072), (513, 256, 256), (256, 256, 512),
              (600, 700, 768)]


@pytest.mark.parametrize("M,N,K,split", [(M, N, K, split) for M, N, K in _V5_SHAPES
                                         for split in (None, "3", "7", "11")
                                         if split is None or int(split) <= K // 128])
def test_gemm_v5_and_k_split(monkeypatch, M, N, K, split):
    # the direct-to-LDS kernel (K % 256 == 0) on ragged tiles, 2 to 24 stages,
    # whole and with the tail tiles' K range split over 3, 7 or 11 workgroups
    # (only where the K range has at least as many 128-wide stages as ways;
    # 11 ways take the reduce kernel's slice loads in two groups of 8 and 3):
    # the splits start items at odd stages and give them odd stage counts,
    # down to one stage, which the paired scale loads treat apart
    monkeypatch.setenv("NVFP4_GEMM_KERNEL", "v5")
    if split:
        monkeypatch.setenv("NVFP4_GEMM_SPLIT", split)
        assert nv.gemm_workspace(M, N, K) is not None
    for epi, bias in (("none", False), ("gelu", True)):
        y, ref = _gemm_case(M, N, K, seed=M + 5 * N + K, bias=bias, epilogue=epi)
        assert_gemm_close(y, ref, f"v5/{split} {M}x{N}x{K} {epi}")


def test_gemm_v5_amax_and_determinism(monkeypatch):
    import torch
    monkeypatch.setenv("NVFP4_GEMM_KERNEL", "v5")
    M, N, K = 700, 600, 1280
    a_bits = W.random_matrix(91, (M, K), "t3")
    w_bits = W.random_matrix(92, (N, K), "normal", 0.02)
    qa, ra = check_quantize(a_bits)
    qw, rw = check_quantize(w_bits)
    for split in (None, "4"):
        if split:
            monkeypatch.setenv("NVFP4_GEMM_SPLIT", split)
        ws = nv.gemm_workspace(M, N, K)
        amax = torch.full((1,), 1e30, dtype=torch.float32, device="cuda")
        y1 = bits_of(nv.gemm(qa, qw, epilogue="gelu", y_amax=amax, workspace=ws))
        assert np.float32(amax.item()) == np.abs(bf16_bits_to_f32(y1)).max()
        y2 = bits_of(nv.gemm(qa, qw, epilogue="gelu", workspace=ws))
        assert np.array_equal(y1, y2)
        ref, _ = gemm_fp64(ra, rw, K, gelu=True)
        assert_gemm_close(y1, ref, f"v5 split {split}")


def test_gemm_k_split_deterministic_with_amax(monkeypatch):
    import torch
    monkeypatch.setenv("NVFP4_GEMM_KERNEL", "pipe")
    monkeypatch.setenv("NVFP4_GEMM_SPLIT", "5")
    M, N, K = 520, 300, 2048
    a_bits = W.random_matrix(81, (M, K), "t3")
    w_bits = W.random_matrix(82, (N, K), "normal", 0.02)
    qa, ra = check_quantize(a_bits)
    qw, rw = check_quantize(w_bits)
    ws = nv.gemm_workspace(M, N, K)
    amax = torch.full((1,), 1e30, dtype=torch.float32, device="cuda")
    y1 = bits_of(nv.gemm(qa, qw, epilogue="gelu", y_amax=amax, workspace=ws))
    assert np.float32(amax.item()) == np.abs(bf16_bits_to_f32(y1)).max()
    y2 = bits_of(nv.gemm(qa, qw, epilogue="gelu", workspace=ws))     # same workspace reused
    assert np.array_equal(y1, y2)
    whole = bits_of(nv.gemm(qa, qw, epilogue="gelu", workspace=None))
    ref, _ = gemm_fp64(ra, rw, K, gelu=True)
    assert_gemm_close(y1, ref, "split")
    assert_gemm_close(whole, ref, "whole")
    assert float((ulp_diff(y1, whole) > 1).mean()) <= 1e-3   # only the fp32 addition order differs


# ------------------------------------------------ NVFP4 output, static scale --

def _gemm_quantized_case(M, N, K, seed, amax_factor, epilogue="none", bias=False):
    import torch
    a_bits = W.random_matrix(seed, (M, K), "t3")
    w_bits = W.random_matrix(seed + 1, (N, K), "normal", 0.02)
    b = to_dev(W.random_matrix(seed + 2, (1, N), "normal", 0.1)[0]) if bias else None
    qa, qw = gpu_quantize(a_bits), gpu_quantize(w_bits)
    amax = torch.empty((1,), dtype=torch.float32, device="cuda")
    y = nv.gemm(qa, qw, bias=b, epilogue=epilogue, y_amax=amax)
    static = amax * amax_factor                       # a calibrated amax, above or below the true one
    fused = nv.gemm_quantized(qa, qw, static, bias=b, epilogue=epilogue)
    two_step = nv.quantize(y, amax=static)
    _sync()
    return y, static, fused, two_step


@pytest.mark.parametrize("M,N,K", [(300, 528, 1088), (257, 16, 64), (64, 1024, 2048),
                                   (300, 528, 1152), (257, 16, 128)])
@pytest.mark.parametrize("kernel", ["tiny", "small", "pipe", "v5"])
def test_gemm_quantized_equals_gemm_then_quantize(monkeypatch, M, N, K, kernel):
    monkeypatch.setenv("NVFP4_GEMM_KERNEL", kernel)
    for factor, epi, bias in ((1.0, "gelu", True), (0.25, "none", False), (8.0, "none", True)):
        y, static, fused, two = _gemm_quantized_case(M, N, K, M + N + K, factor, epi, bias)
        for u, v, what in ((fused.codes, two.codes, "codes"), (fused.scales, two.scales, "scales"),
                           (fused.tensor_scale, two.tensor_scale, "tensor scale")):
            assert torch_equal(u, v), f"{kernel} {M}x{N}x{K} amax*{factor}: {what}"
        # and the quantizer half against the oracle, on the GPU's bf16 output
        ref = o_quantize(bits_of(y), amax=np.float32(static.item()))
        assert_quant_equal(fused, ref, f"oracle {kernel} amax*{factor}")
        if factor < 1.0:
            assert (ref.scales == 0x7E).any()     # the static scale saturates some blocks


def torch_equal(u, v):
    import torch
    return bool(torch.equal(u, v))


@pytest.mark.parametrize("kernel", ["default", "pipe", "one_item"])
def test_gemm_quantized_mlp_up_full_size(monkeypatch, kernel):
    # H of the MLP at 2048^2 written straight in NVFP4 under a static amax
    # (default: v5 on the persistent grid; one_item: v5, one tile per workgroup)
    import torch
    if kernel == "one_item":
        monkeypatch.setenv("NVFP4_GEMM_PERSISTENT", "0")
    elif kernel != "default":
        monkeypatch.setenv("NVFP4_GEMM_KERNEL", kernel)
    x_bits = _mlp()["x"]
    wu_bits, _ = _oracle_weight("w_up")
    qx, qwu = gpu_quantize(x_bits), gpu_quantize(wu_bits)
    amax = torch.empty((1,), dtype=torch.float32, device="cuda")
    h = nv.gemm(qx, qwu, epilogue="gelu", y_amax=amax)
    static = amax * 0.75
    fused = nv.gemm_quantized(qx, qwu, static, epilogue="gelu")
    two = nv.quantize(h, amax=static)
    _sync()
    assert torch_equal(fused.codes, two.codes) and torch_equal(fused.scales, two.scales)
    assert torch_equal(fused.tensor_scale, two.tensor_scale)


def test_gemm_quantized_persistent_ragged():
    # 18 x 17 = 306 tiles of 256x256, more than the compute units: the
    # persistent grid over tiles with ragged rows and columns, GELU and bias,
    # against nvfp4_gemm followed by nvfp4_quantize
    import torch
    M, N, K = 4400, 4112, 512
    for factor, epi, bias in ((1.0, "gelu", True), (0.25, "none", False)):
        y, static, fused, two = _gemm_quantized_case(M, N, K, 4242, factor, epi, bias)
        for u, v, what in ((fused.codes, two.codes, "codes"), (fused.scales, two.scales, "scales"),
                           (fused.tensor_scale, two.tensor_scale, "tensor scale")):
            assert torch_equal(u, v), f"persistent {M}x{N}x{K} amax*{factor}: {what}"


def test_gemm_quantized_nonfinite_amax():
    import torch
    qa = gpu_quantize(W.random_matrix(5, (64, 64)))
    qw = gpu_quantize(W.random_matrix(6, (32, 64), "normal", 0.02))
    fused = nv.gemm_quantized(qa, qw, torch.full((1,), float("inf"), device="cuda"))
    _sync()
    assert np.isnan(fused.tensor_scale.item())


# ------------------------------------------------------- bf16 passthrough --

@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (130, 70, 40), (2, 1000, 3072), (300, 257, 1024),
                                   (1, 5, 8), (8, 777, 520), (7, 33, 4104), (9, 100, 256)])
def test_gemm_bf16(M, N, K):
    x = W.random_matrix(M + N, (M, K), "normal")
    w = W.random_matrix(M + N + 1, (N, K), "normal", 0.02)
    b = W.random_matrix(M + N + 2, (1, N), "normal", 0.1)[0]
    y = bits_of(nv.gemm_bf16(to_dev(x), to_dev(w), bias=to_dev(b)))
    ref = linear_bf16_fp64(x, w, b)
    assert_gemm_close(y, ref, f"bf16 {M}x{N}x{K}")


@pytest.mark.parametrize("M", [2, 150])
def test_gemm_bf16_gelu(M):
    # both the few-row kernel and the tiled one apply the same epilogue
    x = W.random_matrix(M, (M, 1024), "normal")
    w = W.random_matrix(M + 1, (300, 1024), "normal", 0.05)
    b = W.random_matrix(M + 2, (1, 300), "normal", 0.5)[0]
    y = bits_of(nv.gemm_bf16(to_dev(x), to_dev(w), bias=to_dev(b), epilogue="gelu"))
    ref = linear_bf16_fp64(x, w, b, gelu=True)
    assert_gemm_close(y, ref, f"bf16 gelu M={M}")


@pytest.mark.parametrize("kernel", ["tile", "dma", "ksplit"])
@pytest.mark.parametrize("M,N,K,epi", [(300, 257, 1024, "none"), (512, 512, 64, "gelu"),
                                       (257, 258, 128, "none"), (384, 300, 192, "gelu"),
                                       (600, 770, 640, "none"), (513, 1024, 320, "gelu"),
                                       (256, 256, 32, "none"), (270, 300, 96, "gelu"), (140, 130, 40, "gelu"),
                                       (520, 260, 160, "none"), (256, 512, 224, "none")])
def test_gemm_bf16_kernels(monkeypatch, M, N, K, epi, kernel):
    # the three tiled kernels pinned, on shapes with one, two and an odd number of
    # 64-wide K stages, ragged M / N tails, full tiles with N % 4 != 0, and K
    # not a multiple of 64 (the 256x256 kernel does not apply: the pin falls
    # back to 128x128 tiles); ksplit also with a single K step (its second
    # group then adds nothing)
    monkeypatch.setenv("NVFP4_BF16_GEMM_KERNEL", kernel)
    x = W.random_matrix(M + 7, (M, K), "normal")
    w = W.random_matrix(N + 8, (N, K), "normal", 0.03)
    b = W.random_matrix(K + 9, (1, N), "normal", 0.2)[0]
    y = bits_of(nv.gemm_bf16(to_dev(x), to_dev(w), bias=to_dev(b), epilogue=epi))
    ref = linear_bf16_fp64(x, w, b, gelu=epi == "gelu")
    assert_gemm_close(y, ref, f"bf16 {kernel} {M}x{N}x{K} {epi}")


@pytest.mark.parametrize("M,N,K,epi", [(4224, 9216, 3072, "gelu"), (8448, 3072, 12288, "none")])
def test_gemm_bf16_large_sampled_rows(M, N, K, epi):
    # sizes of a DiT block's linears at 4224 and 8448 tokens (the 256x256
    # kernel by the default rule): sampled rows against the float64 sum
    x = W.random_matrix(M + 11, (M, K), "normal")
    w = W.random_matrix(N + 12, (N, K), "normal", 0.02)
    b = W.random_matrix(N + 13, (1, N), "normal", 0.2)[0]
    y = bits_of(nv.gemm_bf16(to_dev(x), to_dev(w), bias=to_dev(b), epilogue=epi))
    rows = _sampled_rows(M, 40, seed=M + 1)
    ref = linear_bf16_fp64(x[rows], w, b, gelu=epi == "gelu")
    assert_gemm_close(y[rows], ref, f"bf16 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,epi", [(16, 3072, 12288, "gelu"), (300, 2000, 6144, "none")])
def test_gemm_bf16_few_tiles_long_k(M, N, K, epi):
    # few 128x128 tiles and a long K: the default dispatch splits K between
    # two wave groups in each tile; against the float64 sum, all rows
    x = W.random_matrix(M + 21, (M, K), "normal")
    w = W.random_matrix(N + 22, (N, K), "normal", 0.02)
    b = W.random_matrix(N + 23, (1, N), "normal", 0.2)[0]
    y = bits_of(nv.gemm_bf16(to_dev(x), to_dev(w), bias=to_dev(b), epilogue=epi))
    ref = linear_bf16_fp64(x, w, b, gelu=epi == "gelu")
    assert_gemm_close(y, ref, f"bf16 {M}x{N}x{K} {epi}")


def test_gemm_bf16_modulation_shape():
    # a modulation linear kept bf16: temb [2,3072] x W [18432,3072]
    temb = W.random_matrix(81, (2, 3072), "normal")
    w_mod = W.random_matrix(82, (18432, 3072), "normal", 0.02)
    y = bits_of(nv.gemm_bf16(to_dev(temb), to_dev(w_mod)))
    ref = linear_bf16_fp64(temb, w_mod)
    assert_gemm_close(y, ref, "modulation [2,3072]x[18432,3072]")


def test_linear_dispatch_by_layer_name():
    d = W.linear_small()
    x = to_dev(d["x"])
    wq = nv.quantize_weight(to_dev(d["w"]))
    y_q = bits_of(nv.linear(x, wq, "transformer_blocks.0.attn.to_q"))
    ra, rw = o_quantize(d["x"]), o_quantize(d["w"])
    ref, _ = gemm_fp64(ra, rw, 1024)
    assert_gemm_close(y_q, ref, "nvfp4 layer")
    y_b = bits_of(nv.linear(x, to_dev(d["w"]), "proj_out"))
    assert_gemm_close(y_b, linear_bf16_fp64(d["x"], d["w"]), "bf16 layer")


@pytest.mark.parametrize("shape", [(300, 1024), (16896, 3072)])
def test_quantize_single_pass_wait_timeout_path(shape, monkeypatch):
    # a zero wait limit makes every workgroup that is not released at once
    # read the whole tensor for its amax itself (the path taken when the grid
    # is not co-resident): the same bytes as the oracle
    monkeypatch.setenv("NVFP4_QUANT_KERNEL", "resident")
    monkeypatch.setenv("NVFP4_QUANT_WAIT_TICKS", "0")
    bits = W.random_matrix(51, shape, "outliers")
    if shape[0] * shape[1] <= 1 << 20:
        check_quantize(bits, label=f"{shape} timeout path")
        return
    q = gpu_quantize(bits)
    amax = np.float32(np.abs(bf16_bits_to_f32(bits)).max())
    rows = np.unique(np.concatenate([stratified_rows(shape[0]),
                                     np.random.default_rng(3).choice(shape[0], 40, replace=False)]))
    ref = o_quantize(bits[rows], amax=amax)
    assert np.array_equal(q.scales.cpu().numpy()[rows], ref.scales)
    assert np.array_equal(q.codes.cpu().numpy()[rows], ref.codes)
    assert q.tensor_scale.cpu().numpy().view(np.uint32)[0] == np.float32(ref.tensor_scale).view(np.uint32)


def test_quantize_workspace_reused_across_kernels(monkeypatch):
    # one zero-filled workspace for many calls: the single-pass kernel never
    # clears its arrival words (each call leaves them ready for the next) and
    # the two-pass kernels' partial maxima sit past them, so interleaved calls
    # of both, on two tensors, all give the oracle's bytes
    ws = nv.quantize_workspace()
    cases = [(W.random_matrix(61, (300, 1024), "outliers"), None),
             (W.random_matrix(62, (513, 1024), "t3"), None)]
    cases = [(b, o_quantize(b), to_dev(b)) for b, _ in cases]
    for kernel in ("resident", "twopass", "resident", "resident", "twopass", "small", "resident"):
        monkeypatch.setenv("NVFP4_QUANT_KERNEL", kernel)
        for bits, ref, x in cases:
            if kernel == "small" and bits.size > (1 << 18):
                continue
            q = nv.quantize(x, workspace=ws)
            _sync()
            assert_quant_equal(q, ref, f"{kernel} {bits.shape}")


def test_quantize_default_workspace_many_calls():
    # the binding's own workspace (one per device and stream, zeroed once):
    # the activation [16896,3072] quantized repeatedly, every call bit-exact
    bits = W.quantize_act()["x"]
    ref = o_quantize(bits)
    x = to_dev(bits)
    for _ in range(5):
        q = nv.quantize(x)
        _sync()
        assert_quant_equal(q, ref, "repeat")


@pytest.mark.parametrize("M,N,K", [(3, 40, 8192), (70, 300, 12288)])
def test_gemm_long_k_small_output(M, N, K):
    # a long K sends even a small output to the 256x256 kernel, whose grid of
    # fewer tiles than compute units takes its K split from the cost model
    a_bits = W.random_matrix(M + 7 * N, (M, K), "t3")
    w_bits = W.random_matrix(N + 5 * M, (N, K), "normal", 0.02)
    qa, ra = check_quantize(a_bits)
    qw, rw = check_quantize(w_bits)
    ws = nv.gemm_workspace(M, N, K)
    assert ws is not None                    # the plan splits
    y = bits_of(nv.gemm(qa, qw, workspace=ws))
    ref, _ = gemm_fp64(ra, rw, K)
    assert_gemm_close(y, ref, f"{M}x{N}x{K}")


def test_gemm_share_of_8_down_sampled_rows():
    # one GPU's share of the MLP down projection when the 2048^2 block is
    # split over 8 GPUs by tokens: H [2112,12288] x W_down [3072,12288]^T, a
    # grid of 108 tiles split 2 ways over K; sampled rows against the exact sum
    M, N, K = 2112, 3072, 12288
    h_bits = W.random_matrix(81, (M, K), "normal", 0.5)
    qh, rh = check_quantize(h_bits)
    wb, rw = _oracle_weight("w_down")
    qw = gpu_quantize(wb)
    y = bits_of(nv.gemm(qh, qw, workspace=nv.gemm_workspace(M, N, K)))
    rows = _sampled_rows(M, 48, seed=5)
    ref, _ = gemm_exact_rows(rh, rw, K, rows)
    assert_gemm_close(y[rows], ref, "down share rows")


def _random_shapes(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.integers(1, 700))
        N = int(rng.integers(1, 700))
        K = 16 * int(rng.choice([rng.integers(1, 24), rng.integers(24, 200), 8 * rng.integers(1, 25)]))
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", _random_shapes())
def test_gemm_random_shapes(M, N, K):
    # seeded random shapes through the default dispatch (64x64, 128x128 or
    # 256x256 tiles, with or without a K split): bias + GELU against the oracle
    a_bits = W.random_matrix(M * 31 + K, (M, K), "t3")
    w_bits = W.random_matrix(N * 17 + K, (N, K), "normal", 0.02)
    b_bits = W.random_matrix(M + N + K, (1, N), "normal", 0.1)[0]
    qa, ra = check_quantize(a_bits, label=f"A {M}x{K}")
    qw, rw = check_quantize(w_bits, label=f"W {N}x{K}")
    y = bits_of(nv.gemm(qa, qw, bias=to_dev(b_bits), epilogue="gelu",
                        workspace=nv.gemm_workspace(M, N, K)))
    ref, _ = gemm_fp64(ra, rw, K, bias_bits=b_bits, gelu=True)
    assert_gemm_close(y, ref, f"{M}x{N}x{K}")


def _random_big_shapes(n=6, seed=77):
    rng = np.random.default_rng(seed)
    # even cases: K a multiple of 128 (v5); odd cases: any multiple of 16 (v3)
    return [(int(rng.integers(2900, 4300)), int(rng.integers(2900, 4300)),
             128 * int(rng.integers(2, 12)) if i % 2 == 0 else 16 * int(rng.integers(8, 80)))
            for i in range(n)]


@pytest.mark.parametrize("M,N,K", _random_big_shapes())
def test_gemm_random_large_shapes_sampled_rows(M, N, K):
    # seeded random shapes large enough for the 256x256 kernels (v5 where
    # K % 128 == 0, else v3; tail split by the default plan): sampled rows
    a_bits = W.random_matrix(M + 3 * K, (M, K), "t3")
    w_bits = W.random_matrix(N + 5 * K, (N, K), "normal", 0.02)
    qa, ra = check_quantize(a_bits, label=f"A {M}x{K}")
    qw, rw = check_quantize(w_bits, label=f"W {N}x{K}")
    y = bits_of(nv.gemm(qa, qw, epilogue="gelu", workspace=nv.gemm_workspace(M, N, K)))
    rows = _sampled_rows(M, 40, seed=M)
    ref, _ = gemm_fp64(ra, rw, K, gelu=True, rows=rows)
    assert_gemm_close(y[rows], ref, f"{M}x{N}x{K}")
