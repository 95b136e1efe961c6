"""HIP-graph capture of library call sequences: every replay must equal the
eager result bit for bit, with eager work and synchronisation between
replays, and replays must follow in-place updates of the captured inputs."""

import numpy as np
import pytest

import nvfp4_block_scaled_05_amd as nv
from nvfp4_block_scaled_05_amd import inputs as W
from nvfp4_block_scaled_05_amd.dit_block import LAYERS, DitBlockLinears
from nvfp4_block_scaled_05_amd.graph import capture
from oracle import gemm_fp64, quantize as o_quantize
from tests.gpu_util import bits_of, rel_frobenius, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load()


def _sync():
    import torch
    torch.cuda.synchronize()


def _linear_small_fn(x, w):
    """C1: both operands quantized on every call, then the GEMM."""
    import torch
    rows, k = x.shape
    n = w.shape[0]
    qx = (torch.empty((rows, k // 2), dtype=torch.uint8, device="cuda"),
          torch.empty((rows, k // 16), dtype=torch.uint8, device="cuda"),
          torch.empty((1,), dtype=torch.float32, device="cuda"))
    qw = (torch.empty((n, k // 2), dtype=torch.uint8, device="cuda"),
          torch.empty((n, k // 16), dtype=torch.uint8, device="cuda"),
          torch.empty((1,), dtype=torch.float32, device="cuda"))
    ws = nv.quantize_workspace()
    ws2 = nv.quantize_workspace()
    y = torch.empty((rows, n), dtype=torch.bfloat16, device="cuda")

    def fn():
        a = nv.quantize(x, workspace=ws, out=qx)
        b = nv.quantize(w, workspace=ws2, out=qw)
        return nv.gemm(a, b, out=y, workspace=None)
    return fn


def test_linear_small_graph_replays_equal_eager():
    d = W.linear_small()
    x, w = to_dev(d["x"]), to_dev(d["w"])
    fn = _linear_small_fn(x, w)
    eager = bits_of(fn()).copy()
    g = capture(fn)
    other = _linear_small_fn(to_dev(W.random_matrix(5, (128, 1024))), w)
    for _ in range(3):
        other()                              # eager work between replays
        _sync()
        assert np.array_equal(bits_of(g.replay()), eager)
    # the oracle agrees with what the graph computes
    ref, _ = gemm_fp64(o_quantize(d["x"]), o_quantize(d["w"]), 1024)
    assert rel_frobenius(bits_of(g.outputs), ref) <= 2e-3
    # in-place update of the captured input is seen by the next replay
    new = W.random_matrix(6, (128, 1024), "t3")
    x.copy_(to_dev(new))
    y_new = bits_of(g.replay()).copy()
    assert np.array_equal(y_new, bits_of(_linear_small_fn(x, w)()))
    assert not np.array_equal(y_new, eager)


def _small_block(seed=0, tokens=512, hidden=256, mlp=1024):
    rng = np.random.default_rng(seed)
    def mat(shape, std):
        return to_dev(W.f32_to_bf16_bits((std * rng.standard_normal(shape)).astype(np.float32)))
    weights = {"w_mod": mat((6 * hidden, hidden), 0.02), "w_qkv": mat((3 * hidden, hidden), 0.02),
               "w_o": mat((hidden, hidden), 0.02), "w_up": mat((mlp, hidden), 0.02),
               "w_down": mat((hidden, mlp), 0.02)}
    acts = [mat((2, hidden), 1.0), mat((tokens, hidden), 1.0), mat((tokens, hidden), 1.0),
            mat((tokens, hidden), 1.0)]
    return weights, acts


def test_dit_block_graph_replays_equal_eager():
    weights, (temb, xq, xo, xm) = _small_block()
    block = DitBlockLinears(weights, tokens=xq.shape[0])
    assert not block.quantized["double_stream_modulation_img.linear"]
    eager = {k: bits_of(v).copy() for k, v in block(temb, xq, xo, xm).items()}
    g = capture(lambda: block(temb, xq, xo, xm))
    for _ in range(3):
        nv.gemm_bf16(xq, weights["w_o"])     # eager work between replays
        _sync()
        out = g.replay()
        for k in LAYERS:
            assert np.array_equal(bits_of(out[k]), eager[k]), k
    # the NVFP4 QKV projection against the oracle
    x_bits = bits_of(xq)
    w_bits = bits_of(weights["w_qkv"])
    ref, _ = gemm_fp64(o_quantize(x_bits), o_quantize(w_bits), x_bits.shape[1])
    assert rel_frobenius(eager["transformer_blocks.0.attn.to_qkv"], ref) <= 2e-3


@pytest.mark.parametrize("kernel", ["resident", "twopass"])
def test_dynamic_quantize_graph_replays(kernel, monkeypatch):
    """The dynamic-amax quantizer captured and replayed: the single-pass
    kernel (forced on a small tensor) with its counter-clearing launch, and
    the two-pass kernels.  Every replay equals the eager bytes and the oracle,
    with eager quantizes of another tensor on the same workspace between
    replays (they leave its counters and partials behind)."""
    import torch
    monkeypatch.setenv("NVFP4_QUANT_KERNEL", kernel)
    bits = W.random_matrix(41, (300, 1024), "outliers")
    x = to_dev(bits)
    ws = nv.quantize_workspace()
    out = (torch.empty((300, 512), dtype=torch.uint8, device="cuda"),
           torch.empty((300, 64), dtype=torch.uint8, device="cuda"),
           torch.empty((1,), dtype=torch.float32, device="cuda"))
    fn = lambda: nv.quantize(x, workspace=ws, out=out)
    q = fn()
    _sync()
    eager = [t.cpu().numpy().copy() for t in (q.codes, q.scales, q.tensor_scale)]
    ref = o_quantize(bits)
    assert np.array_equal(eager[0], ref.codes) and np.array_equal(eager[1], ref.scales)
    g = capture(fn)
    other = to_dev(W.random_matrix(42, (300, 1024), "t3"))
    for _ in range(4):
        nv.quantize(other, workspace=ws)     # eager work on the same workspace
        _sync()
        g.replay()
        _sync()
        got = [t.cpu().numpy() for t in (out[0], out[1], out[2])]
        assert all(np.array_equal(a, b) for a, b in zip(got, eager))
