"""The linear layers of one DiT block at full size -- 2048x2048 image with a
CFG pair: M = 33792 token rows, hidden 3072, MLP 12288 -- run as an NVFP4
model runs them (DitBlockLinears), checked stage by stage against the oracle:

  * every weight's NVFP4 bytes (quantized once, at construction) bit-exact;
  * QKV and output projections: the activation's codes and scales bit-exact
    and the GEMM output within the 2e-3 bar, on rows covering every 256-row
    tile band of the output;
  * MLP up + GELU against the oracle's GELU(G1); the epilogue's amax equal to
    max |H| exactly; quantize(H) with that amax bit-exact; the down projection
    against the oracle's G1 on the GPU's own H (each stage on the previous
    stage's GPU output, so a code flipped at a rounding tie cannot propagate);
  * the modulation linear, kept bf16 by the exclude pattern, against the
    float64 sum.
Sources: "英伟达B200狂飙10.2倍！AI绘图告别龟速！" (nmedialink.com), section
"NVFP4量化" (16-element blocks, the exclude pattern); "NVIDIA介绍用TensorRT LLM
VisualGen加速Blackwell上的FLUX 3 Image Klein…" (sns.style), time-breakdown
paragraph (2048x2048, NVFP4 weights).
"""

import numpy as np
import pytest

import nvfp4_block_scaled_05_amd as nv
from nvfp4_block_scaled_05_amd import inputs as W
from nvfp4_block_scaled_05_amd.dit_block import LAYERS, DitBlockLinears
from oracle import bf16_bits_to_f32, gemm_fp64, linear_bf16_fp64, quantize as o_quantize
from tests.gpu_util import bits_of, rel_frobenius, stratified_rows, to_dev, ulp_diff

pytestmark = pytest.mark.gpu

TOKENS = 33792
NAMES = list(LAYERS)
MOD, QKV, OUT, UP, DOWN = NAMES
GEMM_TOL = 2e-3


@pytest.fixture(scope="module")
def run():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load()
    blk = W.dit_block_2048()
    wts = {k: to_dev(blk[k]) for k in ("w_mod", "w_qkv", "w_o", "w_up", "w_down")}
    acts = [to_dev(blk[k]) for k in ("temb", "x_qkv", "x_o", "x_mlp")]
    block = DitBlockLinears(wts, tokens=TOKENS)
    out = block(*acts)
    torch.cuda.synchronize()
    rows = stratified_rows(TOKENS)
    yield blk, block, out, rows
    _ORACLE_W.clear()
    del block, out, wts, acts
    torch.cuda.empty_cache()


_ORACLE_W = {}


def _oracle_weight(blk, key):
    """The oracle's quantization of a weight, computed once per module."""
    if key not in _ORACLE_W:
        _ORACLE_W[key] = o_quantize(blk[key])
    return _ORACLE_W[key]


def _rows_of(t, rows):
    """Rows of a device tensor on the host (bf16 as uint16 bit patterns)."""
    import torch
    r = t[torch.as_tensor(rows, device=t.device)]
    if r.dtype == torch.bfloat16:
        return r.view(torch.int16).cpu().numpy().view(np.uint16)
    return r.cpu().numpy()


def _check_gemm(y, ref, label):
    err = rel_frobenius(y, ref)
    far = float((ulp_diff(y, ref) > 1).mean())
    assert err <= GEMM_TOL, f"{label}: rel Frobenius {err:.3e}"
    assert far <= 1e-2, f"{label}: {far:.2e} of outputs more than 1 ulp away"


def test_layer_selection(run):
    _, block, _, _ = run
    assert not block.quantized[MOD]          # contains "stream": kept bf16
    assert all(block.quantized[n] for n in (QKV, OUT, UP, DOWN))
    assert block.chain


@pytest.mark.parametrize("name,key", [(QKV, "w_qkv"), (OUT, "w_o"), (UP, "w_up"), (DOWN, "w_down")])
def test_weights_bit_exact(run, name, key):
    blk, block, _, _ = run
    ref = _oracle_weight(blk, key)
    q = block.weights[name]
    assert np.array_equal(q.codes.cpu().numpy(), ref.codes), f"{key} codes"
    assert np.array_equal(q.scales.cpu().numpy(), ref.scales), f"{key} scales"
    assert q.tensor_scale.cpu().numpy().view(np.uint32)[0] == np.float32(ref.tensor_scale).view(np.uint32)


@pytest.mark.parametrize("name,xkey,wkey", [(QKV, "x_qkv", "w_qkv"), (OUT, "x_o", "w_o")])
def test_attention_projections(run, name, xkey, wkey):
    blk, block, out, rows = run
    x = blk[xkey]
    amax = np.float32(np.abs(bf16_bits_to_f32(x)).max())
    rx = o_quantize(x[rows], amax=amax)           # rows of the full-tensor quantization
    codes, scales, ts = block.qbuf[name]
    assert np.array_equal(_rows_of(codes, rows), rx.codes), f"{xkey} codes"
    assert np.array_equal(_rows_of(scales, rows), rx.scales), f"{xkey} scales"
    assert ts.cpu().numpy().view(np.uint32)[0] == np.float32(rx.tensor_scale).view(np.uint32)
    rw = _oracle_weight(blk, wkey)
    ref, _ = gemm_fp64(rx, rw, x.shape[1])
    _check_gemm(_rows_of(out[name], rows), ref, name)


def test_mlp_chain(run):
    blk, block, out, rows = run
    x = blk["x_mlp"]
    # stage 1: H = GELU(Xq @ Wup^T)
    x_amax = np.float32(np.abs(bf16_bits_to_f32(x)).max())
    rx = o_quantize(x[rows], amax=x_amax)
    rwu = _oracle_weight(blk, "w_up")
    h_ref, _ = gemm_fp64(rx, rwu, x.shape[1], gelu=True)
    h = out[UP]
    h_rows = _rows_of(h, rows)
    _check_gemm(h_rows, h_ref, "up + GELU")
    # stage 2: the epilogue amax is max |H| over the whole GPU output, exactly
    h_amax = float(h.abs().max().float().item())
    assert np.float32(block.amax.item()) == np.float32(h_amax)
    # stage 3: quantize(H_gpu) with that amax, bit-exact
    rh = o_quantize(h_rows, amax=np.float32(h_amax))
    codes, scales, ts = block.qbuf[DOWN]
    assert np.array_equal(_rows_of(codes, rows), rh.codes), "H codes"
    assert np.array_equal(_rows_of(scales, rows), rh.scales), "H scales"
    assert ts.cpu().numpy().view(np.uint32)[0] == np.float32(rh.tensor_scale).view(np.uint32)
    # stage 4: Y = Hq @ Wdown^T on the GPU's own H
    rwd = _oracle_weight(blk, "w_down")
    y_ref, _ = gemm_fp64(rh, rwd, h.shape[1])
    _check_gemm(_rows_of(out[DOWN], rows), y_ref, "down")


def test_modulation_bf16(run):
    blk, _, out, _ = run
    ref = linear_bf16_fp64(blk["temb"], blk["w_mod"])
    y = bits_of(out[MOD])
    assert rel_frobenius(y, ref) <= GEMM_TOL
    assert float((ulp_diff(y, ref) > 1).mean()) <= 1e-2
