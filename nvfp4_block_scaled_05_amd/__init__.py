"""MI355X (gfx950) NVFP4: two-level quantize / dequantize, the block-scaled
W4A4 GEMM of the DiT linear layers, a bf16 passthrough GEMM, and the layer
predicate -- Python face of the C ABI in include/nvfp4.h.

Functions mirror the C entry points by name.  Tensors are torch tensors on the
current HIP device (bf16 data as ``torch.bfloat16``, codes and scales as
``torch.uint8``, tensor scales / amax as one-element ``torch.float32``); calls
are enqueued on ``torch.cuda.current_stream()``.  Outputs that are not passed
in are allocated with torch; nothing here computes any part of the method.
"""

from collections import namedtuple

from . import _binding
from ._binding import EPILOGUES, Nvfp4Error, load

Nvfp4Tensor = namedtuple("Nvfp4Tensor", ["codes", "scales", "tensor_scale", "cols"])
Fp8Tensor = namedtuple("Fp8Tensor", ["codes", "scales"])   # E4M3 [rows, cols], float [rows]

__all__ = ["Nvfp4Tensor", "Fp8Tensor", "Nvfp4Error", "load", "abi_version", "status_string",
           "quantize_workspace_bytes", "quantize", "dequantize", "gemm", "gemm_workspace",
           "gemm_quantized", "gemm_bf16", "layer_is_quantized", "quantize_weight", "linear",
           "fp8_quantize", "fp8_gemm", "fp8_gemm_workspace"]


def _torch():
    import torch
    return torch


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def abi_version():
    return load().nvfp4_abi_version()


def status_string(status):
    return load().nvfp4_status_string(status).decode()


def quantize_workspace_bytes(rows, cols):
    return load().nvfp4_quantize_workspace_bytes(rows, cols)


def quantize(x, amax=None, workspace=None, dev_status=None, out=None):
    """NVFP4-quantize a 2-D bf16 tensor.  Returns an ``Nvfp4Tensor``.

    amax: optional one-element float32 device tensor (a producer's amax); when
    None the amax is computed by the library.  out: optional (codes, scales,
    tensor_scale) tensors to write into.
    """
    torch = _torch()
    lib = load()
    rows, cols = x.shape
    dev = x.device
    if out is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
        ts = torch.empty((1,), dtype=torch.float32, device=dev)
    else:
        codes, scales, ts = out
    if amax is None and workspace is None:
        nbytes = lib.nvfp4_quantize_workspace_bytes(rows, cols)
        workspace = torch.empty((max(nbytes, 4),), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _binding.check(lib.nvfp4_quantize(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _ptr(ts),
                                      _ptr(amax), _ptr(workspace), ws_bytes, _ptr(dev_status),
                                      _stream()), "nvfp4_quantize")
    return Nvfp4Tensor(codes, scales, ts, cols)


def dequantize(q, out=None):
    torch = _torch()
    rows = q.codes.shape[0]
    y = out if out is not None else torch.empty((rows, q.cols), dtype=torch.bfloat16,
                                                device=q.codes.device)
    _binding.check(load().nvfp4_dequantize(_ptr(q.codes), _ptr(q.scales), _ptr(q.tensor_scale),
                                           rows, q.cols, _ptr(y), _stream()), "nvfp4_dequantize")
    return y


def gemm_workspace(M, N, K, device="cuda"):
    """A workspace for ``gemm`` on an (M, N, K) problem, or None if it would not split."""
    nbytes = load().nvfp4_gemm_workspace_bytes(M, N, K)
    if nbytes == 0:
        return None
    return _torch().empty(nbytes, dtype=_torch().uint8, device=device)


_NO_WORKSPACE = object()


def gemm(a, w, bias=None, epilogue="none", y_amax=None, out=None, workspace=_NO_WORKSPACE):
    """Y = epi(sA*sW * A_hat @ W_hat^T + bias) in bf16, from two ``Nvfp4Tensor``.

    ``workspace``: a uint8 device tensor from ``gemm_workspace`` (reused across
    calls on one stream), None to compute every tile whole, or left out to have
    one taken from torch's caching allocator for this call.
    """
    torch = _torch()
    M, N, K = a.codes.shape[0], w.codes.shape[0], a.cols
    if w.cols != K:
        raise ValueError("K mismatch")
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=a.codes.device)
    if workspace is _NO_WORKSPACE:
        workspace = gemm_workspace(M, N, K, device=a.codes.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _binding.check(load().nvfp4_gemm(_ptr(a.codes), _ptr(a.scales), _ptr(a.tensor_scale),
                                     _ptr(w.codes), _ptr(w.scales), _ptr(w.tensor_scale),
                                     _ptr(bias), M, N, K, EPILOGUES[epilogue], _ptr(y),
                                     _ptr(y_amax), _ptr(workspace), ws_bytes, _stream()),
                   "nvfp4_gemm")
    return y


def gemm_quantized(a, w, amax, bias=None, epilogue="none", out=None):
    """The GEMM with NVFP4 output under the static amax ``amax`` (one-element
    float32 device tensor): the same bytes as ``quantize(gemm(a, w), amax=amax)``.
    Returns an ``Nvfp4Tensor``; ``out``: optional (codes, scales, tensor_scale)."""
    torch = _torch()
    M, N, K = a.codes.shape[0], w.codes.shape[0], a.cols
    if w.cols != K:
        raise ValueError("K mismatch")
    dev = a.codes.device
    if out is None:
        out = (torch.empty((M, N // 2), dtype=torch.uint8, device=dev),
               torch.empty((M, N // 16), dtype=torch.uint8, device=dev),
               torch.empty((1,), dtype=torch.float32, device=dev))
    codes, scales, ts = out
    _binding.check(load().nvfp4_gemm_quantized(_ptr(a.codes), _ptr(a.scales), _ptr(a.tensor_scale),
                                               _ptr(w.codes), _ptr(w.scales), _ptr(w.tensor_scale),
                                               _ptr(bias), M, N, K, EPILOGUES[epilogue], _ptr(amax),
                                               _ptr(codes), _ptr(scales), _ptr(ts), _stream()),
                   "nvfp4_gemm_quantized")
    return Nvfp4Tensor(codes, scales, ts, N)


def fp8_quantize(x, dev_status=None, out=None):
    """FP8 row-wise quantization of a 2-D bf16 tensor (one scale per row).
    Returns an ``Fp8Tensor``; ``out``: optional (codes, scales)."""
    torch = _torch()
    rows, cols = x.shape
    if out is None:
        out = (torch.empty((rows, cols), dtype=torch.uint8, device=x.device),
               torch.empty((rows,), dtype=torch.float32, device=x.device))
    codes, scales = out
    _binding.check(load().nvfp4_fp8_quantize_rowwise(_ptr(x), rows, cols, _ptr(codes), _ptr(scales),
                                                     _ptr(dev_status), _stream()),
                   "nvfp4_fp8_quantize_rowwise")
    return Fp8Tensor(codes, scales)


def fp8_gemm_workspace(M, N, K, device="cuda"):
    """A workspace for ``fp8_gemm`` on an (M, N, K) problem, or None if it would not split."""
    nbytes = load().nvfp4_fp8_gemm_workspace_bytes(M, N, K)
    if nbytes == 0:
        return None
    return _torch().empty(nbytes, dtype=_torch().uint8, device=device)


def fp8_gemm(a, w, bias=None, epilogue="none", out=None, workspace=_NO_WORKSPACE):
    """Y = epi((A_q @ W_q^T) * dA[m] * dW[n] + bias) in bf16, from two ``Fp8Tensor``.

    ``workspace``: as for ``gemm`` (from ``fp8_gemm_workspace``, None, or left out).
    """
    torch = _torch()
    M, K = a.codes.shape
    N = w.codes.shape[0]
    if w.codes.shape[1] != K:
        raise ValueError("K mismatch")
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=a.codes.device)
    if workspace is _NO_WORKSPACE:
        workspace = fp8_gemm_workspace(M, N, K, device=a.codes.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _binding.check(load().nvfp4_fp8_gemm(_ptr(a.codes), _ptr(a.scales), _ptr(w.codes), _ptr(w.scales),
                                         _ptr(bias), M, N, K, EPILOGUES[epilogue], _ptr(y),
                                         _ptr(workspace), ws_bytes, _stream()),
                   "nvfp4_fp8_gemm")
    return y


def gemm_bf16(x, w, bias=None, epilogue="none", out=None):
    """Y = epi(X @ W^T + bias) in bf16 with fp32 accumulation (bf16 passthrough)."""
    torch = _torch()
    M, K = x.shape
    N = w.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _binding.check(load().nvfp4_gemm_bf16(_ptr(x), _ptr(w), _ptr(bias), M, N, K,
                                          EPILOGUES[epilogue], _ptr(y), _stream()),
                   "nvfp4_gemm_bf16")
    return y


def layer_is_quantized(name, pattern=None):
    """True when the layer runs in NVFP4 under ``pattern`` (default: the page's exclude regex)."""
    r = load().nvfp4_layer_is_quantized(name.encode(), None if pattern is None else pattern.encode())
    if r < 0:
        raise Nvfp4Error(r, "nvfp4_layer_is_quantized")
    return bool(r)


def quantize_weight(w):
    """Quantize a weight once, at load time (quantize_weights=True)."""
    return quantize(w)


def linear(x, weight, name, bias=None, epilogue="none", pattern=None):
    """One linear layer as the patched model runs it: NVFP4 (quantize x, then
    the block-scaled GEMM against the pre-quantized ``weight``) when the layer
    predicate selects it, else the bf16 passthrough on the bf16 ``weight``."""
    if layer_is_quantized(name, pattern):
        return gemm(quantize(x), weight, bias=bias, epilogue=epilogue)
    return gemm_bf16(x, weight, bias=bias, epilogue=epilogue)
