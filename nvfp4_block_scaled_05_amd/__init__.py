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
           "quantize_workspace_bytes", "quantize_workspace", "quantize", "dequantize", "gemm", "gemm_workspace",
           "gemm_quantized", "gemm_bf16", "layer_is_quantized", "quantize_weight", "linear",
           "fp8_quantize", "fp8_gemm", "fp8_gemm_workspace"]


_TORCH = None
_RAW_STREAM = None


def _torch():
    global _TORCH
    if _TORCH is None:
        import torch
        _TORCH = torch
    return _TORCH


def _stream():
    """The current HIP stream of the current device, as a pointer-sized int.
    torch's own raw-stream getter when it has one: building the Stream object
    of torch.cuda.current_stream() costs about 3 us a call, a large part of a
    small call's host time."""
    global _RAW_STREAM
    torch = _torch()
    if _RAW_STREAM is None:
        _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    if _RAW_STREAM:
        return _RAW_STREAM(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _tensor(t, name, dtype, shape=None, min_numel=1):
    """Check one tensor's layout before its pointer goes to the library: a
    torch tensor of ``dtype``, contiguous (the library reads dense row-major
    memory) and of ``shape`` (or at least ``min_numel`` elements).  Where it
    lives is checked by _device, once every operand's layout has passed.
    Raises ValueError."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous (got strides {tuple(t.stride())})")
    if shape is not None and t.shape != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if shape is None and t.numel() < min_numel:
        raise ValueError(f"{name}: needs at least {min_numel} element(s)")
    return t


def _opt(t, name, dtype, shape=None, min_numel=1):
    return None if t is None else _tensor(t, name, dtype, shape, min_numel)


def _device(**named):
    """Every given tensor (None skipped) is on the GPU, all on one device, and
    that device is the current one (the library works on the current device;
    a host pointer or another device's memory would be read by its kernels as
    this device's).  Returns the device."""
    torch = _torch()
    dev = None
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name}: must be a GPU tensor, got device {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name}: on {t.device}, other operands on {dev}")
    if dev is not None and dev.index != torch.cuda.current_device():
        raise ValueError(f"operands on {dev}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    return dev


def _matrix(t, name, dtype):
    """A 2-D tensor: returns (rows, cols) after the checks of _tensor."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"{name}: expected a 2-D torch.Tensor")
    _tensor(t, name, dtype, min_numel=0)          # zero rows: a no-op call
    return tuple(t.shape)


def _epilogue(epilogue):
    if epilogue not in EPILOGUES:
        raise ValueError(f"epilogue must be one of {sorted(EPILOGUES)}, got {epilogue!r}")
    return EPILOGUES[epilogue]


def _nvfp4(q, name):
    """Check an Nvfp4Tensor's parts against its row count and ``cols``;
    returns the row count."""
    torch = _torch()
    if not isinstance(q, Nvfp4Tensor):
        raise ValueError(f"{name}: expected an Nvfp4Tensor")
    rows = q.codes.shape[0] if isinstance(q.codes, torch.Tensor) and q.codes.dim() == 2 else -1
    if rows < 0 or q.cols <= 0 or q.cols % 16:
        raise ValueError(f"{name}: codes must be 2-D and cols a positive multiple of 16")
    _tensor(q.codes, f"{name}.codes", torch.uint8, (rows, q.cols // 2))
    _tensor(q.scales, f"{name}.scales", torch.uint8, (rows, q.cols // 16))
    _tensor(q.tensor_scale, f"{name}.tensor_scale", torch.float32)
    return rows


def _parts(q, name):
    """The tensors of an Nvfp4Tensor / Fp8Tensor by name, for _device."""
    return {f"{name}.{k}": v for k, v in q._asdict().items() if k != "cols"}


def abi_version():
    return load().nvfp4_abi_version()


def status_string(status):
    return load().nvfp4_status_string(status).decode()


def quantize_workspace_bytes(rows, cols):
    return load().nvfp4_quantize_workspace_bytes(rows, cols)


def quantize_workspace(device="cuda"):
    """A quantizer workspace: zero-filled once here, as the library requires
    before first use; calls keep it valid, so it is reused across calls on one
    stream without clearing."""
    torch = _torch()
    return torch.zeros(load().nvfp4_quantize_workspace_bytes(1, 16), dtype=torch.uint8, device=device)


_WORKSPACES = {}


def _default_workspace(dev):
    """The quantizer workspace of the current stream on `dev`, made once."""
    torch = _torch()
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    ws = _WORKSPACES.get(key)
    if ws is None:
        ws = _WORKSPACES[key] = quantize_workspace(dev)
    return ws


def _out_tuple(out, n, name):
    if not isinstance(out, (tuple, list)) or len(out) != n:
        raise ValueError(f"{name}: expected a tuple of {n} tensors")
    return out


def quantize(x, amax=None, workspace=None, dev_status=None, out=None):
    """NVFP4-quantize a 2-D bf16 tensor.  Returns an ``Nvfp4Tensor``.

    amax: optional one-element float32 device tensor (a producer's amax); when
    None the amax is computed by the library, with ``workspace`` (from
    ``quantize_workspace``; by default one kept per device and stream).  out:
    optional (codes, scales, tensor_scale) tensors to write into.
    """
    torch = _torch()
    rows, cols = _matrix(x, "x", torch.bfloat16)
    if cols <= 0 or cols % 16:
        raise ValueError(f"x: cols must be a positive multiple of 16, got {cols}")
    _opt(amax, "amax", torch.float32)
    _opt(workspace, "workspace", torch.uint8)
    _opt(dev_status, "dev_status", torch.int32)
    codes = scales = ts = None
    if out is not None:
        codes, scales, ts = _out_tuple(out, 3, "out")
        _tensor(codes, "out codes", torch.uint8, (rows, cols // 2))
        _tensor(scales, "out scales", torch.uint8, (rows, cols // 16))
        _tensor(ts, "out tensor_scale", torch.float32)
    dev = _device(x=x, amax=amax, workspace=workspace, dev_status=dev_status, out_codes=codes,
                  out_scales=scales, out_tensor_scale=ts)
    if out is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
        ts = torch.empty((1,), dtype=torch.float32, device=dev)
    lib = load()
    if amax is None and workspace is None:
        workspace = _default_workspace(dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    _binding.check(lib.nvfp4_quantize(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _ptr(ts),
                                      _ptr(amax), _ptr(workspace), ws_bytes, _ptr(dev_status),
                                      _stream()), "nvfp4_quantize")
    return Nvfp4Tensor(codes, scales, ts, cols)


def dequantize(q, out=None):
    torch = _torch()
    rows = _nvfp4(q, "q")
    _opt(out, "out", torch.bfloat16, (rows, q.cols))
    dev = _device(**_parts(q, "q"), out=out)
    if out is None:
        out = torch.empty((rows, q.cols), dtype=torch.bfloat16, device=dev)
    _binding.check(load().nvfp4_dequantize(_ptr(q.codes), _ptr(q.scales), _ptr(q.tensor_scale),
                                           rows, q.cols, _ptr(out), _stream()), "nvfp4_dequantize")
    return out


def gemm_workspace(M, N, K, device="cuda"):
    """A workspace for ``gemm`` on an (M, N, K) problem, or None if it would not split."""
    nbytes = load().nvfp4_gemm_workspace_bytes(M, N, K)
    if nbytes == 0:
        return None
    return _torch().empty(nbytes, dtype=_torch().uint8, device=device)


_NO_WORKSPACE = object()


def _gemm_operands(a, w):
    M = _nvfp4(a, "a")
    N = _nvfp4(w, "w")
    if w.cols != a.cols:
        raise ValueError(f"K mismatch: a has {a.cols} columns, w {w.cols}")
    return M, N, a.cols


def gemm(a, w, bias=None, epilogue="none", y_amax=None, out=None, workspace=_NO_WORKSPACE):
    """Y = epi(sA*sW * A_hat @ W_hat^T + bias) in bf16, from two ``Nvfp4Tensor``.

    ``workspace``: a uint8 device tensor from ``gemm_workspace`` (reused across
    calls on one stream), None to compute every tile whole, or left out to have
    one taken from torch's caching allocator for this call.
    """
    torch = _torch()
    M, N, K = _gemm_operands(a, w)
    epi = _epilogue(epilogue)
    _opt(bias, "bias", torch.bfloat16, (N,))
    _opt(y_amax, "y_amax", torch.float32)
    _opt(out, "out", torch.bfloat16, (M, N))
    ws = None if workspace is _NO_WORKSPACE else _opt(workspace, "workspace", torch.uint8)
    dev = _device(**_parts(a, "a"), **_parts(w, "w"), bias=bias, y_amax=y_amax, out=out,
                  workspace=ws)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if workspace is _NO_WORKSPACE:
        workspace = gemm_workspace(M, N, K, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    _binding.check(load().nvfp4_gemm(_ptr(a.codes), _ptr(a.scales), _ptr(a.tensor_scale),
                                     _ptr(w.codes), _ptr(w.scales), _ptr(w.tensor_scale),
                                     _ptr(bias), M, N, K, epi, _ptr(out),
                                     _ptr(y_amax), _ptr(workspace), ws_bytes, _stream()),
                   "nvfp4_gemm")
    return out


def gemm_quantized(a, w, amax, bias=None, epilogue="none", out=None):
    """The GEMM with NVFP4 output under the static amax ``amax`` (one-element
    float32 device tensor): the same bytes as ``quantize(gemm(a, w), amax=amax)``.
    Returns an ``Nvfp4Tensor``; ``out``: optional (codes, scales, tensor_scale)."""
    torch = _torch()
    M, N, K = _gemm_operands(a, w)
    epi = _epilogue(epilogue)
    if N % 16:
        raise ValueError(f"gemm_quantized needs N % 16 == 0, got N = {N}")
    _tensor(amax, "amax", torch.float32)
    _opt(bias, "bias", torch.bfloat16, (N,))
    codes = scales = ts = None
    if out is not None:
        codes, scales, ts = _out_tuple(out, 3, "out")
        _tensor(codes, "out codes", torch.uint8, (M, N // 2))
        _tensor(scales, "out scales", torch.uint8, (M, N // 16))
        _tensor(ts, "out tensor_scale", torch.float32)
    dev = _device(**_parts(a, "a"), **_parts(w, "w"), amax=amax, bias=bias, out_codes=codes,
                  out_scales=scales, out_tensor_scale=ts)
    if out is None:
        codes = torch.empty((M, N // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((M, N // 16), dtype=torch.uint8, device=dev)
        ts = torch.empty((1,), dtype=torch.float32, device=dev)
    _binding.check(load().nvfp4_gemm_quantized(_ptr(a.codes), _ptr(a.scales), _ptr(a.tensor_scale),
                                               _ptr(w.codes), _ptr(w.scales), _ptr(w.tensor_scale),
                                               _ptr(bias), M, N, K, epi, _ptr(amax),
                                               _ptr(codes), _ptr(scales), _ptr(ts), _stream()),
                   "nvfp4_gemm_quantized")
    return Nvfp4Tensor(codes, scales, ts, N)


def fp8_quantize(x, dev_status=None, out=None):
    """FP8 row-wise quantization of a 2-D bf16 tensor (one scale per row).
    Returns an ``Fp8Tensor``; ``out``: optional (codes, scales)."""
    torch = _torch()
    rows, cols = _matrix(x, "x", torch.bfloat16)
    if cols <= 0 or cols % 16:
        raise ValueError(f"x: cols must be a positive multiple of 16, got {cols}")
    _opt(dev_status, "dev_status", torch.int32)
    codes = scales = None
    if out is not None:
        codes, scales = _out_tuple(out, 2, "out")
        _tensor(codes, "out codes", torch.uint8, (rows, cols))
        _tensor(scales, "out scales", torch.float32, (rows,))
    dev = _device(x=x, dev_status=dev_status, out_codes=codes, out_scales=scales)
    if out is None:
        codes = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows,), dtype=torch.float32, device=dev)
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


def _fp8(q, name):
    torch = _torch()
    if not isinstance(q, Fp8Tensor):
        raise ValueError(f"{name}: expected an Fp8Tensor")
    rows, cols = _matrix(q.codes, f"{name}.codes", torch.uint8)
    _tensor(q.scales, f"{name}.scales", torch.float32, (rows,))
    return rows, cols


def fp8_gemm(a, w, bias=None, epilogue="none", out=None, workspace=_NO_WORKSPACE):
    """Y = epi((A_q @ W_q^T) * dA[m] * dW[n] + bias) in bf16, from two ``Fp8Tensor``.

    ``workspace``: as for ``gemm`` (from ``fp8_gemm_workspace``, None, or left out).
    """
    torch = _torch()
    M, K = _fp8(a, "a")
    N, Kw = _fp8(w, "w")
    if Kw != K:
        raise ValueError(f"K mismatch: a has {K} columns, w {Kw}")
    epi = _epilogue(epilogue)
    _opt(bias, "bias", torch.bfloat16, (N,))
    _opt(out, "out", torch.bfloat16, (M, N))
    ws = None if workspace is _NO_WORKSPACE else _opt(workspace, "workspace", torch.uint8)
    dev = _device(**_parts(a, "a"), **_parts(w, "w"), bias=bias, out=out, workspace=ws)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if workspace is _NO_WORKSPACE:
        workspace = fp8_gemm_workspace(M, N, K, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    _binding.check(load().nvfp4_fp8_gemm(_ptr(a.codes), _ptr(a.scales), _ptr(w.codes), _ptr(w.scales),
                                         _ptr(bias), M, N, K, epi, _ptr(out),
                                         _ptr(workspace), ws_bytes, _stream()),
                   "nvfp4_fp8_gemm")
    return out


def gemm_bf16(x, w, bias=None, epilogue="none", out=None):
    """Y = epi(X @ W^T + bias) in bf16 with fp32 accumulation (bf16 passthrough)."""
    torch = _torch()
    M, K = _matrix(x, "x", torch.bfloat16)
    N, Kw = _matrix(w, "w", torch.bfloat16)
    if Kw != K:
        raise ValueError(f"K mismatch: x has {K} columns, w {Kw}")
    epi = _epilogue(epilogue)
    _opt(bias, "bias", torch.bfloat16, (N,))
    _opt(out, "out", torch.bfloat16, (M, N))
    dev = _device(x=x, w=w, bias=bias, out=out)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _binding.check(load().nvfp4_gemm_bf16(_ptr(x), _ptr(w), _ptr(bias), M, N, K, epi, _ptr(out),
                                          _stream()),
                   "nvfp4_gemm_bf16")
    return out


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
