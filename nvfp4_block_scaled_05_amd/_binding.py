"""ctypes binding of ``lib/libnvfp4.so`` (the C ABI in include/nvfp4.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's kernels.  There
is no fallback: if the library is missing or the device is not a gfx950, the
calls raise.
"""

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
# NVFP4_LIBRARY names another build of the same sources (the host-sanitizer
# build of the tests); by default the in-tree library.
LIB_PATH = os.environ.get("NVFP4_LIBRARY") or os.path.join(PKG, "lib", "libnvfp4.so")

NVFP4_OK = 0
STATUS_NAMES = {0: "NVFP4_OK", -1: "NVFP4_ERR_NULL", -2: "NVFP4_ERR_SHAPE",
                -3: "NVFP4_ERR_ALIGN", -4: "NVFP4_ERR_WORKSPACE", -5: "NVFP4_ERR_DEVICE",
                -6: "NVFP4_ERR_ARG", -7: "NVFP4_ERR_HIP", -8: "NVFP4_ERR_NONFINITE"}
EPILOGUES = {"none": 0, "gelu": 1}

#: exported symbols and their (restype, argtypes)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
SIGNATURES = {
    "nvfp4_abi_version": (ctypes.c_int, []),
    "nvfp4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "nvfp4_quantize_workspace_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "nvfp4_quantize": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P]),
    "nvfp4_quantize_no_alloc": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P, _P]),
    "nvfp4_dequantize": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P, _P]),
    "nvfp4_gemm": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P, _P,
                                  _P, ctypes.c_size_t, _P]),
    "nvfp4_gemm_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "nvfp4_gemm_quantized": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64,
                                            ctypes.c_int, _P, _P, _P, _P, _P]),
    "nvfp4_gemm_bf16": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P, _P]),
    "nvfp4_fp8_quantize_rowwise": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P]),
    "nvfp4_fp8_gemm": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P, _P,
                                      ctypes.c_size_t, _P]),
    "nvfp4_fp8_gemm_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "nvfp4_graph_begin": (ctypes.c_int, [_P]),
    "nvfp4_graph_end": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_void_p)]),
    "nvfp4_graph_launch": (ctypes.c_int, [_P, _P]),
    "nvfp4_graph_destroy": (ctypes.c_int, [_P]),
    "nvfp4_layer_is_quantized": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_char_p]),
}

_lib = None
_lock = threading.Lock()


class Nvfp4Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}")


class _SignedLibrary:
    """The loaded library, exposing only the functions in SIGNATURES (each
    with its argument and result types set).  A function called without its
    argument types would have its pointer arguments cut to a C int by ctypes;
    here such a call fails with AttributeError instead of reaching the GPU."""

    def __init__(self, lib):
        self._lib = lib
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
            setattr(self, name, fn)

    def __getattr__(self, name):
        raise AttributeError(f"{name}: not an exported function with a declared signature")


def load(path=LIB_PATH):
    """Load (once) and return the library; raises if it is not built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is not built; run `python -m nvfp4_block_scaled_05_amd.build`")
            _lib = _SignedLibrary(ctypes.CDLL(path))
        return _lib


def check(status, where):
    if status != NVFP4_OK:
        raise Nvfp4Error(status, where)
    return status
