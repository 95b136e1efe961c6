"""nvfp4_quantize_no_alloc (the quantizer with a library-owned scratch array,
for callers that cannot allocate) against nvfp4_quantize (caller-provided
workspace), both called through the C ABI: the same codes, scales, tensor
scale and status on two calls in a row, the second on a smaller input -- the
scratch keeps the first call's contents -- and once more on the first input,
through each kernel that uses the scratch."""

import ctypes

import numpy as np
import pytest

import nvfp4_block_scaled_05_amd as nv
from nvfp4_block_scaled_05_amd import _binding
from nvfp4_block_scaled_05_amd import inputs as W

pytestmark = pytest.mark.gpu


def _entry_points():
    """The two C entry points, with their argument types set here (pointers
    as void*, sizes as int64) whatever the binding holds."""
    lib = ctypes.CDLL(_binding.LIB_PATH)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    na = lib.nvfp4_quantize_no_alloc
    na.argtypes = [P, I64, I64, P, P, P, P, P]
    na.restype = ctypes.c_int
    q = lib.nvfp4_quantize
    q.argtypes = [P, I64, I64, P, P, P, P, P, ctypes.c_size_t, P, P]
    q.restype = ctypes.c_int
    return na, q


def _quantize_pair(lib, x):
    """(no_alloc outputs, reference outputs) for bf16 device tensor x."""
    import torch
    rows, cols = x.shape
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    outs = []
    for which in ("no_alloc", "ref"):
        codes = torch.full((rows, cols // 2), 0xAB, dtype=torch.uint8, device="cuda")
        scales = torch.full((rows, cols // 16), 0xCD, dtype=torch.uint8, device="cuda")
        ts = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
        st = torch.full((1,), 99, dtype=torch.int32, device="cuda")
        if which == "no_alloc":
            rc = lib[0](x.data_ptr(), rows, cols, codes.data_ptr(), scales.data_ptr(),
                        ts.data_ptr(), st.data_ptr(), stream)
        else:
            ws = nv.quantize_workspace()
            rc = lib[1](x.data_ptr(), rows, cols, codes.data_ptr(), scales.data_ptr(),
                        ts.data_ptr(), None, ws.data_ptr(), ws.numel(), st.data_ptr(), stream)
        assert rc == 0, (which, rc)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (codes, scales, ts, st)])
    return outs


@pytest.mark.parametrize("kernel", ["default", "resident", "twopass"])
def test_no_alloc_matches_workspace_entry(kernel, monkeypatch):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if kernel != "default":
        monkeypatch.setenv("NVFP4_QUANT_KERNEL", kernel)
    nv.load()
    lib = _entry_points()
    big = W.quantize_act()["x"]                                   # [16896, 3072]
    small = W.random_matrix(7, (1000, 3072), "t3")                # smaller, second call
    for bits in (big, small, big):
        x = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
        got, ref = _quantize_pair(lib, x)
        for g, r, what in zip(got, ref, ("codes", "scales", "tensor scale", "status")):
            assert np.array_equal(g, r), f"{kernel} {bits.shape}: {what}"
        assert got[3][0] == 0
