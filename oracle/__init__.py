"""CPU oracle for the NVFP4 quantize / dequantize / block-scaled GEMM path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything in this package.  The
product path (the HIP library and its Python binding) never imports, links or
calls it, and the oracle never imports the product path: the two share no code.
Inputs reach both sides only through the seeded generators in
``nvfp4_block_scaled_05_amd/inputs.py``, which hold none of the method's
arithmetic.

Everything here is a plain, slow, readable restatement of what the method
computes, written with explicit ``numpy.float32`` operations where the method
is specified in binary32 and in float64 / exact integers / ``fractions`` where
it is specified as an exact value.

Sources (the web pages this path is built from):
  [P1] "英伟达B200狂飙10.2倍！AI绘图告别龟速！" (nmedialink.com), section
       "NVFP4量化：在精度与速度之间寻得最佳平衡" -- two-level micro-block
       scaling: an FP32 per-tensor scale (static or dynamic) and a per-block
       scale computed dynamically over 16-element blocks; layers kept in higher
       precision through the exclude_pattern regex.
  [P2] "NVIDIA介绍用TensorRT LLM VisualGen加速Blackwell上的FLUX 3 Image Klein"
       (sns.style), time-breakdown paragraph -- NVFP4 weights in the DiT
       linears, up to 1.62x over BF16.
  [P3] "NVIDIA показала, как сократить генерацию FLUX 3 Image Klein с 22 до 6
       секунд" (xalabuda.com), section "Квантование NVFP4 и оптимизация
       вычислительных ядер" -- NVFP4 GEMM kernels for the linear layers.

Where the pages are silent (element and scale encodings, rounding, bit and
byte order, the tensor-scale formula, degenerate inputs) each function names
the reading it implements; the readings are numbered R-1 ... R-19, and each
function's docstring names the ones it follows.

Module map:
  formats.py -- E2M1 element codes, E4M3 scale bytes, bf16 rounding.
  quant.py   -- two-level quantize and dequantize.
  gemm.py    -- block-scaled GEMM (exact integer form and fp64 form), GELU,
                bf16 passthrough linear.
  layers.py  -- the exclude-pattern layer predicate.
  fp8.py     -- the FP8 row-wise variant ("fp8r"): quantize, dequantize, W8A8
                GEMM (reading R-22: the pages name the variant, not its recipe).
"""

from .formats import (E2M1_MAGNITUDES, e2m1_encode_magnitude, e2m1_value,
                      e4m3_encode_nonneg, e4m3_value, bf16_bits_to_f32,
                      round_to_bf16_bits, bf16_bits_to_f64)
from .quant import NonFiniteInput, Quantized, quantize, dequantize, unpack_codes
from .gemm import (block_values_f64, gemm_fp64, gemm_exact_rows, gelu_f64,
                   epilogue_to_bf16, linear_bf16_fp64)
from .layers import EXCLUDE_PATTERN, layer_is_quantized
from .fp8 import (Fp8Rowwise, quantize_fp8_rowwise, dequantize_fp8_rowwise,
                  gemm_fp8_exact_rows, gemm_fp8_fp64)

__all__ = [
    "E2M1_MAGNITUDES", "e2m1_encode_magnitude", "e2m1_value",
    "e4m3_encode_nonneg", "e4m3_value", "bf16_bits_to_f32",
    "round_to_bf16_bits", "bf16_bits_to_f64",
    "NonFiniteInput", "Quantized", "quantize", "dequantize", "unpack_codes",
    "block_values_f64", "gemm_fp64", "gemm_exact_rows", "gelu_f64",
    "epilogue_to_bf16", "linear_bf16_fp64",
    "EXCLUDE_PATTERN", "layer_is_quantized",
    "Fp8Rowwise", "quantize_fp8_rowwise", "dequantize_fp8_rowwise",
    "gemm_fp8_exact_rows", "gemm_fp8_fp64",
]
