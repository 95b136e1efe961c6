"""MI355X-native NVFP4 quantize / dequantize / block-scaled GEMM (placeholder; binding added next)."""
