// Internal launch interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Compute units of the current device (256 if the query fails).
int compute_units();

// Upper bound on the partial maxima the amax pass writes (workspace words).
static constexpr int kMaxAmaxPartials = 1024;

// Quantizer workspace, in 32-bit words: the single-pass kernel's arrival
// counters, release words and tagged partial slots in [0, kQuantSyncWords)
// (they must start zeroed and every call leaves them consistent), the
// two-pass kernels' partial maxima after them (written before they are read
// by every call).
static constexpr int kQuantSyncWords = 1024;
static constexpr int kQuantTwoPassWords = kMaxAmaxPartials;
static constexpr int kQuantWorkspaceWords = kQuantSyncWords + kQuantTwoPassWords;

int amax_partial_count(int64_t numel);

// The library-owned quantizer workspace of the current device (a static
// device array of static_scratch_bytes(), zero when loaded): its device
// address, looked up once per device.
hipError_t static_scratch(uint32_t** out);
size_t static_scratch_bytes();

hipError_t launch_quantize(const void* x, int64_t rows, int64_t cols, uint8_t* codes,
                           uint8_t* scales, float* tensor_scale, const float* amax_in,
                           uint32_t* workspace, size_t workspace_bytes, int32_t* dev_status,
                           hipStream_t stream);

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales,
                             const float* tensor_scale, int64_t rows, int64_t cols, void* y,
                             hipStream_t stream);

hipError_t launch_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales,
                             const float* a_tensor_scale, const uint8_t* w_codes,
                             const uint8_t* w_scales, const float* w_tensor_scale,
                             const void* bias, int64_t M, int64_t N, int64_t K, int epilogue,
                             void* y, float* y_amax, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

// The same GEMM writing Y as NVFP4 (codes, scales, tensor scale) quantized
// with the static amax *y_amax_static; N % 16 == 0.
hipError_t launch_gemm_nvfp4_quantized(const uint8_t* a_codes, const uint8_t* a_scales,
                                       const float* a_tensor_scale, const uint8_t* w_codes,
                                       const uint8_t* w_scales, const float* w_tensor_scale,
                                       const void* bias, int64_t M, int64_t N, int64_t K,
                                       int epilogue, const float* y_amax_static, uint8_t* y_codes,
                                       uint8_t* y_scales, float* y_tensor_scale,
                                       hipStream_t stream);

// Workspace bytes launch_gemm_nvfp4 can use to split the tail tiles over K
// (0: no split for this shape).
size_t gemm_nvfp4_workspace_bytes(int64_t M, int64_t N, int64_t K);

// The FP8 row-wise variant.
hipError_t launch_fp8_quantize_rowwise(const void* x, int64_t rows, int64_t cols, uint8_t* codes,
                                       float* row_scales, int32_t* dev_status, hipStream_t stream);
hipError_t launch_gemm_fp8(const uint8_t* a_codes, const float* a_scales, const uint8_t* w_codes,
                           const float* w_scales, const void* bias, int64_t M, int64_t N,
                           int64_t K, int epilogue, void* y, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);
// Workspace bytes launch_gemm_fp8 can use to split the tail tiles over K.
size_t gemm_fp8_workspace_bytes(int64_t M, int64_t N, int64_t K);

hipError_t launch_gemm_bf16(const void* x, const void* w, const void* bias, int64_t M, int64_t N,
                            int64_t K, int epilogue, void* y, hipStream_t stream);

}  // namespace nvfp4
