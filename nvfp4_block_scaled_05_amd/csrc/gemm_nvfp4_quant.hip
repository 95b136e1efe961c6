// The NVFP4-output instance of the v5 GEMM kernel (gemm_v5.hpp): the GEMM of
// gemm_nvfp4.hip with its bf16 result quantized in the epilogue under the
// static tensor scale derived from *out.amax_static.  A translation unit of
// its own so that it compiles in parallel with the bf16-output instance.
#include "gemm_v5.hpp"

namespace nvfp4 {

hipError_t launch_v5_quant(const uint8_t* a_codes, const uint8_t* a_scales, const float* sa,
                           const uint8_t* w_codes, const uint8_t* w_scales, const float* sw,
                           const uint16_t* bias, int64_t M, int64_t N, int64_t K, int epi,
                           const Out& out, int64_t tiles, int64_t grid, hipStream_t stream) {
  const SplitK whole{nullptr, tiles, 1};
  hipLaunchKernelGGL(gemm_nvfp4_v5_kernel<true>, dim3((unsigned)grid), dim3(kVNT), 0, stream,
                     a_codes, a_scales, sa, w_codes, w_scales, sw, bias, M, N, K, epi, out, whole,
                     tiles);
  return hipGetLastError();
}

}  // namespace nvfp4
