// extern "C" entry points declared in include/nvfp4.h: argument validation,
// the gfx950 device check, and launches on the caller's stream.
//
// Validation never touches the GPU: sizes, NULL pointers of non-empty buffers,
// shape multiples, alignment and workspace are checked first, in that order,
// then the current device is checked (once per device, cached), then the
// kernels are enqueued.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <regex>
#include <string>
#include <string_view>

#include "kernels.hpp"
#include "nvfp4.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

std::atomic<int> g_arch_ok[64];   // 0 unknown, 1 gfx950, -1 other / error

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return NVFP4_ERR_DEVICE;
  int c = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      c = -1;
    else
      c = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_arch_ok[dev].store(c, std::memory_order_relaxed);
  }
  return c == 1 ? NVFP4_OK : NVFP4_ERR_DEVICE;
}

int hip_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

bool bad_dim(int64_t v) { return v < 0 || v >= kMaxDim; }

// The page's exclude pattern, ^(?!.*(embedder|norm_out|proj_out|to_add_out|
// to_added_qkv|stream)).*, matched from the start of the name: the lookahead
// fails exactly when one of these words occurs before the name's first line
// terminator (the pattern's `.` stops at \n and \r).  Evaluated as that
// substring search, so a name of any length costs one linear scan.
constexpr const char* kExcludedWords[] = {"embedder", "norm_out",     "proj_out",
                                          "to_add_out", "to_added_qkv", "stream"};

int page_pattern_matches(const char* name) {
  std::string_view s(name);
  s = s.substr(0, s.find_first_of("\n\r"));
  for (const char* w : kExcludedWords)
    if (s.find(w) != std::string_view::npos) return 0;
  return 1;
}

// The regex engine recurses once per character of the subject, so a caller's
// pattern is only applied to names up to this length.
constexpr size_t kMaxPatternName = 1024;

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "null pointer";
    case NVFP4_ERR_SHAPE: return "invalid shape";
    case NVFP4_ERR_ALIGN: return "misaligned pointer";
    case NVFP4_ERR_WORKSPACE: return "workspace too small";
    case NVFP4_ERR_DEVICE: return "no gfx950 device";
    case NVFP4_ERR_ARG: return "invalid argument";
    case NVFP4_ERR_HIP: return "HIP error";
    case NVFP4_ERR_NONFINITE: return "non-finite input";
    default: return "unknown status";
  }
}

size_t nvfp4_quantize_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || bad_dim(rows) || bad_dim(cols)) return 0;
  // the single-pass kernel's arrival words and partial slots, then the
  // two-pass kernels' partial maxima
  return 4u * (size_t)nvfp4::kQuantWorkspaceWords;
}

int nvfp4_quantize(const void* x_bf16, int64_t rows, int64_t cols, uint8_t* codes,
                   uint8_t* scales, float* tensor_scale, const float* amax_in, void* workspace,
                   size_t workspace_bytes, int32_t* dev_status, void* stream) {
  if (bad_dim(rows) || bad_dim(cols) || rows * cols >= ((int64_t)1 << 40)) return NVFP4_ERR_SHAPE;
  const bool empty = rows == 0;
  if (!tensor_scale) return NVFP4_ERR_NULL;
  if (!empty && (!x_bf16 || !codes || !scales)) return NVFP4_ERR_NULL;
  if (!empty && !amax_in && !workspace) return NVFP4_ERR_NULL;
  if (cols == 0 || cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(codes, 8) || !aligned(tensor_scale, 4) ||
      !aligned(amax_in, 4) || !aligned(workspace, 8) || !aligned(dev_status, 4))
    return NVFP4_ERR_ALIGN;
  if (!empty && !amax_in && workspace_bytes < nvfp4_quantize_workspace_bytes(rows, cols))
    return NVFP4_ERR_WORKSPACE;
  int st = check_device();
  if (st != NVFP4_OK) return st;
  if (empty) return NVFP4_OK;
  return hip_status(nvfp4::launch_quantize(x_bf16, rows, cols, codes, scales, tensor_scale,
                                           amax_in, static_cast<uint32_t*>(workspace),
                                           workspace_bytes, dev_status,
                                           static_cast<hipStream_t>(stream)));
}

int nvfp4_quantize_no_alloc(const void* x_bf16, int64_t rows, int64_t cols, uint8_t* codes,
                            uint8_t* scales, float* tensor_scale, int32_t* dev_status,
                            void* stream) {
  if (bad_dim(rows) || bad_dim(cols) || rows * cols >= ((int64_t)1 << 40)) return NVFP4_ERR_SHAPE;
  const bool empty = rows == 0;
  if (!tensor_scale) return NVFP4_ERR_NULL;
  if (!empty && (!x_bf16 || !codes || !scales)) return NVFP4_ERR_NULL;
  if (cols == 0 || cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(codes, 8) || !aligned(tensor_scale, 4) ||
      !aligned(dev_status, 4))
    return NVFP4_ERR_ALIGN;
  if (nvfp4_quantize_workspace_bytes(rows, cols) > nvfp4::static_scratch_bytes())
    return NVFP4_ERR_WORKSPACE;
  int st = check_device();
  if (st != NVFP4_OK) return st;
  if (empty) return NVFP4_OK;
  uint32_t* ws = nullptr;
  if (nvfp4::static_scratch(&ws) != hipSuccess) return NVFP4_ERR_HIP;
  return hip_status(nvfp4::launch_quantize(x_bf16, rows, cols, codes, scales, tensor_scale,
                                           nullptr, ws, nvfp4::static_scratch_bytes(), dev_status,
                                           static_cast<hipStream_t>(stream)));
}

int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                     int64_t rows, int64_t cols, void* y_bf16, void* stream) {
  if (bad_dim(rows) || bad_dim(cols) || rows * cols >= ((int64_t)1 << 40)) return NVFP4_ERR_SHAPE;
  const bool empty = rows == 0;
  if (!empty && (!codes || !scales || !tensor_scale || !y_bf16)) return NVFP4_ERR_NULL;
  if (cols == 0 || cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!aligned(codes, 8) || !aligned(tensor_scale, 4) || !aligned(y_bf16, 16))
    return NVFP4_ERR_ALIGN;
  int st = check_device();
  if (st != NVFP4_OK) return st;
  if (empty) return NVFP4_OK;
  return hip_status(nvfp4::launch_dequantize(codes, scales, tensor_scale, rows, cols, y_bf16,
                                             static_cast<hipStream_t>(stream)));
}

size_t nvfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (bad_dim(M) || bad_dim(N) || bad_dim(K) || K % 16 != 0) return 0;
  return nvfp4::gemm_nvfp4_workspace_bytes(M, N, K);
}

int nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
               const uint8_t* w_codes, const uint8_t* w_scales, const float* w_tensor_scale,
               const void* bias_bf16, int64_t M, int64_t N, int64_t K, int epilogue, void* y_bf16,
               float* y_amax, void* workspace, size_t workspace_bytes, void* stream) {
  if (bad_dim(M) || bad_dim(N) || bad_dim(K)) return NVFP4_ERR_SHAPE;
  const bool empty = M == 0 || N == 0;
  if (!empty && (!a_codes || !a_scales || !a_tensor_scale || !w_codes || !w_scales ||
                 !w_tensor_scale || !y_bf16))
    return NVFP4_ERR_NULL;
  if (K == 0 || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (((M + 127) / 128) * ((N + 127) / 128) >= ((int64_t)1 << 24)) return NVFP4_ERR_SHAPE;
  if (!aligned(a_codes, 8) || !aligned(w_codes, 8) || !aligned(a_tensor_scale, 4) ||
      !aligned(w_tensor_scale, 4) || !aligned(bias_bf16, 2) || !aligned(y_bf16, 2) ||
      !aligned(y_amax, 4) || !aligned(workspace, 256))
    return NVFP4_ERR_ALIGN;
  if (epilogue != NVFP4_EPI_NONE && epilogue != NVFP4_EPI_GELU) return NVFP4_ERR_ARG;
  int st = check_device();
  if (st != NVFP4_OK) return st;
  return hip_status(nvfp4::launch_gemm_nvfp4(a_codes, a_scales, a_tensor_scale, w_codes, w_scales,
                                             w_tensor_scale, bias_bf16, M, N, K, epilogue, y_bf16,
                                             y_amax, workspace, workspace ? workspace_bytes : 0,
                                             static_cast<hipStream_t>(stream)));
}

int nvfp4_gemm_quantized(const uint8_t* a_codes, const uint8_t* a_scales,
                         const float* a_tensor_scale, const uint8_t* w_codes,
                         const uint8_t* w_scales, const float* w_tensor_scale,
                         const void* bias_bf16, int64_t M, int64_t N, int64_t K, int epilogue,
                         const float* y_amax, uint8_t* y_codes, uint8_t* y_scales,
                         float* y_tensor_scale, void* stream) {
  if (bad_dim(M) || bad_dim(N) || bad_dim(K)) return NVFP4_ERR_SHAPE;
  const bool empty = M == 0 || N == 0;
  if (!empty && (!a_codes || !a_scales || !a_tensor_scale || !w_codes || !w_scales ||
                 !w_tensor_scale || !y_amax || !y_codes || !y_scales || !y_tensor_scale))
    return NVFP4_ERR_NULL;
  if (K == 0 || K % 16 != 0 || N % 16 != 0) return NVFP4_ERR_SHAPE;
  if (((M + 127) / 128) * ((N + 127) / 128) >= ((int64_t)1 << 24)) return NVFP4_ERR_SHAPE;
  if (!aligned(a_codes, 8) || !aligned(w_codes, 8) || !aligned(a_tensor_scale, 4) ||
      !aligned(w_tensor_scale, 4) || !aligned(bias_bf16, 2) || !aligned(y_amax, 4) ||
      !aligned(y_codes, 8) || !aligned(y_tensor_scale, 4))
    return NVFP4_ERR_ALIGN;
  if (epilogue != NVFP4_EPI_NONE && epilogue != NVFP4_EPI_GELU) return NVFP4_ERR_ARG;
  int st = check_device();
  if (st != NVFP4_OK) return st;
  if (empty) return NVFP4_OK;
  return hip_status(nvfp4::launch_gemm_nvfp4_quantized(
      a_codes, a_scales, a_tensor_scale, w_codes, w_scales, w_tensor_scale, bias_bf16, M, N, K,
      epilogue, y_amax, y_codes, y_scales, y_tensor_scale, static_cast<hipStream_t>(stream)));
}

int nvfp4_fp8_quantize_rowwise(const void* x_bf16, int64_t rows, int64_t cols, uint8_t* codes,
                               float* row_scales, int32_t* dev_status, void* stream) {
  if (bad_dim(rows) || bad_dim(cols) || rows * cols >= ((int64_t)1 << 40)) return NVFP4_ERR_SHAPE;
  const bool empty = rows == 0;
  if (!empty && (!x_bf16 || !codes || !row_scales)) return NVFP4_ERR_NULL;
  if (cols == 0 || cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(codes, 8) || !aligned(row_scales, 4) ||
      !aligned(dev_status, 4))
    return NVFP4_ERR_ALIGN;
  int st = check_device();
  if (st != NVFP4_OK) return st;
  return hip_status(nvfp4::launch_fp8_quantize_rowwise(x_bf16, rows, cols, codes, row_scales,
                                                       dev_status,
                                                       static_cast<hipStream_t>(stream)));
}

size_t nvfp4_fp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (bad_dim(M) || bad_dim(N) || bad_dim(K) || K % 16 != 0) return 0;
  return nvfp4::gemm_fp8_workspace_bytes(M, N, K);
}

int nvfp4_fp8_gemm(const uint8_t* a_codes, const float* a_scales, const uint8_t* w_codes,
                   const float* w_scales, const void* bias_bf16, int64_t M, int64_t N, int64_t K,
                   int epilogue, void* y_bf16, void* workspace, size_t workspace_bytes,
                   void* stream) {
  if (bad_dim(M) || bad_dim(N) || bad_dim(K)) return NVFP4_ERR_SHAPE;
  const bool empty = M == 0 || N == 0;
  if (!empty && (!a_codes || !a_scales || !w_codes || !w_scales || !y_bf16)) return NVFP4_ERR_NULL;
  if (K == 0 || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (((M + 255) / 256) * ((N + 255) / 256) >= ((int64_t)1 << 24)) return NVFP4_ERR_SHAPE;
  if (!aligned(a_codes, 16) || !aligned(w_codes, 16) || !aligned(a_scales, 4) ||
      !aligned(w_scales, 4) || !aligned(bias_bf16, 2) || !aligned(y_bf16, 2) ||
      !aligned(workspace, 256))
    return NVFP4_ERR_ALIGN;
  if (epilogue != NVFP4_EPI_NONE && epilogue != NVFP4_EPI_GELU) return NVFP4_ERR_ARG;
  int st = check_device();
  if (st != NVFP4_OK) return st;
  if (empty) return NVFP4_OK;
  return hip_status(nvfp4::launch_gemm_fp8(a_codes, a_scales, w_codes, w_scales, bias_bf16, M, N,
                                           K, epilogue, y_bf16, workspace,
                                           workspace ? workspace_bytes : 0,
                                           static_cast<hipStream_t>(stream)));
}

int nvfp4_gemm_bf16(const void* x_bf16, const void* w_bf16, const void* bias_bf16, int64_t M,
                    int64_t N, int64_t K, int epilogue, void* y_bf16, void* stream) {
  if (bad_dim(M) || bad_dim(N) || bad_dim(K)) return NVFP4_ERR_SHAPE;
  const bool empty = M == 0 || N == 0;
  if (!empty && (!x_bf16 || !w_bf16 || !y_bf16)) return NVFP4_ERR_NULL;
  if (K == 0 || K % 8 != 0) return NVFP4_ERR_SHAPE;
  if (((M + 127) / 128) * ((N + 127) / 128) >= ((int64_t)1 << 24)) return NVFP4_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(w_bf16, 16) || !aligned(bias_bf16, 2) ||
      !aligned(y_bf16, 2))
    return NVFP4_ERR_ALIGN;
  if (epilogue != NVFP4_EPI_NONE && epilogue != NVFP4_EPI_GELU) return NVFP4_ERR_ARG;
  int st = check_device();
  if (st != NVFP4_OK) return st;
  if (empty) return NVFP4_OK;
  return hip_status(nvfp4::launch_gemm_bf16(x_bf16, w_bf16, bias_bf16, M, N, K, epilogue, y_bf16,
                                            static_cast<hipStream_t>(stream)));
}

int nvfp4_graph_begin(void* stream) {
  if (!stream) return NVFP4_ERR_NULL;
  int st = check_device();
  if (st != NVFP4_OK) return st;
  return hip_status(
      hipStreamBeginCapture(static_cast<hipStream_t>(stream), hipStreamCaptureModeThreadLocal));
}

int nvfp4_graph_end(void* stream, void** graph) {
  if (!stream || !graph) return NVFP4_ERR_NULL;
  hipGraph_t g = nullptr;
  if (hipStreamEndCapture(static_cast<hipStream_t>(stream), &g) != hipSuccess || !g)
    return NVFP4_ERR_HIP;
  hipGraphExec_t exec = nullptr;
  const hipError_t e = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
  // the instantiated graph does not need the captured one
  static_cast<void>(hipGraphDestroy(g));
  if (e != hipSuccess) return NVFP4_ERR_HIP;
  *graph = exec;
  return NVFP4_OK;
}

int nvfp4_graph_launch(void* graph, void* stream) {
  if (!graph) return NVFP4_ERR_NULL;
  return hip_status(
      hipGraphLaunch(static_cast<hipGraphExec_t>(graph), static_cast<hipStream_t>(stream)));
}

int nvfp4_graph_destroy(void* graph) {
  if (!graph) return NVFP4_ERR_NULL;
  return hip_status(hipGraphExecDestroy(static_cast<hipGraphExec_t>(graph)));
}

int nvfp4_layer_is_quantized(const char* layer_name, const char* pattern) {
  if (!layer_name) return NVFP4_ERR_NULL;
  if (!pattern) return page_pattern_matches(layer_name);
  try {
    const std::regex re(pattern, std::regex::ECMAScript);
    const std::string name(layer_name);
    if (name.size() > kMaxPatternName) return NVFP4_ERR_ARG;
    return std::regex_search(name, re, std::regex_constants::match_continuous) ? 1 : 0;
  } catch (const std::exception&) {
    return NVFP4_ERR_ARG;
  }
}

}  // extern "C"
