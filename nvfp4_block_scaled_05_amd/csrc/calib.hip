// Measurement probes behind calib.h: a matrix-core loop with known FLOPs and
// the shader clock it ran at, and streaming HBM read / copy kernels with
// known bytes.  They give the sustained rates of the part the roofline
// fractions are also reported against.
#include "calib.h"
#include "device_common.hpp"

namespace {

using namespace nvfp4;

constexpr int kCalibThreads = 256;   // 4 waves: one per SIMD
constexpr int kReadGrid = 4096;

// A 32-bit mix of the lane's coordinates (splitmix-style finalizer) for
// pseudo-random fp16 operand values.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

// An fp16 value shaped like a decoded NVFP4 operand: a signed E2M1 value
// (code from bits 0-3) times an E4M3-like scale 2^(e-3) * (1 + m/8) (bits
// 4-6 and 7-9): at most 6 significant bits, as the GEMM's decoded operands.
__device__ __forceinline__ float nvfp4_like(uint32_t h) {
  const uint32_t c = h & 7u;   // E2M1 magnitude code: 0, .5, 1, 1.5, 2, 3, 4, 6
  const float mag = c < 2u ? 0.5f * (float)c
                           : __builtin_ldexpf(1.0f + 0.5f * (float)(c & 1u), (int)(c >> 1) - 1);
  const float v = (h & 8u) ? -mag : mag;
  const float s = __builtin_ldexpf(1.0f + (float)((h >> 7) & 7u) * 0.125f, (int)((h >> 4) & 7u) - 3);
  return v * s;
}

__global__ __launch_bounds__(kCalibThreads, 1) void calib_mfma_kernel(int iters, int mode,
                                                                      float* __restrict__ sink,
                                                                      uint64_t* __restrict__ clocks) {
  f16x8 a[4], b[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = mix32((blockIdx.x * kCalibThreads + threadIdx.x) * 64u + u * 8u + e);
      float va = 0.5f, vb = 0.25f;
      if (mode == 1) {
        va = (float)(h & 0xFFFFu) * (1.0f / 32768.0f) - 1.0f;
        vb = (float)(h >> 16) * (1.0f / 32768.0f) - 1.0f;
      } else if (mode == 2) {
        va = nvfp4_like(h);
        vb = nvfp4_like(h >> 12);
      }
      a[u][e] = (_Float16)va;
      b[u][e] = (_Float16)vb;
    }
  f32x16 acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = f32x16{};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[k & 3], b[k >> 2], acc[k], 0, 0, 0);
  }
  // the accumulators are complete once they are read below; the counters are
  // taken after the last MFMA result is consumed
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  sink[blockIdx.x * kCalibThreads + threadIdx.x] = s;
  __builtin_amdgcn_s_waitcnt(0);
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if ((threadIdx.x & 63) == 0) {
    const int w = blockIdx.x * (kCalibThreads / 64) + (threadIdx.x >> 6);
    clocks[2 * w] = t1 - t0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

__global__ __launch_bounds__(256) void calib_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  u32x4 x = u32x4{0u, 0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u];
  }
  for (; i < n16; i += stride) x ^= __builtin_nontemporal_load(src + i);
  uint32_t w = x.x ^ x.y ^ x.z ^ x.w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) w ^= __shfl_xor(w, off, 64);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(256) void calib_copy_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, int64_t n16) {
  constexpr int U = 4;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

int units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 0;
  return n;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int launched() { return hipGetLastError() == hipSuccess ? 0 : -7; }

}  // namespace

extern "C" {

int nvfp4_calib_units(void) { return units(); }

int nvfp4_calib_mfma_f16(int iters, int mode, float* sink, uint64_t* clocks, void* stream) {
  if (!sink || !clocks) return -1;
  if (iters < 1 || mode < 0 || mode > 2) return -2;
  const int n = units();
  if (n <= 0) return -7;
  hipLaunchKernelGGL(calib_mfma_kernel, dim3(n), dim3(kCalibThreads), 0,
                     static_cast<hipStream_t>(stream), iters, mode, sink, clocks);
  return launched();
}

int nvfp4_calib_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return -1;
  if (bytes == 0 || bytes % 16) return -2;
  if (!aligned16(src)) return -3;
  hipLaunchKernelGGL(calib_read_kernel, dim3(kReadGrid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     (int64_t)(bytes / 16), sink);
  return launched();
}

int nvfp4_calib_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return -1;
  if (bytes == 0 || bytes % 16) return -2;
  if (!aligned16(src) || !aligned16(dst)) return -3;
  hipLaunchKernelGGL(calib_copy_kernel, dim3(kReadGrid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), (int64_t)(bytes / 16));
  return launched();
}

}  // extern "C"
