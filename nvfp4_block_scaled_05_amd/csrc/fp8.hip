// The FP8 row-wise variant of the DiT linear layers on gfx950.
//
// The pages select FP8 as the other quantized variant of the same model
// ("NVIDIA показала, как сократить генерацию FLUX 3 Image Klein с 22 до 6
// секунд", xalabuda.com, the paragraph on run options: --variant fp8r) and
// give no recipe.  Here "fp8r" is FP8 with row-wise scales: one FP32 scale per
// activation row (per token, dynamic on every call) and per weight row (per
// output channel, at load time), E4M3 elements, and
//
//   Y[m,n] = bf16( epi( (sum_k qA[m,k] * qW[n,k]) * (dA[m] * dW[n]) + bias[n] ) ).
//
// Quantize: a row's max needs no other row, so a workgroup holds its row in
// registers and reads it from HBM once; the E4M3 encode is the gfx950 packed
// conversion on values clamped to 448 (pinned against the oracle's encoder
// over every binary32 pattern).  GEMM: gfx950 runs E4M3 x E4M3 on the matrix cores natively
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit E8M0 scales), so unlike NVFP4
// nothing is decoded: operand bytes go from HBM through LDS into the MFMA.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nvfp4 {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// --------------------------------------------------------------- quantize --

constexpr int kQThreads = 256;

// E4M3 bytes of 4 bf16 values (two words) times s, sign in bit 7: |x| * s in
// binary32, clamped to 448 (saturation), then the packed hardware conversion.
__device__ __forceinline__ uint32_t encode4_fp8(uint32_t w0, uint32_t w1, float s) {
  const float v0 = __builtin_fminf(__uint_as_float((w0 & 0x7FFFu) << 16) * s, 448.0f);
  const float v1 = __builtin_fminf(__uint_as_float(w0 & 0x7FFF0000u) * s, 448.0f);
  const float v2 = __builtin_fminf(__uint_as_float((w1 & 0x7FFFu) << 16) * s, 448.0f);
  const float v3 = __builtin_fminf(__uint_as_float(w1 & 0x7FFF0000u) * s, 448.0f);
  const uint32_t signs = ((w0 >> 8) & 0x80u) | ((w0 >> 16) & 0x8000u) | ((w1 << 8) & 0x800000u) |
                         (w1 & 0x80000000u);
  return e4m3_pack4(v0, v1, v2, v3) | signs;
}

__global__ __launch_bounds__(kQThreads) void fp8_quantize_rowwise_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, uint8_t* __restrict__ codes,
    float* __restrict__ row_scales, int32_t* __restrict__ dev_status) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kQThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* xr = x + row * cols;
  u16x2 m = {0, 0};
  for (int64_t k = (int64_t)lane * 8; k < cols; k += 512) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xr + k);
    m = max_u16x2(m, max8(v));
  }
  const uint32_t amax_bits = wave_max_u32(m.x > m.y ? m.x : m.y) << 16;
  if (amax_bits >= 0x7F800000u) {                 // Inf / NaN in the row
    if (lane == 0) {
      row_scales[row] = __uint_as_float(0x7FC00000u);
      if (dev_status) *dev_status = -8;           // NVFP4_ERR_NONFINITE
    }
    return;
  }
  const float amax = __uint_as_float(amax_bits);
  const bool degenerate = amax < 0x1p-96f;
  const float s = degenerate ? 1.0f : 448.0f / amax;
  if (lane == 0) row_scales[row] = degenerate ? 1.0f : 1.0f / s;
  uint8_t* cr = codes + row * cols;
  for (int64_t k = (int64_t)lane * 8; k < cols; k += 512) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xr + k);
    *reinterpret_cast<u32x2*>(cr + k) = u32x2{encode4_fp8(v.x, v.y, s), encode4_fp8(v.z, v.w, s)};
  }
}

// One workgroup per row, the row held in registers (chunks of 8 elements,
// thread t holding chunks t, t + 256, ...; indices past the row's end are
// clamped to its last chunk, which leaves the max unchanged and is not
// stored): the input is read from HBM exactly once.  Rows of up to
// 2048 * MAXC elements.
template <int MAXC>
__global__ __launch_bounds__(kQThreads) void fp8_quantize_row_resident_kernel(
    const uint16_t* __restrict__ x, int64_t cols, uint8_t* __restrict__ codes,
    float* __restrict__ row_scales, int32_t* __restrict__ dev_status) {
  __shared__ uint32_t red[kQThreads / 64];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int nch = (int)(cols / 8);
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + row * cols);
  u32x4 v[MAXC];
  u16x2 m = {0, 0};
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = min(tid + i * kQThreads, nch - 1);
    v[i] = __builtin_nontemporal_load(xr + c);
    m = max_u16x2(m, max8(v[i]));
  }
  const uint32_t wm = wave_max_u32(m.x > m.y ? m.x : m.y);
  if ((tid & 63) == 0) red[tid >> 6] = wm;
  __syncthreads();
  const uint32_t amax_bits = max(max(red[0], red[1]), max(red[2], red[3])) << 16;
  if (amax_bits >= 0x7F800000u) {                 // Inf / NaN in the row
    if (tid == 0) {
      row_scales[row] = __uint_as_float(0x7FC00000u);
      if (dev_status) *dev_status = -8;           // NVFP4_ERR_NONFINITE
    }
    return;
  }
  const float amax = __uint_as_float(amax_bits);
  const bool degenerate = amax < 0x1p-96f;
  const float s = degenerate ? 1.0f : 448.0f / amax;
  if (tid == 0) row_scales[row] = degenerate ? 1.0f : 1.0f / s;
  u32x2* cr = reinterpret_cast<u32x2*>(codes + row * cols);
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = tid + i * kQThreads;
    if (c < nch) cr[c] = u32x2{encode4_fp8(v[i].x, v[i].y, s), encode4_fp8(v[i].z, v[i].w, s)};
  }
}

__global__ void zero_status_kernel(int32_t* p) { *p = 0; }

// ------------------------------------------------------------------- GEMM --

// Workgroup of 8 waves in 4x2 over a 256x256 tile, each wave 64x128 (2x4
// MFMA tiles of 32x32).  K advances 64 per stage: the stage's 64 operand
// bytes of each of the 256 A rows and 256 W rows sit in LDS (rows padded to
// 80 B, conflict-free 16-byte reads); the next stage is loaded into registers
// while the current one is computed.  K order inside a stage is the same for
// A and W: lanes 0-31 give bytes 0-31 of a row, lanes 32-63 bytes 32-63.
constexpr int kBM = 256, kBN = 256, kBK = 64, kNT = 512;
constexpr int kWGM = 4, kWGN = 2, kWM = kBM / kWGM, kWN = kBN / kWGN;
constexpr int kTM = kWM / 32, kTN = kWN / 32;
constexpr int kPitch = 80;
constexpr int kStage = (kBM + kBN) * kPitch;

struct Fp8Staged {
  u32x4 a[2], w[2];   // 32 B of one A row and one W row: half (q & 1) of the stage
};

template <bool kEdge>
__device__ __forceinline__ void fp8_load(const uint8_t* __restrict__ a, const uint8_t* __restrict__ w,
                                         int64_t M, int64_t N, int64_t K, int64_t m0, int64_t n0,
                                         int64_t k0, Fp8Staged& s) {
  const int q = threadIdx.x;
  const int64_t ra = m0 + (q >> 1), rw = n0 + (q >> 1);
  const int64_t k = k0 + (q & 1) * 32;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if constexpr (kEdge) {
      const bool kin = k + 16 * h < K;
      s.a[h] = (ra < M && kin) ? *reinterpret_cast<const u32x4*>(a + ra * K + k + 16 * h)
                               : u32x4{0u, 0u, 0u, 0u};
      s.w[h] = (rw < N && kin) ? *reinterpret_cast<const u32x4*>(w + rw * K + k + 16 * h)
                               : u32x4{0u, 0u, 0u, 0u};
    } else {
      s.a[h] = *reinterpret_cast<const u32x4*>(a + ra * K + k + 16 * h);
      s.w[h] = *reinterpret_cast<const u32x4*>(w + rw * K + k + 16 * h);
    }
  }
}

__device__ __forceinline__ void fp8_store(const Fp8Staged& s, uint8_t* stage) {
  const int q = threadIdx.x;
  u32x4* pa = reinterpret_cast<u32x4*>(stage + (q >> 1) * kPitch + (q & 1) * 32);
  u32x4* pw = reinterpret_cast<u32x4*>(stage + (kBM + (q >> 1)) * kPitch + (q & 1) * 32);
  pa[0] = s.a[0];
  pa[1] = s.a[1];
  pw[0] = s.w[0];
  pw[1] = s.w[1];
}

__device__ __forceinline__ i32x8 fp8_frag(const uint8_t* stage, int row) {
  const int h = (threadIdx.x & 63) >> 5;
  const u32x4* p = reinterpret_cast<const u32x4*>(stage + row * kPitch + h * 32);
  const u32x4 lo = p[0], hi = p[1];
  return __builtin_bit_cast(i32x8, (u32x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ void fp8_compute(const uint8_t* stage, f32x16 (&acc)[kTM][kTN]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWGN, wn = wave % kWGN;
  const int r = lane & 31;
  i32x8 av[kTM], bv[kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i) av[i] = fp8_frag(stage, wm * kWM + i * 32 + r);
#pragma unroll
  for (int j = 0; j < kTN; ++j) bv[j] = fp8_frag(stage, kBM + wn * kWN + j * 32 + r);
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)   // E4M3 x E4M3, E8M0 scales 127 (x1)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[i], bv[j], acc[i][j], 0, 0, 0,
                                                                   127, 0, 127);
}

template <bool kEdge>
__device__ __forceinline__ void fp8_main_loop(const uint8_t* a, const uint8_t* w, int64_t M,
                                              int64_t N, int64_t K, int64_t m0, int64_t n0,
                                              uint8_t* lds, f32x16 (&acc)[kTM][kTN]) {
  const int nk = (int)((K + kBK - 1) / kBK);
  Fp8Staged st;
  fp8_load<kEdge>(a, w, M, N, K, m0, n0, 0, st);
  fp8_store(st, lds);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    uint8_t* cur = lds + (kt & 1) * kStage;
    uint8_t* nxt = lds + ((kt + 1) & 1) * kStage;
    const int kn = kt + 1 < nk ? kt + 1 : kt;       // unconditional prefetch
    fp8_load<kEdge>(a, w, M, N, K, m0, n0, (int64_t)kn * kBK, st);
    __builtin_amdgcn_sched_barrier(0);
    fp8_compute(cur, acc);
    __builtin_amdgcn_sched_barrier(0);
    fp8_store(st, nxt);
    __syncthreads();
  }
}

__global__ __launch_bounds__(kNT, 1) void gemm_fp8_kernel(
    const uint8_t* __restrict__ a, const float* __restrict__ da, const uint8_t* __restrict__ w,
    const float* __restrict__ dw, const uint16_t* __restrict__ bias, int64_t M, int64_t N,
    int64_t K, int epi, uint16_t* __restrict__ y, int vec) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];
  __shared__ float row_scale[kBM], col_scale[kBN];
  const int64_t tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
  int64_t tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * kBM, n0 = tn * kBN;
  if (threadIdx.x < kBM) {
    const int64_t r = m0 + threadIdx.x;
    row_scale[threadIdx.x] = r < M ? da[r] : 0.0f;
  } else {
    const int64_t c = n0 + threadIdx.x - kBM;
    col_scale[threadIdx.x - kBM] = c < N ? dw[c] : 0.0f;
  }
  f32x16 acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = f32x16{};
  if (m0 + kBM <= M && n0 + kBN <= N && K % kBK == 0 && vec)
    fp8_main_loop<false>(a, w, M, N, K, m0, n0, lds, acc);
  else
    fp8_main_loop<true>(a, w, M, N, K, m0, n0, lds, acc);

  // epilogue: (acc * (dA[m] * dW[n]) + bias) -> GELU -> bf16
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWGN, wn = wave % kWGN;
#pragma unroll
  for (int j = 0; j < kTN; ++j) {
    const int cl = wn * kWN + j * 32 + (lane & 31);
    const int64_t col = n0 + cl;
    if (col >= N) continue;
    const float bv = bias ? bf16_bits_to_f32(bias[col]) : 0.0f;
    const float cs = col_scale[cl];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const int rl = wm * kWM + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        float v0 = __builtin_fmaf(acc[i][j][e], row_scale[rl] * cs, bv);
        float v1 = __builtin_fmaf(acc[i][j][e + 1], row_scale[rl + 1] * cs, bv);
        if (epi == 1) {
          v0 = gelu_erf(v0);
          v1 = gelu_erf(v1);
        }
        const uint32_t pk = bf16x2_rne(v0, v1);
        if (m0 + rl < M) y[(m0 + rl) * N + col] = (uint16_t)pk;
        if (m0 + rl + 1 < M) y[(m0 + rl + 1) * N + col] = (uint16_t)(pk >> 16);
      }
  }
}

}  // namespace

hipError_t launch_fp8_quantize_rowwise(const void* x, int64_t rows, int64_t cols, uint8_t* codes,
                                       float* row_scales, int32_t* dev_status,
                                       hipStream_t stream) {
  if (dev_status) {
    hipLaunchKernelGGL(zero_status_kernel, dim3(1), dim3(1), 0, stream, dev_status);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (rows == 0) return hipSuccess;
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
  if (cols <= 2048 * 2) {
    hipLaunchKernelGGL(fp8_quantize_row_resident_kernel<2>, dim3((unsigned)rows), dim3(kQThreads),
                       0, stream, xb, cols, codes, row_scales, dev_status);
    return hipGetLastError();
  }
  if (cols <= 2048 * 6) {
    hipLaunchKernelGGL(fp8_quantize_row_resident_kernel<6>, dim3((unsigned)rows), dim3(kQThreads),
                       0, stream, xb, cols, codes, row_scales, dev_status);
    return hipGetLastError();
  }
  // longer rows: a wave per row, the encode pass re-reading the row
  const int64_t wgs = (rows + kQThreads / 64 - 1) / (kQThreads / 64);
  hipLaunchKernelGGL(fp8_quantize_rowwise_kernel, dim3((unsigned)wgs), dim3(kQThreads), 0, stream,
                     reinterpret_cast<const uint16_t*>(x), rows, cols, codes, row_scales,
                     dev_status);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8(const uint8_t* a_codes, const float* a_scales, const uint8_t* w_codes,
                           const float* w_scales, const void* bias, int64_t M, int64_t N,
                           int64_t K, int epilogue, void* y, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  const uintptr_t al = reinterpret_cast<uintptr_t>(a_codes) | reinterpret_cast<uintptr_t>(w_codes);
  hipLaunchKernelGGL(gemm_fp8_kernel, dim3((unsigned)tiles), dim3(kNT), 0, stream, a_codes, a_scales,
                     w_codes, w_scales, reinterpret_cast<const uint16_t*>(bias), M, N, K, epilogue,
                     reinterpret_cast<uint16_t*>(y), (al & 15) == 0 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace nvfp4
