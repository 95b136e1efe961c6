// bf16 passthrough GEMM for gfx950: the linear layers kept in higher precision
// by the exclude pattern ("英伟达B200狂飙10.2倍！AI绘图告别龟速！",
// nmedialink.com, section "NVFP4量化").
//
//   Y[m,n] = bf16( epi( sum_k X[m,k]*W[n,k] + bias[n] ) ), fp32 accumulation.
//
// Tiling: 128x128 output tile per 256-thread workgroup, K step 64, LDS
// double-buffered with a register prefetch of the next K step; each of the 4
// waves owns a 64x64 sub-tile = 2x2 v_mfma_f32_32x32x16_bf16 tiles.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nvfp4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

static constexpr int BM = 128, BN = 128, BK = 64;
static constexpr int PITCH = BK + 8;   // halves per LDS row: 144 B, conflict-free b128 reads
static constexpr int NT = 256;
static constexpr int TILE_ELEMS = BM * PITCH;

// ------------------------------------------------------------------ loaders --

// bf16 operand [rows, K], K % 8 == 0.  Per K step: 128 rows x 8 chunks of
// 8 bf16 = 1024 chunks; 4 per thread.
struct Bf16Tile {
  u32x4 v[4];
};

__device__ __forceinline__ void load_bf16(const uint16_t* __restrict__ x, int64_t rows, int64_t K,
                                          int64_t row0, int64_t k0, Bf16Tile& t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = threadIdx.x + i * NT;
    const int64_t row = row0 + (q >> 3);
    const int64_t k = k0 + (q & 7) * 8;
    if (row < rows && k < K)
      t.v[i] = *reinterpret_cast<const u32x4*>(x + row * K + k);
    else
      t.v[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void store_bf16(const Bf16Tile& t, uint16_t* __restrict__ lds) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = threadIdx.x + i * NT;
    *reinterpret_cast<u32x4*>(lds + (q >> 3) * PITCH + (q & 7) * 8) = t.v[i];
  }
}

// ------------------------------------------------------------------ compute --

template <bool kF16>
__device__ __forceinline__ void mma_step(const uint16_t* __restrict__ As,
                                         const uint16_t* __restrict__ Bs, f32x16 (&acc)[2][2]) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int r = lane & 31, kh = (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    u32x4 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      a[i] = *reinterpret_cast<const u32x4*>(As + (wm * 64 + i * 32 + r) * PITCH + kk * 16 + kh);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      b[j] = *reinterpret_cast<const u32x4*>(Bs + (wn * 64 + j * 32 + r) * PITCH + kk * 16 + kh);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (kF16)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(f16x8, a[i]), __builtin_bit_cast(f16x8, b[j]), acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a[i]), __builtin_bit_cast(bf16x8, b[j]), acc[i][j], 0, 0, 0);
      }
  }
}

// ----------------------------------------------------------------- epilogue --

__device__ __forceinline__ void epilogue(const f32x16 (&acc)[2][2], float scale,
                                         const uint16_t* __restrict__ bias, int epi, int64_t M,
                                         int64_t N, int64_t m0, int64_t n0,
                                         uint16_t* __restrict__ y, uint32_t* __restrict__ y_amax) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  uint32_t amax = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
    const bool col_ok = col < N;
    const float bv = (bias && col_ok) ? bf16_bits_to_f32(bias[col]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (col_ok && row < M) {
          float v = acc[i][j][r] * scale + bv;
          if (epi == 1) v = gelu_erf(v);
          const uint32_t h = bf16_rne_bits(v);
          y[row * N + col] = (uint16_t)h;
          const uint32_t mag = (h & 0x7FFFu) << 16;
          amax = amax > mag ? amax : mag;
        }
      }
  }
  if (y_amax) {
    amax = wave_max_u32(amax);
    if (lane == 0) atomicMax(y_amax, amax);
  }
}

// ------------------------------------------------------------------- kernels --

__global__ __launch_bounds__(NT, 2) void gemm_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ bias, int64_t M, int64_t N, int64_t K, int epi,
    uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][TILE_ELEMS];
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * BM;
  const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * BN;
  const int nk = (int)((K + BK - 1) / BK);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  Bf16Tile ta, tb;
  load_bf16(x, M, K, m0, 0, ta);
  load_bf16(w, N, K, n0, 0, tb);
  store_bf16(ta, lds[0][0]);
  store_bf16(tb, lds[0][1]);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      load_bf16(x, M, K, m0, (int64_t)(kt + 1) * BK, ta);
      load_bf16(w, N, K, n0, (int64_t)(kt + 1) * BK, tb);
    }
    mma_step<false>(lds[cur][0], lds[cur][1], acc);
    if (more) {
      store_bf16(ta, lds[cur ^ 1][0]);
      store_bf16(tb, lds[cur ^ 1][1]);
    }
    __syncthreads();
  }
  epilogue(acc, 1.0f, bias, epi, M, N, m0, n0, y, nullptr);
}

// Few-row case (M <= kGemvMaxRows, e.g. the modulation linear on the timestep
// embedding, M = 2): the weight read is the whole cost, so no tiles and no
// MFMA.  Each wave owns kGemvRows weight rows; lane l reads 8 consecutive k
// per 512-wide step of every row (16 B loads, a wave covers 1 KB of a row),
// multiplies by the same k of every X row (L2-resident, read through the
// cache), and accumulates in fp32; the 64 lanes' partial sums are then added
// by a butterfly across the wave.
static constexpr int kGemvMaxRows = 8;
static constexpr int kGemvRows = 4;      // weight rows per wave

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int MR>
__global__ __launch_bounds__(256) void gemv_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ bias, int64_t N, int64_t K, int epi, uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t n0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kGemvRows;
  if (n0 >= N) return;
  float acc[kGemvRows][MR];
#pragma unroll
  for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[r][m] = 0.0f;
  for (int64_t k = (int64_t)lane * 8; k < K; k += 512) {
    u32x4 wv[kGemvRows], xv[MR];
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
      const int64_t n = n0 + r < N ? n0 + r : N - 1;
      wv[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w + n * K + k));
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) xv[m] = *reinterpret_cast<const u32x4*>(x + m * K + k);
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[r][m] = __builtin_fmaf(bf16_lo(wv[r][e]), bf16_lo(xv[m][e]), acc[r][m]);
          acc[r][m] = __builtin_fmaf(bf16_hi(wv[r][e]), bf16_hi(xv[m][e]), acc[r][m]);
        }
  }
#pragma unroll
  for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) acc[r][m] += __shfl_xor(acc[r][m], off);
  // lane r*MR + m writes output (m, n0 + r)
#pragma unroll
  for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
    for (int m = 0; m < MR; ++m)
      if (lane == r * MR + m && n0 + r < N) {
        float v = acc[r][m] + (bias ? bf16_bits_to_f32(bias[n0 + r]) : 0.0f);
        if (epi == 1) v = gelu_erf(v);
        y[m * N + n0 + r] = (uint16_t)bf16_rne_bits(v);
      }
}

template <int MR>
hipError_t launch_gemv(const void* x, const void* w, const void* bias, int64_t N, int64_t K,
                       int epilogue, void* y, hipStream_t stream) {
  const int64_t waves = (N + kGemvRows - 1) / kGemvRows;
  hipLaunchKernelGGL((gemv_bf16_kernel<MR>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                     stream, reinterpret_cast<const uint16_t*>(x),
                     reinterpret_cast<const uint16_t*>(w), reinterpret_cast<const uint16_t*>(bias),
                     N, K, epilogue, reinterpret_cast<uint16_t*>(y));
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers --

hipError_t launch_gemm_bf16(const void* x, const void* w, const void* bias, int64_t M, int64_t N,
                            int64_t K, int epilogue, void* y, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  switch (M) {   // few rows: the weight-streaming kernel
    case 1: return launch_gemv<1>(x, w, bias, N, K, epilogue, y, stream);
    case 2: return launch_gemv<2>(x, w, bias, N, K, epilogue, y, stream);
    case 3: return launch_gemv<3>(x, w, bias, N, K, epilogue, y, stream);
    case 4: return launch_gemv<4>(x, w, bias, N, K, epilogue, y, stream);
    case 5: return launch_gemv<5>(x, w, bias, N, K, epilogue, y, stream);
    case 6: return launch_gemv<6>(x, w, bias, N, K, epilogue, y, stream);
    case 7: return launch_gemv<7>(x, w, bias, N, K, epilogue, y, stream);
    case 8: return launch_gemv<8>(x, w, bias, N, K, epilogue, y, stream);
    default: break;
  }
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3((unsigned)tiles), dim3(NT), 0, stream,
                     reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(w),
                     reinterpret_cast<const uint16_t*>(bias), M, N, K, epilogue,
                     reinterpret_cast<uint16_t*>(y));
  return hipGetLastError();
}

}  // namespace nvfp4
