// Block-scaled W4A4 NVFP4 GEMM and the bf16 passthrough GEMM for gfx950.
//
// The DiT linear layers run an NVFP4 GEMM on NVFP4 weights and activations
// ("NVIDIA介绍用TensorRT LLM VisualGen加速Blackwell上的FLUX 3 Image Klein",
// sns.style, time-breakdown paragraph; "NVIDIA показала, как сократить
// генерацию FLUX 3 Image Klein с 22 до 6 секунд", xalabuda.com, section
// "Квантование NVFP4 и оптимизация вычислительных ядер"); layers matched by
// the exclude pattern stay bf16 ("英伟达B200狂飙10.2倍！AI绘图告别龟速！",
// nmedialink.com, section "NVFP4量化").
//
//   Y[m,n] = bf16( epi( sA*sW * sum_k Ahat[m,k]*What[n,k] + bias[n] ) )
//
// Exact decode.  value(E2M1) * E4M3 has at most 6 significant bits and lies
// in [2^-10, 2688], so it is exact in fp16 (normal range).  The loader turns
// each 16-element block into fp16 with the gfx950 packed E2M1->fp16
// conversion (scale operand 1.0, which it applies as an exponent only) and one
// packed fp16 multiply by the block scale, and stores the fp16 tile in LDS.
// The MFMA v_mfma_f32_32x32x16_f16 then accumulates exact products in fp32,
// and the per-tensor scales are applied once in the epilogue.
//
// Tiling: 128x128 output tile per 256-thread workgroup, K step 64 (four
// 16-blocks), LDS double-buffered with a register prefetch of the next K step;
// each of the 4 waves owns a 64x64 sub-tile = 2x2 MFMA 32x32 tiles.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nvfp4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

static constexpr int BM = 128, BN = 128, BK = 64;
static constexpr int PITCH = BK + 8;   // halves per LDS row: 144 B, conflict-free b128 reads
static constexpr int NT = 256;
static constexpr int TILE_ELEMS = BM * PITCH;

// ------------------------------------------------------------------ loaders --

// NVFP4 operand: codes [rows, K/2], scales [rows, K/16].  Per K step a tile
// holds 128 rows x 4 blocks = 512 blocks; each thread moves 2 of them.
struct Nvfp4Tile {
  uint2 c[2];
  uint32_t s[2];
};

__device__ __forceinline__ void load_nvfp4(const uint8_t* __restrict__ codes,
                                           const uint8_t* __restrict__ scales, int64_t rows,
                                           int64_t kblocks, int64_t row0, int64_t kb0,
                                           Nvfp4Tile& t) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + i * NT;
    const int64_t row = row0 + (q >> 2);
    const int64_t kb = kb0 + (q & 3);
    if (row < rows && kb < kblocks) {
      t.c[i] = *reinterpret_cast<const uint2*>(codes + row * (kblocks * 8) + kb * 8);
      t.s[i] = scales[row * kblocks + kb];
    } else {
      t.c[i] = make_uint2(0u, 0u);
      t.s[i] = 0u;
    }
  }
}

__device__ __forceinline__ uint4 decode8_f16(uint32_t w, f16x2 s2) {
  const f16x2 p0 = e2m1_unpack2_f16<0>(w) * s2;
  const f16x2 p1 = e2m1_unpack2_f16<1>(w) * s2;
  const f16x2 p2 = e2m1_unpack2_f16<2>(w) * s2;
  const f16x2 p3 = e2m1_unpack2_f16<3>(w) * s2;
  return make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                    __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
}

__device__ __forceinline__ void store_nvfp4(const Nvfp4Tile& t, uint16_t* __restrict__ lds) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + i * NT;
    const _Float16 s = (_Float16)e4m3_to_f32(t.s[i]);   // exact in fp16
    const f16x2 s2 = {s, s};
    uint4* dst = reinterpret_cast<uint4*>(lds + (q >> 2) * PITCH + (q & 3) * 16);
    dst[0] = decode8_f16(t.c[i].x, s2);
    dst[1] = decode8_f16(t.c[i].y, s2);
  }
}

// bf16 operand [rows, K], K % 8 == 0.  Per K step: 128 rows x 8 chunks of
// 8 bf16 = 1024 chunks; 4 per thread.
struct Bf16Tile {
  uint4 v[4];
};

__device__ __forceinline__ void load_bf16(const uint16_t* __restrict__ x, int64_t rows, int64_t K,
                                          int64_t row0, int64_t k0, Bf16Tile& t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = threadIdx.x + i * NT;
    const int64_t row = row0 + (q >> 3);
    const int64_t k = k0 + (q & 7) * 8;
    if (row < rows && k < K)
      t.v[i] = *reinterpret_cast<const uint4*>(x + row * K + k);
    else
      t.v[i] = make_uint4(0u, 0u, 0u, 0u);
  }
}

__device__ __forceinline__ void store_bf16(const Bf16Tile& t, uint16_t* __restrict__ lds) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = threadIdx.x + i * NT;
    *reinterpret_cast<uint4*>(lds + (q >> 3) * PITCH + (q & 7) * 8) = t.v[i];
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
    uint4 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      a[i] = *reinterpret_cast<const uint4*>(As + (wm * 64 + i * 32 + r) * PITCH + kk * 16 + kh);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      b[j] = *reinterpret_cast<const uint4*>(Bs + (wn * 64 + j * 32 + r) * PITCH + kk * 16 + kh);
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

__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

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

__global__ __launch_bounds__(NT, 2) void gemm_nvfp4_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ sa, const uint8_t* __restrict__ w_codes,
    const uint8_t* __restrict__ w_scales, const float* __restrict__ sw,
    const uint16_t* __restrict__ bias, int64_t M, int64_t N, int64_t K, int epi,
    uint16_t* __restrict__ y, uint32_t* __restrict__ y_amax) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][TILE_ELEMS];
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * BM;
  const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * BN;
  const int64_t kblocks = K / 16;
  const int nk = (int)((K + BK - 1) / BK);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  Nvfp4Tile ta, tb;
  load_nvfp4(a_codes, a_scales, M, kblocks, m0, 0, ta);
  load_nvfp4(w_codes, w_scales, N, kblocks, n0, 0, tb);
  store_nvfp4(ta, lds[0][0]);
  store_nvfp4(tb, lds[0][1]);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      load_nvfp4(a_codes, a_scales, M, kblocks, m0, (int64_t)(kt + 1) * (BK / 16), ta);
      load_nvfp4(w_codes, w_scales, N, kblocks, n0, (int64_t)(kt + 1) * (BK / 16), tb);
    }
    mma_step<true>(lds[cur][0], lds[cur][1], acc);
    if (more) {
      store_nvfp4(ta, lds[cur ^ 1][0]);
      store_nvfp4(tb, lds[cur ^ 1][1]);
    }
    __syncthreads();
  }
  const float scale = (*sa) * (*sw);
  epilogue(acc, scale, bias, epi, M, N, m0, n0, y, y_amax);
}

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

__global__ void zero_word_kernel(uint32_t* p) { *p = 0u; }

// ---------------------------------------------------------------- launchers --

hipError_t launch_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales,
                             const float* a_tensor_scale, const uint8_t* w_codes,
                             const uint8_t* w_scales, const float* w_tensor_scale,
                             const void* bias, int64_t M, int64_t N, int64_t K, int epilogue,
                             void* y, float* y_amax, hipStream_t stream) {
  uint32_t* amax_bits = reinterpret_cast<uint32_t*>(y_amax);
  if (amax_bits) {
    hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(1), 0, stream, amax_bits);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL(gemm_nvfp4_kernel, dim3((unsigned)tiles), dim3(NT), 0, stream, a_codes,
                     a_scales, a_tensor_scale, w_codes, w_scales, w_tensor_scale,
                     reinterpret_cast<const uint16_t*>(bias), M, N, K, epilogue,
                     reinterpret_cast<uint16_t*>(y), amax_bits);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const void* x, const void* w, const void* bias, int64_t M, int64_t N,
                            int64_t K, int epilogue, void* y, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3((unsigned)tiles), dim3(NT), 0, stream,
                     reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(w),
                     reinterpret_cast<const uint16_t*>(bias), M, N, K, epilogue,
                     reinterpret_cast<uint16_t*>(y));
  return hipGetLastError();
}

}  // namespace nvfp4
