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
#include <algorithm>
#include <cstdlib>
#include <cstring>

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

// ------------------------------------------------- GEMM, direct-to-LDS --
//
// For K % 128 == 0.  Workgroup of 4 waves in 2x2 over a 256x256 tile, each
// wave 128x128 (4x4 MFMA tiles, 256 fp32 accumulators per lane): half the LDS
// reads per flop of the 8-wave layout above.  K advances 128 per stage (two
// MFMA k-steps of 64), double-buffered in LDS (2 x 64 KB).
//   * Operand bytes go from global memory straight into LDS (the gfx950
//     16-byte global->LDS load: one instruction fills 1 KB, lane L's 16 bytes
//     at offset 16 L), so they pass through no registers.  One instruction
//     covers 8 rows x 128 bytes; inside a row the 16-byte pieces are permuted
//     by an XOR with (row / 2) % 8, which makes every fragment read below
//     (16 lanes, 16 consecutive rows, the same logical piece) touch 16
//     different bank groups.
//   * Fragments: lane (r = lane % 32, h = lane / 32) of an MFMA takes 32 bytes
//     of row r: pieces 4s + 2h and 4s + 2h + 1 for k-step s.  A and W use the
//     same order, so the sum over k is the same.
//   * Each stage has one barrier; the MFMAs of its second k-step run after
//     the next barrier, while the first LDS reads of the next stage are in
//     flight, so the matrix pipe does not drain at every barrier.
// Rows past M or N are read clamped to the last row (valid memory); their
// results are never stored.
constexpr int kDBM = 256, kDBN = 256, kDBK = 128, kDNT = 256;
constexpr int kDWM = 128, kDWN = 128, kDTM = kDWM / 32, kDTN = kDWN / 32;
constexpr int kDOp = kDBM * kDBK;          // bytes of one operand per stage
constexpr int kDStage = 2 * kDOp;          // A then W

// This lane's source offsets (bytes from the operand's start; rows * K
// < 2^32 is checked on the host), one per 8-row chunk it loads.
struct DmaPtrs {
  uint32_t a[kDBM / 8 / 4];
  uint32_t w[kDBN / 8 / 4];
};

__device__ __forceinline__ void dma_setup(int64_t M, int64_t N, int64_t K, int64_t m0, int64_t n0,
                                          DmaPtrs& d) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kDBM / 8 / 4; ++i) {
    const int c = wave * (kDBM / 8 / 4) + i;             // chunk: rows 8c .. 8c+7
    const int row = 8 * c + (lane >> 3);
    const int piece = (lane & 7) ^ ((row >> 1) & 7);
    const int64_t ra = m0 + row < M ? m0 + row : M - 1;
    const int64_t rw = n0 + row < N ? n0 + row : N - 1;
    d.a[i] = (uint32_t)(ra * K + piece * 16);
    d.w[i] = (uint32_t)(rw * K + piece * 16);
  }
}

__device__ __forceinline__ void dma_issue(const uint8_t* __restrict__ a, const uint8_t* __restrict__ w,
                                          const DmaPtrs& d, int64_t k0, uint8_t* stage) {
  const int wave = wave_id();
#pragma unroll
  for (int i = 0; i < kDBM / 8 / 4; ++i) {
    const int c = wave * (kDBM / 8 / 4) + i;
    buffer_load_lds<16>(a, d.a[i], (int)k0, stage + c * 1024);
    buffer_load_lds<16>(w, d.w[i], (int)k0, stage + kDOp + c * 1024);
  }
}

struct DmaFrags {
  i32x8 a[kDTM], b[kDTN];
};

// Fragments of k-step s from one stage.  row_off: this lane's byte offset of
// its row in the wave's first A / W tile; sw = (row / 2) % 8.
template <int S>
__device__ __forceinline__ void dma_frags(const uint8_t* stage, int a_off, int b_off, int h, int sw,
                                          DmaFrags& f) {
  const int p0 = ((4 * S + 2 * h) ^ sw) << 4, p1 = ((4 * S + 2 * h + 1) ^ sw) << 4;
#pragma unroll
  for (int i = 0; i < kDTM; ++i) {
    const uint8_t* r = stage + a_off + i * 32 * kDBK;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(r + p0);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(r + p1);
    f.a[i] = __builtin_bit_cast(i32x8, (u32x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
#pragma unroll
  for (int j = 0; j < kDTN; ++j) {
    const uint8_t* r = stage + kDOp + b_off + j * 32 * kDBK;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(r + p0);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(r + p1);
    f.b[j] = __builtin_bit_cast(i32x8, (u32x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

// The weight fragment is the MFMA's first operand and the activation the
// second, so acc[i][j] holds the transposed 32x32 tile: lane (r, h) has row
// m = i*32 + r of Y and columns n = j*32 + 8g + 4h + t at element 4g + t --
// four consecutive columns of one row per g, stored as one 8-byte write.
__device__ __forceinline__ void dma_mfma(const DmaFrags& f, f32x16 (&acc)[kDTM][kDTN]) {
#pragma unroll
  for (int i = 0; i < kDTM; ++i)
#pragma unroll
    for (int j = 0; j < kDTN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], acc[i][j], 0, 0, 0,
                                                                   127, 0, 127);
}

// Every DMA of this wave has landed in LDS (vmcnt 0), then the workgroup
// barrier: all waves' data for the next stage is visible and all reads of the
// buffer about to be refilled are done.
__device__ __forceinline__ void dma_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// One stage: refill `nxt` with the stage after this one (REFILL), read this
// stage's fragments from `cur`, and run the previous stage's second k-step and
// this stage's first.  MFMAs are interleaved with the LDS reads and the DMA
// issues, one load per MFMA over the first half of the stage: early enough to
// land before the next barrier (two buffers leave one stage of latency), and
// not in a burst, which would hold the matrix pipe idle while the compute
// unit's address unit takes the loads.  REFILL is compile-time so that the
// loads sit in the MFMAs' basic block instead of a branch of their own.
template <bool REFILL>
__device__ __forceinline__ void dma_stage(const uint8_t* __restrict__ a, const uint8_t* __restrict__ w,
                                          const uint8_t* cur, uint8_t* nxt, const DmaPtrs& ptr,
                                          int64_t k_next, int a_off, int b_off, int h, int sw,
                                          DmaFrags& f0, DmaFrags& f1, f32x16 (&acc)[kDTM][kDTN]) {
  dma_barrier();
  if (REFILL) dma_issue(a, w, ptr, k_next, nxt);
  dma_frags<0>(cur, a_off, b_off, h, sw, f0);
  dma_mfma(f1, acc);                        // previous stage, k-step 1
  dma_frags<1>(cur, a_off, b_off, h, sw, f1);
  dma_mfma(f0, acc);
#pragma unroll
  for (int m = 0; m < 2 * kDTM * kDTN; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    if (REFILL && m < kDTM * kDTN) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM (DMA issue)
  }
}

// 32 rows x 128 columns of a wave's tile, staged in LDS by the epilogue of
// gemm_fp8_dma_kernel, to bf16: lane takes 4 consecutive columns of a row per
// step (32 lanes cover the row segment, so the 8-byte stores complete whole
// lines).
template <int EPI>
__device__ __forceinline__ void fp8_slice_out(const float* st, const float* rs, f32x4 cs, f32x4 bv,
                                              int64_t row0, int64_t col, int64_t M, int64_t N,
                                              bool vec, uint16_t* __restrict__ y, int lane) {
  const int c = lane & 31;
  asm volatile("" : "+v"(row0));   // row offsets computed here, not hoisted (see opaque_lane)
  // four rows' reads first, then their 16 values (GELU one step across all
  // 16), then the stores: one LDS wait per 16 values and independent chains
  for (int it0 = 0; it0 < 16; it0 += 4) {
    f32x4 v[4];
    float rsc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int rr = (it0 + u) * 2 + (lane >> 5);
      v[u] = *reinterpret_cast<const f32x4*>(st + rr * 128 + ((c ^ rr) << 2));
      rsc[u] = rs[rr];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < 4; ++t) v[u][t] = __builtin_fmaf(v[u][t], rsc[u] * cs[t], bv[t]);
    if (EPI == 1) gelu_erf16(v);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x2 pk = {bf16x2_rne(v[u][0], v[u][1]), bf16x2_rne(v[u][2], v[u][3])};
      const int64_t row = row0 + (it0 + u) * 2 + (lane >> 5);
      if (vec) {
        *reinterpret_cast<u32x2*>(y + row * N + col) = pk;
      } else if (row < M) {
        const uint16_t hv[4] = {(uint16_t)pk.x, (uint16_t)(pk.x >> 16), (uint16_t)pk.y, (uint16_t)(pk.y >> 16)};
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (col + t < N) y[row * N + col + t] = hv[t];
      }
    }
  }
}

// Work item b of a launch: a whole tile, or one K range of a tail tile
// (split_coords_of on item b), with its first and last stage.
struct DmaItem {
  int64_t m0, n0, tail;
  int split, kb, ke;
};

__device__ __forceinline__ DmaItem dma_item(int64_t b, int64_t tiles_m, int64_t tiles_n,
                                            const SplitK& sk, int nk) {
  DmaItem it;
  int64_t tm, tn;
  split_coords_of(b, tiles_m, tiles_n, sk, tm, tn, it.tail, it.split);
  it.m0 = tm * kDBM;
  it.n0 = tn * kDBN;
  // the stage range is uniform; readfirstlane keeps it in scalar registers
  // (the loads take their K offset as a scalar operand)
  it.kb = __builtin_amdgcn_readfirstlane(it.split < 0 ? 0 : (int)((int64_t)it.split * nk / sk.ways));
  it.ke = __builtin_amdgcn_readfirstlane(it.split < 0 ? nk : (int)((int64_t)(it.split + 1) * nk / sk.ways));
  return it;
}

// Persistent: workgroup b takes work items b, b + gridDim.x, ... below
// `items` (the grid is a multiple of the 8 XCDs, so every item of a
// workgroup maps to its XCD's range of the tile order, as a one-item launch
// would).  The epilogue stages the accumulators in buffer 1 only, so the next
// item's first stage is loaded into buffer 0 while this item's epilogue runs.
__global__ __launch_bounds__(kDNT, 1) void gemm_fp8_dma_kernel(
    const uint8_t* __restrict__ a, const float* __restrict__ da, const uint8_t* __restrict__ w,
    const float* __restrict__ dw, const uint16_t* __restrict__ bias, int64_t M, int64_t N,
    int64_t K, int epi, uint16_t* __restrict__ y, SplitK sk, int64_t items) {
  // two separately declared buffers, so that reads of one are seen not to
  // alias DMA writes into the other
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kDStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kDStage];
  __shared__ float row_scale[kDBM];
  __shared__ __attribute__((aligned(16))) float col_scale[kDBN], col_bias[kDBN];
  static_assert(4 * 16384 <= kDStage, "the epilogue's staging fits in one buffer");
  const int64_t tiles_m = (M + kDBM - 1) / kDBM, tiles_n = (N + kDBN - 1) / kDBN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, h = lane >> 5, sw = (r >> 1) & 7;
  const int a_off = (wm * kDWM + r) * kDBK, b_off = (wn * kDWN + r) * kDBK;
  const int nk = (int)(K / kDBK);

  int64_t b = blockIdx.x;
  DmaItem it = dma_item(b, tiles_m, tiles_n, sk, nk);
  DmaPtrs ptr;
  dma_setup(M, N, K, it.m0, it.n0, ptr);
  dma_issue(a, w, ptr, (int64_t)it.kb * kDBK, lds0);
  for (;;) {
    {
      const int64_t rr = it.m0 + threadIdx.x, c = it.n0 + threadIdx.x;
      row_scale[threadIdx.x] = rr < M ? da[rr] : 0.0f;
      col_scale[threadIdx.x] = c < N ? dw[c] : 0.0f;
      col_bias[threadIdx.x] = (bias && c < N) ? bf16_bits_to_f32(bias[c]) : 0.0f;
    }
    f32x16 acc[kDTM][kDTN];
#pragma unroll
    for (int i = 0; i < kDTM; ++i)
#pragma unroll
      for (int j = 0; j < kDTN; ++j) acc[i][j] = f32x16{};

    // stages [kb, ke) of 128 K: all of them, or this split's share; the
    // first one is already issued
    const int kb = it.kb, ns = it.ke - it.kb;
    DmaFrags f0, f1;
    dma_barrier();
    if (ns > 1) dma_issue(a, w, ptr, (int64_t)(kb + 1) * kDBK, lds1);
    dma_frags<0>(lds0, a_off, b_off, h, sw, f0);
    dma_frags<1>(lds0, a_off, b_off, h, sw, f1);
    dma_mfma(f0, acc);
    // stage kb + t reads buffer t % 2 and refills the other with stage
    // kb + t + 1; whole pairs of stages, then at most one more.  Both stages
    // of a pair load: the second stage of the last pair, with no stage left
    // to load, loads its own stage again into the buffer nothing reads any
    // more (a branch around its loads would take them out of the MFMAs'
    // basic block); those loads are waited for before the epilogue or the
    // partial stores.
    int t = 1;
    for (; t + 1 < ns; t += 2) {
      dma_stage<true>(a, w, lds1, lds0, ptr, (int64_t)(kb + t + 1) * kDBK, a_off, b_off, h, sw, f0,
                      f1, acc);
      const int k2 = t + 2 < ns ? kb + t + 2 : kb + t + 1;
      dma_stage<true>(a, w, lds0, lds1, ptr, (int64_t)k2 * kDBK, a_off, b_off, h, sw, f0, f1, acc);
    }
    if (t < ns) dma_stage<false>(a, w, lds1, lds0, ptr, 0, a_off, b_off, h, sw, f0, f1, acc);
    dma_mfma(f1, acc);
    __builtin_amdgcn_s_waitcnt(0);           // every load into LDS has landed

    const DmaItem cur = it;
    const int64_t nb = b + gridDim.x;
    const bool has_next = nb < items;
    if (cur.split >= 0) {
      // a tail split: fp32 partial sums into its slice in accumulator order --
      // float4 number (((wave * 4 + i) * 4 + j) * 64 + lane) * 4 + g holds
      // acc[i][j][4g .. 4g+3], so each wave writes 4 KB contiguous per tile
      f32x4* slice =
          reinterpret_cast<f32x4*>(sk.part + (cur.tail * sk.ways + cur.split) * (int64_t)(kDBM * kDBN));
#pragma unroll
      for (int i = 0; i < kDTM; ++i)
#pragma unroll
        for (int j = 0; j < kDTN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            slice[(((wave * kDTM + i) * kDTN + j) * 64 + lane) * 4 + g] =
                f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
      if (!has_next) break;
      asm volatile("s_barrier" ::: "memory");   // every wave is done reading this item's buffers
      b = nb;
      it = dma_item(b, tiles_m, tiles_n, sk, nk);
      dma_setup(M, N, K, it.m0, it.n0, ptr);
      dma_issue(a, w, ptr, (int64_t)it.kb * kDBK, lds0);
      continue;
    }
    __syncthreads();   // every wave is done with the stage buffers
    if (has_next) {    // the next item's first stage, into buffer 0, under the epilogue
      b = nb;
      it = dma_item(b, tiles_m, tiles_n, sk, nk);
      dma_setup(M, N, K, it.m0, it.n0, ptr);
      dma_issue(a, w, ptr, (int64_t)it.kb * kDBK, lds0);
    }

    // epilogue: (acc * (dA[m] * dW[n]) + bias) -> GELU -> bf16, the
    // operations of gemm_fp8_kernel's epilogue in the same order.  Fully
    // unrolled over 256 accumulators per lane this would be more code than
    // the instruction cache holds, so each wave moves 32 rows of its
    // accumulators at a time into its own 16 KB of buffer 1 (fp32, 16-byte
    // chunks of a 512-byte row permuted by XOR with the row) and a short loop
    // takes them back 4 columns per lane.
    const int le = opaque_lane(), re = le & 31, he = le >> 5;
    float* st = reinterpret_cast<float*>(lds1 + wave * 16384);
    const bool vec = cur.m0 + kDBM <= M && cur.n0 + kDBN <= N && N % 4 == 0 &&
                     (reinterpret_cast<uintptr_t>(y) & 7) == 0;
    const int cq = wn * kDWN + re * 4;                      // this lane's 4 columns on read-back
    const f32x4 cs = *reinterpret_cast<const f32x4*>(col_scale + cq);
    const f32x4 bv = *reinterpret_cast<const f32x4*>(col_bias + cq);
#pragma unroll
    for (int i = 0; i < kDTM; ++i) {
#pragma unroll
      for (int j = 0; j < kDTN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = j * 8 + g * 2 + he;
          *reinterpret_cast<f32x4*>(st + re * 128 + ((c ^ re) << 2)) =
              f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);                     // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
      const int rl0 = wm * kDWM + i * 32;
      if (epi == 1)
        fp8_slice_out<1>(st, row_scale + rl0, cs, bv, cur.m0 + rl0, cur.n0 + cq, M, N, vec, y, le);
      else
        fp8_slice_out<0>(st, row_scale + rl0, cs, bv, cur.m0 + rl0, cur.n0 + cq, M, N, vec, y, le);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_wave_barrier();
    }
    if (!has_next) break;
    // every wave is done with the staging and the row and column arrays
    // before the next item's second stage refills buffer 1 and its scales
    // are written
    asm volatile("s_barrier" ::: "memory");
  }
}

// Sums the slices of the tail tiles in split order and applies the epilogue
// of the whole tiles (same operations, same order).  Slices are in the
// accumulator order of gemm_fp8_dma_kernel; thread q of a tile takes float4 q
// (4 consecutive columns of one row), so every slice is read contiguously.  A
// thread issues the loads of up to 8 slices before it adds them (in split
// order), with one workgroup per 256 float4 of a tile, and interior rows
// store their 4 outputs at once.
constexpr int kFp8ReduceWgs = 64;             // workgroups per tail tile

__global__ __launch_bounds__(256) void fp8_split_reduce_kernel(
    const float* __restrict__ part, int64_t main_tiles, int ways, const float* __restrict__ da,
    const float* __restrict__ dw, const uint16_t* __restrict__ bias, int64_t M, int64_t N, int epi,
    uint16_t* __restrict__ y) {
  constexpr int kQuads = kDBM * kDBN / 4;       // float4 per slice
  constexpr int kPerWg = kQuads / kFp8ReduceWgs;
  static_assert(kPerWg % 256 == 0, "whole rounds of the workgroup's threads");
  const int64_t tail = blockIdx.x / kFp8ReduceWgs;
  const int64_t tiles_m = (M + kDBM - 1) / kDBM, tiles_n = (N + kDBN - 1) / kDBN;
  int64_t tm, tn;
  grouped_tile(main_tiles + tail, tiles_m, tiles_n, tm, tn);
  const f32x4* slices = reinterpret_cast<const f32x4*>(part) + tail * ways * (int64_t)kQuads;
  const bool vec = N % 4 == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0;
  for (int q = (int)(blockIdx.x % kFp8ReduceWgs) * kPerWg + threadIdx.x;
       q < (int)(blockIdx.x % kFp8ReduceWgs + 1) * kPerWg; q += 256) {
    // q = (((wave * 4 + i) * 4 + j) * 64 + lane) * 4 + g
    const int g = q & 3, lane = (q >> 2) & 63, j = (q >> 8) & 3, i = (q >> 10) & 3, wave = q >> 12;
    const int rl = (wave >> 1) * kDWM + i * 32 + (lane & 31);
    const int cl = (wave & 1) * kDWN + j * 32 + g * 8 + (lane >> 5) * 4;
    const int64_t row = tm * kDBM + rl, col = tn * kDBN + cl;
    if (row >= M) continue;
    f32x4 sum = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < ways; s0 += 8) {
      f32x4 p[8];
#pragma unroll
      for (int s = 0; s < 8; ++s)
        if (s0 + s < ways) p[s] = slices[(s0 + s) * (int64_t)kQuads + q];
#pragma unroll
      for (int s = 0; s < 8; ++s)
        if (s0 + s < ways) sum += p[s];
    }
    const float rs = da[row];
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool ok = col + k < N;
      const float cs = ok ? dw[col + k] : 0.0f;
      const float bv = (bias && ok) ? bf16_bits_to_f32(bias[col + k]) : 0.0f;
      v[k] = __builtin_fmaf(sum[k], rs * cs, bv);
      if (epi == 1) v[k] = gelu_erf(v[k]);
    }
    const uint32_t p01 = bf16x2_rne(v[0], v[1]), p23 = bf16x2_rne(v[2], v[3]);
    uint16_t* dst = y + row * N + col;
    if (vec && col + 3 < N) {
      *reinterpret_cast<u32x2*>(dst) = u32x2{p01, p23};
    } else {
      const uint16_t hv[4] = {(uint16_t)p01, (uint16_t)(p01 >> 16), (uint16_t)p23,
                              (uint16_t)(p23 >> 16)};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (col + k < N) dst[k] = hv[k];
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

namespace {

// The direct-to-LDS kernel needs K % 128 == 0, 16-byte aligned code rows and
// operands below 4 GiB; NVFP4_FP8_GEMM_KERNEL=reg pins the register-staged
// kernel (testing).
bool use_fp8_dma(int64_t M, int64_t N, int64_t K, uintptr_t align_bits) {
  if (const char* f = getenv("NVFP4_FP8_GEMM_KERNEL"))
    if (!strcmp(f, "reg")) return false;
  const int64_t limit = (int64_t)1 << 32;   // 32-bit source offsets
  return K % kDBK == 0 && (align_bits & 15) == 0 && M * K < limit && N * K < limit;
}

struct Fp8SplitPlan {
  int64_t tiles = 0, main_tiles = 0, tail = 0;
  int ways = 1;
  size_t bytes = 0;
};

// Tail split for the direct-to-LDS kernel: the tiles past the last whole
// round over the compute units are split into `ways` K ranges of at least
// kFp8MinSplitStages stages, as many as fill the round, at most kFp8MaxWays
// (each way adds a slice of partial sums to write and read back).  Below
// kFp8MinWays the partial-sum traffic costs about what the split saves
// (measured on the DiT up projection: 96 tail tiles, 2 ways), so the tail is
// computed whole.  NVFP4_FP8_GEMM_SPLIT=n forces n ways on the tail (testing).
constexpr int kFp8MinSplitStages = 4;
constexpr int kFp8MinWays = 3;
constexpr int kFp8MaxWays = 8;

Fp8SplitPlan plan_fp8_split(int64_t M, int64_t N, int64_t K) {
  Fp8SplitPlan p;
  p.tiles = p.main_tiles = ((M + kDBM - 1) / kDBM) * ((N + kDBN - 1) / kDBN);
  if (p.tiles == 0 || K % kDBK != 0) return p;
  const int cus = compute_units();
  const int64_t nk = K / kDBK;
  const int64_t tail = p.tiles % cus;
  if (tail == 0) return p;
  int64_t ways = std::min<int64_t>(std::min<int64_t>(cus / tail, nk / kFp8MinSplitStages),
                                   kFp8MaxWays);
  if (ways < kFp8MinWays) ways = 1;
  if (const char* f = getenv("NVFP4_FP8_GEMM_SPLIT")) ways = std::min<int64_t>(atoi(f), nk);
  if (ways < 2) return p;
  p.tail = tail;
  p.main_tiles = p.tiles - tail;
  p.ways = (int)ways;
  p.bytes = (size_t)tail * ways * kDBM * kDBN * sizeof(float);
  return p;
}

}  // namespace

size_t gemm_fp8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || !use_fp8_dma(M, N, K, 0)) return 0;
  return plan_fp8_split(M, N, K).bytes;
}

hipError_t launch_gemm_fp8(const uint8_t* a_codes, const float* a_scales, const uint8_t* w_codes,
                           const float* w_scales, const void* bias, int64_t M, int64_t N,
                           int64_t K, int epilogue, void* y, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const uintptr_t al = reinterpret_cast<uintptr_t>(a_codes) | reinterpret_cast<uintptr_t>(w_codes);
  if (use_fp8_dma(M, N, K, al)) {
    const Fp8SplitPlan plan = plan_fp8_split(M, N, K);
    const bool split = plan.ways > 1 && workspace && workspace_bytes >= plan.bytes;
    const SplitK sk = split ? SplitK{static_cast<float*>(workspace), plan.main_tiles, plan.ways}
                            : SplitK{nullptr, plan.tiles, 1};
    const int64_t items = split ? plan.main_tiles + plan.tail * plan.ways : plan.tiles;
    // persistent grid, one workgroup per compute unit, when there are more
    // items than compute units and the units divide into whole XCD groups
    // (NVFP4_GEMM_PERSISTENT=0: one item per workgroup)
    const int cus = compute_units();
    const char* pe = getenv("NVFP4_GEMM_PERSISTENT");
    const bool persistent = items > cus && cus % kXcds == 0 && !(pe && strcmp(pe, "0") == 0);
    const int64_t grid = persistent ? cus : items;
    const uint16_t* b16 = reinterpret_cast<const uint16_t*>(bias);
    uint16_t* y16 = reinterpret_cast<uint16_t*>(y);
    hipLaunchKernelGGL(gemm_fp8_dma_kernel, dim3((unsigned)grid), dim3(kDNT), 0, stream, a_codes,
                       a_scales, w_codes, w_scales, b16, M, N, K, epilogue, y16, sk, items);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !split) return e;
    hipLaunchKernelGGL(fp8_split_reduce_kernel, dim3((unsigned)(plan.tail * kFp8ReduceWgs)),
                       dim3(256), 0, stream, static_cast<const float*>(workspace), plan.main_tiles,
                       plan.ways, a_scales, w_scales, b16, M, N, epilogue, y16);
    return hipGetLastError();
  }
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  hipLaunchKernelGGL(gemm_fp8_kernel, dim3((unsigned)tiles), dim3(kNT), 0, stream, a_codes, a_scales,
                     w_codes, w_scales, reinterpret_cast<const uint16_t*>(bias), M, N, K, epilogue,
                     reinterpret_cast<uint16_t*>(y), (al & 15) == 0 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace nvfp4
