// Block-scaled W4A4 NVFP4 GEMM for gfx950.
//
// The DiT linear layers run an NVFP4 GEMM on NVFP4 weights and dynamically
// quantized NVFP4 activations ("NVIDIA介绍用TensorRT LLM VisualGen加速Blackwell
// 上的FLUX 3 Image Klein", sns.style, time-breakdown paragraph; "NVIDIA
// показала, как сократить генерацию FLUX 3 Image Klein с 22 до 6 секунд",
// xalabuda.com, section "Квантование NVFP4 и оптимизация вычислительных ядер"):
//
//   Y[m,n] = bf16( epi( sA*sW * sum_k Ahat[m,k]*What[n,k] + bias[n] ) )
//
// Exact decode.  value(E2M1) * E4M3 has at most 6 significant bits and lies
// in [2^-10, 2688]: it is exact in fp16.  Each wave decodes its own operand
// fragments in registers -- the gfx950 packed E2M1->fp16 conversion (scale 1.0,
// which it applies as an exponent only) and one packed fp16 multiply by the
// block scale -- and feeds v_mfma_f32_32x32x16_f16, so the products are exact
// and only the fp32 accumulation rounds.  The per-tensor scales are applied
// once in the epilogue.
//
// Layout of the work:
//   * workgroup = 4 waves in 2x2, output tile BM x BN, each wave BM/2 x BN/2
//     (4x4 MFMA 32x32 tiles at 256x256 -> 256 fp32 accumulators per lane);
//   * K advances 128 elements (8 blocks) per step; LDS holds the packed codes
//     (64 B per row and step, rows padded to 80 B) and the block scales already
//     turned into fp16 pairs (32 B per row, padded to 40 B), double-buffered,
//     with the next step's global loads held in registers meanwhile;
//   * K is permuted inside a step, identically for A and W: lanes 0-31 of a
//     wave take elements 0-63 of the step, lanes 32-63 elements 64-127, so a
//     lane's codes for the whole step are 32 contiguous bytes of its row (two
//     128-bit LDS reads) and each lane's 8 elements of one MFMA share a scale.
//     The MFMA sums over whichever 16 k's it is given; A and W agree on them.
//   * the tile order is renumbered so each XCD (workgroups are dealt to the 8
//     XCDs round-robin) walks a contiguous, row-grouped range of tiles and
//     reuses A and W panels in its own L2.
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "device_common.hpp"
#include "gemm_v5.hpp"
#include "kernels.hpp"

namespace nvfp4 {
namespace {

constexpr int kBK = 128;               // K elements per step
constexpr int kCodePitch = 80;         // LDS bytes per row of codes (64 used)
constexpr int kScalePitch = 20;        // LDS bytes per row of fp16 scales (16 used)

// Tile shape BM x BN, WGM x WGN waves (each owns a WM x WN sub-tile of 32x32
// MFMA tiles), MINB workgroups per CU requested from the register allocator.
template <int BM_, int BN_, int WGM_, int WGN_, int MINB_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, MINB = MINB_;
  static constexpr int NT = 64 * WGM * WGN;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int A_CODES = 0;
  static constexpr int B_CODES = A_CODES + BM * kCodePitch;
  static constexpr int A_SC = B_CODES + BN * kCodePitch;
  static constexpr int B_SC = A_SC + BM * kScalePitch;
  static constexpr int STAGE = B_SC + BN * kScalePitch;
  static constexpr int A_CHUNKS = BM * 4 / NT;   // 16-byte code chunks per thread
  static constexpr int B_CHUNKS = BN * 4 / NT;
  static_assert(BM * 4 % NT == 0 && BN * 4 % NT == 0, "loader split");
  static_assert(BM <= NT && BN <= NT, "one scale row per thread");
  static_assert(TM >= 1 && TN >= 1, "wave tile");
};

struct Operand {
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t rows;
};

template <class C>
struct Staged {
  u32x4 a[C::A_CHUNKS];
  u32x4 b[C::B_CHUNKS];
  u32x2 sa, sb;
};

// 16 bytes of codes = 2 blocks of row `row`, starting at block `kb`.
__device__ __forceinline__ u32x4 load_code_chunk(const Operand& op, int64_t row, int64_t kb,
                                                 int64_t kblocks, bool vec16) {
  if (row >= op.rows || kb >= kblocks) return u32x4{0u, 0u, 0u, 0u};
  const uint8_t* p = op.codes + row * (kblocks * 8) + kb * 8;
  if (kb + 2 <= kblocks) {
    if (vec16) return *reinterpret_cast<const u32x4*>(p);
    const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 8);
    return u32x4{lo.x, lo.y, hi.x, hi.y};
  }
  const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
  return u32x4{lo.x, lo.y, 0u, 0u};
}

// The 8 scale bytes of row `row` for blocks kb .. kb+7 (zero past the end).
__device__ __forceinline__ u32x2 load_scale8(const Operand& op, int64_t row, int64_t kb,
                                             int64_t kblocks, bool vec8) {
  if (row >= op.rows) return u32x2{0u, 0u};
  const uint8_t* p = op.scales + row * kblocks + kb;
  if (vec8 && kb + 8 <= kblocks) return *reinterpret_cast<const u32x2*>(p);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (kb + i < kblocks) w[i >> 2] |= (uint32_t)p[i] << (8 * (i & 3));
  return u32x2{w[0], w[1]};
}

// Global -> registers for K step kt.  kEdge: rows or K may run past the end
// (zero fill, narrow loads); otherwise every access is a full 16 / 8-byte load.
template <class C, bool kEdge>
__device__ __forceinline__ void load_stage(const Operand& A, const Operand& W, int64_t m0,
                                           int64_t n0, int kt, int64_t kblocks, bool vec16,
                                           bool vec8, Staged<C>& s) {
  using T = C;
  constexpr int BM = C::BM, BN = C::BN;
  const int64_t kb0 = (int64_t)kt * (kBK / 16);
#pragma unroll
  for (int i = 0; i < T::A_CHUNKS; ++i) {
    const int q = threadIdx.x + i * C::NT;
    if constexpr (kEdge)
      s.a[i] = load_code_chunk(A, m0 + (q >> 2), kb0 + (q & 3) * 2, kblocks, vec16);
    else
      s.a[i] = *reinterpret_cast<const u32x4*>(A.codes + (m0 + (q >> 2)) * (kblocks * 8) +
                                               (kb0 + (q & 3) * 2) * 8);
  }
#pragma unroll
  for (int i = 0; i < T::B_CHUNKS; ++i) {
    const int q = threadIdx.x + i * C::NT;
    if constexpr (kEdge)
      s.b[i] = load_code_chunk(W, n0 + (q >> 2), kb0 + (q & 3) * 2, kblocks, vec16);
    else
      s.b[i] = *reinterpret_cast<const u32x4*>(W.codes + (n0 + (q >> 2)) * (kblocks * 8) +
                                               (kb0 + (q & 3) * 2) * 8);
  }
  if constexpr (kEdge) {
    if (threadIdx.x < BM) s.sa = load_scale8(A, m0 + threadIdx.x, kb0, kblocks, vec8);
    if (threadIdx.x < BN) s.sb = load_scale8(W, n0 + threadIdx.x, kb0, kblocks, vec8);
  } else {
    if (threadIdx.x < BM)
      s.sa = *reinterpret_cast<const u32x2*>(A.scales + (m0 + threadIdx.x) * kblocks + kb0);
    if (threadIdx.x < BN)
      s.sb = *reinterpret_cast<const u32x2*>(W.scales + (n0 + threadIdx.x) * kblocks + kb0);
  }
}

// Eight E4M3 scale bytes -> eight fp16 (exact) in LDS, two per dword.
__device__ __forceinline__ void store_scales(u32x2 sc, uint8_t* dst) {
  uint32_t* d = reinterpret_cast<uint32_t*>(dst);
  d[0] = __builtin_bit_cast(uint32_t, e4m3_pair_to_f16x2<false>(sc.x));
  d[1] = __builtin_bit_cast(uint32_t, e4m3_pair_to_f16x2<true>(sc.x));
  d[2] = __builtin_bit_cast(uint32_t, e4m3_pair_to_f16x2<false>(sc.y));
  d[3] = __builtin_bit_cast(uint32_t, e4m3_pair_to_f16x2<true>(sc.y));
}

template <class C>
__device__ __forceinline__ void store_stage(const Staged<C>& s, uint8_t* stage) {
  using T = C;
  constexpr int BM = C::BM, BN = C::BN;
#pragma unroll
  for (int i = 0; i < T::A_CHUNKS; ++i) {
    const int q = threadIdx.x + i * C::NT;
    *reinterpret_cast<u32x4*>(stage + T::A_CODES + (q >> 2) * kCodePitch + (q & 3) * 16) = s.a[i];
  }
#pragma unroll
  for (int i = 0; i < T::B_CHUNKS; ++i) {
    const int q = threadIdx.x + i * C::NT;
    *reinterpret_cast<u32x4*>(stage + T::B_CODES + (q >> 2) * kCodePitch + (q & 3) * 16) = s.b[i];
  }
  if (threadIdx.x < BM) store_scales(s.sa, stage + T::A_SC + threadIdx.x * kScalePitch);
  if (threadIdx.x < BN) store_scales(s.sb, stage + T::B_SC + threadIdx.x * kScalePitch);
}

template <class C>
__device__ __forceinline__ void compute_stage(const uint8_t* stage,
                                              f32x16 (&acc)[C::TM][C::TN]) {
  using T = C;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    u32x4 ca[T::TM], cb[T::TN];
    f16x2 sa[T::TM], sb[T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
      const int row = wm * T::WM + i * 32 + r;
      ca[i] = *reinterpret_cast<const u32x4*>(stage + T::A_CODES + row * kCodePitch + h * 32 + half * 16);
      sa[i] = *reinterpret_cast<const f16x2*>(stage + T::A_SC + row * kScalePitch + h * 8 + half * 4);
    }
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
      const int row = wn * T::WN + j * 32 + r;
      cb[j] = *reinterpret_cast<const u32x4*>(stage + T::B_CODES + row * kCodePitch + h * 32 + half * 16);
      sb[j] = *reinterpret_cast<const f16x2*>(stage + T::B_SC + row * kScalePitch + h * 8 + half * 4);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      f16x8 av[T::TM], bv[T::TN];
#pragma unroll
      for (int i = 0; i < T::TM; ++i) {
        const uint32_t w = kk == 0 ? ca[i].x : kk == 1 ? ca[i].y : kk == 2 ? ca[i].z : ca[i].w;
        av[i] = decode8(w, kk < 2 ? sa[i].x : sa[i].y);
      }
#pragma unroll
      for (int j = 0; j < T::TN; ++j) {
        const uint32_t w = kk == 0 ? cb[j].x : kk == 1 ? cb[j].y : kk == 2 ? cb[j].z : cb[j].w;
        bv[j] = decode8(w, kk < 2 ? sb[j].x : sb[j].y);
      }
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
  }
}

template <class C, bool kEdge>
__device__ __forceinline__ void main_loop(const Operand& A, const Operand& Wt, int64_t m0,
                                          int64_t n0, int64_t K, bool vec16, bool vec8,
                                          uint8_t* lds,
                                          f32x16 (&acc)[C::TM][C::TN]) {
  using T = C;
  const int64_t kblocks = K / 16;
  const int nk = (int)((K + kBK - 1) / kBK);
  Staged<C> st;
  load_stage<C, kEdge>(A, Wt, m0, n0, 0, kblocks, vec16, vec8, st);
  store_stage<C>(st, lds);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    uint8_t* cur = lds + (kt & 1) * T::STAGE;
    uint8_t* nxt = lds + ((kt + 1) & 1) * T::STAGE;
    // Prefetch the next step unconditionally (the last step re-reads itself
    // into the idle buffer): a conditional prefetch gets sunk next to its LDS
    // stores, and every step then waits out the full memory latency.
    const int kn = kt + 1 < nk ? kt + 1 : kt;
    load_stage<C, kEdge>(A, Wt, m0, n0, kn, kblocks, vec16, vec8, st);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage<C>(cur, acc);
    __builtin_amdgcn_sched_barrier(0);
    store_stage<C>(st, nxt);
    __syncthreads();
  }
}

// Epilogue: acc * sA*sW + bias (one fused multiply-add), optional GELU, bf16
// round-to-nearest-even, optional max |bf16 y| (one atomic per workgroup),
// an integer max of the bf16 magnitudes, so a NaN output makes it non-finite.
// A lane holds, per 32x32 tile, column (lane % 32) of rows
// (e/4)*8 + (lane/32)*4 + e%4; rows e, e+1 are packed by one conversion.
template <class C>
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[C::TM][C::TN], float scale,
                                         const uint16_t* __restrict__ bias, int epi, int64_t M,
                                         int64_t N, int64_t m0, int64_t n0,
                                         uint16_t* __restrict__ y, uint32_t* __restrict__ y_amax) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int64_t r0 = m0 + wm * C::WM + (lane >> 5) * 4;
  const int64_t c0 = n0 + wn * C::WN + (lane & 31);
  const bool full = m0 + C::BM <= M && n0 + C::BN <= N && (int64_t)C::BM * N < ((int64_t)1 << 30);
  uint16_t* __restrict__ yt = y + r0 * N + c0;   // this lane's first element
  u16x2 amax = {0, 0};
#pragma unroll
  for (int j = 0; j < C::TN; ++j) {
    const int64_t col = c0 + j * 32;
    const bool col_ok = col < N;
    const float bv = (bias && col_ok) ? bf16_bits_to_f32(bias[col]) : 0.0f;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const int dr = i * 32 + (e >> 2) * 8 + (e & 3);       // row offset from r0
        float v0 = __builtin_fmaf(acc[i][j][e], scale, bv);
        float v1 = __builtin_fmaf(acc[i][j][e + 1], scale, bv);
        if (epi == 1) {
          v0 = gelu_erf(v0);
          v1 = gelu_erf(v1);
        }
        const uint32_t pk = bf16x2_rne(v0, v1);
        if (full) {
          const uint32_t off = (uint32_t)dr * (uint32_t)N + (uint32_t)(j * 32);
          yt[off] = (uint16_t)pk;
          yt[off + (uint32_t)N] = (uint16_t)(pk >> 16);
          amax = amax_bf16x2(amax, pk);
        } else if (col_ok) {
          uint32_t kept = 0;
          if (r0 + dr < M) {
            y[(r0 + dr) * N + col] = (uint16_t)pk;
            kept |= 0xFFFFu;
          }
          if (r0 + dr + 1 < M) {
            y[(r0 + dr + 1) * N + col] = (uint16_t)(pk >> 16);
            kept |= 0xFFFF0000u;
          }
          amax = amax_bf16x2(amax, pk & kept);
        }
      }
  }
  if (y_amax) {   // one atomic per workgroup
    __shared__ uint32_t wave_amax[C::NT / 64];
    uint32_t a = (uint32_t)(amax.x > amax.y ? amax.x : amax.y) << 16;
    a = wave_max_u32(a);
    if (lane == 0) wave_amax[wave] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t m = 0;
#pragma unroll
      for (int w = 0; w < C::NT / 64; ++w) m = max(m, wave_amax[w]);
      atomicMax(y_amax, m);
    }
  }
}

// NVFP4 output.  The tile's bf16 values (computed exactly as in epilogue())
// are staged row-major in LDS half a tile at a time; then each thread takes
// whole 16-element blocks of a row through quantize_block(), the quantizer's
// own routine.  Needs N % 16 == 0 and (BM/2) * (BN+8) halves of LDS.
template <class C>
__device__ __forceinline__ void epilogue_quant(const f32x16 (&acc)[C::TM][C::TN], float scale,
                                               const uint16_t* __restrict__ bias, int epi,
                                               int64_t M, int64_t N, int64_t m0, int64_t n0,
                                               const Out& out, uint8_t* lds) {
  constexpr int kHalf = C::BM / 2;
  constexpr int kPitch = C::BN + 8;      // halves per staged row (spreads the banks)
  constexpr int kBlocks = C::BN / 16;    // 16-blocks per staged row
  static_assert(kHalf % C::WM == 0, "each wave's rows lie in one half of the tile");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  uint16_t* stage = reinterpret_cast<uint16_t*>(lds);
  // tensor scales as the quantizer derives them from a given amax
  const uint32_t amax_bits = __float_as_uint(*out.amax_static) & 0x7FFFFFFFu;
  if (amax_bits >= 0x7F800000u) {                  // Inf / NaN amax: no scale exists
    if (blockIdx.x == 0 && threadIdx.x == 0) *out.tensor_scale = __uint_as_float(0x7FC00000u);
    return;
  }
  bool degenerate;
  float s_enc, s_dec;
  tensor_scales(__uint_as_float(amax_bits), degenerate, s_enc, s_dec);
  if (blockIdx.x == 0 && threadIdx.x == 0) *out.tensor_scale = s_dec;
  const int64_t code_pitch = N / 2, scale_pitch = N / 16;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((wm * C::WM) / kHalf == half) {
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int cl = wn * C::WN + j * 32 + (lane & 31);
        const int64_t col = n0 + cl;
        const float bv = (bias && col < N) ? bf16_bits_to_f32(bias[col]) : 0.0f;
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int e = 0; e < 16; e += 2) {
            const int rl = wm * C::WM + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3) - half * kHalf;
            float v0 = __builtin_fmaf(acc[i][j][e], scale, bv);
            float v1 = __builtin_fmaf(acc[i][j][e + 1], scale, bv);
            if (epi == 1) {
              v0 = gelu_erf(v0);
              v1 = gelu_erf(v1);
            }
            const uint32_t pk = bf16x2_rne(v0, v1);
            stage[rl * kPitch + cl] = (uint16_t)pk;
            stage[(rl + 1) * kPitch + cl] = (uint16_t)(pk >> 16);
          }
      }
    }
    __syncthreads();
    for (int b = threadIdx.x; b < kHalf * kBlocks; b += C::NT) {
      const int rl = b / kBlocks, cb = b % kBlocks;
      const int64_t row = m0 + half * kHalf + rl, col = n0 + cb * 16;
      if (row < M && col < N) {
        const u32x4* src = reinterpret_cast<const u32x4*>(stage + rl * kPitch + cb * 16);
        u32x2 c;
        uint32_t S;
        quantize_block(src[0], src[1], degenerate, s_enc, s_dec, c, S);
        *reinterpret_cast<u32x2*>(out.codes + row * code_pitch + col / 2) = c;
        out.scales[row * scale_pitch + col / 16] = (uint8_t)S;
      }
    }
    __syncthreads();
  }
}

template <class C>
__device__ __forceinline__ void finish_tile(const f32x16 (&acc)[C::TM][C::TN], float scale,
                                            const uint16_t* __restrict__ bias, int epi, int64_t M,
                                            int64_t N, int64_t m0, int64_t n0, const Out& out,
                                            uint8_t* lds) {
  if (out.codes)
    epilogue_quant<C>(acc, scale, bias, epi, M, N, m0, n0, out, lds);
  else
    epilogue<C>(acc, scale, bias, epi, M, N, m0, n0, out.y, out.y_amax);
}

template <class C>
__global__ __launch_bounds__(C::NT, C::MINB) void gemm_nvfp4_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ sa, const uint8_t* __restrict__ w_codes,
    const uint8_t* __restrict__ w_scales, const float* __restrict__ sw,
    const uint16_t* __restrict__ bias, int64_t M, int64_t N, int64_t K, int epi, Out out,
    int vec_flags) {
  using T = C;
  constexpr int BM = C::BM, BN = C::BN;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * T::STAGE];
  static_assert(BM / 2 * (BN + 8) * 2 <= 2 * T::STAGE, "LDS for the NVFP4 epilogue");

  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int64_t tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const bool vec16 = vec_flags & 1, vec8 = vec_flags & 2;
  const Operand A{a_codes, a_scales, M}, Wt{w_codes, w_scales, N};

  f32x16 acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j) acc[i][j] = f32x16{};

  const bool interior = m0 + BM <= M && n0 + BN <= N && K % kBK == 0 && vec16 && vec8;
  if (interior)
    main_loop<C, false>(A, Wt, m0, n0, K, vec16, vec8, lds, acc);
  else
    main_loop<C, true>(A, Wt, m0, n0, K, vec16, vec8, lds, acc);

  finish_tile<C>(acc, (*sa) * (*sw), bias, epi, M, N, m0, n0, out, lds);
}

// ---------------------------------------------------------------------------
// v2: the weight operand is decoded once per workgroup into LDS as fp16 and
// shared by every wave-row; the activation operand stays packed in LDS and is
// decoded by each wave in registers.  K advances 64 elements per step.  Same
// K permutation as above at half width: lanes 0-31 take elements 0-31 of the
// step, lanes 32-63 elements 32-63.
// ---------------------------------------------------------------------------
constexpr int kBK2 = 64;
constexpr int kACodePitch2 = 48;      // 32 B of codes per row and step
constexpr int kAScalePitch2 = 12;     // 4 fp16 block scales per row and step
constexpr int kWPitch2 = 144;         // 64 fp16 of decoded weight per row and step

template <class C>
struct Lay2 {
  static constexpr int A_CODES = 0;
  static constexpr int A_SC = A_CODES + C::BM * kACodePitch2;
  static constexpr int W_F16 = A_SC + C::BM * kAScalePitch2;
  static constexpr int STAGE = W_F16 + C::BN * kWPitch2;
  static_assert(C::BM * 2 == C::NT && C::BN * 2 == C::NT, "one 16-byte chunk of A and W per thread");
};

struct Staged2 {
  u32x4 a;        // 16 B of A codes: 2 blocks
  u32x4 w;        // 16 B of W codes: 2 blocks
  uint32_t sa;    // 4 A scale bytes (threads < BM)
  uint32_t sw;    // 2 W scale bytes for this thread's chunk
};

template <class C, bool kEdge>
__device__ __forceinline__ void load_stage2(const Operand& A, const Operand& W, int64_t m0,
                                            int64_t n0, int kt, int64_t kblocks, Staged2& s) {
  const int q = threadIdx.x;
  const int64_t kb0 = (int64_t)kt * (kBK2 / 16);
  const int64_t ra = m0 + (q >> 1), rw = n0 + (q >> 1);
  const int64_t kb = kb0 + (q & 1) * 2;
  if constexpr (kEdge) {
    s.a = load_code_chunk(A, ra, kb, kblocks, false);
    s.w = load_code_chunk(W, rw, kb, kblocks, false);
    uint32_t sa = 0, sw = 0;
    if (q < C::BM && m0 + q < A.rows) {
      const uint8_t* p = A.scales + (m0 + q) * kblocks;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (kb0 + i < kblocks) sa |= (uint32_t)p[kb0 + i] << (8 * i);
    }
    if (rw < W.rows) {
      const uint8_t* p = W.scales + rw * kblocks;
      if (kb < kblocks) sw |= p[kb];
      if (kb + 1 < kblocks) sw |= (uint32_t)p[kb + 1] << 8;
    }
    s.sa = sa;
    s.sw = sw;
  } else {
    s.a = *reinterpret_cast<const u32x4*>(A.codes + ra * (kblocks * 8) + kb * 8);
    s.w = *reinterpret_cast<const u32x4*>(W.codes + rw * (kblocks * 8) + kb * 8);
    if (q < C::BM) s.sa = *reinterpret_cast<const uint32_t*>(A.scales + (m0 + q) * kblocks + kb0);
    s.sw = *reinterpret_cast<const uint16_t*>(W.scales + rw * kblocks + kb);
  }
}

template <class C>
__device__ __forceinline__ void store_stage2(const Staged2& s, uint8_t* stage) {
  using L = Lay2<C>;
  const int q = threadIdx.x;
  const int row = q >> 1, c = q & 1;
  *reinterpret_cast<u32x4*>(stage + L::A_CODES + row * kACodePitch2 + c * 16) = s.a;
  if (q < C::BM) {
    uint32_t* d = reinterpret_cast<uint32_t*>(stage + L::A_SC + q * kAScalePitch2);
    d[0] = __builtin_bit_cast(uint32_t, e4m3_pair_to_f16x2<false>(s.sa));
    d[1] = __builtin_bit_cast(uint32_t, e4m3_pair_to_f16x2<true>(s.sa));
  }
  // decode this thread's 32 weight elements (2 blocks) to fp16
  const uint32_t sp = __builtin_bit_cast(uint32_t, e4m3_pair_to_f16x2<false>(s.sw));
  const _Float16 s0 = __builtin_bit_cast(_Float16, (uint16_t)(sp & 0xFFFFu));
  const _Float16 s1 = __builtin_bit_cast(_Float16, (uint16_t)(sp >> 16));
  u32x4* d = reinterpret_cast<u32x4*>(stage + L::W_F16 + row * kWPitch2 + c * 64);
  d[0] = __builtin_bit_cast(u32x4, decode8(s.w.x, s0));
  d[1] = __builtin_bit_cast(u32x4, decode8(s.w.y, s0));
  d[2] = __builtin_bit_cast(u32x4, decode8(s.w.z, s1));
  d[3] = __builtin_bit_cast(u32x4, decode8(s.w.w, s1));
}

// v3: v2 with the work of one K step software-pipelined inside each wave --
// the LDS reads and activation decode of MFMA step kk+1, and (in the second
// half of the step) the next stage's stores and weight decode, are issued
// between the MFMAs of step kk, so the matrix pipe runs while the vector ALU
// decodes (one wave keeps both busy).
template <class C>
__device__ __forceinline__ void store_a_stage2(const Staged2& s, uint8_t* stage) {
  using L = Lay2<C>;
  const int q = threadIdx.x;
  *reinterpret_cast<u32x4*>(stage + L::A_CODES + (q >> 1) * kACodePitch2 + (q & 1) * 16) = s.a;
  if (q < C::BM) {
    uint32_t* d = reinterpret_cast<uint32_t*>(stage + L::A_SC + q * kAScalePitch2);
    d[0] = __builtin_bit_cast(uint32_t, e4m3_pair_to_f16x2<false>(s.sa));
    d[1] = __builtin_bit_cast(uint32_t, e4m3_pair_to_f16x2<true>(s.sa));
  }
}

// Quarter `part` (0..3) of this thread's weight decode: 8 elements.
template <class C>
__device__ __forceinline__ void store_w_part2(const Staged2& s, uint8_t* stage, int part) {
  using L = Lay2<C>;
  const int q = threadIdx.x;
  const uint32_t sp = __builtin_bit_cast(uint32_t, e4m3_pair_to_f16x2<false>(s.sw));
  const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)(part < 2 ? (sp & 0xFFFFu) : (sp >> 16)));
  const uint32_t w = part == 0 ? s.w.x : part == 1 ? s.w.y : part == 2 ? s.w.z : s.w.w;
  u32x4* d = reinterpret_cast<u32x4*>(stage + L::W_F16 + (q >> 1) * kWPitch2 + (q & 1) * 64);
  d[part] = __builtin_bit_cast(u32x4, decode8(w, sc));
}

template <class C>
__device__ __forceinline__ void compute_stage3(const uint8_t* stage, const Staged2& st,
                                               uint8_t* nxt, f32x16 (&acc)[C::TM][C::TN]) {
  using L = Lay2<C>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int r = lane & 31, h = lane >> 5;
  u32x4 ca[C::TM];
  f16x2 sa[C::TM];
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int row = wm * C::WM + i * 32 + r;
    ca[i] = *reinterpret_cast<const u32x4*>(stage + L::A_CODES + row * kACodePitch2 + h * 16);
    sa[i] = *reinterpret_cast<const f16x2*>(stage + L::A_SC + row * kAScalePitch2 + h * 4);
  }
  f16x8 av[2][C::TM], bv[2][C::TN];
#pragma unroll
  for (int j = 0; j < C::TN; ++j) {
    const int row = wn * C::WN + j * 32 + r;
    bv[0][j] = *reinterpret_cast<const f16x8*>(stage + L::W_F16 + row * kWPitch2 + h * 64);
  }
#pragma unroll
  for (int i = 0; i < C::TM; ++i) av[0][i] = decode8(ca[i].x, sa[i].x);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int cur = kk & 1, nx = cur ^ 1;
    if (kk < 3) {
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int row = wn * C::WN + j * 32 + r;
        bv[nx][j] = *reinterpret_cast<const f16x8*>(stage + L::W_F16 + row * kWPitch2 + h * 64 + (kk + 1) * 16);
      }
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const uint32_t w = kk == 0 ? ca[i].y : kk == 1 ? ca[i].z : ca[i].w;
        av[nx][i] = decode8(w, kk + 1 < 2 ? sa[i].x : sa[i].y);
      }
    }
    // the next stage's data is stored in the second half of the step, giving
    // its global loads (issued at the top of the step) time to arrive
    if (kk == 2) {
      store_a_stage2<C>(st, nxt);
      store_w_part2<C>(st, nxt, 0);
      store_w_part2<C>(st, nxt, 1);
    } else if (kk == 3) {
      store_w_part2<C>(st, nxt, 2);
      store_w_part2<C>(st, nxt, 3);
    }
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[cur][i], bv[cur][j], acc[i][j], 0, 0, 0);
    // interleave: each MFMA followed by a few vector ops and LDS accesses
#pragma unroll
    for (int m = 0; m < C::TM * C::TN; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
    }
  }
}

// Stages [kb, ke) of the K loop (a stage is 64 elements of K).
template <class C, bool kEdge>
__device__ __forceinline__ void main_loop3(const Operand& A, const Operand& Wt, int64_t m0,
                                           int64_t n0, int64_t K, int kb, int ke, uint8_t* lds,
                                           f32x16 (&acc)[C::TM][C::TN]) {
  using L = Lay2<C>;
  const int64_t kblocks = K / 16;
  Staged2 st;
  load_stage2<C, kEdge>(A, Wt, m0, n0, kb, kblocks, st);
  store_stage2<C>(st, lds);
  __syncthreads();
  for (int kt = kb; kt < ke; ++kt) {
    uint8_t* cur = lds + ((kt - kb) & 1) * L::STAGE;
    uint8_t* nxt = lds + ((kt - kb + 1) & 1) * L::STAGE;
    const int kn = kt + 1 < ke ? kt + 1 : kt;
    load_stage2<C, kEdge>(A, Wt, m0, n0, kn, kblocks, st);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage3<C>(cur, st, nxt, acc);
    __syncthreads();
  }
}

// Split K for the tail.  When the tiles do not fill a whole number of rounds
// of workgroups over the compute units, the last, partial round leaves units
// idle.  Its tiles are then each split into `ways` ranges of K stages given to
// different workgroups, which store their fp32 partial sums, row-major, in
// their own slice of the workspace; a second kernel adds the slices in split
// order (the result does not depend on timing) and applies the epilogue
// (SplitK and split_coords describe the assignment).

// This workgroup's partial sums into its slice, at their tile positions (the
// accumulator layout of the epilogue).
template <class C>
__device__ __forceinline__ void store_partial(const f32x16 (&acc)[C::TM][C::TN], const SplitK& sk,
                                              int64_t tail, int split) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  float* slice = sk.part + (tail * sk.ways + split) * (int64_t)(C::BM * C::BN);
  float* base = slice + (wm * C::WM + (lane >> 5) * 4) * C::BN + wn * C::WN + (lane & 31);
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        base[(i * 32 + (e >> 2) * 8 + (e & 3)) * C::BN + j * 32] = acc[i][j][e];
}

// Sums the slices of the tail tiles in split order and applies the epilogue
// of the whole tiles (same operations, same order).  A workgroup covers
// kReduceRows rows of a tile, each thread 4 consecutive outputs of a row per
// step; the output amax is reduced in the workgroup first, so the amax word
// sees one atomic per workgroup rather than a burst of one per wave.
constexpr int kReduceRows = 64;

template <class C>
__global__ __launch_bounds__(256) void split_reduce_kernel(
    const float* __restrict__ part, int64_t main_tiles, int ways, const float* __restrict__ sa,
    const float* __restrict__ sw, const uint16_t* __restrict__ bias, int64_t M, int64_t N,
    int epi, uint16_t* __restrict__ y, uint32_t* __restrict__ y_amax) {
  constexpr int kPerTile = C::BM / kReduceRows;
  constexpr int kCols4 = C::BN / 4;              // threads per tile row
  constexpr int kRowStep = 256 / kCols4;         // rows per step
  static_assert(256 % kCols4 == 0 && kReduceRows % kRowStep == 0, "reduce layout");
  const int64_t tail = blockIdx.x / kPerTile;
  const int r0 = (int)(blockIdx.x % kPerTile) * kReduceRows + threadIdx.x / kCols4;
  const int c = (threadIdx.x % kCols4) * 4;
  const int64_t tiles_m = (M + C::BM - 1) / C::BM, tiles_n = (N + C::BN - 1) / C::BN;
  int64_t tm, tn;
  grouped_tile(main_tiles + tail, tiles_m, tiles_n, tm, tn);
  const int64_t col = tn * C::BN + c;
  const float scale = (*sa) * (*sw);
  float bv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) bv[k] = (bias && col + k < N) ? bf16_bits_to_f32(bias[col + k]) : 0.0f;
  const float* slices = part + tail * ways * (int64_t)(C::BM * C::BN);
  u16x2 amax = {0, 0};
  for (int r = r0; r < r0 + kReduceRows; r += kRowStep) {
    const int64_t row = tm * C::BM + r;
    const f32x4* src = reinterpret_cast<const f32x4*>(slices + r * C::BN + c);
    f32x4 sum = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int w = 0; w < ways; ++w) sum += src[w * (C::BM * C::BN / 4)];
    if (row >= M) continue;
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = __builtin_fmaf(sum[k], scale, bv[k]);
      if (epi == 1) v[k] = gelu_erf(v[k]);
    }
    const uint32_t p01 = bf16x2_rne(v[0], v[1]), p23 = bf16x2_rne(v[2], v[3]);
    const uint16_t h[4] = {(uint16_t)p01, (uint16_t)(p01 >> 16), (uint16_t)p23, (uint16_t)(p23 >> 16)};
    uint16_t* dst = y + row * N + col;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (col + k < N) {
        dst[k] = h[k];
        amax = max_u16x2(amax, u16x2{(unsigned short)(h[k] & 0x7FFFu), 0});
      }
  }
  if (y_amax) {
    __shared__ uint32_t wave_amax[4];
    uint32_t a = (uint32_t)(amax.x > amax.y ? amax.x : amax.y) << 16;
    a = wave_max_u32(a);
    if ((threadIdx.x & 63) == 0) wave_amax[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t m = max(max(wave_amax[0], wave_amax[1]), max(wave_amax[2], wave_amax[3]));
      atomicMax(y_amax, m);
    }
  }
}

template <class C>
__global__ __launch_bounds__(C::NT, C::MINB) void gemm_nvfp4_pipe_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ sa, const uint8_t* __restrict__ w_codes,
    const uint8_t* __restrict__ w_scales, const float* __restrict__ sw,
    const uint16_t* __restrict__ bias, int64_t M, int64_t N, int64_t K, int epi, Out out,
    int vec_flags, SplitK sk) {
  using L = Lay2<C>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * L::STAGE];
  static_assert(C::BM / 2 * (C::BN + 8) * 2 <= 2 * L::STAGE, "LDS for the NVFP4 epilogue");
  const int64_t tiles_m = (M + C::BM - 1) / C::BM, tiles_n = (N + C::BN - 1) / C::BN;
  int64_t tm, tn, tail;
  int split;
  split_coords(tiles_m, tiles_n, sk, tm, tn, tail, split);
  const int64_t m0 = tm * C::BM, n0 = tn * C::BN;
  const Operand A{a_codes, a_scales, M}, Wt{w_codes, w_scales, N};
  const int nk = (int)((K + kBK2 - 1) / kBK2);
  const int kb = split < 0 ? 0 : (int)((int64_t)split * nk / sk.ways);
  const int ke = split < 0 ? nk : (int)((int64_t)(split + 1) * nk / sk.ways);
  f32x16 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = f32x16{};
  const bool interior = m0 + C::BM <= M && n0 + C::BN <= N && K % kBK2 == 0 && (vec_flags & 4);
  if (interior)
    main_loop3<C, false>(A, Wt, m0, n0, K, kb, ke, lds, acc);
  else
    main_loop3<C, true>(A, Wt, m0, n0, K, kb, ke, lds, acc);
  if (split >= 0) {
    store_partial<C>(acc, sk, tail, split);
    return;
  }
  finish_tile<C>(acc, (*sa) * (*sw), bias, epi, M, N, m0, n0, out, lds);
}

// Sums the slices of v5's tail tiles in split order and applies v5's epilogue
// (same operations, same order).  Slices are in v5's accumulator order;
// thread q of a tile takes float4 q (4 consecutive columns of one row), so
// every slice is read contiguously.  A thread issues the loads of up to 8
// slices before it adds them (in split order), and one workgroup per 256
// float4 of a tile gives the loads enough threads to cover their latency.
// The output amax is reduced in the workgroup first: one atomic per
// workgroup.
constexpr int kV5ReduceWgs = 64;            // workgroups per tail tile

__global__ __launch_bounds__(256) void v5_split_reduce_kernel(
    const float* __restrict__ part, int64_t main_tiles, int ways, const float* __restrict__ sa,
    const float* __restrict__ sw, const uint16_t* __restrict__ bias, int64_t M, int64_t N,
    int epi, uint16_t* __restrict__ y, uint32_t* __restrict__ y_amax) {
  constexpr int kQuads = kVBM * kVBN / 4;
  constexpr int kPerWg = kQuads / kV5ReduceWgs;
  static_assert(kPerWg % 256 == 0, "whole rounds of the workgroup's threads");
  const int64_t tail = blockIdx.x / kV5ReduceWgs;
  const int64_t tiles_m = (M + kVBM - 1) / kVBM, tiles_n = (N + kVBN - 1) / kVBN;
  int64_t tm, tn;
  grouped_tile(main_tiles + tail, tiles_m, tiles_n, tm, tn);
  const float scale = (*sa) * (*sw);
  const f32x4* slices = reinterpret_cast<const f32x4*>(part) + tail * ways * (int64_t)kQuads;
  const bool vec = N % 4 == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0;
  u16x2 amax = {0, 0};
  for (int q = (int)(blockIdx.x % kV5ReduceWgs) * kPerWg + threadIdx.x;
       q < (int)(blockIdx.x % kV5ReduceWgs + 1) * kPerWg; q += 256) {
    // q = (((wave * 4 + i) * 4 + j) * 64 + lane) * 4 + g
    const int g = q & 3, lane = (q >> 2) & 63, j = (q >> 8) & 3, i = (q >> 10) & 3, wave = q >> 12;
    const int rl = (wave >> 1) * kVWM + i * 32 + (lane & 31);
    const int cl = (wave & 1) * kVWN + j * 32 + g * 8 + (lane >> 5) * 4;
    const int64_t row = tm * kVBM + rl, col = tn * kVBN + cl;
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
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float bv = (bias && col + k < N) ? bf16_bits_to_f32(bias[col + k]) : 0.0f;
      v[k] = __builtin_fmaf(sum[k], scale, bv);
      if (epi == 1) v[k] = gelu_erf(v[k]);
    }
    const uint32_t p01 = bf16x2_rne(v[0], v[1]), p23 = bf16x2_rne(v[2], v[3]);
    uint16_t* dst = y + row * N + col;
    if (vec && col + 3 < N) {
      *reinterpret_cast<u32x2*>(dst) = u32x2{p01, p23};
      amax = amax_bf16x2(amax_bf16x2(amax, p01), p23);
    } else {
      const uint16_t hv[4] = {(uint16_t)p01, (uint16_t)(p01 >> 16), (uint16_t)p23,
                              (uint16_t)(p23 >> 16)};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (col + k < N) {
          dst[k] = hv[k];
          amax = max_u16x2(amax, u16x2{(unsigned short)(hv[k] & 0x7FFFu), 0});
        }
    }
  }
  if (y_amax) {
    __shared__ uint32_t wave_amax[4];
    uint32_t a = (uint32_t)(amax.x > amax.y ? amax.x : amax.y) << 16;
    a = wave_max_u32(a);
    if ((threadIdx.x & 63) == 0) wave_amax[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t m = max(max(wave_amax[0], wave_amax[1]), max(wave_amax[2], wave_amax[3]));
      atomicMax(y_amax, m);
    }
  }
}

__global__ void zero_word_kernel(uint32_t* p) { *p = 0u; }

template <class C>
hipError_t launch_tile(const uint8_t* a_codes, const uint8_t* a_scales, const float* sa,
                       const uint8_t* w_codes, const uint8_t* w_scales, const float* sw,
                       const void* bias, int64_t M, int64_t N, int64_t K, int epi,
                       const Out& out, hipStream_t stream) {
  const int64_t tiles = ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  const uintptr_t align_bits = reinterpret_cast<uintptr_t>(a_codes) | reinterpret_cast<uintptr_t>(w_codes);
  const bool vec16 = (K % 32 == 0) && (align_bits & 15) == 0;
  const uintptr_t salign = reinterpret_cast<uintptr_t>(a_scales) | reinterpret_cast<uintptr_t>(w_scales);
  const bool vec8 = ((K / 16) % 8 == 0) && (salign & 7) == 0;
  hipLaunchKernelGGL((gemm_nvfp4_kernel<C>), dim3((unsigned)tiles), dim3(C::NT), 0, stream,
                     a_codes, a_scales, sa, w_codes, w_scales, sw,
                     reinterpret_cast<const uint16_t*>(bias), M, N, K, epi, out,
                     (vec16 ? 1 : 0) | (vec8 ? 2 : 0));
  return hipGetLastError();
}

using CfgPipe = Cfg<256, 256, 4, 2, 1>;    // 8 waves of 64x128 (v3)
using CfgSmall = Cfg<128, 128, 2, 2, 2>;   // 4 waves of 64x64, 2 workgroups per CU (v1)
using CfgTiny = Cfg<64, 64, 2, 2, 2>;      // 4 waves of 32x32 (v1), for few-tile problems

// DiT-sized problems run v5 (K % 256 == 0, aligned buffers) or v3 on 256x256
// tiles; small ones v1 on 128x128 tiles, two workgroups per CU, or on 64x64
// tiles when 128x128 ones would leave more than half the compute units idle.
// NVFP4_GEMM_KERNEL=tiny|small|pipe|v5 pins one (testing; v5 only where it
// applies).
bool use_pipe(int64_t M, int64_t N, int64_t K) {
  if (const char* f = getenv("NVFP4_GEMM_KERNEL")) {
    if (!strcmp(f, "pipe") || !strcmp(f, "v5")) return true;
    if (!strcmp(f, "small") || !strcmp(f, "tiny")) return false;
  }
  // a long K favours the 256x256 kernels and their K split even when the
  // output is small (2112 x 3072 x 12288: 171 us against 240 on 128x128 tiles)
  return M * N > (int64_t)256 * 256 * 128 || K >= 8192;
}

bool use_tiny(int64_t M, int64_t N) {
  if (const char* f = getenv("NVFP4_GEMM_KERNEL")) {
    if (!strcmp(f, "tiny")) return true;
    if (!strcmp(f, "small")) return false;
  }
  const int64_t tiles128 = ((M + 127) / 128) * ((N + 127) / 128);
  return 2 * tiles128 < compute_units();
}

// v5 needs K % 256 == 0 (an even number of stages; scale rows of a multiple
// of 16 bytes), 16-byte aligned code and scale buffers and code bytes below
// 4 GiB per operand (32-bit source offsets).
bool v5_applies(int64_t M, int64_t N, int64_t K, uintptr_t code_bits, uintptr_t scale_bits) {
  if (const char* f = getenv("NVFP4_GEMM_KERNEL"))
    if (!strcmp(f, "pipe") || !strcmp(f, "small")) return false;
  const int64_t limit = (int64_t)1 << 32;
  return K % (2 * kVBK) == 0 && (code_bits & 15) == 0 && (scale_bits & 15) == 0 &&
         M * (K / 2) < limit && N * (K / 2) < limit;
}

struct SplitPlan {
  int64_t tiles = 0;        // all tiles
  int64_t main_tiles = 0;   // tiles computed whole
  int64_t tail = 0;         // tiles split over K
  int ways = 1;
  size_t bytes = 0;         // workspace needed
};

// Tail split for the v3 kernel: the tiles past the last whole round of
// workgroups over the compute units are split into `ways` K ranges of at least
// 4 stages, as many as fill the round.  Below 4 ways the partial-sum traffic
// and the reduce kernel cost about what the split saves (measured on the DiT
// up projection: 96 tail tiles, 2 ways), so the tail is computed whole.
// NVFP4_GEMM_SPLIT=n forces n ways on the tail (testing).
SplitPlan plan_split(int64_t M, int64_t N, int64_t K) {
  using C = CfgPipe;
  SplitPlan p;
  p.tiles = p.main_tiles = ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  if (p.tiles == 0) return p;
  const int cus = compute_units();
  const int64_t nk = (K + kBK2 - 1) / kBK2;
  const int64_t tail = p.tiles % cus;
  if (tail == 0) return p;
  int64_t ways = std::min<int64_t>(cus / tail, nk / 4);
  if (ways < 4) ways = 1;
  if (const char* f = getenv("NVFP4_GEMM_SPLIT")) ways = std::min<int64_t>(atoi(f), nk);
  if (ways < 2) return p;
  p.tail = tail;
  p.main_tiles = p.tiles - tail;
  p.ways = (int)ways;
  p.bytes = (size_t)tail * ways * C::BM * C::BN * sizeof(float);
  return p;
}

hipError_t launch_pipe(const uint8_t* a_codes, const uint8_t* a_scales, const float* sa,
                       const uint8_t* w_codes, const uint8_t* w_scales, const float* sw,
                       const void* bias, int64_t M, int64_t N, int64_t K, int epi,
                       const Out& out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  using C = CfgPipe;
  const uintptr_t cal = reinterpret_cast<uintptr_t>(a_codes) | reinterpret_cast<uintptr_t>(w_codes);
  const uintptr_t sal = reinterpret_cast<uintptr_t>(a_scales) | reinterpret_cast<uintptr_t>(w_scales);
  // interior fast path: 16-byte code rows, 4-byte scale rows
  const bool vec = (K % 64 == 0) && (cal & 15) == 0 && (sal & 3) == 0;
  const SplitPlan plan = plan_split(M, N, K);
  // (NVFP4 output is written by whole tiles only)
  const bool split = plan.ways > 1 && workspace && workspace_bytes >= plan.bytes && !out.codes;
  const SplitK sk = split ? SplitK{static_cast<float*>(workspace), plan.main_tiles, plan.ways}
                          : SplitK{nullptr, plan.tiles, 1};
  const int64_t grid = split ? plan.main_tiles + plan.tail * plan.ways : plan.tiles;
  hipLaunchKernelGGL((gemm_nvfp4_pipe_kernel<C>), dim3((unsigned)grid), dim3(C::NT), 0, stream,
                     a_codes, a_scales, sa, w_codes, w_scales, sw,
                     reinterpret_cast<const uint16_t*>(bias), M, N, K, epi, out, vec ? 4 : 0,
                     sk);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  hipLaunchKernelGGL((split_reduce_kernel<C>), dim3((unsigned)(plan.tail * (C::BM / kReduceRows))),
                     dim3(256), 0, stream, static_cast<const float*>(workspace), plan.main_tiles,
                     plan.ways, sa, sw, reinterpret_cast<const uint16_t*>(bias), M, N, epi, out.y,
                     out.y_amax);
  return hipGetLastError();
}

// Tail split for v5: as plan_split, with stages of 128 K, at least 3 and at
// most 8 ways (each way adds a slice of partial sums to write and read back;
// the DiT up projection's 96 tail tiles would split only 2 ways, which
// measured slower than computing them whole).
// Ways for a grid whose tiles are all tail tiles (fewer tiles than compute
// units): minimise, in stage times, the rounds over the compute units times
// the stages per split, plus the split's cost -- each fp32 partial tile
// (256 KB written and read back, about 0.2 us) and the reduce launch (about
// 5 us), at about 2.9 us per stage.  A K-heavy grid of 108 tiles (2112 x 3072
// x 12288) splits 2 ways; grids whose second round would be mostly idle, or
// whose K is short, stay whole.
int64_t all_tail_ways(int64_t tiles, int64_t nk, int cus) {
  int64_t best = 1;
  double best_cost = (double)nk;
  for (int64_t w = 2; w <= 8 && w <= nk; ++w) {
    const int64_t rounds = (tiles * w + cus - 1) / cus;
    const double cost = (double)(rounds * ((nk + w - 1) / w)) + ((double)(tiles * w) * 0.2 + 5.0) / 2.9;
    if (cost < best_cost) {
      best_cost = cost;
      best = w;
    }
  }
  return best;
}

SplitPlan plan_split_v5(int64_t M, int64_t N, int64_t K) {
  SplitPlan p;
  p.tiles = p.main_tiles = ((M + kVBM - 1) / kVBM) * ((N + kVBN - 1) / kVBN);
  if (p.tiles == 0 || K % kVBK != 0) return p;
  const int cus = compute_units();
  const int64_t nk = K / kVBK;
  const int64_t tail = p.tiles % cus;
  if (tail == 0) return p;
  int64_t ways = std::min<int64_t>(std::min<int64_t>(cus / tail, nk / 4), 8);
  if (ways < 3) ways = 1;
  if (p.tiles < cus) ways = all_tail_ways(p.tiles, nk, cus);
  if (const char* f = getenv("NVFP4_GEMM_SPLIT")) ways = std::min<int64_t>(atoi(f), nk);
  if (ways < 2) return p;
  p.tail = tail;
  p.main_tiles = p.tiles - tail;
  p.ways = (int)ways;
  p.bytes = (size_t)tail * ways * kVBM * kVBN * sizeof(float);
  return p;
}

hipError_t launch_v5(const uint8_t* a_codes, const uint8_t* a_scales, const float* sa,
                     const uint8_t* w_codes, const uint8_t* w_scales, const float* sw,
                     const void* bias, int64_t M, int64_t N, int64_t K, int epi, const Out& out,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const SplitPlan plan = plan_split_v5(M, N, K);
  const bool split = plan.ways > 1 && workspace && workspace_bytes >= plan.bytes;
  const SplitK sk = split ? SplitK{static_cast<float*>(workspace), plan.main_tiles, plan.ways}
                          : SplitK{nullptr, plan.tiles, 1};
  const int64_t items = split ? plan.main_tiles + plan.tail * plan.ways : plan.tiles;
  const uint16_t* b16 = reinterpret_cast<const uint16_t*>(bias);
  // persistent grid, one workgroup per compute unit, when there are more
  // items than compute units and the units divide into whole XCD groups
  // (NVFP4_GEMM_PERSISTENT=0: one item per workgroup)
  const int cus = compute_units();
  const char* pe = getenv("NVFP4_GEMM_PERSISTENT");
  const bool no_persist = pe && strcmp(pe, "0") == 0;
  if (out.codes) {   // NVFP4 output: whole tiles
    const bool persistent = plan.tiles > cus && cus % kXcds == 0 && !no_persist;
    return launch_v5_quant(a_codes, a_scales, sa, w_codes, w_scales, sw, b16, M, N, K, epi, out,
                           plan.tiles, persistent ? cus : plan.tiles, stream);
  }
  const bool persistent = items > cus && cus % kXcds == 0 && !no_persist;
  const int64_t grid = persistent ? cus : items;
  hipLaunchKernelGGL(gemm_nvfp4_v5_kernel<false>, dim3((unsigned)grid), dim3(kVNT), 0, stream, a_codes,
                     a_scales, sa, w_codes, w_scales, sw, b16, M, N, K, epi, out, sk, items);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  hipLaunchKernelGGL(v5_split_reduce_kernel, dim3((unsigned)(plan.tail * kV5ReduceWgs)), dim3(256), 0,
                     stream, static_cast<const float*>(workspace), plan.main_tiles, plan.ways, sa, sw,
                     b16, M, N, epi, out.y, out.y_amax);
  return hipGetLastError();
}

}  // namespace

int compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

size_t gemm_nvfp4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || !use_pipe(M, N, K)) return 0;
  // the plan of the kernel that runs with aligned operands
  return v5_applies(M, N, K, 0, 0) ? plan_split_v5(M, N, K).bytes : plan_split(M, N, K).bytes;
}

namespace {

hipError_t launch_any(const uint8_t* a_codes, const uint8_t* a_scales, const float* sa,
                      const uint8_t* w_codes, const uint8_t* w_scales, const float* sw,
                      const void* bias, int64_t M, int64_t N, int64_t K, int epilogue,
                      const Out& out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  if (out.y_amax) {
    hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(1), 0, stream, out.y_amax);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (M == 0 || N == 0) return hipSuccess;
  const uintptr_t code_bits = reinterpret_cast<uintptr_t>(a_codes) | reinterpret_cast<uintptr_t>(w_codes);
  const uintptr_t scale_bits = reinterpret_cast<uintptr_t>(a_scales) | reinterpret_cast<uintptr_t>(w_scales);
  if (use_pipe(M, N, K) && v5_applies(M, N, K, code_bits, scale_bits))
    return launch_v5(a_codes, a_scales, sa, w_codes, w_scales, sw, bias, M, N, K, epilogue, out,
                     workspace, workspace_bytes, stream);
  if (use_pipe(M, N, K))
    return launch_pipe(a_codes, a_scales, sa, w_codes, w_scales, sw, bias, M, N, K, epilogue, out,
                       workspace, workspace_bytes, stream);
  if (use_tiny(M, N))
    return launch_tile<CfgTiny>(a_codes, a_scales, sa, w_codes, w_scales, sw, bias, M, N, K,
                                epilogue, out, stream);
  return launch_tile<CfgSmall>(a_codes, a_scales, sa, w_codes, w_scales, sw, bias, M, N, K,
                               epilogue, out, stream);
}

}  // namespace

hipError_t launch_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales,
                             const float* a_tensor_scale, const uint8_t* w_codes,
                             const uint8_t* w_scales, const float* w_tensor_scale,
                             const void* bias, int64_t M, int64_t N, int64_t K, int epilogue,
                             void* y, float* y_amax, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  const Out out{reinterpret_cast<uint16_t*>(y), reinterpret_cast<uint32_t*>(y_amax), nullptr,
                nullptr, nullptr, nullptr};
  return launch_any(a_codes, a_scales, a_tensor_scale, w_codes, w_scales, w_tensor_scale, bias, M,
                    N, K, epilogue, out, workspace, workspace_bytes, stream);
}

hipError_t launch_gemm_nvfp4_quantized(const uint8_t* a_codes, const uint8_t* a_scales,
                                       const float* a_tensor_scale, const uint8_t* w_codes,
                                       const uint8_t* w_scales, const float* w_tensor_scale,
                                       const void* bias, int64_t M, int64_t N, int64_t K,
                                       int epilogue, const float* y_amax_static, uint8_t* y_codes,
                                       uint8_t* y_scales, float* y_tensor_scale,
                                       hipStream_t stream) {
  const Out out{nullptr, nullptr, y_codes, y_scales, y_tensor_scale, y_amax_static};
  return launch_any(a_codes, a_scales, a_tensor_scale, w_codes, w_scales, w_tensor_scale, bias, M,
                    N, K, epilogue, out, nullptr, 0, stream);
}

}  // namespace nvfp4
