// bf16 passthrough GEMM for gfx950: the linear layers kept in higher precision
// by the exclude pattern ("英伟达B200狂飙10.2倍！AI绘图告别龟速！",
// nmedialink.com, section "NVFP4量化").
//
//   Y[m,n] = bf16( epi( sum_k X[m,k]*W[n,k] + bias[n] ) ), fp32 accumulation.
//
// Three kernels, chosen by shape:
//  * gemv_bf16_kernel (M <= 8): streams the weight once, no tiles;
//  * gemm_bf16_dma_kernel (large problems): 256x256 tiles, operands loaded
//    straight into LDS, 4 waves of 128x128;
//  * gemm_bf16_kernel (the rest): 128x128 output tile per 256-thread
//    workgroup, K step 64, LDS double-buffered with a register prefetch of
//    the next K step; each of the 4 waves owns a 64x64 sub-tile = 2x2
//    v_mfma_f32_32x32x16_bf16 tiles;
//  * gemm_bf16_ksplit_kernel (fewer 128x128 tiles than compute units): the
//    same tile with two such wave groups splitting K.
#include <cstdlib>
#include <cstring>

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

// tid: the thread's index within its group of NT threads
__device__ __forceinline__ void load_bf16(const uint16_t* __restrict__ x, int64_t rows, int64_t K,
                                          int64_t row0, int64_t k0, Bf16Tile& t, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + i * NT;
    const int64_t row = row0 + (q >> 3);
    const int64_t k = k0 + (q & 7) * 8;
    if (row < rows && k < K)
      t.v[i] = *reinterpret_cast<const u32x4*>(x + row * K + k);
    else
      t.v[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void store_bf16(const Bf16Tile& t, uint16_t* __restrict__ lds, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + i * NT;
    *reinterpret_cast<u32x4*>(lds + (q >> 3) * PITCH + (q & 7) * 8) = t.v[i];
  }
}

// ------------------------------------------------------------------ compute --

template <bool kF16>
__device__ __forceinline__ void mma_step(const uint16_t* __restrict__ As,
                                         const uint16_t* __restrict__ Bs, f32x16 (&acc)[2][2],
                                         int tid) {
  const int lane = tid & 63;
  const int w = tid >> 6;
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
  const int tid = threadIdx.x;
  load_bf16(x, M, K, m0, 0, ta, tid);
  load_bf16(w, N, K, n0, 0, tb, tid);
  store_bf16(ta, lds[0][0], tid);
  store_bf16(tb, lds[0][1], tid);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      load_bf16(x, M, K, m0, (int64_t)(kt + 1) * BK, ta, tid);
      load_bf16(w, N, K, n0, (int64_t)(kt + 1) * BK, tb, tid);
    }
    mma_step<false>(lds[cur][0], lds[cur][1], acc, tid);
    if (more) {
      store_bf16(ta, lds[cur ^ 1][0], tid);
      store_bf16(tb, lds[cur ^ 1][1], tid);
    }
    __syncthreads();
  }
  epilogue(acc, 1.0f, bias, epi, M, N, m0, n0, y, nullptr);
}

// Few tiles (fewer 128x128 tiles than compute units): two groups of 4 waves
// share each tile, group g taking the K steps g, g + 2, g + 4, ...; group 1
// hands its sums to group 0 through LDS before the epilogue.  Twice the waves
// per tile, no workspace.  (The two halves of the K sum are added at the end,
// so the rounding differs from gemm_bf16_kernel's within fp32 accumulation.)
__global__ __launch_bounds__(2 * NT, 1) void gemm_bf16_ksplit_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ bias, int64_t M, int64_t N, int64_t K, int epi,
    uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][2][TILE_ELEMS];   // group, stage, operand
  static_assert(sizeof(lds[1]) >= NT * 64 * sizeof(float), "group 1's buffers hold its sums");
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * BM;
  const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * BN;
  const int nk = (int)((K + BK - 1) / BK);
  const int g = (int)(threadIdx.x / NT), tid = (int)(threadIdx.x % NT);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  Bf16Tile ta, tb;
  if (g < nk) {
    load_bf16(x, M, K, m0, (int64_t)g * BK, ta, tid);
    load_bf16(w, N, K, n0, (int64_t)g * BK, tb, tid);
    store_bf16(ta, lds[g][0][0], tid);
    store_bf16(tb, lds[g][0][1], tid);
  }
  __syncthreads();
  const int steps = (nk + 1) / 2;          // group 0's count; group 1 has nk / 2
  for (int s = 0; s < steps; ++s) {        // every thread reaches every barrier
    const int cur = s & 1;
    const int kt = g + 2 * s;
    const bool have = kt < nk, more = kt + 2 < nk;
    if (more) {
      load_bf16(x, M, K, m0, (int64_t)(kt + 2) * BK, ta, tid);
      load_bf16(w, N, K, n0, (int64_t)(kt + 2) * BK, tb, tid);
    }
    if (have) mma_step<false>(lds[g][cur][0], lds[g][cur][1], acc, tid);
    if (more) {
      store_bf16(ta, lds[g][cur ^ 1][0], tid);
      store_bf16(tb, lds[g][cur ^ 1][1], tid);
    }
    __syncthreads();
  }
  float* red = reinterpret_cast<float*>(&lds[1][0][0][0]);   // group 1's buffers, now free
  if (g == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((i * 2 + j) * 16 + r) * NT + tid] = acc[i][j][r];
  }
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] += red[((i * 2 + j) * 16 + r) * NT + tid];
    epilogue(acc, 1.0f, bias, epi, M, N, m0, n0, y, nullptr);
  }
}

// Large problems (256x256 tiles covering at least half the compute units,
// K % 64 == 0, 16-byte aligned operands): each workgroup computes a 256x256
// tile with 4 waves of 128x128 (256 fp32 accumulators per lane, in AGPRs at one
// wave per SIMD).  Operands go from global memory straight into LDS with the
// gfx950 global->LDS load (lane L's 16 bytes land at offset 16 L of the 1 KB
// the instruction fills): per stage 64 K, i.e. 128 bytes of bf16 per row, in
// two separately declared 64 KB buffers, so the compiler sees that a stage's
// LDS reads do not alias the load in flight into the other buffer.  Inside a
// 128-byte row the 16-byte pieces are permuted by XOR with (row / 2) % 8: the
// fragment reads (16 lanes, 16 consecutive rows, one logical piece) then hit
// distinct bank groups.  v_mfma_f32_32x32x16_bf16 takes one piece per lane and
// row: k-step s of a stage is piece 2s + h for lane half h.  The weight
// fragment is the MFMA's first operand, so each lane holds four consecutive
// columns of one output row, and the epilogue moves 32 rows at a time through
// LDS to write 8-byte stores.
constexpr int kEBM = 256, kEBN = 256, kEBK = 64, kENT = 256;
constexpr int kEWM = 128, kEWN = 128, kETM = 4, kETN = 4;
constexpr int kERow = kEBK * 2;              // 128 bytes per row and stage
constexpr int kEOp = kEBM * kERow;           // 32 KB per operand and stage
constexpr int kEStage = 2 * kEOp;            // A, then W

// This lane's source offsets (bytes from the operand's start; rows * K * 2 <
// 2^32 is checked on the host), one per 8-row chunk it loads.
struct BDmaPtrs {
  uint32_t a[kEBM / 8 / 4];
  uint32_t w[kEBN / 8 / 4];
};

__device__ __forceinline__ void bdma_setup(int64_t M, int64_t N, int64_t K, int64_t m0, int64_t n0,
                                           BDmaPtrs& d) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t pitch = K * 2;
#pragma unroll
  for (int i = 0; i < kEBM / 8 / 4; ++i) {
    const int c = wave * (kEBM / 8 / 4) + i;             // chunk: rows 8c .. 8c+7
    const int row = 8 * c + (lane >> 3);
    const int piece = (lane & 7) ^ ((row >> 1) & 7);
    const int64_t ra = m0 + row < M ? m0 + row : M - 1;
    const int64_t rw = n0 + row < N ? n0 + row : N - 1;
    d.a[i] = (uint32_t)(ra * pitch + piece * 16);
    d.w[i] = (uint32_t)(rw * pitch + piece * 16);
  }
}

__device__ __forceinline__ void bdma_issue(const uint8_t* __restrict__ a, const uint8_t* __restrict__ w,
                                           const BDmaPtrs& d, int64_t kbyte, uint8_t* stage) {
  const int wave = wave_id();
#pragma unroll
  for (int i = 0; i < kEBM / 8 / 4; ++i) {
    const int c = wave * (kEBM / 8 / 4) + i;
    buffer_load_lds<16>(a, d.a[i], (int)kbyte, stage + c * 1024);
    buffer_load_lds<16>(w, d.w[i], (int)kbyte, stage + kEOp + c * 1024);
  }
}

struct BFrags {
  u32x4 a[kETM], b[kETN];
};

// Fragments of k-step S (0..3) of a stage; a_off / b_off: this lane's byte
// offset of its row in the wave's first A / W tile; sw = (row / 2) % 8.
template <int S>
__device__ __forceinline__ void bfrags(const uint8_t* stage, int a_off, int b_off, int h, int sw,
                                       BFrags& f) {
  const int p = ((2 * S + h) ^ sw) << 4;
#pragma unroll
  for (int i = 0; i < kETM; ++i)
    f.a[i] = *reinterpret_cast<const u32x4*>(stage + a_off + i * 32 * kERow + p);
#pragma unroll
  for (int j = 0; j < kETN; ++j)
    f.b[j] = *reinterpret_cast<const u32x4*>(stage + kEOp + b_off + j * 32 * kERow + p);
}

__device__ __forceinline__ void bmfma(const BFrags& f, f32x16 (&acc)[kETM][kETN]) {
#pragma unroll
  for (int i = 0; i < kETM; ++i)
#pragma unroll
    for (int j = 0; j < kETN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.b[j]),
                                                          __builtin_bit_cast(bf16x8, f.a[i]),
                                                          acc[i][j], 0, 0, 0);
}

// Every load of this wave has landed in LDS (vmcnt 0), then the workgroup
// barrier: the next stage is visible and all reads of the buffer about to be
// refilled are done.
__device__ __forceinline__ void bdma_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// One stage: refill `nxt` with the stage after this one (REFILL), read this
// stage's four k-steps from `cur` and run the previous stage's last k-step
// and this stage's first three, MFMAs interleaved with the reads and loads.
// REFILL is compile-time so that the loads sit in the MFMAs' basic block (a
// branch around them issues them in a burst with the matrix pipe idle).
template <bool REFILL>
__device__ __forceinline__ void bdma_stage(const uint8_t* __restrict__ a, const uint8_t* __restrict__ w,
                                           const uint8_t* cur, uint8_t* nxt, const BDmaPtrs& ptr,
                                           int64_t kbyte_next, int a_off, int b_off, int h, int sw,
                                           BFrags& f0, BFrags& f1, f32x16 (&acc)[kETM][kETN]) {
  bdma_barrier();
  if (REFILL) bdma_issue(a, w, ptr, kbyte_next, nxt);
  bfrags<0>(cur, a_off, b_off, h, sw, f0);
  bmfma(f1, acc);                          // previous stage, k-step 3
  bfrags<1>(cur, a_off, b_off, h, sw, f1);
  bmfma(f0, acc);
  bfrags<2>(cur, a_off, b_off, h, sw, f0);
  bmfma(f1, acc);
  bfrags<3>(cur, a_off, b_off, h, sw, f1);
  bmfma(f0, acc);
#pragma unroll
  for (int m = 0; m < kETM * kETN; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    if (REFILL) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM (load issue)
  }
#pragma unroll
  for (int m = 0; m < 3 * kETM * kETN; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// 32 rows x 128 columns of a wave's tile, staged in LDS, to bf16: a lane takes
// 4 consecutive columns of a row per step, so 32 lanes cover a 128-column row
// segment and the 8-byte stores complete whole lines.
template <int EPI>
__device__ __forceinline__ void bdma_slice_out(const float* st, f32x4 bv, int64_t row0, int64_t col,
                                               int64_t M, int64_t N, bool vec,
                                               uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63, c = lane & 31;
  // four rows' reads first, then their 16 values (GELU one step across all
  // 16), then the stores: one LDS wait per 16 values and independent chains
  for (int it0 = 0; it0 < 16; it0 += 4) {
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int rr = (it0 + u) * 2 + (lane >> 5);
      v[u] = *reinterpret_cast<const f32x4*>(st + rr * 128 + ((c ^ rr) << 2));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < 4; ++t) v[u][t] = v[u][t] + bv[t];
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

__global__ __launch_bounds__(kENT, 1) void gemm_bf16_dma_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ w, const uint16_t* __restrict__ bias,
    int64_t M, int64_t N, int64_t K, int epi, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kEStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kEStage];
  __shared__ __attribute__((aligned(16))) float col_bias[kEBN];
  const int64_t tiles_m = (M + kEBM - 1) / kEBM, tiles_n = (N + kEBN - 1) / kEBN;
  int64_t tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * kEBM, n0 = tn * kEBN;
  {
    const int64_t c = n0 + threadIdx.x;
    col_bias[threadIdx.x] = (bias && c < N) ? bf16_bits_to_f32(bias[c]) : 0.0f;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, h = lane >> 5, sw = (r >> 1) & 7;
  const int a_off = (wm * kEWM + r) * kERow, b_off = (wn * kEWN + r) * kERow;

  BDmaPtrs ptr;
  bdma_setup(M, N, K, m0, n0, ptr);
  f32x16 acc[kETM][kETN];
#pragma unroll
  for (int i = 0; i < kETM; ++i)
#pragma unroll
    for (int j = 0; j < kETN; ++j) acc[i][j] = f32x16{};

  const int ns = (int)(K / kEBK);
  BFrags f0, f1;
  bdma_issue(x, w, ptr, 0, lds0);
  bdma_barrier();
  if (ns > 1) bdma_issue(x, w, ptr, kERow, lds1);
  bfrags<0>(lds0, a_off, b_off, h, sw, f0);
  bfrags<1>(lds0, a_off, b_off, h, sw, f1);
  bmfma(f0, acc);
  bfrags<2>(lds0, a_off, b_off, h, sw, f0);
  bmfma(f1, acc);
  bfrags<3>(lds0, a_off, b_off, h, sw, f1);
  bmfma(f0, acc);
  // stage t reads buffer t % 2 and refills the other with stage t + 1; whole
  // pairs of stages, then at most one more
  // pairs of stages, then at most one more.  Both stages of a pair load: the
  // second stage of the last pair, with no stage left, loads its own stage
  // again into the buffer nothing reads any more; every load into LDS is
  // waited for before the epilogue.
  int t = 1;
  for (; t + 1 < ns; t += 2) {
    bdma_stage<true>(x, w, lds1, lds0, ptr, (int64_t)(t + 1) * kERow, a_off, b_off, h, sw, f0, f1,
                     acc);
    const int t2 = t + 2 < ns ? t + 2 : t + 1;
    bdma_stage<true>(x, w, lds0, lds1, ptr, (int64_t)t2 * kERow, a_off, b_off, h, sw, f0, f1, acc);
  }
  if (t < ns) bdma_stage<false>(x, w, lds1, lds0, ptr, 0, a_off, b_off, h, sw, f0, f1, acc);
  bmfma(f1, acc);
  __builtin_amdgcn_s_waitcnt(0);           // every load into LDS has landed

  // epilogue: acc + bias -> GELU -> bf16, the operations of gemm_bf16_kernel
  __syncthreads();   // every wave is done with the stage buffers
  float* st = reinterpret_cast<float*>(lds0 + wave * 16384);
  const bool vec = m0 + kEBM <= M && n0 + kEBN <= N && N % 4 == 0 &&
                   (reinterpret_cast<uintptr_t>(y) & 7) == 0;
  const int cq = wn * kEWN + (lane & 31) * 4;             // this lane's 4 columns on read-back
  const f32x4 bv = *reinterpret_cast<const f32x4*>(col_bias + cq);
#pragma unroll
  for (int i = 0; i < kETM; ++i) {
#pragma unroll
    for (int j = 0; j < kETN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = j * 8 + g * 2 + h;
        *reinterpret_cast<f32x4*>(st + r * 128 + ((c ^ r) << 2)) =
            f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);                     // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    const int64_t row0 = m0 + wm * kEWM + i * 32;
    if (epi == 1)
      bdma_slice_out<1>(st, bv, row0, n0 + cq, M, N, vec, y);
    else
      bdma_slice_out<0>(st, bv, row0, n0 + cq, M, N, vec, y);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
  }
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
  static_assert(kGemvMaxRows == 8, "the cases below cover M = 1 .. kGemvMaxRows");
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
  // the 256x256 direct-to-LDS kernel when its tiles cover at least half the
  // compute units (measured: 0.68-0.83x the 128x128 kernel's time from 144
  // tiles on, 1.1-1.7x at 108 and fewer) and its layout applies;
  // NVFP4_BF16_GEMM_KERNEL=tile|dma pins one (dma only where it applies)
  const int64_t big_tiles = ((M + kEBM - 1) / kEBM) * ((N + kEBN - 1) / kEBN);
  const uintptr_t bits = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w);
  const int64_t limit = (int64_t)1 << 32;
  const bool dma_ok = K > 0 && K % kEBK == 0 && (bits & 15) == 0 && M * K * 2 < limit && N * K * 2 < limit;
  const char* pin = getenv("NVFP4_BF16_GEMM_KERNEL");
  const bool want_dma = pin ? strcmp(pin, "dma") == 0 : 2 * big_tiles >= compute_units();
  if (dma_ok && want_dma) {
    hipLaunchKernelGGL(gemm_bf16_dma_kernel, dim3((unsigned)big_tiles), dim3(kENT), 0, stream,
                       reinterpret_cast<const uint8_t*>(x), reinterpret_cast<const uint8_t*>(w),
                       reinterpret_cast<const uint16_t*>(bias), M, N, K, epilogue,
                       reinterpret_cast<uint16_t*>(y));
    return hipGetLastError();
  }
  // fewer 128x128 tiles than compute units: two wave groups split K in each
  // tile (NVFP4_BF16_GEMM_KERNEL=ksplit|tile pins one)
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const bool ksplit = pin ? strcmp(pin, "ksplit") == 0 : tiles < compute_units() && K > BK;
  if (ksplit) {
    hipLaunchKernelGGL(gemm_bf16_ksplit_kernel, dim3((unsigned)tiles), dim3(2 * NT), 0, stream,
                       reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(w),
                       reinterpret_cast<const uint16_t*>(bias), M, N, K, epilogue,
                       reinterpret_cast<uint16_t*>(y));
    return hipGetLastError();
  }
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3((unsigned)tiles), dim3(NT), 0, stream,
                     reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(w),
                     reinterpret_cast<const uint16_t*>(bias), M, N, K, epilogue,
                     reinterpret_cast<uint16_t*>(y));
  return hipGetLastError();
}

}  // namespace nvfp4
