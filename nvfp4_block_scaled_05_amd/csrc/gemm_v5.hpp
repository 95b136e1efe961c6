// The v5 NVFP4 GEMM kernel (device code), shared by the two translation units
// that instantiate it: gemm_nvfp4.hip (bf16 output, the persistent grid and
// the split-K tail) and gemm_nvfp4_quant.hip (NVFP4 output under a static
// tensor scale), which compile in parallel.  The operation, its exactness and
// the sources it follows are described at the top of gemm_nvfp4.hip.
#pragma once

#include "device_common.hpp"

namespace nvfp4 {

// Where a tile's results go: bf16 Y (with an optional amax), or -- when
// `codes` is set -- Y quantized to NVFP4 with the static tensor scale derived
// from *amax_static, the same bytes as quantizing the bf16 Y with that amax.
struct Out {
  uint16_t* y;
  uint32_t* y_amax;
  uint8_t* codes;
  uint8_t* scales;
  float* tensor_scale;
  const float* amax_static;
};

namespace {

// ---------------------------------------------------------------------------
// v5: direct-to-LDS operands, both decoded in registers.  For K % 256 == 0
// (an even number of 128-wide stages, and 16-byte aligned scale rows for the
// paired scale loads).
// Workgroup of 4 waves in 2x2 over a 256x256 tile, each wave 128x128 (4x4
// MFMA tiles, 256 fp32 accumulators per lane).  K advances 128 per stage
// (eight 16-K MFMA steps), triple-buffered in LDS; a stage holds per row 64
// bytes of codes of each operand and room for 16 block-scale bytes (the
// scales of two stages, loaded every other stage) (40 KB).
//   * Codes and scales go from global memory straight into LDS (the gfx950
//     buffer load with the LDS destination: one instruction fills 1 KB with
//     16-byte pieces, lane L's at offset 16 L).  Inside a 64-byte code row
//     the 16-byte pieces are permuted by an XOR with
//     (row / 4) % 4, which makes the fragment reads (16 lanes, 16 consecutive
//     rows, one logical piece) hit 16 different bank groups.
//   * Same K permutation as v1-v3 at this width: lanes 0-31 of a wave take
//     elements 0-63 of the stage, lanes 32-63 elements 64-127; MFMA step s
//     takes code word s of each lane's 32 bytes, so A and W agree on k.
//   * Each wave decodes its own 128 rows of A and 128 rows of W from the
//     packed codes (no fp16 copy in LDS): LDS traffic is the codes only.
//   * Three stage slots in LDS (120 KB): the loads of stage t+2 are issued
//     during stage t, after its packed operands have all been read into
//     registers, so no LDS read waits on a load in flight.
//   * The decode of step s+1 is interleaved with the MFMAs of step s; the
//     MFMAs of a stage's last two steps run after the next barrier, while the
//     next stage's LDS reads, scale conversion and first decode are done.
//   * The weight fragment is the MFMA's first operand, so acc[i][j] holds the
//     transposed tile: lane (r, h) has row m = i*32 + r and the four
//     consecutive columns n = j*32 + 8g + 4h + t at elements 4g + t.
// Rows past M or N are read clamped to the last row; their results are never
// stored.
// ---------------------------------------------------------------------------
constexpr int kVBM = 256, kVBN = 256, kVBK = 128, kVNT = 256;
constexpr int kVWM = 128, kVWN = 128, kVTM = 4, kVTN = 4;
constexpr int kVCodeRow = kVBK / 2;                 // 64 code bytes per row and stage
constexpr int kVScaleRow = kVBK / 16;               // 8 scale bytes per row and stage
constexpr int kVScalePair = 2 * kVScaleRow;         // a row's scales of two stages
constexpr int kVA = 0;                              // A codes
constexpr int kVW = kVA + kVBM * kVCodeRow;         // W codes
constexpr int kVSA = kVW + kVBN * kVCodeRow;        // A scales, two stages per row
constexpr int kVSW = kVSA + kVBM * kVScalePair;     // W scales, two stages per row
constexpr int kVStage = kVSW + kVBN * kVScalePair;  // 40 KB

// This lane's source offsets (bytes from the start of the operand's codes /
// scales; rows * K / 2 < 2^32 is checked on the host).
struct V5Src {
  uint32_t ac[4], wc[4];     // code chunks of 16 rows
  uint32_t as, ws;           // start of the scale row this lane loads (row 64 * wave + lane)
};

__device__ __forceinline__ void v5_setup(int64_t M, int64_t N, int64_t K, int64_t m0, int64_t n0,
                                         V5Src& d) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t cpitch = K / 2, spitch = K / 16;
  const int piece = (lane & 3) ^ ((lane >> 4) & 3);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * (wave * 4 + i) + (lane >> 2);
    const int64_t ra = m0 + row < M ? m0 + row : M - 1;
    const int64_t rw = n0 + row < N ? n0 + row : N - 1;
    d.ac[i] = (uint32_t)(ra * cpitch + piece * 16);
    d.wc[i] = (uint32_t)(rw * cpitch + piece * 16);
  }
  {
    const int row = 64 * wave + lane;
    const int64_t ra = m0 + row < M ? m0 + row : M - 1;
    const int64_t rw = n0 + row < N ? n0 + row : N - 1;
    d.as = (uint32_t)(ra * spitch);
    d.ws = (uint32_t)(rw * spitch);
  }
}

// The global->LDS loads of one stage into `stage`: parts 0-3 the code chunks
// i of A and W (two instructions each), part 4 the block scales.  Scales go in
// pairs of stages: one 16-byte load per row brings a row's scales of stages
// `pair` and `pair` + 1 (8 bytes each), so only every other stage loads them
// (and an item's first stage, whatever its parity: the pair that holds it).
// A stage of odd index then reads its scales from the slot of the stage
// before it.  Inside the K loop the parts are spread over the stage's MFMA
// steps: issuing a load occupies the wave while the compute unit's address
// unit takes its 64 addresses, and all of a stage's loads in a row (four
// waves at once) leave the matrix pipe idle for hundreds of clocks; the scale
// loads, two of the old eight per wave and stage, cost as much to issue as
// code loads that carry four times the bytes.
struct V5Refill {
  const uint8_t* ac;
  const uint8_t* as;
  const uint8_t* wc;
  const uint8_t* ws;
  const V5Src* src;
  int kt;          // the stage's K index (codes)
  int pair;        // the first stage of the scale pair to load, or -1: none
  uint8_t* stage;
};

template <int P>
__device__ __forceinline__ void v5_issue_part(const V5Refill& r) {
  const int wave = wave_id();
  if constexpr (P < 4) {
    const int c = wave * 4 + P;
    buffer_load_lds<16>(r.ac, r.src->ac[P], r.kt * kVCodeRow, r.stage + kVA + c * 1024);
    buffer_load_lds<16>(r.wc, r.src->wc[P], r.kt * kVCodeRow, r.stage + kVW + c * 1024);
  } else {
    // rows 64 * wave + lane, 16 bytes each: 1 KB per wave and operand
    buffer_load_lds<16>(r.as, r.src->as, r.pair * kVScaleRow, r.stage + kVSA + wave * 1024);
    buffer_load_lds<16>(r.ws, r.src->ws, r.pair * kVScaleRow, r.stage + kVSW + wave * 1024);
  }
}

// A whole stage at once (the first stages of an item): the scales first, so a
// wait that lets the codes of the stage after stay in flight has them.
__device__ __forceinline__ void v5_issue(const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
                                         const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws,
                                         const V5Src& d, int kt, int pair, uint8_t* stage) {
  const V5Refill r{ac, as, wc, ws, &d, kt, pair, stage};
  if (pair >= 0) v5_issue_part<4>(r);
  v5_issue_part<0>(r);
  v5_issue_part<1>(r);
  v5_issue_part<2>(r);
  v5_issue_part<3>(r);
}

// The scale pair an item's stage t (K index g = kb + t) loads: its own pair at
// an even g, the pair holding it at the item's first stage, none otherwise.
__device__ __forceinline__ int v5_pair(int g, int t) {
  return (g & 1) == 0 ? g : t == 0 ? g - 1 : -1;
}

// One lane's packed operands for a stage: tiles 0-3 are A (i), 4-7 are W (j).
struct V5Packed {
  u32x4 lo[8], hi[8];   // code words 0-3 and 4-7 (MFMA steps)
  f16x2 s01[8], s23[8]; // block scales (4 blocks) as fp16
};

struct V5Ops {
  f16x8 v[8];
};

// `scl`: the scales of this stage -- its own slot's pair area, or the
// previous stage's, plus 8 bytes for the second stage of a pair.
__device__ __forceinline__ void v5_read(const uint8_t* stage, const uint8_t* scl, int a_row,
                                        int w_row, int h, int x, V5Packed& p, uint32_t (&sc)[8]) {
  const int p0 = ((2 * h) ^ x) << 4, p1 = ((2 * h + 1) ^ x) << 4;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int row = (t < 4 ? a_row + t * 32 : w_row + (t - 4) * 32);
    const uint8_t* cr = stage + (t < 4 ? kVA : kVW) + row * kVCodeRow;
    p.lo[t] = *reinterpret_cast<const u32x4*>(cr + p0);
    p.hi[t] = *reinterpret_cast<const u32x4*>(cr + p1);
    sc[t] = *reinterpret_cast<const uint32_t*>(scl + (t < 4 ? kVSA : kVSW) + row * kVScalePair + h * 4);
  }
}

__device__ __forceinline__ void v5_scales(const uint32_t (&sc)[8], V5Packed& p) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    p.s01[t] = e4m3_pair_to_f16x2<false>(sc[t]);
    p.s23[t] = e4m3_pair_to_f16x2<true>(sc[t]);
  }
}

// decode8 of the step's 8 fragments, written as all 32 conversions and then
// all 32 scale products: in this order the scheduler hands the MFMA groups
// independent conversions and products, instead of pairs in which each
// product waits for the conversion issued just before it.
template <int S>
__device__ __forceinline__ void v5_decode(const V5Packed& p, V5Ops& o) {
  f16x2 c[8][4];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t w = S < 4 ? p.lo[t][S & 3] : p.hi[t][S & 3];
    c[t][0] = e2m1_unpack2_f16<0>(w);
    c[t][1] = e2m1_unpack2_f16<1>(w);
    c[t][2] = e2m1_unpack2_f16<2>(w);
    c[t][3] = e2m1_unpack2_f16<3>(w);
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const _Float16 s = (S >> 1) == 0 ? p.s01[t].x : (S >> 1) == 1 ? p.s01[t].y
                     : (S >> 1) == 2 ? p.s23[t].x : p.s23[t].y;
    const f16x2 s2 = {s, s};
    o.v[t] = __builtin_bit_cast(f16x8, u32x4{__builtin_bit_cast(uint32_t, c[t][0] * s2),
                                             __builtin_bit_cast(uint32_t, c[t][1] * s2),
                                             __builtin_bit_cast(uint32_t, c[t][2] * s2),
                                             __builtin_bit_cast(uint32_t, c[t][3] * s2)});
  }
}

__device__ __forceinline__ void v5_mfma(const V5Ops& o, f32x16 (&acc)[kVTM][kVTN]) {
#pragma unroll
  for (int i = 0; i < kVTM; ++i)
#pragma unroll
    for (int j = 0; j < kVTN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(o.v[4 + j], o.v[i], acc[i][j], 0, 0, 0);
}

// MFMAs of step S-1 (in `cur`) interleaved with the decode of step S (into
// `nxt`); with LOAD, steps 1-4 also issue code part S - 1 of the refill, one
// load after the 8th and one after the 16th MFMA.
template <int S, bool LOAD>
__device__ __forceinline__ void v5_step(const V5Packed& p, const V5Ops& cur, V5Ops& nxt,
                                        f32x16 (&acc)[kVTM][kVTN], const V5Refill& r) {
  constexpr bool L = LOAD && S <= 4;
  v5_decode<S>(p, nxt);
  v5_mfma(cur, acc);
  if constexpr (L) v5_issue_part<S - 1>(r);
#pragma unroll
  for (int m = 0; m < kVTM * kVTN; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU (decode)
    if (L && m % 8 == 7) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM (load)
  }
}

// Steps of a stage whose step-0 operands are in `y` (`x` free): the MFMAs of
// steps 0-5 and the decode of steps 1-7.  Leaves step 6's operands in `y`,
// step 7's in `c`, and `x` free: those two steps run after the next barrier.
// With LOAD the refill's code loads `r` are issued along the way, one part
// per step.
template <bool LOAD>
__device__ __forceinline__ void v5_body(const V5Packed& p, V5Ops& x, V5Ops& y, V5Ops& c,
                                        f32x16 (&acc)[kVTM][kVTN], const V5Refill& r) {
  v5_step<1, LOAD>(p, y, x, acc, r);
  v5_step<2, LOAD>(p, x, y, acc, r);
  v5_step<3, LOAD>(p, y, x, acc, r);
  v5_step<4, LOAD>(p, x, y, acc, r);
  v5_step<5, LOAD>(p, y, x, acc, r);
  v5_decode<6>(p, y);                      // MFMAs of step 5 with two decodes
  v5_decode<7>(p, c);
  v5_mfma(x, acc);
#pragma unroll
  for (int m = 0; m < kVTM * kVTN; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // VALU (decode)
  }
}

// Stage data in LDS: this wave's loads for it have landed (vmcnt; with
// `next_in_flight` the 8 code loads of the following stage, its last loads,
// may still be outstanding -- its scales went out before them; loads complete
// in order, and any later memory instruction only makes the wait stricter),
// then the workgroup barrier
// makes every wave's loads visible and ends every read of the slot about to
// be refilled.
// (__syncthreads() would add a release fence, which waits for every load in
// flight; the waits here are explicit, and the asm barrier with a memory
// clobber keeps the compiler from moving memory accesses across it.)
__device__ __forceinline__ void v5_barrier(bool next_in_flight) {
  if (next_in_flight)
    __builtin_amdgcn_s_waitcnt(0x0078);   // vmcnt(8) lgkmcnt(0)
  else
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// One stage after the first, from slot `cur`.  The previous stage left the
// operands of its steps 6 and 7 in `s6` and `c`; their 32 MFMAs run here,
// first while this stage's packed operands are read (all of them, so no LDS
// read follows the refill loads), then while its scales are converted and
// step 0 is decoded into `s6` (free once the step-6 MFMAs have issued), so
// the matrix pipe stays busy across the barrier.  The body alternates `s6`
// and `x` from step to step and leaves this stage's step 6 in `s6`, step 7 in
// `c` and `x` free: the same roles the next stage expects, so the operand
// sets are never copied.
// `scl`: where this stage's scales are (see v5_read).  `next_in_flight`: the
// following stage's loads are outstanding.  REFILL: this stage issues the
// loads of stage t + 2 into `refill` (its scale pair `pair_refill`, if any,
// then its codes over steps 1-4), after every LDS read of the stage, so no
// read waits on them; compile-time, so the code loads sit in the same basic
// blocks as the MFMAs they are interleaved with.
template <bool REFILL>
__device__ __forceinline__ void v5_stage(const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
                                         const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws,
                                         const V5Src& src, const uint8_t* cur, const uint8_t* scl,
                                         uint8_t* refill, bool next_in_flight, int k_refill,
                                         int pair_refill, int a_row, int w_row, int h, int x_sw,
                                         V5Packed& p, V5Ops& x, V5Ops& s6, V5Ops& c,
                                         f32x16 (&acc)[kVTM][kVTN]) {
  v5_barrier(next_in_flight);
  uint32_t sc[8];
  v5_read(cur, scl, a_row, w_row, h, x_sw, p, sc);
  v5_mfma(s6, acc);                        // previous stage, step 6
#pragma unroll
  for (int m = 0; m < 12; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  __builtin_amdgcn_sched_barrier(0);
  const V5Refill r{ac, as, wc, ws, &src, k_refill, pair_refill, refill};
  // the refill's scale pair, if it loads one, first: the next stage's wait
  // lets only its code loads stay in flight
  if (REFILL && pair_refill >= 0) v5_issue_part<4>(r);
  v5_scales(sc, p);
  v5_decode<0>(p, s6);
  v5_mfma(c, acc);                         // previous stage, step 7
#pragma unroll
  for (int m = 0; m < kVTM * kVTN; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU (scales, decode, addresses)
  }
  __builtin_amdgcn_sched_barrier(0);
  v5_body<REFILL>(p, x, s6, c, acc, r);
}

// Epilogue of v5: acc * sA*sW + bias (one fused multiply-add), optional GELU,
// bf16 round-to-nearest-even, optional max |bf16 y| (one atomic per
// workgroup) -- the operations of epilogue(), in the same order.
// Fully unrolled over 256 accumulators per lane this is ~100 KB of code, more
// than the instruction cache holds; instead each wave moves 32 rows of its
// accumulators at a time into its own 16 KB of LDS (fp32, 16-byte chunks of a
// 512-byte row permuted by XOR with the row, conflict-free both ways) and a
// short loop takes them back 4 consecutive columns per lane: 32 lanes cover
// a 128-column row segment, so the 8-byte stores complete whole lines.
template <int EPI>
__device__ __forceinline__ u16x2 v5_slice_out(const float* st, float scale, f32x4 bv, int64_t row0,
                                              int64_t col, int64_t M, int64_t N, bool vec,
                                              uint16_t* __restrict__ y) {
  const int lane = opaque_lane(), c = lane & 31;
  asm volatile("" : "+v"(row0));   // row offsets computed here, not hoisted (see opaque_lane)
  u16x2 amax = {0, 0};
  // four rows' reads first, then their 16 values, then the stores: one LDS
  // wait per 16 values and 16 independent chains for the scheduler to
  // interleave (a lone dependent chain issues at about half the rate)
  for (int it0 = 0; it0 < 16; it0 += 4) {
    f32x4 a4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int rr = (it0 + u) * 2 + (lane >> 5);
      a4[u] = *reinterpret_cast<const f32x4*>(st + rr * 128 + ((c ^ rr) << 2));
    }
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < 4; ++t) v[u][t] = __builtin_fmaf(a4[u][t], scale, bv[t]);
    if (EPI == 1) gelu_erf16(v);
    u32x2 pk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      pk[u] = u32x2{bf16x2_rne(v[u][0], v[u][1]), bf16x2_rne(v[u][2], v[u][3])};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t row = row0 + (it0 + u) * 2 + (lane >> 5);
      if (vec) {
        *reinterpret_cast<u32x2*>(y + row * N + col) = pk[u];
        amax = amax_bf16x2(amax_bf16x2(amax, pk[u].x), pk[u].y);
      } else if (row < M) {
        const uint16_t hv[4] = {(uint16_t)pk[u].x, (uint16_t)(pk[u].x >> 16), (uint16_t)pk[u].y,
                                (uint16_t)(pk[u].y >> 16)};
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (col + t < N) {
            y[row * N + col + t] = hv[t];
            amax = max_u16x2(amax, u16x2{(unsigned short)(hv[t] & 0x7FFFu), 0});
          }
      }
    }
  }
  return amax;
}

__device__ __forceinline__ u16x2 v5_epilogue(const f32x16 (&acc)[kVTM][kVTN], float scale,
                                             const float* col_bias, int epi, int64_t M, int64_t N,
                                             int64_t m0, int64_t n0, uint16_t* __restrict__ y,
                                             float* st) {
  const int lane = opaque_lane(), wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, r = lane & 31, h = lane >> 5;
  const bool vec = m0 + kVBM <= M && n0 + kVBN <= N && N % 4 == 0 &&
                   (reinterpret_cast<uintptr_t>(y) & 7) == 0;
  const int cl = wn * kVWN + (lane & 31) * 4;               // this lane's 4 columns when reading back
  const f32x4 bv = *reinterpret_cast<const f32x4*>(col_bias + cl);
  u16x2 amax = {0, 0};
#pragma unroll
  for (int i = 0; i < kVTM; ++i) {
    // rows i*32 .. i*32+31 of the wave's tile: lane (r, h) holds row r, and
    // 4 consecutive columns j*32 + 8g + 4h at elements 4g .. 4g+3
#pragma unroll
    for (int j = 0; j < kVTN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = j * 8 + g * 2 + h;                    // 16-byte chunk of the 512-byte row
        *reinterpret_cast<f32x4*>(st + r * 128 + ((c ^ r) << 2)) =
            f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);                     // lgkmcnt(0): the wave's writes landed
    __builtin_amdgcn_wave_barrier();
    const int64_t row0 = m0 + wm * kVWM + i * 32;
    const u16x2 a = epi == 1 ? v5_slice_out<1>(st, scale, bv, row0, n0 + cl, M, N, vec, y)
                             : v5_slice_out<0>(st, scale, bv, row0, n0 + cl, M, N, vec, y);
    amax = max_u16x2(amax, a);
    __builtin_amdgcn_s_waitcnt(0xC07F);                     // reads done before the next slice's writes
    __builtin_amdgcn_wave_barrier();
  }
  return amax;   // this lane's max |bf16 y| (16-bit magnitudes)
}

// NVFP4 output of v5 under the static tensor scale derived from
// *out.amax_static: the bf16 values of v5_slice_out (same operations) are
// staged in the wave's LDS, 32 rows x 128 columns at a time, and every lane
// then quantizes whole 16-element blocks with the quantizer's own routine --
// the bytes nvfp4_quantize writes for the bf16 output.  N % 16 == 0.
// The bf16 rows (272-byte pitch) overlay the fp32 rows they come from
// (512-byte pitch) in the same area: bf16 row R ends at byte 272 R + 272,
// never past the start of fp32 row R + 1, so a row's bf16 values only
// overwrite fp32 rows already read; the rows are read and written in
// increasing order, and a compiler fence keeps each group's reads before its
// writes (the hardware runs a wave's LDS accesses in order).
template <int EPI>
__device__ __forceinline__ void v5_slice_quant(const float* st, uint16_t* st16, float scale, f32x4 bv,
                                               int64_t row0, int64_t col_w, int64_t M, int64_t N,
                                               bool degenerate, float s_enc, const float* e_of,
                                               const Out& out) {
  const int lane = opaque_lane(), c = lane & 31;
  asm volatile("" : "+v"(row0));   // row offsets computed here, not hoisted (see opaque_lane)
  // four rows' reads first, then their 16 values (as in v5_slice_out)
  for (int it0 = 0; it0 < 16; it0 += 4) {
    f32x4 a4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int rr = (it0 + u) * 2 + (lane >> 5);
      a4[u] = *reinterpret_cast<const f32x4*>(st + rr * 128 + ((c ^ rr) << 2));
    }
    // the group's reads stay before its writes: a lane's bf16 row can
    // overlay another lane's fp32 row of the same group
    asm volatile("" ::: "memory");
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < 4; ++t) v[u][t] = __builtin_fmaf(a4[u][t], scale, bv[t]);
    if (EPI == 1) gelu_erf16(v);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int rr = (it0 + u) * 2 + (lane >> 5);
      *reinterpret_cast<u32x2*>(st16 + rr * 136 + c * 4) =
          u32x2{bf16x2_rne(v[u][0], v[u][1]), bf16x2_rne(v[u][2], v[u][3])};
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);                       // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  const int64_t code_pitch = N / 2, scale_pitch = N / 16;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int b = lane + 64 * k, rr = b >> 3, blk = b & 7;   // 32 rows x 8 blocks
    const int64_t row = row0 + rr, col = col_w + blk * 16;
    const u32x4* src = reinterpret_cast<const u32x4*>(st16 + rr * 136 + blk * 16);
    u32x2 cw;
    uint32_t S;
    quantize_block_tab(src[0], src[1], bf16_bits_to_f32(block_max_bits(src[0], src[1])), degenerate,
                       s_enc, e_of, cw, S);
    if (row < M && col < N) {
      *reinterpret_cast<u32x2*>(out.codes + row * code_pitch + col / 2) = cw;
      out.scales[row * scale_pitch + col / 16] = (uint8_t)S;
    }
  }
}

__device__ __forceinline__ void v5_epilogue_quant(const f32x16 (&acc)[kVTM][kVTN], float scale,
                                                  const float* col_bias, int epi, int64_t M,
                                                  int64_t N, int64_t m0, int64_t n0, const Out& out,
                                                  float* st, uint16_t* st16, float* e_of) {
  const int lane = opaque_lane(), wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, r = lane & 31, h = lane >> 5;
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
  // the wave's table of encode factors (visible after the first slice's wait)
  e_of[lane] = encode_factor(lane, s_dec);
  e_of[lane + 64] = encode_factor(lane + 64, s_dec);
  const f32x4 bv = *reinterpret_cast<const f32x4*>(col_bias + wn * kVWN + (lane & 31) * 4);
#pragma unroll
  for (int i = 0; i < kVTM; ++i) {
#pragma unroll
    for (int j = 0; j < kVTN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = j * 8 + g * 2 + h;
        *reinterpret_cast<f32x4*>(st + r * 128 + ((c ^ r) << 2)) =
            f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
    const int64_t row0 = m0 + wm * kVWM + i * 32, col_w = n0 + wn * kVWN;
    if (epi == 1)
      v5_slice_quant<1>(st, st16, scale, bv, row0, col_w, M, N, degenerate, s_enc, e_of, out);
    else
      v5_slice_quant<0>(st, st16, scale, bv, row0, col_w, M, N, degenerate, s_enc, e_of, out);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
  }
}

// Work item b of a v5 launch: a whole tile, or one K range of a tail tile
// (split_coords on item b), with its first and last stage.
struct V5Item {
  int64_t m0, n0, tail;
  int split, kb, ke;
};

__device__ __forceinline__ V5Item v5_item(int64_t b, int64_t tiles_m, int64_t tiles_n,
                                          const SplitK& sk, int nk) {
  V5Item it;
  int64_t tm, tn;
  split_coords_of(b, tiles_m, tiles_n, sk, tm, tn, it.tail, it.split);
  it.m0 = tm * kVBM;
  it.n0 = tn * kVBN;
  it.kb = it.split < 0 ? 0 : (int)((int64_t)it.split * nk / sk.ways);
  it.ke = it.split < 0 ? nk : (int)((int64_t)(it.split + 1) * nk / sk.ways);
  return it;
}

// kQuant: NVFP4 output (out.codes, out.scales, out.tensor_scale) instead of
// bf16 (out.y, out.y_amax); whole tiles only.
// Persistent: workgroup b takes work items b, b + gridDim.x, ... below
// `items` (the grid is a multiple of the 8 XCDs, so every item of a
// workgroup maps to its XCD's range of the tile order, as a one-item launch
// would).  Stage t of an item lives in slot (t + 2) % 3, so its first stage
// lands in slot 2, which the epilogue's staging (the first 64 KB) leaves
// alone: the next item's first stage is loaded while this item's epilogue
// runs, and the next item starts with it in LDS.  The output amax is
// carried across items and reduced once per workgroup.
template <bool kQuant>
__global__ __launch_bounds__(kVNT, 1) void gemm_nvfp4_v5_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ sa, const uint8_t* __restrict__ w_codes,
    const uint8_t* __restrict__ w_scales, const float* __restrict__ sw,
    const uint16_t* __restrict__ bias, int64_t M, int64_t N, int64_t K, int epi, Out out,
    SplitK sk, int64_t items) {
  // three stage slots: the loads of stage t + 2 are issued while stage t runs
  __shared__ __attribute__((aligned(1024))) uint8_t lds[3 * kVStage];
  static_assert(32 * 136 * 2 <= 16384, "a wave's bf16 rows fit in its fp32 staging area");
  static_assert(4 * 16384 + 4 * 512 <= 2 * kVStage,
                "the epilogue's staging and encode-factor tables leave slot 2 free");
  __shared__ __attribute__((aligned(16))) float col_bias[kVBN];
#define V5_SLOT(t) (lds + (((t) + 2) % 3) * kVStage)
  // the scales of the item's stage t (K index kb + t): in the pair its own
  // slot holds, or -- at an odd K index past the item's first stage -- in the
  // second half of the pair the stage before it loaded
#define V5_SCL(t)                                                                       \
  ((((it.kb + (t)) & 1) && (t) > 0) ? V5_SLOT((t) - 1) + kVScaleRow                    \
                                    : V5_SLOT(t) + ((it.kb + (t)) & 1) * kVScaleRow)
  const int64_t tiles_m = (M + kVBM - 1) / kVBM, tiles_n = (N + kVBN - 1) / kVBN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, h = lane >> 5, x = (r >> 2) & 3;
  const int a_row = wm * kVWM + r, w_row = wn * kVWN + r;
  const int nk = (int)(K / kVBK);
  const float scale = (*sa) * (*sw);

  int64_t b = blockIdx.x;
  V5Item it = v5_item(b, tiles_m, tiles_n, sk, nk);
  V5Src src;
  v5_setup(M, N, K, it.m0, it.n0, src);
  v5_issue(a_codes, a_scales, w_codes, w_scales, src, it.kb, v5_pair(it.kb, 0), V5_SLOT(0));
  u16x2 amax = {0, 0};
  for (;;) {
    {
      const int64_t c = it.n0 + threadIdx.x;
      col_bias[threadIdx.x] = (bias && c < N) ? bf16_bits_to_f32(bias[c]) : 0.0f;
    }
    f32x16 acc[kVTM][kVTN];
#pragma unroll
    for (int i = 0; i < kVTM; ++i)
#pragma unroll
      for (int j = 0; j < kVTN; ++j) acc[i][j] = f32x16{};

    // stages [kb, ke) of 128 K: all of them, or this split's share; the
    // first one is already issued
    const int ns = it.ke - it.kb;
    V5Packed p;
    V5Ops oa, ob, oc;
    if (ns > 1)
      v5_issue(a_codes, a_scales, w_codes, w_scales, src, it.kb + 1, v5_pair(it.kb + 1, 1),
               V5_SLOT(1));
    v5_barrier(ns > 1);
    {
      uint32_t sc[8];
      v5_read(V5_SLOT(0), V5_SCL(0), a_row, w_row, h, x, p, sc);
      if (ns > 2)
        v5_issue(a_codes, a_scales, w_codes, w_scales, src, it.kb + 2, v5_pair(it.kb + 2, 2),
                 V5_SLOT(2));
      v5_scales(sc, p);
    }
    v5_decode<0>(p, oa);
    v5_body<false>(p, ob, oa, oc, acc, V5Refill{});   // steps 6, 7 pending in oa, oc
    // every stage leaves its step 6 in oa and step 7 in oc, as this one
    int t = 1;
    for (; t + 2 < ns; ++t)                  // the stage two ahead is loaded
      v5_stage<true>(a_codes, a_scales, w_codes, w_scales, src, V5_SLOT(t), V5_SCL(t),
                     V5_SLOT(t + 2), true, it.kb + t + 2, v5_pair(it.kb + t + 2, t + 2), a_row,
                     w_row, h, x, p, ob, oa, oc, acc);
    for (; t < ns; ++t)                      // the last two: nothing more to load
      v5_stage<false>(a_codes, a_scales, w_codes, w_scales, src, V5_SLOT(t), V5_SCL(t), nullptr,
                      t + 1 < ns, 0, -1, a_row, w_row, h, x, p, ob, oa, oc, acc);
    v5_mfma(oa, acc);
    v5_mfma(oc, acc);

    const V5Item cur = it;
    const int64_t nb = b + gridDim.x;
    const bool has_next = nb < items;
    if (!kQuant && cur.split >= 0) {
      // a tail split: fp32 partial sums into its slice in accumulator order --
      // float4 number (((wave * 4 + i) * 4 + j) * 64 + lane) * 4 + g holds
      // acc[i][j][4g .. 4g+3], so each wave writes 4 KB contiguous per tile
      f32x4* slice =
          reinterpret_cast<f32x4*>(sk.part + (cur.tail * sk.ways + cur.split) * (int64_t)(kVBM * kVBN));
#pragma unroll
      for (int i = 0; i < kVTM; ++i)
#pragma unroll
        for (int j = 0; j < kVTN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            slice[(((wave * kVTM + i) * kVTN + j) * 64 + lane) * 4 + g] =
                f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
      if (!has_next) break;
      asm volatile("s_barrier" ::: "memory");   // every wave is done reading this item's slots
      b = nb;
      it = v5_item(b, tiles_m, tiles_n, sk, nk);
      v5_setup(M, N, K, it.m0, it.n0, src);
      v5_issue(a_codes, a_scales, w_codes, w_scales, src, it.kb, v5_pair(it.kb, 0), V5_SLOT(0));
      continue;
    }
    __syncthreads();   // every wave is done with the stage buffers
    if (has_next) {    // the next item's first stage, into slot 2, under the epilogue
      b = nb;
      it = v5_item(b, tiles_m, tiles_n, sk, nk);
      v5_setup(M, N, K, it.m0, it.n0, src);
      v5_issue(a_codes, a_scales, w_codes, w_scales, src, it.kb, v5_pair(it.kb, 0), V5_SLOT(0));
    }
    float* st = reinterpret_cast<float*>(lds + wave * 16384);
    if (kQuant)   // bf16 rows over the wave's fp32 area; encode factors after the four areas
      v5_epilogue_quant(acc, scale, col_bias, epi, M, N, cur.m0, cur.n0, out, st,
                        reinterpret_cast<uint16_t*>(st),
                        reinterpret_cast<float*>(lds + 4 * 16384 + wave * 512));
    else
      amax = max_u16x2(amax, v5_epilogue(acc, scale, col_bias, epi, M, N, cur.m0, cur.n0, out.y, st));
    if (!has_next) break;
    // every wave is done with the epilogue's staging and col_bias before the
    // next item's loads refill slots 0 and 1 and its bias is written
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
  }
#undef V5_SCL
#undef V5_SLOT
  if (!kQuant && out.y_amax) {   // one atomic per workgroup
    __shared__ uint32_t wave_amax[kVNT / 64];
    uint32_t a = (uint32_t)(amax.x > amax.y ? amax.x : amax.y) << 16;
    a = wave_max_u32(a);
    if (lane == 0) wave_amax[wave] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t m = 0;
#pragma unroll
      for (int w = 0; w < kVNT / 64; ++w) m = max(m, wave_amax[w]);
      atomicMax(out.y_amax, m);
    }
  }
}

}  // namespace

// gemm_nvfp4_v5_kernel<true> over `tiles` whole tiles on `grid` workgroups
// (tiles, or the persistent grid; defined in gemm_nvfp4_quant.hip).
hipError_t launch_v5_quant(const uint8_t* a_codes, const uint8_t* a_scales, const float* sa,
                           const uint8_t* w_codes, const uint8_t* w_scales, const float* sw,
                           const uint16_t* bias, int64_t M, int64_t N, int64_t K, int epi,
                           const Out& out, int64_t tiles, int64_t grid, hipStream_t stream);

}  // namespace nvfp4
