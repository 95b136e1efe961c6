// NVFP4 quantize / dequantize kernels for gfx950.
//
// Two-level scaling ("英伟达B200狂飙10.2倍！AI绘图告别龟速！", nmedialink.com,
// section "NVFP4量化"): one FP32 per-tensor scale, computed dynamically here
// from the tensor amax, and one scale per block of 16 elements computed in the
// same pass that encodes the elements.
//
// With the amax computed here, a small tensor (up to 512 KB of bf16) takes a
// one-launch kernel whose workgroups each fold the whole amax, and one that
// fits on chip (up to 109 MB on 256 compute units) the single-pass kernel
// further down, which reads it from HBM once; otherwise quantization is two
// launches, both HBM-bound:
//   amax_partial_kernel  every workgroup reads a grid-strided slice with
//                        128-bit loads (ordinary loads, so the tensor stays in
//                        the last-level cache for the second pass) and writes one partial max|x| (as the
//                        binary32 bit pattern of a bf16 magnitude; integer max
//                        of the magnitude bits, so no ordering or NaN issues).
//   quantize_kernel      every workgroup first folds the partials (or the
//                        producer's amax) into amax, derives s_enc / s_dec,
//                        then each thread encodes whole 16-element blocks: two
//                        128-bit loads, block max by integer max, E4M3 scale,
//                        E2M1 codes by the gfx950 packed conversion, one 64-bit
//                        code store and one scale byte.
//
// The arithmetic is binary32 round-to-nearest-even throughout: divisions are
// correctly rounded (no fast-math) and the file is built with FP contraction
// off, so every value equals the CPU oracle's bit for bit.
#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "device_common.hpp"
#include "kernels.hpp"

namespace nvfp4 {

static constexpr int kQuantThreads = 256;

// Partial amax: workgroup b scans its contiguous chunk of 16-byte words, U
// loads in flight per thread, and writes max |x| of the chunk.
template <int U>
__global__ __launch_bounds__(kQuantThreads) void amax_partial_kernel(
    const u32x4* __restrict__ x, int64_t n16, int64_t chunk, uint32_t* __restrict__ partial) {
  u16x2 m = {0, 0};
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = lo + chunk < n16 ? lo + chunk : n16;
  int64_t i = lo + threadIdx.x;
  for (; i + (U - 1) * kQuantThreads < hi; i += U * kQuantThreads) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = x[i + u * kQuantThreads];
#pragma unroll
    for (int u = 0; u < U; ++u) m = max_u16x2(m, max8(v[u]));
  }
  for (; i < hi; i += kQuantThreads) m = max_u16x2(m, max8(x[i]));
  uint32_t v = m.x > m.y ? m.x : m.y;
  v = wave_max_u32(v);
  __shared__ uint32_t red[kQuantThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (int w = 1; w < kQuantThreads / 64; ++w) r = r > red[w] ? r : red[w];
    partial[blockIdx.x] = r << 16;   // binary32 bits of the bf16 magnitude
  }
}

// Fold n words of binary32 magnitude bits into one (workgroup-wide).
__device__ __forceinline__ uint32_t fold_amax_words(const uint32_t* __restrict__ w, int n) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < n; i += kQuantThreads) {
    uint32_t v = w[i] & 0x7FFFFFFFu;
    m = m > v ? m : v;
  }
  m = wave_max_u32(m);
  __shared__ uint32_t red[kQuantThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < kQuantThreads / 64; ++i) r = r > red[i] ? r : red[i];
  return r;
}

// Every workgroup folds the amax words, derives s_enc / s_dec, then each
// thread quantizes U blocks per round (all 2U loads issued first).
template <int U>
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(
    const u32x4* __restrict__ x, int64_t nblocks, const uint32_t* __restrict__ amax_words,
    int n_amax, u32x2* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ tensor_scale, int32_t* __restrict__ dev_status) {
  const uint32_t amax_bits = fold_amax_words(amax_words, n_amax);
  const bool first = blockIdx.x == 0 && threadIdx.x == 0;
  if (amax_bits >= 0x7F800000u) {                       // Inf or NaN in the input
    if (first) {
      *tensor_scale = __uint_as_float(0x7FC00000u);
      if (dev_status) *dev_status = -8;                 // NVFP4_ERR_NONFINITE
    }
    return;
  }
  bool degenerate;
  float s_enc, s_dec;
  tensor_scales(__uint_as_float(amax_bits), degenerate, s_enc, s_dec);
  if (first) {
    *tensor_scale = s_dec;
    if (dev_status) *dev_status = 0;
  }
  __shared__ float e_of[128];                      // encode factor of every scale byte
  if (threadIdx.x < 128) e_of[threadIdx.x] = encode_factor(threadIdx.x, s_dec);
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * kQuantThreads * U;
  int64_t b = (int64_t)blockIdx.x * kQuantThreads * U + threadIdx.x;
  for (; b + (U - 1) * kQuantThreads < nblocks; b += stride) {
    u32x4 lo[U], hi[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      lo[u] = __builtin_nontemporal_load(x + 2 * (b + u * kQuantThreads));
      hi[u] = __builtin_nontemporal_load(x + 2 * (b + u * kQuantThreads) + 1);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      u32x2 c;
      uint32_t S;
      quantize_block_tab(lo[u], hi[u], bf16_bits_to_f32(block_max_bits(lo[u], hi[u])), degenerate,
                         s_enc, e_of, c, S);
      codes[b + u * kQuantThreads] = c;
      scales[b + u * kQuantThreads] = (uint8_t)S;
    }
  }
  for (; b < nblocks; b += kQuantThreads) {
    const u32x4 lo = x[2 * b], hi = x[2 * b + 1];
    u32x2 c;
    uint32_t S;
    quantize_block_tab(lo, hi, bf16_bits_to_f32(block_max_bits(lo, hi)), degenerate, s_enc, e_of, c, S);
    codes[b] = c;
    scales[b] = (uint8_t)S;
  }
}

// One-launch quantizer for small tensors (at most kSmallMaxElems elements,
// 512 KB of bf16): every workgroup folds the amax of the whole tensor itself
// (the first reads come from HBM, the rest mostly from L2), then encodes its
// own range of blocks.  No workspace, no second launch, no waiting on other
// workgroups; the same bytes as the other kernels.
static constexpr int kSmallThreads = 512;
static constexpr int kSmallMaxGrid = 16;
static constexpr int64_t kSmallMaxElems = (int64_t)1 << 18;

__global__ __launch_bounds__(kSmallThreads) void quantize_small_kernel(
    const u32x4* __restrict__ x, uint32_t nblocks, uint32_t chunk, u32x2* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tensor_scale,
    int32_t* __restrict__ dev_status) {
  constexpr int NW = kSmallThreads / 64;
  __shared__ uint32_t red[NW];
  __shared__ float e_of[128];
  const uint32_t n16 = 2 * nblocks;
  u16x2 m = {0, 0};
  uint32_t w = threadIdx.x;
  for (; w + 7 * kSmallThreads < n16; w += 8 * kSmallThreads) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = x[w + u * kSmallThreads];
#pragma unroll
    for (int u = 0; u < 8; ++u) m = max_u16x2(m, max8(v[u]));
  }
  for (; w < n16; w += kSmallThreads) m = max_u16x2(m, max8(x[w]));
  const uint32_t r = wave_max_u32(m.x > m.y ? m.x : m.y);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = r;
  __syncthreads();
  uint32_t amax16 = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) amax16 = amax16 > red[i] ? amax16 : red[i];
  const uint32_t amax_bits = amax16 << 16;
  const bool first = blockIdx.x == 0 && threadIdx.x == 0;
  if (amax_bits >= 0x7F800000u) {                 // Inf or NaN in the input
    if (first) {
      *tensor_scale = __uint_as_float(0x7FC00000u);
      if (dev_status) *dev_status = -8;           // NVFP4_ERR_NONFINITE
    }
    return;
  }
  bool degenerate;
  float s_enc, s_dec;
  tensor_scales(__uint_as_float(amax_bits), degenerate, s_enc, s_dec);
  if (first) {
    *tensor_scale = s_dec;
    if (dev_status) *dev_status = 0;
  }
  if (threadIdx.x < 128) e_of[threadIdx.x] = encode_factor(threadIdx.x, s_dec);
  __syncthreads();
  const uint32_t lo = blockIdx.x * chunk;
  const uint32_t end = lo + chunk < nblocks ? lo + chunk : nblocks;
  for (uint32_t b = lo + threadIdx.x; b < end; b += kSmallThreads) {
    const u32x4 v0 = x[2 * b], v1 = x[2 * b + 1];
    u32x2 c;
    uint32_t S;
    quantize_block_tab(v0, v1, bf16_bits_to_f32(block_max_bits(v0, v1)), degenerate, s_enc, e_of, c, S);
    codes[b] = c;
    scales[b] = (uint8_t)S;
  }
}

// Dequantize: y = bf16_rne((value * S) * s_dec).  One lane per 8 elements
// (half a block): a 4-byte code load, its block's scale byte (shared by the
// lane pair), one 16-byte streaming store, so each wave instruction writes
// 1 KB contiguous; two half-blocks per lane per round keep more in flight.
// The products are binary32 (the first is exact); the packed conversion
// rounds to nearest-even.
static constexpr int kDequantU = 2;

__global__ __launch_bounds__(kQuantThreads) void dequantize_kernel(
    const uint32_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ tensor_scale, int64_t nhalves, u32x4* __restrict__ y) {
  const float s_dec = *tensor_scale;
  const int64_t stride = (int64_t)gridDim.x * kQuantThreads * kDequantU;
  for (int64_t h0 = (int64_t)blockIdx.x * kQuantThreads * kDequantU + threadIdx.x; h0 < nhalves;
       h0 += stride) {
    uint32_t w[kDequantU], sb[kDequantU];
#pragma unroll
    for (int u = 0; u < kDequantU; ++u) {
      const int64_t h = h0 + u * kQuantThreads;
      if (h < nhalves) {
        w[u] = __builtin_nontemporal_load(codes + h);
        sb[u] = scales[h >> 1];
      }
    }
#pragma unroll
    for (int u = 0; u < kDequantU; ++u) {
      const int64_t h = h0 + u * kQuantThreads;
      if (h < nhalves) {
        const float S = e4m3_to_f32(sb[u]);
        const f32x2 p[4] = {e2m1_unpack2_f32<0>(w[u]), e2m1_unpack2_f32<1>(w[u]),
                            e2m1_unpack2_f32<2>(w[u]), e2m1_unpack2_f32<3>(w[u])};
        uint32_t out[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = bf16x2_rne((p[j].x * S) * s_dec, (p[j].y * S) * s_dec);
        __builtin_nontemporal_store(u32x4{out[0], out[1], out[2], out[3]}, y + h);
      }
    }
  }
}

// Single-pass quantizer for a tensor that fits on chip.  One workgroup per
// compute unit (its LDS use admits no second one).  Workgroup g owns the
// contiguous blocks [g*chunk, (g+1)*chunk):
//   1. it reads them all at once, R blocks per thread into registers and L
//      per thread straight into LDS (global->LDS loads into a wave-private
//      region), keeps each block's max|x| and folds them into one partial;
//   2. it publishes the partial, counts itself in, and waits until every
//      workgroup has arrived;
//   3. it folds the partials into the tensor amax, derives s_enc / s_dec,
//      tabulates the encode factor of every scale byte, and encodes its
//      blocks from registers and LDS, so X crosses HBM once.
// The bytes are those of quantize_block (quantize_block_tab computes the same
// function).  The loads are unconditional: indexes past the range are clamped
// to its last block (for an empty range, the tensor's last block), which the
// maxima already count, so the compiler can overlap the maxima with the data
// still arriving.  Codes and scales are streamed out with nontemporal stores.
// The arrival (below) uses only agent-coherent atomic words.  The grid is not
// launched cooperatively (that launch path costs tens of microseconds), so
// nothing guarantees that all workgroups are resident together: another
// stream's kernels may hold compute units.  The wait is therefore bounded in
// time: a workgroup that has not been released after wait_ticks folds the
// partials already published and reads only the ranges of the workgroups
// whose partial is missing (slower, but the same value), so the kernel always
// completes and always gives the same bytes.
// The kernel is instantiated for three footprints, R 16-element blocks per
// thread in registers and L more in LDS: <9, 4> (13 blocks: up to 13,312 per
// workgroup, 54.5 M elements on 256 compute units; 4 * 32 B * 1024 = 128 KB
// of LDS), <4, 0> and <2, 0>.  A call takes the smallest that holds its
// range, so a mid-size tensor does not issue the loads of the large
// footprint (clamped to its last block) for nothing.
static constexpr int kResThreads = 1024;
static constexpr int kResR = 9;   // the large footprint: blocks per thread in registers
static constexpr int kResL = 4;   // ... and in LDS
static constexpr uint64_t kResWaitTicks = 20000;   // 200 us of the 100 MHz real-time counter

// Workspace words of the arrival.  Workgroups are dealt to kXcds groups
// (blockIdx % 8, which is also the XCD they run on); each group counts its
// arrivals on its own 128-byte line, the last of a group counts the group in
// on the top counter, and the last group raises every group's release word,
// which that group's workgroups poll.  No line sees more than 32 arrivals or
// pollers.  Nothing is ever cleared: the counters only grow (64-bit), every
// call adds exactly the same count to each (one arrival per workgroup, one
// workgroup per compute unit), so count / arrivals-per-call is the number of
// calls made before -- the call's epoch -- and the release word of a group
// holds the epoch + 1 of the last call released.  Each workgroup publishes
// its partial max in its own slot tagged with (epoch + 1) mod 2^16, in the
// same 32-bit atomic store, so a reader can tell a published partial from a
// stale one by the slot alone; the counters and release words only say when
// to look.  The workspace must hold zeros before its first use; calls then
// keep it consistent (counters at whole multiples of a call's arrivals, slots
// all tagged with the last epoch), which is what the next call relies on.
static constexpr int kResLine = 32;                              // words per 128-byte line
static constexpr int kResTop = 0;                                // u64 top counter
static constexpr int kResGroupCount = kResLine;                  // + 32 * g: u64 group counter
static constexpr int kResGroupFlag = kResLine * (1 + kXcds);     // + 32 * g: u64 release epoch
static constexpr int kResSlots = kResLine * (1 + 2 * kXcds);     // + workgroup: tag << 16 | max
static constexpr int kResMaxUnits = kQuantSyncWords - kResSlots; // slots that fit

__device__ __forceinline__ uint64_t* res_u64(uint32_t* sync, int word) {
  return reinterpret_cast<uint64_t*>(sync + word);
}

// One 16-byte global load per lane straight into LDS (lane L's bytes at
// byte 16 L of the wave's destination).  A plain device function: called in
// the body of a kernel template, the builtin made the host-side
// instantiation fail silently and the kernel's launch stub was never emitted.
__device__ __forceinline__ void load16_to_lds(const u32x4* src, u32x4* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

template <int R, int L>
__global__ __launch_bounds__(kResThreads) void quantize_resident_kernel(
    const u32x4* __restrict__ x, uint32_t nblocks, uint32_t chunk, u32x2* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tensor_scale, int32_t* __restrict__ dev_status,
    uint32_t* __restrict__ sync, uint64_t wait_ticks) {
  constexpr int T = kResThreads, NW = T / 64;
  __shared__ u32x4 stage[NW][L > 0 ? L : 1][128];   // wave w, slot s: 64 blocks = 128 words
  __shared__ float e_of[128];           // encode factor of every scale byte
  __shared__ uint32_t red[NW];
  __shared__ uint32_t shared_ok, shared_tag;
  __shared__ uint32_t missing[kResMaxUnits / 32];   // workgroups whose partial did not arrive
  const int wave = wave_id();
  const int lane = threadIdx.x & 63;
  const uint32_t lo = blockIdx.x * chunk;
  const uint32_t end = lo + chunk < nblocks ? lo + chunk : nblocks;   // may be below lo: empty
  const uint32_t last = end > lo ? end - 1 : nblocks - 1;
  __shared__ uint64_t shared_count;

  // 1. loads: the LDS part first (no registers held), then the register part
#pragma unroll
  for (int s = 0; s < L; ++s) {
    const uint32_t blk0 = lo + (uint32_t)((R + s) * T + wave * 64);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t word = 2 * blk0 + (uint32_t)(64 * i + lane);
      load16_to_lds(x + (word < 2 * last + 1 ? word : 2 * last + 1), &stage[wave][s][64 * i]);
    }
  }
  u32x4 a[R], b[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    uint32_t blk = lo + (uint32_t)(k * T) + threadIdx.x;
    blk = blk < last ? blk : last;
    a[k] = __builtin_nontemporal_load(x + 2 * blk);
    b[k] = __builtin_nontemporal_load(x + 2 * blk + 1);
  }
  // the group counter before this workgroup arrives, read while the loads
  // above are in flight (its value gives the call's epoch; see the arrival)
  if (threadIdx.x == 0)
    shared_count = __hip_atomic_load(res_u64(sync, kResGroupCount + kResLine * (blockIdx.x % kXcds)),
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // block maxima, two 16-bit magnitudes per word
  uint32_t bm[(R + L + 1) / 2];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const uint32_t v = block_max_bits(a[k], b[k]);
    bm[k / 2] = k % 2 ? bm[k / 2] | (v << 16) : v;
  }
  __builtin_amdgcn_sched_barrier(0);    // the maxima above stay ahead of the wait below
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): the LDS part has landed
#pragma unroll
  for (int s = 0; s < L; ++s) {
    const uint32_t v = block_max_bits(stage[wave][s][2 * lane], stage[wave][s][2 * lane + 1]);
    const int k = R + s;
    bm[k / 2] = k % 2 ? bm[k / 2] | (v << 16) : v;
  }
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < (R + L + 1) / 2; ++k) {
    const u16x2 p = __builtin_bit_cast(u16x2, bm[k]);
    m = m > p.x ? m : p.x;
    m = m > p.y ? m : p.y;
  }

  // 2. partial max of the workgroup: publish it, arrive, wait (bounded)
  m = wave_max_u32(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  const uint32_t grp = blockIdx.x % kXcds;
  const uint32_t groups = gridDim.x < kXcds ? gridDim.x : kXcds;
  const uint32_t in_group = (gridDim.x - grp + kXcds - 1) / kXcds;
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = r > red[w] ? r : red[w];
    // this call's epoch, from the group counter read before any arrival of
    // this workgroup (it lies in [epoch * in_group, (epoch + 1) * in_group))
    const uint64_t epoch = shared_count / in_group;
    __hip_atomic_store(sync + kResSlots + blockIdx.x, (((uint32_t)epoch + 1u) << 16) | r,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0070);             // vmcnt(0) lgkmcnt(0): slot written first
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    uint64_t* gcount = res_u64(sync, kResGroupCount + kResLine * grp);
    if (__hip_atomic_fetch_add(gcount, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) %
                in_group == in_group - 1 &&
        __hip_atomic_fetch_add(res_u64(sync, kResTop), (uint64_t)1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT) % groups == groups - 1) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      for (uint32_t q = 0; q < groups; ++q)
        __hip_atomic_store(res_u64(sync, kResGroupFlag + kResLine * q), epoch + 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    bool ok = true;
    while (__hip_atomic_load(res_u64(sync, kResGroupFlag + kResLine * grp), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT) != epoch + 1) {
      if (__builtin_amdgcn_s_memrealtime() - t0 > wait_ticks) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    shared_ok = ok;
    shared_tag = ((uint32_t)epoch + 1u) & 0xFFFFu;
  }
  if (threadIdx.x < kResMaxUnits / 32) missing[threadIdx.x] = 0u;
  __syncthreads();
  // the partials, one slot per thread: a slot tagged with this call's epoch
  // holds its workgroup's max.  Released, every slot is tagged or about to be
  // (its store may still be on its way): poll it, within the same time limit.
  // Not released in time, a slot not yet tagged is counted as missing.
  uint32_t r = 0;
  if (threadIdx.x < gridDim.x) {
    const uint32_t tag = shared_tag;
    uint32_t w = __hip_atomic_load(sync + kResSlots + threadIdx.x, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    if (shared_ok && (w >> 16) != tag) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while ((w >> 16) != tag && __builtin_amdgcn_s_memrealtime() - t0 <= wait_ticks) {
        __builtin_amdgcn_s_sleep(1);
        w = __hip_atomic_load(sync + kResSlots + threadIdx.x, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if ((w >> 16) == tag)
      r = (w & 0xFFFFu) << 16;
    else
      atomicOr(&missing[threadIdx.x >> 5], 1u << (threadIdx.x & 31));
  }
  __syncthreads();
  // workgroups whose partial is missing (not resident in time): read their
  // ranges here -- only theirs -- and fold them in
  {
    u16x2 mm = {0, 0};
    for (int i = 0; i < kResMaxUnits / 32; ++i) {
      uint32_t bits = missing[i];                 // the same word for every thread
      while (bits) {
        const uint32_t g = 32u * i + (uint32_t)__builtin_ctz(bits);
        bits &= bits - 1u;
        const uint32_t glo = g * chunk;
        const uint32_t gend = glo + chunk < nblocks ? glo + chunk : nblocks;
        for (uint32_t w = 2 * glo + threadIdx.x; w < 2 * gend; w += T) mm = max_u16x2(mm, max8(x[w]));
      }
    }
    const uint32_t f = (uint32_t)(mm.x > mm.y ? mm.x : mm.y) << 16;
    r = r > f ? r : f;
  }
  r = wave_max_u32(r);
  __syncthreads();                                // red[] is free again
  if (lane == 0) red[wave] = r;
  __syncthreads();
  uint32_t amax_bits = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) amax_bits = amax_bits > red[w] ? amax_bits : red[w];

  // 3. scales, the encode factors, then encode from registers and LDS
  if (amax_bits >= 0x7F800000u) {                // Inf or NaN in the input
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *tensor_scale = __uint_as_float(0x7FC00000u);
      if (dev_status) *dev_status = -8;           // NVFP4_ERR_NONFINITE
    }
    return;
  }
  bool degenerate;
  float s_enc, s_dec;
  tensor_scales(__uint_as_float(amax_bits), degenerate, s_enc, s_dec);
  if (threadIdx.x < 128) e_of[threadIdx.x] = encode_factor(threadIdx.x, s_dec);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *tensor_scale = s_dec;
    if (dev_status) *dev_status = 0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const uint32_t blk = lo + (uint32_t)(k * T) + threadIdx.x;
    if (blk < end) {
      const float a_b = bf16_bits_to_f32((bm[k / 2] >> (16 * (k % 2))) & 0xFFFFu);
      u32x2 c;
      uint32_t S;
      quantize_block_tab(a[k], b[k], a_b, degenerate, s_enc, e_of, c, S);
      __builtin_nontemporal_store(c, codes + blk);
      __builtin_nontemporal_store((uint8_t)S, scales + blk);
    }
  }
#pragma unroll
  for (int s = 0; s < L; ++s) {
    const int k = R + s;
    const uint32_t blk = lo + (uint32_t)(k * T + wave * 64 + lane);
    if (blk < end) {
      const float a_b = bf16_bits_to_f32((bm[k / 2] >> (16 * (k % 2))) & 0xFFFFu);
      u32x2 c;
      uint32_t S;
      quantize_block_tab(stage[wave][s][2 * lane], stage[wave][s][2 * lane + 1], a_b, degenerate,
                         s_enc, e_of, c, S);
      __builtin_nontemporal_store(c, codes + blk);
      __builtin_nontemporal_store((uint8_t)S, scales + blk);
    }
  }
}

// ---------------------------------------------------------------- launchers --

static int grid_for(int64_t work, int per_thread, int cap) {
  int64_t g = (work + (int64_t)kQuantThreads * per_thread - 1) / ((int64_t)kQuantThreads * per_thread);
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

// Launch shape.  Defaults: the amax pass reads with 8 loads in flight per
// thread over at most kMaxAmaxPartials workgroups; the quantizer handles 2
// blocks per thread and round over at most 2048 workgroups, so every
// workgroup's fold of the partials stays a small L2 read.
struct QuantShape {
  int amax_u = 8, quant_u = 2, quant_grid = 2048, amax_grid = kMaxAmaxPartials;
};

static QuantShape quant_shape() {
  QuantShape q;
  // debug pinning: "amax_u,amax_grid,quant_u,quant_grid"
  if (const char* e = getenv("NVFP4_QUANT_SHAPE")) {
    int a, ag, u, g;
    if (sscanf(e, "%d,%d,%d,%d", &a, &ag, &u, &g) == 4) {
      q.amax_u = a;
      q.amax_grid = ag < kMaxAmaxPartials ? ag : kMaxAmaxPartials;
      q.quant_u = u;
      q.quant_grid = g;
    }
  }
  return q;
}

int amax_partial_count(int64_t numel) {
  return grid_for(numel / 8, 8, kMaxAmaxPartials);
}

// The single-pass kernel is used when the amax is computed here, the tensor
// fits on chip (at most units * (R + L) * 1024 blocks of 16: 109 MB of bf16 on
// 256 compute units), it is above the one-launch kernel's size (back to back
// through the C ABI the single pass in its small footprints takes 7.6 us a
// call at 0.5-1 M elements and 13 us at 14 M, the two passes 8.5 and 15), and
// the workspace holds the counters,
// the release words and one slot per compute unit.  NVFP4_QUANT_KERNEL=twopass
// turns it off, =resident also takes it for the smallest tensors.  One launch
// per call: the arrival words are never cleared (see above), so no clearing
// kernel runs before it.
static constexpr int64_t kResMinElems = kSmallMaxElems + 1;

static bool try_resident(const u32x4* xv, int64_t nblocks, u32x2* codes, uint8_t* scales,
                         float* tensor_scale, uint32_t* workspace, size_t workspace_bytes,
                         int32_t* dev_status, hipStream_t stream) {
  const char* env = getenv("NVFP4_QUANT_KERNEL");
  const bool forced = env && strcmp(env, "resident") == 0;
  if (env && strcmp(env, "twopass") == 0) return false;
  if (!forced && nblocks * 16 < kResMinElems) return false;
  const int units = compute_units();
  if (nblocks > (int64_t)units * (kResR + kResL) * kResThreads) return false;
  if (units > kResMaxUnits || workspace_bytes < 4u * (size_t)kQuantSyncWords) return false;
  uint32_t nb = (uint32_t)nblocks;
  uint32_t chunk = (uint32_t)((nblocks + units - 1) / units);
  // NVFP4_QUANT_WAIT_TICKS shortens the wait (tests: 0 sends the
  // workgroups not released at once down the path that reads the missing
  // partials' ranges themselves)
  uint64_t wait_ticks = kResWaitTicks;
  if (const char* w = getenv("NVFP4_QUANT_WAIT_TICKS")) wait_ticks = strtoull(w, nullptr, 10);
  if (chunk <= 2u * kResThreads)
    quantize_resident_kernel<2, 0><<<dim3(units), dim3(kResThreads), 0, stream>>>(
        xv, nb, chunk, codes, scales, tensor_scale, dev_status, workspace, wait_ticks);
  else if (chunk <= 4u * kResThreads)
    quantize_resident_kernel<4, 0><<<dim3(units), dim3(kResThreads), 0, stream>>>(
        xv, nb, chunk, codes, scales, tensor_scale, dev_status, workspace, wait_ticks);
  else
    quantize_resident_kernel<kResR, kResL><<<dim3(units), dim3(kResThreads), 0, stream>>>(
        xv, nb, chunk, codes, scales, tensor_scale, dev_status, workspace, wait_ticks);
  return true;
}

hipError_t launch_quantize(const void* x, int64_t rows, int64_t cols, uint8_t* codes,
                           uint8_t* scales, float* tensor_scale, const float* amax_in,
                           uint32_t* workspace, size_t workspace_bytes, int32_t* dev_status,
                           hipStream_t stream) {
  const QuantShape qs = quant_shape();
  const int64_t numel = rows * cols;
  const int64_t nblocks = numel / 16;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  const char* kind = getenv("NVFP4_QUANT_KERNEL");
  if (!amax_in && (kind ? strcmp(kind, "small") == 0 : numel <= kSmallMaxElems) &&
      numel <= kSmallMaxElems) {
    const int g = (int)std::min<int64_t>(kSmallMaxGrid, (nblocks + kSmallThreads - 1) / kSmallThreads);
    const uint32_t chunk = (uint32_t)((nblocks + g - 1) / g);
    hipLaunchKernelGGL(quantize_small_kernel, dim3(g), dim3(kSmallThreads), 0, stream, xv,
                       (uint32_t)nblocks, chunk, reinterpret_cast<u32x2*>(codes), scales,
                       tensor_scale, dev_status);
    return hipGetLastError();
  }
  if (!amax_in && try_resident(xv, nblocks, reinterpret_cast<u32x2*>(codes), scales, tensor_scale,
                               workspace, workspace_bytes, dev_status, stream))
    return hipGetLastError();
  const uint32_t* words;
  int n_words;
  if (amax_in) {
    words = reinterpret_cast<const uint32_t*>(amax_in);
    n_words = 1;
  } else {
    int g = amax_partial_count(numel);
    if (g > qs.amax_grid) g = qs.amax_grid;
    const int64_t n16 = numel / 8;
    const int64_t chunk = (n16 + g - 1) / g;
    uint32_t* partials = workspace + kQuantSyncWords;   // past the single-pass words
    if (qs.amax_u == 4)
      hipLaunchKernelGGL(amax_partial_kernel<4>, dim3(g), dim3(kQuantThreads), 0, stream, xv, n16, chunk, partials);
    else if (qs.amax_u == 16)
      hipLaunchKernelGGL(amax_partial_kernel<16>, dim3(g), dim3(kQuantThreads), 0, stream, xv, n16, chunk, partials);
    else
      hipLaunchKernelGGL(amax_partial_kernel<8>, dim3(g), dim3(kQuantThreads), 0, stream, xv, n16, chunk, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    words = partials;
    n_words = g;
  }
  const int u = qs.quant_u == 1 || qs.quant_u == 4 ? qs.quant_u : 2;
  const int g = grid_for(nblocks, u, qs.quant_grid > 0 ? qs.quant_grid : 1 << 30);
  u32x2* cv = reinterpret_cast<u32x2*>(codes);
  if (u == 1)
    hipLaunchKernelGGL(quantize_kernel<1>, dim3(g), dim3(kQuantThreads), 0, stream, xv, nblocks,
                       words, n_words, cv, scales, tensor_scale, dev_status);
  else if (u == 4)
    hipLaunchKernelGGL(quantize_kernel<4>, dim3(g), dim3(kQuantThreads), 0, stream, xv, nblocks,
                       words, n_words, cv, scales, tensor_scale, dev_status);
  else
    hipLaunchKernelGGL(quantize_kernel<2>, dim3(g), dim3(kQuantThreads), 0, stream, xv, nblocks,
                       words, n_words, cv, scales, tensor_scale, dev_status);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                             int64_t rows, int64_t cols, void* y, hipStream_t stream) {
  const int64_t nhalves = rows * cols / 8;
  const int g = grid_for(nhalves, kDequantU, 16384);
  hipLaunchKernelGGL(dequantize_kernel, dim3(g), dim3(kQuantThreads), 0, stream,
                     reinterpret_cast<const uint32_t*>(codes), scales, tensor_scale, nhalves,
                     reinterpret_cast<u32x4*>(y));
  return hipGetLastError();
}

// ---------------------------------------------------- library-owned scratch --
// The quantizer workspace of nvfp4_quantize_no_alloc, for callers that cannot
// allocate: one copy of this array per GPU, created zero-filled when the code
// object is loaded on that GPU (the state the single-pass kernel's arrival
// words need before their first use; each call leaves them valid for the
// next) and held until the process ends.  In host code the name `scratch`
// is a host-side stand-in, not a device address: the device address comes
// from hipGetSymbolAddress, once per device with that device current, and
// only that address is passed to kernels.
static __device__ __align__(256) uint32_t scratch[kQuantWorkspaceWords] = {};

static constexpr int kMaxScratchDevices = 64;
static std::atomic<uint32_t*> g_scratch[kMaxScratchDevices];
static std::mutex g_scratch_lock;

size_t static_scratch_bytes() { return sizeof(uint32_t) * kQuantWorkspaceWords; }

hipError_t static_scratch(uint32_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  uint32_t* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_lock);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      p = static_cast<uint32_t*>(addr);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace nvfp4
