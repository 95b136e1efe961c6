// Device helpers shared by the gfx950 kernels of the NVFP4 library.
//
// Formats (NVFP4): E2M1 elements, sign in bit 3, magnitudes 0, .5, 1, 1.5, 2,
// 3, 4, 6; E4M3 block scales (OCP "fn", bias 7, max 448 = 0x7E, subnormal
// quantum 2^-9); bf16 = the top half of a binary32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Largest |x| of the two bf16 halves of a word, as a 16-bit magnitude pattern.
__device__ __forceinline__ u16x2 abs_halves(uint32_t w) {
  return __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
}

__device__ __forceinline__ u16x2 max_u16x2(u16x2 a, u16x2 b) {
  return __builtin_elementwise_max(a, b);
}

// binary32 -> E4M3 byte for t >= 0: nearest, ties to the even byte, saturating
// at 448.  Below 2^-6 the E4M3 grid is uniform with quantum 2^-9, so t * 512
// (exact) rounded to an integer with the hardware's nearest-even rounding is
// the byte (0..8; 8 is the smallest normal, 0x08).  From 2^-6 up, the binary32
// significand is rounded to 3 bits, nearest-even, by integer arithmetic, and
// the exponent is rebiased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_from_f32_rne(float t) {
  // both candidates are computed and one selected: no divergent branch
  const uint32_t sub = (uint32_t)__builtin_rintf(t * 512.0f);
  const uint32_t u = __float_as_uint(t);
  const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
  const uint32_t byte = ((((r >> 23) - 127u + 7u)) << 3) | ((r >> 20) & 7u);
  return t < 0.015625f ? sub : (byte > 0x7Eu ? 0x7Eu : byte);
}

// E4M3 bytes of four values in [0, 448] through the gfx950 packed FP8
// conversion (OCP E4M3, nearest-even); v0 lands in the low byte.  Callers
// clamp to 448, which makes the conversion saturate exactly like
// e4m3_from_f32_rne.
__device__ __forceinline__ uint32_t e4m3_pack4(float v0, float v1, float v2, float v3) {
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
}

// E4M3 scale byte (0x00..0x7E: non-negative, finite) -> exact binary32.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t e = b >> 3, m = b & 7u;
  return e == 0 ? (float)m * 0.001953125f                     // m * 2^-9, exact
                : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// binary32 -> bf16 bits, nearest-even (finite input; overflow gives Inf).
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two binary32 -> two bf16 (low half = lo), round-to-nearest-even, through the
// gfx950 packed conversion.
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// erf-form GELU, z * Phi(z) with Phi(z) = erfc(-z / sqrt 2) / 2.  With
// x = |z| / sqrt 2 and t = 1 / (1 + |z| / (2 sqrt 2)), h = Phi(-|z|) =
// erfc(x) / 2 is t * 2^(Q(t) - 1 - z^2 log2(e) / 2), Q a degree-5 polynomial
// fitted to log2(erfcx(x) / t) on |z| <= 14 (fractional error of erfc below
// 8e-6; gelu_fit.py beside this file derives the coefficients; the constant
// term below includes the -1).  Then z * Phi(z) = max(z, 0) - |z| * h for
// either sign, one FMA.  The result is accurate relative to |GELU(z)| in both
// tails, to about 1e-5 -- hundreds of times below the bf16 rounding the
// epilogues apply to it.
__device__ __forceinline__ float gelu_erf(float z) {
  const float az = __builtin_fabsf(z);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(az, 0.353553391f, 1.0f));
  float q = 0.33010265f;
  q = __builtin_fmaf(q, t, -1.0232246f);
  q = __builtin_fmaf(q, t, 0.68463063f);
  q = __builtin_fmaf(q, t, 0.36704522f);
  q = __builtin_fmaf(q, t, 1.4686911f);
  q = __builtin_fmaf(q, t, -2.827234f);
  const float arg = __builtin_fmaf(z * -0.72134752f, z, q);
  const float h = t * __builtin_amdgcn_exp2f(arg);           // Phi(-|z|)
  return __builtin_fmaf(-az, h, __builtin_fmaxf(z, 0.0f));
}

// gelu_erf on 16 independent values, one step across all of them before the
// next (the same operations per value, so the same bits).  One wave issues a
// dependent chain at about half the rate of independent instructions, and
// left to itself the compiler runs the chains one after another.  The empty
// asm statements between the steps take all 16 values as operands, so every
// value's step k is done before any value's step k+1; they emit nothing.
__device__ __forceinline__ void tie16(f32x4 (&v)[4]) {
  asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
}

__device__ __forceinline__ void gelu_erf16(f32x4 (&z)[4]) {
  f32x4 t[4], q[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) t[u][e] = __builtin_fmaf(__builtin_fabsf(z[u][e]), 0.353553391f, 1.0f);
  tie16(t);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) t[u][e] = __builtin_amdgcn_rcpf(t[u][e]);
  tie16(t);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) q[u][e] = __builtin_fmaf(0.33010265f, t[u][e], -1.0232246f);
  tie16(q);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) q[u][e] = __builtin_fmaf(q[u][e], t[u][e], 0.68463063f);
  tie16(q);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) q[u][e] = __builtin_fmaf(q[u][e], t[u][e], 0.36704522f);
  tie16(q);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) q[u][e] = __builtin_fmaf(q[u][e], t[u][e], 1.4686911f);
  tie16(q);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) q[u][e] = __builtin_fmaf(q[u][e], t[u][e], -2.827234f);
  tie16(q);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) q[u][e] = __builtin_fmaf(z[u][e] * -0.72134752f, z[u][e], q[u][e]);
  tie16(q);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) q[u][e] = __builtin_amdgcn_exp2f(q[u][e]);
  tie16(q);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      z[u][e] = __builtin_fmaf(-__builtin_fabsf(z[u][e]), t[u][e] * q[u][e], __builtin_fmaxf(z[u][e], 0.0f));
}

// Running max |bf16| of two packed bf16 values (the output amax), as 16-bit
// magnitudes: an integer max, so a NaN output makes the amax non-finite.
__device__ __forceinline__ u16x2 amax_bf16x2(u16x2 m, uint32_t pair) {
  return max_u16x2(m, abs_halves(pair));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Two binary32 values -> two E2M1 codes in byte `sel` of `old`, element `a`
// in the low nibble.  The gfx950 conversion rounds to nearest-even, saturates
// at 6 and keeps the sign of zero; with scale 1.0 it applies no scaling.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Byte `SEL` of `w` (two E2M1 codes) -> two fp16 E2M1 values, exact.  The
// conversion's scale operand only contributes its exponent; 1.0 adds nothing.
template <int SEL>
__device__ __forceinline__ f16x2 e2m1_unpack2_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// Two E4M3 bytes of `w` (bytes 0,1 or, with HI, bytes 2,3) -> two fp16, exact
// (every finite E4M3 value, subnormals included, is an fp16 normal or zero).
// The gfx950 conversion reads OCP E4M3; scale 1.0 adds nothing.
template <bool HI>
__device__ __forceinline__ f16x2 e4m3_pair_to_f16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

template <int SEL>
__device__ __forceinline__ f32x2 e2m1_unpack2_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// 8 E2M1 codes (one dword, element 0 in the low nibble) times their block
// scale s (one fp16, broadcast), as an fp16x8 MFMA operand.  value * scale
// has at most 6 significant bits and lies in [2^-10, 2688], so both the
// conversion and the product are exact.  The packed results are consumed
// whole: this compiler mis-simplifies a scalar extract of the high half of
// the packed conversion's result.
__device__ __forceinline__ f16x8 decode8(uint32_t w, _Float16 s) {
  const f16x2 s2 = {s, s};
  const f16x2 p0 = e2m1_unpack2_f16<0>(w) * s2;
  const f16x2 p1 = e2m1_unpack2_f16<1>(w) * s2;
  const f16x2 p2 = e2m1_unpack2_f16<2>(w) * s2;
  const f16x2 p3 = e2m1_unpack2_f16<3>(w) * s2;
  return __builtin_bit_cast(f16x8, u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                                         __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)});
}

// Index of this wave in the workgroup as a scalar (the compiler cannot see
// that threadIdx.x >> 6 is uniform across a wave): LDS destinations of the
// global->LDS loads, which go through M0, are then computed in scalar
// registers instead of one v_readfirstlane per load.
// The lane index through an empty asm statement.  A persistent kernel's
// epilogue takes its lane-derived addresses from this, so they are computed
// in the epilogue instead of being hoisted out of the item loop, where they
// would hold registers through the main loop (and spill).
__device__ __forceinline__ int opaque_lane() {
  int l = (int)(threadIdx.x & 63);
  asm volatile("" : "+v"(l));
  return l;
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Global -> LDS load in the gfx950 buffer form: lane L's BYTES (4 or 16)
// from base + lane_off + scalar_off land at lds + L * BYTES (lds is wave
// uniform and goes through M0).  The 32-bit per-lane offset and the scalar
// offset need no 64-bit address arithmetic per load.  The resource has record
// count 0xFFFFFFFF (no range clamping: callers keep every offset inside the
// buffer) and word 3 of the raw 32-bit data format used for untyped dword
// access.
constexpr int kBufferWord3 = 0x00020000;

template <int BYTES>
__device__ __forceinline__ void buffer_load_lds(const void* base, uint32_t lane_off, int scalar_off,
                                                void* lds) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xFFFFFFFF, kBufferWord3);
  auto* dst = (__attribute__((address_space(3))) void*)lds;
  if constexpr (BYTES == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, lane_off, scalar_off, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, lane_off, scalar_off, 0, 0);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}


// ------------------------------------------------------------- quantizer --
// Shared by the quantize kernel and the GEMM epilogue that writes NVFP4
// output, so both produce the same bytes for the same bf16 values.

// Largest |x| of 8 bf16 values (one 16-byte word), as two 16-bit magnitudes.
__device__ __forceinline__ u16x2 max8(u32x4 a) {
  return max_u16x2(max_u16x2(abs_halves(a.x), abs_halves(a.y)),
                   max_u16x2(abs_halves(a.z), abs_halves(a.w)));
}

// Max |x| of a 16-element block (two 16-byte words) as a 16-bit bf16 magnitude.
__device__ __forceinline__ uint32_t block_max_bits(u32x4 lo, u32x4 hi) {
  const u16x2 m = max_u16x2(max8(lo), max8(hi));
  return m.x > m.y ? m.x : m.y;
}

// Per-tensor scales from the tensor amax (a finite binary32): s_enc = 2688 /
// amax and s_dec = 1 / s_enc, both correctly rounded; below 2^-96 the tensor
// is degenerate (s_enc = s_dec = 1, every block scale 0).
__device__ __forceinline__ void tensor_scales(float amax, bool& degenerate, float& s_enc,
                                              float& s_dec) {
  degenerate = amax < 0x1p-96f;
  s_enc = degenerate ? 1.0f : 2688.0f / amax;
  s_dec = degenerate ? 1.0f : 1.0f / s_enc;
}

// E2M1 codes of 8 bf16 values (one 16-byte word) times e, packed.
__device__ __forceinline__ uint32_t encode8(u32x4 v, float e) {
  uint32_t c = 0;
  c = e2m1_pack2<0>(c, bf16_bits_to_f32(v.x & 0xFFFFu) * e, bf16_bits_to_f32(v.x >> 16) * e);
  c = e2m1_pack2<1>(c, bf16_bits_to_f32(v.y & 0xFFFFu) * e, bf16_bits_to_f32(v.y >> 16) * e);
  c = e2m1_pack2<2>(c, bf16_bits_to_f32(v.z & 0xFFFFu) * e, bf16_bits_to_f32(v.z >> 16) * e);
  c = e2m1_pack2<3>(c, bf16_bits_to_f32(v.w & 0xFFFFu) * e, bf16_bits_to_f32(v.w >> 16) * e);
  return c;
}

// Sign-only codes (block scale 0): nibble = 8 for a negative input, else 0.
__device__ __forceinline__ uint32_t signs8(u32x4 v) {
  uint32_t c = 0;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c |= ((w[j] >> 15) & 1u) << (8 * j + 3);
    c |= ((w[j] >> 31) & 1u) << (8 * j + 7);
  }
  return c;
}

// a / 6 in binary32, correctly rounded, for every bf16 value a >= 0: one
// multiply by RN(1/6) and two FMA corrections.  (Not for every binary32: some
// subnormal quotients differ; an exhaustive comparison over the bf16
// magnitudes with the IEEE division finds no difference.)
__device__ __forceinline__ float div6_bf16(float a) {
  const float c = 0x1.555556p-3f;
  const float q0 = a * c;
  const float r = __builtin_fmaf(-q0, 6.0f, a);
  return __builtin_fmaf(r, c, q0);
}

// Block scale byte E4M3_RNE_sat((a_b / 6) * s_enc) for a bf16 block max a_b:
// the same byte as e4m3_from_f32_rne, through the clamp and the packed
// hardware conversion.
__device__ __forceinline__ uint32_t block_scale_e4m3(float a_b, float s_enc) {
  const float t = div6_bf16(a_b) * s_enc;
  return __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fminf(t, 448.0f), 0.0f, 0, false) & 0xFFu;
}

// Encode factor e_S = 1 / (S * s_dec) of scale byte S (1..126), correctly
// rounded; 0 for S = 0, which makes encode8 give the sign-only codes (every
// product is a signed zero, and the conversion keeps the sign of zero).
// Kernels tabulate it once per tensor: 126 values replace a division per block.
__device__ __forceinline__ float encode_factor(uint32_t S, float s_dec) {
  return S == 0 || S > 0x7Eu ? 0.0f : 1.0f / (e4m3_to_f32(S) * s_dec);
}

// One 16-element block whose bf16 max |x| is a_b: scale byte S and 8 bytes of
// codes, with e_of[] the encode factors of every scale byte.  The same bytes
// as quantize_block.
__device__ __forceinline__ void quantize_block_tab(u32x4 lo, u32x4 hi, float a_b, bool degenerate,
                                                   float s_enc, const float* e_of, u32x2& c,
                                                   uint32_t& S) {
  S = degenerate ? 0u : block_scale_e4m3(a_b, s_enc);
  const float e = e_of[S];
  c = u32x2{encode8(lo, e), encode8(hi, e)};
}

// One 16-element block: scale byte and 8 bytes of codes.
__device__ __forceinline__ void quantize_block(u32x4 lo, u32x4 hi, bool degenerate, float s_enc,
                                               float s_dec, u32x2& c, uint32_t& S) {
  const u16x2 m = max_u16x2(max8(lo), max8(hi));
  const float a_b = bf16_bits_to_f32(m.x > m.y ? m.x : m.y);
  S = degenerate ? 0u : e4m3_from_f32_rne((a_b / 6.0f) * s_enc);
  if (S == 0) {
    c = u32x2{signs8(lo), signs8(hi)};
  } else {
    const float e = 1.0f / (e4m3_to_f32(S) * s_dec);
    c = u32x2{encode8(lo, e), encode8(hi, e)};
  }
}


// ------------------------------------------------------------ tile order --
// Workgroups are dealt to the 8 XCDs round-robin and each XCD has its own L2:
// tiles are renumbered so each XCD walks a contiguous range of the
// row-grouped order, and neighbouring tiles share operand panels in one L2.
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

// Position, in XCD-contiguous order, of workgroup b among the first T
// workgroups: they are dealt to the XCDs round-robin, so the ones on XCD k
// (b % 8 == k) take the k-th contiguous range of positions.
__device__ __forceinline__ int64_t xcd_order(int64_t b, int64_t T) {
  const int64_t xcd = b % kXcds, slot = b / kXcds;
  // workgroups with id % 8 == k: n_k = ceil((T - k) / 8); start_k = sum_{j<k} n_j
  int64_t start = 0;
  for (int64_t k = 0; k < xcd; ++k) start += (T - k + kXcds - 1) / kXcds;
  return start + slot;
}

// Tile (tm, tn) at position t of the row-grouped order: groups of kGroupM
// tile-rows, column-major inside a group, so neighbours share A and W panels.
__device__ __forceinline__ void grouped_tile(int64_t t, int64_t tiles_m, int64_t tiles_n,
                                             int64_t& tm, int64_t& tn) {
  const int64_t per_group = kGroupM * tiles_n;
  const int64_t group = t / per_group;
  const int64_t first_m = group * kGroupM;
  const int64_t gsize = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  const int64_t in_group = t - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// Split K for the tail of a tiled GEMM: workgroups 0 .. main_tiles-1 compute
// whole tiles; the remaining tiles are each split into `ways` ranges of K
// stages, one workgroup per range, whose fp32 partial sums go to their own
// slice of `part` for a second kernel to add in split order.
struct SplitK {
  float* part;         // [tail tiles][ways][BM][BN] fp32 partial sums
  int64_t main_tiles;  // tiles computed whole, by workgroups 0 .. main_tiles-1
  int ways;            // K ranges per tail tile (1: no split)
};

// Work item b: tile (tm, tn), and for a tail tile its index among the tail
// tiles and its split (split < 0 for a whole tile).  Item b runs on XCD b % 8
// (one item per workgroup, or a persistent grid that is a multiple of 8).
__device__ __forceinline__ void split_coords_of(int64_t b, int64_t tiles_m, int64_t tiles_n,
                                                const SplitK& sk, int64_t& tm, int64_t& tn,
                                                int64_t& tail, int& split) {
  if (b < sk.main_tiles) {
    grouped_tile(xcd_order(b, sk.main_tiles), tiles_m, tiles_n, tm, tn);
    tail = -1;
    split = -1;
  } else {
    const int64_t u = b - sk.main_tiles;
    tail = u / sk.ways;
    split = (int)(u - tail * sk.ways);
    grouped_tile(sk.main_tiles + tail, tiles_m, tiles_n, tm, tn);
  }
}

// Work of this workgroup (one item per workgroup).
__device__ __forceinline__ void split_coords(int64_t tiles_m, int64_t tiles_n, const SplitK& sk,
                                             int64_t& tm, int64_t& tn, int64_t& tail,
                                             int& split) {
  split_coords_of(blockIdx.x, tiles_m, tiles_n, sk, tm, tn, tail, split);
}

// Tile index of this workgroup: XCD-contiguous ranges, then row-grouped order.
__device__ __forceinline__ void tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                            int64_t& tn) {
  grouped_tile(xcd_order(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
}

}  // namespace nvfp4
