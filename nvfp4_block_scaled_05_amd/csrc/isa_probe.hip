// Probes of the gfx950 conversions the NVFP4 kernels rely on, exposed through
// isa_probe.h (beside this file) so tests can compare them with the CPU oracle on
// every input the kernels can give them.  Each probe calls the same device
// helpers the kernels call (device_common.hpp), never a copy of them.
//
//   * E2M1 encode (quantizer): a monotone step function of the binary32 bit
//     pattern, so scanning every pattern of a range and reporting where the
//     code changes characterises it completely.  All four byte positions of
//     the packed conversion are exercised and must agree.
//   * E4M3 encode (quantizer, integer arithmetic): the same scan.
//   * E4M3 encode of the FP8 row quantizer (clamp to 448, packed hardware
//     conversion): the same scan, all four byte positions.
//   * E2M1 decode to fp16 / fp32 and E4M3 decode to fp16 / fp32 (GEMM
//     loader, dequantizer): every byte value in every byte position.
//   * The block-scale path of the single-pass quantizer (a / 6 by FMA
//     corrections, the hardware E4M3 conversion, encode factor 0 for scale
//     byte 0): every bf16 pattern.
#include "device_common.hpp"
#include "isa_probe.h"

namespace {

using namespace nvfp4;

template <int MODE>
__device__ __forceinline__ uint32_t probe_code(uint32_t bits) {
  const float v = __uint_as_float(bits);
  if constexpr (MODE == 0) {
    // pack the same value into both nibbles of each byte position
    uint32_t w = 0;
    w = e2m1_pack2<0>(w, v, v);
    w = e2m1_pack2<1>(w, v, v);
    w = e2m1_pack2<2>(w, v, v);
    w = e2m1_pack2<3>(w, v, v);
    return w;   // 8 nibbles that must all be equal
  } else if constexpr (MODE == 1) {
    return e4m3_from_f32_rne(v);
  } else {
    // the FP8 row quantizer's element encode: clamp to 448, then the packed
    // conversion; the same value in all four byte positions
    const float c = __builtin_fminf(v, 448.0f);
    return e4m3_pack4(c, c, c, c);
  }
}

template <int MODE>
__global__ __launch_bounds__(256) void transitions_kernel(uint32_t lo, uint32_t nchunks,
                                                          uint32_t* list, uint32_t cap,
                                                          uint32_t* count, uint32_t* mismatch) {
  const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nchunks) return;
  const uint32_t base = lo + (uint32_t)(t * 256u);
  uint32_t prev = 0;
  for (uint32_t i = 0; i <= 256; ++i) {
    const uint32_t p = base + i;
    uint32_t c = probe_code<MODE>(p);
    if constexpr (MODE == 0) {
      if (c != (c & 0xFu) * 0x11111111u) atomicAdd(mismatch, 1u);
      c &= 0xFu;
    } else if constexpr (MODE == 2) {
      if (c != (c & 0xFFu) * 0x01010101u) atomicAdd(mismatch, 1u);
      c &= 0xFFu;
    }
    if (i > 0 && c != prev) {
      const uint32_t slot = atomicAdd(count, 1u);
      if (slot < cap) {
        list[3 * slot] = p;
        list[3 * slot + 1] = prev;
        list[3 * slot + 2] = c;
      }
    }
    prev = c;
  }
}

template <int MODE>
__global__ __launch_bounds__(256) void encode_kernel(const uint32_t* bits, int n, uint32_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = probe_code<MODE>(bits[i]);
}

// For item i (word w = words[i], E4M3 byte b = sbytes[i] & 0xFF):
//   e2m1_f16 [i][8]: the GEMM operand decode8(w, fp16(b)), element 0 first;
//   e2m1_f32 [i][8]: the dequantizer's E2M1 -> fp32 conversion of w;
//   e4m3_f16 [i][4]: the four bytes of w as E4M3 through the hardware pair
//                    conversion the GEMM loader uses;
//   e4m3_f32 [i][4]: the four bytes of w through the integer E4M3 decoder.
// Outputs are written as whole packed words.
__global__ __launch_bounds__(256) void decode_kernel(const uint32_t* words, const uint32_t* sbytes,
                                                     int n, uint32_t* e2m1_f16, float* e2m1_f32,
                                                     uint32_t* e4m3_f16, float* e4m3_f32) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t w = words[i];
  const uint32_t sp = __builtin_bit_cast(uint32_t, e4m3_pair_to_f16x2<false>(sbytes[i] & 0xFFu));
  const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)(sp & 0xFFFFu));
  const u32x4 d = __builtin_bit_cast(u32x4, decode8(w, s));
  reinterpret_cast<u32x4*>(e2m1_f16)[i] = d;
  const f32x2 f[4] = {e2m1_unpack2_f32<0>(w), e2m1_unpack2_f32<1>(w), e2m1_unpack2_f32<2>(w),
                      e2m1_unpack2_f32<3>(w)};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    e2m1_f32[8 * i + 2 * j] = f[j].x;
    e2m1_f32[8 * i + 2 * j + 1] = f[j].y;
  }
  e4m3_f16[2 * i] = __builtin_bit_cast(uint32_t, e4m3_pair_to_f16x2<false>(w));
  e4m3_f16[2 * i + 1] = __builtin_bit_cast(uint32_t, e4m3_pair_to_f16x2<true>(w));
#pragma unroll
  for (int j = 0; j < 4; ++j) e4m3_f32[4 * i + j] = e4m3_to_f32((w >> (8 * j)) & 0xFFu);
}

// bf16[i] = bf16 rounding of in[i] through the epilogue's packed conversion
// (pairs i, i+1 converted together); gelu[i] = the epilogue's GELU of in[i].
__global__ __launch_bounds__(256) void bf16_gelu_kernel(const float* in, int n, uint32_t* bf16,
                                                        float* gelu) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (2 * i + 1 < n) bf16[i] = bf16x2_rne(in[2 * i], in[2 * i + 1]);
  if (i < n) gelu[i] = gelu_erf(in[i]);
  if (i + (n + 1) / 2 < n) gelu[i + (n + 1) / 2] = gelu_erf(in[i + (n + 1) / 2]);
}

// out[16 t .. 16 t + 15] = the GEMM epilogues' 16-wide GELU (gelu_erf16) of
// in[16 t .. 16 t + 15], one thread per 16 values.
__global__ __launch_bounds__(256) void gelu16_kernel(const float* in, int groups, float* out) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= groups) return;
  f32x4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = reinterpret_cast<const f32x4*>(in)[4 * t + u];
  gelu_erf16(v);
#pragma unroll
  for (int u = 0; u < 4; ++u) reinterpret_cast<f32x4*>(out)[4 * t + u] = v[u];
}

// For bf16 pattern h = bits[i] & 0xFFFF: quot[i] = div6_bf16(|h|) (the
// quotient behind the block scale), scale[i] = block_scale_e4m3(|h|, s_enc),
// zero_codes[i] = encode8 of eight copies of h with encode factor 0 (the
// codes of a block whose scale byte is 0).
__global__ __launch_bounds__(256) void block_scale_kernel(const uint32_t* bits, int n, float s_enc,
                                                          float* quot, uint32_t* scale,
                                                          uint32_t* zero_codes) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t h = bits[i] & 0xFFFFu;
  const float a = bf16_bits_to_f32(h & 0x7FFFu);
  quot[i] = div6_bf16(a);
  scale[i] = block_scale_e4m3(a, s_enc);
  const uint32_t w = h | (h << 16);
  zero_codes[i] = encode8(u32x4{w, w, w, w}, 0.0f);
}

bool bad_ptr(const void* p) { return p == nullptr; }

}  // namespace

extern "C" {

int nvfp4_probe_transitions(int which, uint32_t lo, uint32_t nchunks, uint32_t* list, uint32_t cap,
                            uint32_t* count, uint32_t* mismatch, void* stream) {
  if (bad_ptr(list) || bad_ptr(count) || bad_ptr(mismatch)) return -1;
  if (which < 0 || which > 2 || nchunks == 0 || (uint64_t)lo + (uint64_t)nchunks * 256u > 0xFFFFFFFFull)
    return -2;
  const dim3 grid((nchunks + 255) / 256), block(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (which == 0)
    hipLaunchKernelGGL(transitions_kernel<0>, grid, block, 0, s, lo, nchunks, list, cap, count, mismatch);
  else if (which == 1)
    hipLaunchKernelGGL(transitions_kernel<1>, grid, block, 0, s, lo, nchunks, list, cap, count, mismatch);
  else
    hipLaunchKernelGGL(transitions_kernel<2>, grid, block, 0, s, lo, nchunks, list, cap, count, mismatch);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int nvfp4_probe_encode(int which, const uint32_t* bits, int n, uint32_t* out, void* stream) {
  if (bad_ptr(bits) || bad_ptr(out)) return -1;
  if (which < 0 || which > 2 || n <= 0) return -2;
  const dim3 grid((n + 255) / 256), block(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (which == 0)
    hipLaunchKernelGGL(encode_kernel<0>, grid, block, 0, s, bits, n, out);
  else if (which == 1)
    hipLaunchKernelGGL(encode_kernel<1>, grid, block, 0, s, bits, n, out);
  else
    hipLaunchKernelGGL(encode_kernel<2>, grid, block, 0, s, bits, n, out);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int nvfp4_probe_decode(const uint32_t* words, const uint32_t* sbytes, int n, uint16_t* e2m1_f16,
                       float* e2m1_f32, uint16_t* e4m3_f16, float* e4m3_f32, void* stream) {
  if (bad_ptr(words) || bad_ptr(sbytes) || bad_ptr(e2m1_f16) || bad_ptr(e2m1_f32) ||
      bad_ptr(e4m3_f16) || bad_ptr(e4m3_f32))
    return -1;
  if (n <= 0) return -2;
  hipLaunchKernelGGL(decode_kernel, dim3((n + 255) / 256), dim3(256), 0,
                     static_cast<hipStream_t>(stream), words, sbytes, n,
                     reinterpret_cast<uint32_t*>(e2m1_f16), e2m1_f32,
                     reinterpret_cast<uint32_t*>(e4m3_f16), e4m3_f32);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int nvfp4_probe_bf16_gelu(const float* in, int n, uint16_t* bf16, float* gelu, void* stream) {
  if (bad_ptr(in) || bad_ptr(bf16) || bad_ptr(gelu)) return -1;
  if (n <= 0 || (n & 1)) return -2;
  const int threads = (n + 1) / 2;
  hipLaunchKernelGGL(bf16_gelu_kernel, dim3((threads + 255) / 256), dim3(256), 0,
                     static_cast<hipStream_t>(stream), in, n, reinterpret_cast<uint32_t*>(bf16), gelu);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int nvfp4_probe_gelu16(const float* in, int n, float* out, void* stream) {
  if (bad_ptr(in) || bad_ptr(out)) return -1;
  if (n <= 0 || (n % 16)) return -2;
  if ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15) return -3;
  const int groups = n / 16;
  hipLaunchKernelGGL(gelu16_kernel, dim3((groups + 255) / 256), dim3(256), 0,
                     static_cast<hipStream_t>(stream), in, groups, out);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int nvfp4_probe_block_scale(const uint32_t* bits, int n, float s_enc, float* quot, uint32_t* scale,
                            uint32_t* zero_codes, void* stream) {
  if (bad_ptr(bits) || bad_ptr(quot) || bad_ptr(scale) || bad_ptr(zero_codes)) return -1;
  if (n <= 0) return -2;
  hipLaunchKernelGGL(block_scale_kernel, dim3((n + 255) / 256), dim3(256), 0,
                     static_cast<hipStream_t>(stream), bits, n, s_enc, quot, scale, zero_codes);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
