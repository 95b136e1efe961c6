/*
 * isa_probe.h -- test-only probes of the gfx950 conversion helpers the
 * NVFP4 kernels use (library lib/libnvfp4_probes.so).  They let a test
 * compare each helper with the CPU oracle on every input the kernels can give
 * it.  Not part of the NVFP4 computation; nothing in libnvfp4.so calls them.
 *
 * All pointers are device pointers; calls enqueue on `stream` (a hipStream_t,
 * NULL = null stream) and return 0, -1 for a NULL pointer, -2 for a bad size
 * or selector, -7 for a launch failure.
 */
#ifndef NVFP4_ISA_PROBE_H
#define NVFP4_ISA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* which = 0: E2M1 encode of binary32 patterns through the packed conversion
 *            (all four byte positions, both nibbles; a disagreement between
 *            them increments *mismatch);
 * which = 1: E4M3 encode of binary32 patterns (the quantizer's block scale);
 * which = 2: E4M3 encode of the FP8 row quantizer (min(v, 448) through the
 *            packed hardware conversion, all four byte positions; a
 *            disagreement between them increments *mismatch).
 * Scans the bit patterns lo .. lo + 256*nchunks (must not pass 2^32 - 1) and
 * appends every pattern p whose code differs from that of p - 1 to `list` as
 * the triple (p, code(p-1), code(p)), up to `cap` triples; *count receives the
 * total number found (zero *count and *mismatch before the call). */
int nvfp4_probe_transitions(int which, uint32_t lo, uint32_t nchunks, uint32_t* list,
                            uint32_t cap, uint32_t* count, uint32_t* mismatch, void* stream);

/* out[i] = encode(bits[i]) for n patterns (which as above; for E2M1 the eight
 * nibbles of the packed word are returned). */
int nvfp4_probe_encode(int which, const uint32_t* bits, int n, uint32_t* out, void* stream);

/* For n items (word w = words[i], E4M3 byte b = sbytes[i] & 0xFF):
 *   e2m1_f16 [n][8]: the eight E2M1 codes of w (low nibble of byte 0 first)
 *                    times E4M3 value b, as the GEMM decodes its operands (fp16
 *                    bits);
 *   e2m1_f32 [n][8]: the eight codes of w as the dequantizer decodes them;
 *   e4m3_f16 [n][4] / e4m3_f32 [n][4]: the four bytes of w as E4M3, through
 *                    the hardware pair conversion (fp16 bits) and the integer
 *                    decoder (fp32).  16-byte aligned e2m1_f16, 4-byte others. */
int nvfp4_probe_decode(const uint32_t* words, const uint32_t* sbytes, int n, uint16_t* e2m1_f16,
                       float* e2m1_f32, uint16_t* e4m3_f16, float* e4m3_f32, void* stream);

/* For n (even) binary32 inputs: bf16[i] = their bf16 rounding through the GEMM
 * epilogue's packed conversion (4-byte aligned output); gelu[i] = the
 * epilogue's erf-form GELU. */
int nvfp4_probe_bf16_gelu(const float* in, int n, uint16_t* bf16, float* gelu, void* stream);

/* For n binary32 inputs (n > 0, n % 16 == 0; in and out 16-byte aligned):
 * out[i] = the GEMM epilogues' GELU taken 16 values at a time, one step
 * across all 16 before the next (the operations of the scalar GELU above, in
 * another order across values).  Returns 0, -1 on a null pointer, -2 on a bad
 * n, -3 on misalignment, -7 on a launch failure. */
int nvfp4_probe_gelu16(const float* in, int n, float* out, void* stream);

/* For n bf16 patterns h = bits[i] & 0xFFFF (4-byte aligned outputs):
 *   quot[i]       = the quantizer's a / 6 of a = |h| (one multiply, two FMA
 *                   corrections);
 *   scale[i]      = its block scale byte E4M3((a / 6) * s_enc) through the
 *                   clamp and the hardware conversion;
 *   zero_codes[i] = the packed E2M1 codes of eight copies of h encoded with
 *                   factor 0 (a block whose scale byte is 0). */
int nvfp4_probe_block_scale(const uint32_t* bits, int n, float s_enc, float* quot,
                            uint32_t* scale, uint32_t* zero_codes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_ISA_PROBE_H */
