/*
 * calib.h -- measurement probes for the roofline figures (library
 * lib/libnvfp4_probes.so, not part of the NVFP4 computation; nothing in
 * libnvfp4.so calls them).  They measure what this particular part sustains,
 * next to the published peaks: the fp16 matrix-core rate, the shader clock
 * under that load, and the HBM streaming rates, each with a kernel whose work
 * is known exactly.
 *
 * All pointers are device pointers; calls enqueue on `stream` (a hipStream_t,
 * NULL = null stream) and return 0, -1 for a NULL pointer, -2 for a bad size,
 * -3 for a misaligned pointer, -7 for a launch failure.
 */
#ifndef NVFP4_CALIB_H
#define NVFP4_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Compute units of the current device (the grid of nvfp4_calib_mfma_f16). */
int nvfp4_calib_units(void);

/*
 * fp16 matrix-core loop: one workgroup of 4 waves per compute unit (one wave
 * per SIMD), each wave issuing `iters` rounds of 16 independent
 * v_mfma_f32_32x32x16_f16 (32x32x16: 32768 FLOP each) into 16 accumulator
 * tiles, nothing else inside the loop.  FLOP of the launch:
 *   units * 4 * iters * 16 * 32768.
 * mode 0: every MFMA multiplies the same two constant fragments;
 * mode 1: 4 A and 4 B fragments of pseudo-random fp16 values in (-1, 1), a
 *         different (A, B) pair for each accumulator (data-bearing operands,
 *         which draw more power than constant ones);
 * mode 2: as mode 1 with values shaped like decoded NVFP4 operands: a random
 *         signed E2M1 value times a random E4M3-like scale (at most 6
 *         significant bits, the operands the block-scaled GEMM feeds its
 *         MFMAs).
 *   sink    out, units * 256 floats (one sum of accumulators per lane).
 *   clocks  out, units * 4 pairs of uint64: per wave, the shader-clock
 *           counter (s_memtime) and the 100 MHz real-time counter
 *           (s_memrealtime) elapsed over the loop; their ratio times 100 MHz
 *           is the shader clock the wave ran at.
 */
int nvfp4_calib_mfma_f16(int iters, int mode, float* sink, uint64_t* clocks, void* stream);

/*
 * Streaming read of `bytes` (a multiple of 16; src 16-byte aligned): every
 * 16-byte word loaded once, 8 loads in flight per thread, XOR-folded into one
 * word per workgroup written to sink[blockIdx] (sink: 4096 words).
 */
int nvfp4_calib_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * Streaming copy of `bytes` (a multiple of 16; both 16-byte aligned): every
 * 16-byte word read once and written once.  Also the known-size kernel the
 * HBM byte counters are calibrated against.
 */
int nvfp4_calib_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_CALIB_H */
