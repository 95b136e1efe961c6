/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 library: two-level NVFP4
 * quantize / dequantize, the block-scaled W4A4 GEMM that consumes the
 * quantized operands, a bf16 passthrough GEMM for layers kept in higher
 * precision, and the layer predicate that chooses between the two.
 *
 * Sources.  The pages this library follows describe NVFP4 only in outline:
 *   [P1] "英伟达B200狂飙10.2倍！AI绘图告别龟速！" (nmedialink.com), section
 *        "NVFP4量化：在精度与速度之间寻得最佳平衡": two-level micro-block
 *        scaling, an FP32 per-tensor scale (static or dynamic), a per-block
 *        scale computed dynamically over blocks of 16 elements, the
 *        exclude_pattern regex naming layers kept in higher precision, and
 *        apply_visual_gen_linear(load_parameters, quantize_weights, ...).
 *   [P2] "NVIDIA介绍用TensorRT LLM VisualGen加速Blackwell上的FLUX 3 Image
 *        Klein" (sns.style), time-breakdown paragraph: NVFP4 weights in the
 *        DiT linear layers; a tuned NVFP4 GEMM kernel.
 *   [P3] "NVIDIA показала, как сократить генерацию FLUX 3 Image Klein с 22 до
 *        6 секунд" (xalabuda.com), section "Квантование NVFP4 и оптимизация
 *        вычислительных ядер": NVFP4 GEMM kernels for the linear layers.
 * The element and scale encodings are those of the NVFP4 format: E2M1 4-bit
 * elements (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; sign in bit 3), two per
 * byte with the lower-indexed element in the low nibble, and one E4M3 (OCP
 * "fn", max 448) byte per 16-element block.
 *
 * Conventions shared by every call:
 *   - All tensors are row-major and contiguous.  A weight is [N, K] (the
 *     nn.Linear layout), so a linear layer computes Y = X * W^T.
 *   - Every pointer argument except `layer_name` and `pattern` is a DEVICE
 *     pointer on the current HIP device.  The caller owns every buffer; the
 *     library never allocates or frees memory and keeps no state beyond a
 *     cached per-device architecture check.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work on it and return without synchronizing.  Outputs are ready when the
 *     stream reaches that point.
 *   - Every call returns an nvfp4_status synchronously.  Checks run in the
 *     order: null pointers -> shapes -> alignment -> workspace -> device ->
 *     launch, and all argument checks happen before any HIP call, so a bad
 *     argument is reported without touching the GPU.  A launch failure is
 *     reported as NVFP4_ERR_HIP.  Data-dependent errors (Inf / NaN input) are
 *     reported on the device through the optional `dev_status` word.
 *   - Sizes are elements unless named *_bytes.  A zero row count is a no-op
 *     that returns NVFP4_OK.
 *   - Calls on one stream are ordered; calls that share output buffers on
 *     different streams race.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 6
#define NVFP4_BLOCK 16 /* elements per block scale, [P1] "NVFP4量化" */

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = -1,      /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = -2,     /* negative size, or cols / K not a positive multiple of 16 */
  NVFP4_ERR_ALIGN = -3,     /* a pointer misses its required alignment */
  NVFP4_ERR_WORKSPACE = -4, /* workspace smaller than nvfp4_quantize_workspace_bytes() */
  NVFP4_ERR_DEVICE = -5,    /* no HIP device, or the current device is not gfx950 */
  NVFP4_ERR_ARG = -6,       /* unknown epilogue or other invalid argument */
  NVFP4_ERR_HIP = -7,       /* a HIP launch or runtime call failed */
  NVFP4_ERR_NONFINITE = -8  /* (device status word only) Inf or NaN in the input */
} nvfp4_status;

typedef enum {
  NVFP4_EPI_NONE = 0, /* y = acc * sA * sW + bias */
  NVFP4_EPI_GELU = 1  /* y = gelu_erf(acc * sA * sW + bias), gelu_erf(z) = z/2 (1 + erf(z/sqrt 2)) */
} nvfp4_epilogue;

/* NVFP4_ABI_VERSION of the loaded library. */
int nvfp4_abi_version(void);

/* Static, NUL-terminated text for a status code (never NULL). */
const char* nvfp4_status_string(int status);

/* Bytes of device workspace nvfp4_quantize needs for a [rows, cols] input when
 * it computes the tensor amax itself (amax_in == NULL): 8192 (the single-pass
 * kernel's arrival counters, release words and partial slots, then the
 * two-pass kernels' partial maxima).  0 when rows or cols is not positive. */
size_t nvfp4_quantize_workspace_bytes(int64_t rows, int64_t cols);

/*
 * nvfp4_quantize -- two-level NVFP4 quantization of a bf16 tensor
 * ([P1] "NVFP4量化": an FP32 per-tensor scale plus a scale computed
 * dynamically for every block of 16 elements; here along each row).
 *
 *   x_bf16        [rows, cols] bf16, 16-byte aligned.
 *   rows, cols    rows >= 0; cols > 0 and cols % 16 == 0.
 *   codes         out [rows, cols/2] bytes: element 2j in the low nibble of
 *                 byte j, element 2j+1 in the high nibble; 8-byte aligned.
 *   scales        out [rows, cols/16] E4M3 bytes, row-major.
 *   tensor_scale  out, 1 float: the stored FP32 per-tensor scale s_dec.
 *   amax_in       NULL: the tensor amax = max|x| is computed here (uses
 *                 `workspace`).  Non-NULL: 1 device float holding the amax
 *                 as a producer computed it (the GEMM epilogue's y_amax);
 *                 the input is then read once.
 *   workspace     device scratch of at least nvfp4_quantize_workspace_bytes()
 *                 bytes, 8-byte aligned, needed only when amax_in == NULL.
 *                 It must be zero-filled once before its first use; every
 *                 call leaves it valid for the next, so a workspace kept for
 *                 reuse is never cleared again (no clearing launch per
 *                 call).  It belongs to one device, and calls that share it
 *                 must be ordered (one stream).  With other contents the
 *                 results are unspecified.
 *   dev_status    optional device int32: written with NVFP4_OK, or
 *                 NVFP4_ERR_NONFINITE when the amax is Inf / NaN, in which
 *                 case *tensor_scale is set to NaN and codes / scales are
 *                 left unspecified.
 *
 * The arithmetic, in binary32 round-to-nearest-even:
 *   amax < 2^-96 (all-zero input included): s_enc = s_dec = 1, every scale 0.
 *   otherwise s_enc = 2688 / amax, s_dec = 1 / s_enc      (2688 = 6 * 448)
 *   per block b: a_b = max|x| over the block;  S_b = E4M3((a_b / 6) * s_enc),
 *     nearest-even, saturating at 448;
 *   S_b == 0: every code is its input's sign bit (code 8 for negatives);
 *   else e_b = 1 / (S_b * s_dec), code = sign | E2M1(|x| * e_b), nearest-even,
 *     saturating at 6.
 * Deterministic: the same input gives the same bytes on every call.
 * rows == 0: nothing is launched and *tensor_scale is not written.
 * When the amax is computed here and the tensor has more than 262,144
 * elements and fits on chip (at most 212,992 elements per compute unit: 54.5 M
 * elements, 109 MB of bf16, on 256 units), it is read from HBM once: one
 * workgroup per compute unit holds its share on chip while the amax is
 * agreed, then encodes it.  The workgroups of that kernel wait for each other; if another
 * stream's work keeps some of them from starting, the waiting ones time out
 * after 200 us and compute the amax themselves, so the call still completes
 * with the same bytes, only slower.  A tensor of at most 262,144 elements
 * is quantized in one launch whose workgroups each fold the whole amax
 * themselves.  Other sizes take two passes over the input.
 * NVFP4_QUANT_KERNEL=twopass|resident|small (environment) forces a kernel.
 */
int nvfp4_quantize(const void* x_bf16, int64_t rows, int64_t cols,
                   uint8_t* codes, uint8_t* scales, float* tensor_scale,
                   const float* amax_in, void* workspace, size_t workspace_bytes,
                   int32_t* dev_status, void* stream);

/*
 * nvfp4_quantize_no_alloc -- nvfp4_quantize with the amax computed here and
 * no workspace argument: for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It allocates nothing: its kernels use a scratch array the
 * library owns, 8192 bytes per GPU (the whole of what the quantizer needs
 * for any input this ABI accepts), created zero-filled when the library's
 * code object is loaded on that GPU and kept until the process ends.
 *
 *   x_bf16, rows, cols, codes, scales, tensor_scale, dev_status
 *                 as nvfp4_quantize (same checks, same bytes).
 * Every call on one GPU shares that GPU's scratch, and each call leaves it
 * ready for the next, so calls on one GPU must be ordered (one stream, or
 * explicit synchronization); calls that overlap on one GPU race.  Returns
 * NVFP4_ERR_WORKSPACE if an input ever needed more scratch than the array
 * holds (none does), NVFP4_ERR_HIP if the array's device address cannot be
 * looked up (once per device, on the first call there).
 */
int nvfp4_quantize_no_alloc(const void* x_bf16, int64_t rows, int64_t cols, uint8_t* codes,
                            uint8_t* scales, float* tensor_scale, int32_t* dev_status,
                            void* stream);

/*
 * nvfp4_dequantize -- NVFP4 back to bf16.  [P1] "NVFP4量化" defines what a
 * quantized element stands for under the two-level scaling: its 4-bit value
 * times its 16-element block's scale times the FP32 per-tensor scale.  This
 * call computes that value and rounds it to bf16:
 *   y = bf16_rne( (value(code) * S_b) * s_dec ), binary32 products (the first
 *   is exact; the order of the two products is this library's reading, since
 *   the page gives no formula).
 *
 *   codes         [rows, cols/2] bytes, element 2j in the low nibble of byte
 *                 j (as written by nvfp4_quantize); 8-byte aligned.
 *   scales        [rows, cols/16] E4M3 bytes.
 *   tensor_scale  1 device float: s_dec.
 *   rows, cols    rows >= 0; cols > 0 and cols % 16 == 0.
 *   y_bf16        out [rows, cols] bf16, 16-byte aligned.
 * Code 8 (negative zero) gives -0.0.  Errors: NVFP4_ERR_NULL, _SHAPE, _ALIGN,
 * _DEVICE, _HIP as for every call; nothing is data-dependent.
 */
int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales,
                     const float* tensor_scale, int64_t rows, int64_t cols,
                     void* y_bf16, void* stream);

/*
 * nvfp4_gemm -- block-scaled W4A4 GEMM of a DiT linear layer
 * ([P2] time-breakdown paragraph; [P3] "Квантование NVFP4 ..."):
 *
 *   Y[m,n] = bf16_rne( epi( sA * sW * sum_k Ahat[m,k] * What[n,k] + bias[n] ) )
 *
 * with Ahat = value(codeA) * S_A[m, k/16] and What = value(codeW) *
 * S_W[n, k/16] decoded exactly (each product of an E2M1 value and an E4M3
 * scale is exact in fp16), fp32 accumulation, and the per-tensor scales
 * sA = *a_tensor_scale, sW = *w_tensor_scale applied once in the epilogue.
 *
 *   a_codes/a_scales  [M, K/2] / [M, K/16] as written by nvfp4_quantize.
 *   w_codes/w_scales  [N, K/2] / [N, K/16].
 *   bias_bf16         optional [N] bf16.
 *   M, N >= 0; K > 0, K % 16 == 0.  Code pointers 8-byte aligned.
 *   epilogue          an nvfp4_epilogue value.
 *   y_bf16            out [M, N] bf16, 2-byte aligned; any N >= 0.
 *   y_amax            optional device float: set to max |Y| over the bf16
 *                     outputs (the call zeroes it first, on `stream`), ready
 *                     to be passed as amax_in of the next nvfp4_quantize.
 *                     A NaN output makes it non-finite, which that quantize
 *                     then reports as NVFP4_ERR_NONFINITE.
 *   workspace         optional device scratch, 256-byte aligned, owned by the
 *                     call until it completes on `stream`; contents on entry
 *                     irrelevant.  With at least nvfp4_gemm_workspace_bytes
 *                     (M, N, K) bytes the tiles that do not fill a whole round
 *                     of workgroups over the compute units are split over K
 *                     and their fp32 partial sums added there, in a fixed
 *                     order, by a second kernel on `stream`; NULL or a
 *                     smaller size computes every tile whole.  Either way the
 *                     result is deterministic; the two differ only in the
 *                     order of the fp32 additions.
 */
int nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
               const uint8_t* w_codes, const uint8_t* w_scales, const float* w_tensor_scale,
               const void* bias_bf16, int64_t M, int64_t N, int64_t K, int epilogue,
               void* y_bf16, float* y_amax, void* workspace, size_t workspace_bytes,
               void* stream);

/*
 * nvfp4_gemm_quantized -- the same GEMM with its output written in NVFP4
 * under a static (calibrated) per-tensor scale ([P1] "NVFP4量化": the FP32
 * tensor scale may be computed statically or dynamically), so the next
 * layer's activation needs no bf16 round trip and no quantize pass.
 *
 * The bytes are exactly those of nvfp4_gemm (same inputs, bf16 Y) followed
 * by nvfp4_quantize(Y, amax_in = y_amax): every output value is first rounded
 * to bf16, then quantized in 16-element blocks along each row.
 *
 *   inputs, bias, M, N, K, epilogue  as nvfp4_gemm; additionally N % 16 == 0.
 *   y_amax           device float, the static amax the tensor scale is
 *                    derived from (s_enc = 2688 / amax, as in
 *                    nvfp4_quantize); values above it saturate.  An Inf / NaN
 *                    amax sets *y_tensor_scale to NaN and leaves the codes
 *                    unspecified.
 *   y_codes          out [M, N/2] bytes, 8-byte aligned.
 *   y_scales         out [M, N/16] E4M3 bytes.
 *   y_tensor_scale   out, 1 float (s_dec).
 * Tiles are computed whole (no K split).  M == 0 or N == 0: nothing is
 * launched and *y_tensor_scale is not written (as nvfp4_quantize with no rows).
 */
int nvfp4_gemm_quantized(const uint8_t* a_codes, const uint8_t* a_scales,
                         const float* a_tensor_scale, const uint8_t* w_codes,
                         const uint8_t* w_scales, const float* w_tensor_scale,
                         const void* bias_bf16, int64_t M, int64_t N, int64_t K, int epilogue,
                         const float* y_amax, uint8_t* y_codes, uint8_t* y_scales,
                         float* y_tensor_scale, void* stream);

/*
 * nvfp4_gemm_workspace_bytes -- workspace bytes nvfp4_gemm can use for an
 * (M, N, K) problem on the current device (0: it would not split).  Host
 * only; at most 256 KiB per compute unit (64 MiB on a 256-CU device).
 */
size_t nvfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * The FP8 row-wise variant ("fp8r").  [P3] selects FP8 as the other quantized
 * variant of the model (the paragraph on run options) and gives no recipe;
 * here it is FP8 with row-wise scales: one FP32 scale per row of the
 * activation (per token, dynamic on every call) and per row of the weight
 * (per output channel, when the weights are loaded), E4M3 elements (sign in
 * bit 7), and a GEMM on the native FP8 matrix cores with the two row scales
 * applied in the epilogue.
 *
 * nvfp4_fp8_quantize_rowwise -- per row r of x [rows, cols]:
 *   amax_r = max|x|;  s_r = 448 / amax_r;  d_r = 1 / s_r  (binary32, RNE);
 *   amax_r < 2^-96: s_r = d_r = 1;
 *   codes[r, k] = sign(x) << 7 | E4M3(|x| * s_r), nearest-even, saturating.
 *   x_bf16      [rows, cols] bf16, 16-byte aligned; cols > 0, cols % 16 == 0.
 *   codes       out [rows, cols] E4M3 bytes, 8-byte aligned.
 *   row_scales  out [rows] float: d_r.
 *   dev_status  optional device int32: NVFP4_OK, or NVFP4_ERR_NONFINITE if a
 *               row holds Inf / NaN (that row's scale is NaN, its codes
 *               unspecified).
 */
int nvfp4_fp8_quantize_rowwise(const void* x_bf16, int64_t rows, int64_t cols, uint8_t* codes,
                               float* row_scales, int32_t* dev_status, void* stream);

/*
 * nvfp4_fp8_gemm -- Y[m,n] = bf16_rne( epi( (sum_k value(A[m,k]) * value(W[n,k]))
 *                                            * (a_scales[m] * w_scales[n]) + bias[n] ) ),
 * fp32 accumulation of the exact E4M3 products, the scale product in binary32.
 *   a_codes / a_scales  [M, K] / [M] from nvfp4_fp8_quantize_rowwise;
 *   w_codes / w_scales  [N, K] / [N];  code pointers 16-byte aligned.
 *   bias_bf16 optional [N];  M, N >= 0, K > 0, K % 16 == 0.
 *   y_bf16 out [M, N] bf16, 2-byte aligned.
 *   workspace  optional device scratch, 256-byte aligned, owned by the call
 *              until it completes on `stream`; contents on entry irrelevant.
 *              With at least nvfp4_fp8_gemm_workspace_bytes(M, N, K) bytes the
 *              tiles past the last whole round of workgroups over the compute
 *              units are split over K and their fp32 partial sums added there,
 *              in a fixed order, by a second kernel on `stream`; NULL or a
 *              smaller size computes every tile whole.  Either way the result
 *              is deterministic; the two differ only in the order of the fp32
 *              additions.
 */
int nvfp4_fp8_gemm(const uint8_t* a_codes, const float* a_scales, const uint8_t* w_codes,
                   const float* w_scales, const void* bias_bf16, int64_t M, int64_t N, int64_t K,
                   int epilogue, void* y_bf16, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * nvfp4_fp8_gemm_workspace_bytes -- workspace bytes nvfp4_fp8_gemm can use for
 * an (M, N, K) problem on the current device (0: it would not split).  Host
 * only; at most 256 KiB per compute unit (64 MiB on a 256-CU device).
 */
size_t nvfp4_fp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * nvfp4_gemm_bf16 -- the bf16 passthrough for layers kept in higher precision
 * ([P1] "NVFP4量化": chosen layers keep their original precision):
 *   Y[m,n] = bf16_rne( epi( sum_k X[m,k] * W[n,k] + bias[n] ) ), fp32 accumulation.
 *   x_bf16 [M, K], w_bf16 [N, K], bias_bf16 optional [N], y_bf16 [M, N];
 *   M, N >= 0, K > 0, K % 8 == 0; x / w 16-byte aligned, bias / y 2-byte aligned.
 * Kernels:
 *   - M <= 8: the weight is streamed once (one pass, no tiles).
 *   - 256x256 tiles loaded straight into LDS: when they cover at least half
 *     the compute units, K % 64 == 0 and rows * K * 2 < 2^32 for both
 *     operands.
 *   - 128x128 tiles: otherwise.  When there are fewer of them than compute
 *     units, two wave groups split K inside each tile.
 * The 256x256 and plain 128x128 kernels sum in the same order and give
 * identical bits; the K split adds its two halves at the end.
 * NVFP4_BF16_GEMM_KERNEL=tile|dma|ksplit pins one of them (dma only where it
 * applies).  Returns 0, or an error code on invalid arguments or a launch
 * failure.
 */
int nvfp4_gemm_bf16(const void* x_bf16, const void* w_bf16, const void* bias_bf16,
                    int64_t M, int64_t N, int64_t K, int epilogue, void* y_bf16,
                    void* stream);

/*
 * Graph capture of a sequence of library calls.  [P1] section "CUDA Graphs"
 * runs the DiT forward pass as one graph launch instead of one launch per
 * kernel; these four calls do the same with HIP graphs for any sequence of
 * this library's calls (every kernel here is capture-safe: no memset nodes,
 * flags and counters are cleared or kept consistent by kernels).
 *
 * nvfp4_graph_begin  starts capturing what later calls enqueue on `stream`
 *                    (a stream the caller created; the null stream cannot be
 *                    captured).  Thread-local capture: other threads' HIP
 *                    calls are unaffected; this thread must not allocate
 *                    device memory until nvfp4_graph_end.
 * nvfp4_graph_end    ends the capture on `stream` and instantiates it;
 *                    *graph receives an opaque handle.
 * nvfp4_graph_launch enqueues the captured kernels on `stream` (any stream),
 *                    with the pointers and sizes they were captured with:
 *                    refresh inputs in place between launches.
 * nvfp4_graph_destroy releases the handle.
 * Returns NVFP4_ERR_NULL for a NULL stream (begin / end) or graph, else
 * NVFP4_OK or NVFP4_ERR_HIP (capture or instantiation failed; a failed
 * nvfp4_graph_end leaves no capture running).
 */
int nvfp4_graph_begin(void* stream);
int nvfp4_graph_end(void* stream, void** graph);
int nvfp4_graph_launch(void* graph, void* stream);
int nvfp4_graph_destroy(void* graph);

/*
 * nvfp4_layer_is_quantized -- the exclude-pattern predicate of [P1]
 * "NVFP4量化".  Host only; touches no device.
 *   layer_name  NUL-terminated module path, e.g. "transformer_blocks.0.attn.to_q".
 *   pattern     NUL-terminated ECMAScript regex, or NULL for the page's
 *               pattern ^(?!.*(embedder|norm_out|proj_out|to_add_out|to_added_qkv|stream)).*
 * Returns 1 when the pattern matches a prefix of the name (the layer runs in
 * NVFP4), 0 when it does not (the layer stays bf16), NVFP4_ERR_NULL for a NULL
 * name, NVFP4_ERR_ARG for a pattern that does not compile or, with a pattern
 * given, a name longer than 1024 bytes (the regex engine's recursion grows
 * with the name).  The default pattern is evaluated as the substring search it
 * amounts to (none of the six words before the name's first \n or \r), for
 * names of any length.
 */
int nvfp4_layer_is_quantized(const char* layer_name, const char* pattern);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
