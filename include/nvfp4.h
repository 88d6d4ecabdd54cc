/*
 * nvfp4.h -- C ABI of libnvfp4.so: NVFP4 block quantization, the
 * block-scaled 4-bit GEMM that consumes it, and the symmetric INT4
 * per-group weight-only GEMM/GEMV, as hand-written HIP kernels for gfx950.
 *
 * Formats (pages cited by title and section):
 *  - "Tu pipeline NVFP4: meter 62 GB de modelo en 24 GB de laptop",
 *    section 2 ("Qué es realmente NVFP4"): each value is E2M1 (1 sign,
 *    2 exponent, 1 mantissa bit, largest magnitude 6); 16 consecutive
 *    values share one scale stored as FP8 E4M3; the scale is chosen from
 *    the block's largest magnitude.
 *  - "NVFP4 en difusión: la misma cuantización, un motor completamente
 *    distinto", section 2 ("NVFP4 sin vLLM"): the weight is a uint8
 *    tensor (out, in/2) holding two FP4 values per byte, the scale a
 *    float8_e4m3fn tensor (out, in/16); the activation is quantized the
 *    same way on every forward; the matmul multiplies the two decoded
 *    operands (the weight transposed) and emits bfloat16.
 *  - "Cuantización e inferencia local" (course class 085), formula block:
 *    symmetric b-bit quantization s = max|x| / (2^(b-1) - 1),
 *    q = clamp(round(x/s)), x ~ s*q, with one scale per group of weights.
 *
 * Layouts (all row-major, contiguous, no padding):
 *  - bf16 matrices: [rows, cols] of IEEE bfloat16 bit patterns.
 *  - NVFP4 codes:  uint8 [rows, cols/2]; element 2j of a row sits in bits
 *    0-3 of byte j, element 2j+1 in bits 4-7.  A code is sign<<3 | E2M1
 *    magnitude code (0..7 = 0, .5, 1, 1.5, 2, 3, 4, 6).
 *  - NVFP4 scales: uint8 [rows, cols/16], E4M3 (OCP "fn") bit patterns.
 *    The GEMM entry points take the scale bytes the quantizers write:
 *    non-negative and finite (sign bit clear, not 0x7F).  For other bytes
 *    (negative scales, NaN) the decode kernels' results are unspecified.
 *  - NVFP4 global scale: one fp32 in device memory.  The value of element
 *    (r, c) is E2M1(code) * E4M3(scale[r][c/16]) * global_scale.
 *  - INT4 codes: uint8 [N, K/2], two's-complement nibbles in [-7, 7],
 *    element 2j in bits 0-3 of byte j; INT4 scales: fp16 [N, K/group].
 *
 * Ownership and streams: the caller allocates and frees every buffer.  All
 * pointers except `stream` are device pointers.  The library allocates no
 * memory, keeps no global state, never synchronizes the host and never
 * reads device data back: every entry point only enqueues kernels on
 * `stream` (a hipStream_t; NULL is the default stream) and returns.  All
 * entry points are re-entrant; calls on different streams that share an
 * output buffer race.
 *
 * Errors: arguments are validated on the host before any HIP call; a
 * failed check returns an error status, enqueues nothing and records a
 * message readable with nvfp4_last_error() (thread-local).  A kernel
 * launch failure returns NVFP4_ERR_HIP.  Faults inside a kernel surface at
 * the caller's next synchronization.  Empty outputs (M, N or rows == 0)
 * return NVFP4_OK and enqueue nothing.  Alignment: every pointer must be
 * 16-byte aligned (256-byte aligned allocations from HIP or torch satisfy
 * this), except the fp32 global-scale pointers and the quantize workspace
 * (4-byte).
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_ARG = 1, /* null pointer, negative size, aliasing */
  NVFP4_ERR_SHAPE = 2,       /* a dimension that breaks the format's rules */
  NVFP4_ERR_ALIGNMENT = 3,   /* a pointer below the required alignment */
  NVFP4_ERR_UNSUPPORTED = 4, /* a valid request this build does not handle */
  NVFP4_ERR_HIP = 5          /* the HIP runtime reported an error */
} nvfp4_status;

/* Version of this ABI; bumped on any incompatible change. */
int nvfp4_abi_version(void);

/* Device bytes of the workspace nvfp4_quantize needs (per-workgroup
 * partial maxima of the global-amax pass).  The content needs no
 * initialization and is overwritten by every call. */
size_t nvfp4_quantize_workspace_bytes(void);

/*
 * NVFP4-quantize a bf16 matrix x [rows, cols] (cols % 16 == 0).
 * Passages: the E2M1 / 16-value-block / E4M3-scale format and absmax scale
 * choice ("Tu pipeline NVFP4", section 2); two codes per byte and the
 * (out, in/2) / (out, in/16) layouts, with the activation quantized on
 * every forward ("NVFP4 en difusión", section 2).
 *
 * Steps, each an fp32 operation with one round-to-nearest-even:
 *   g   = amax(|x|) / 2688     (2688 = 6 * 448), computed on the device
 *         and written to *global_scale, unless use_given_global_scale != 0,
 *         in which case *global_scale is read (finite, >= 0) and not written;
 *   per row and 16-block b: s = E4M3_RNE_saturating((amax_b / 6) / g),
 *         or 0 when g == 0;
 *   d = s * g;  per element: code = sign(x) | E2M1_RNE(|x| / d), ties to
 *         the even code, saturating at 6; magnitude 0 when d == 0.
 * Outputs: codes [rows, cols/2], scales [rows, cols/16], *global_scale.
 * workspace: >= nvfp4_quantize_workspace_bytes() device bytes, not shared
 * with a concurrent call.  Outputs must not overlap x or each other.
 */
nvfp4_status nvfp4_quantize(const void* x_bf16, int64_t rows, int64_t cols,
                            uint8_t* codes, uint8_t* scales, float* global_scale,
                            int use_given_global_scale, void* workspace, void* stream);

/*
 * nvfp4_quantize without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same steps, arguments, outputs and
 * errors as nvfp4_quantize (absmax rule); codes, scales and g are
 * byte-identical to its results.  The first pass's partial maxima go to a
 * static 4 KB device array that the library holds on each GPU it runs on
 * until the process ends (1024 slots, the most the pass ever writes, so
 * every size nvfp4_quantize accepts fits).  The entry point itself allocates
 * nothing; its first call on a device looks up that array's address once.
 * Every call on one GPU shares the array: calls that overlap on one GPU
 * (different streams without ordering) race and may produce wrong results.
 */
nvfp4_status nvfp4_quantize_noalloc(const void* x_bf16, int64_t rows, int64_t cols,
                                    uint8_t* codes, uint8_t* scales, float* global_scale,
                                    int use_given_global_scale, void* stream);

/* Block-scale selection rules for nvfp4_quantize_ex. */
typedef enum nvfp4_scale_rule {
  NVFP4_SCALE_ABSMAX = 0,        /* the block max maps to 6 (nvfp4_quantize) */
  NVFP4_SCALE_FOUR_OVER_SIX = 1, /* max -> 6 or max -> 4, the lower error */
  NVFP4_SCALE_MSE = 2            /* least error over a one-binade window */
} nvfp4_scale_rule;

/*
 * nvfp4_quantize with a choice of block-scale rule.  Passage: the table of
 * scale algorithms in "Tu pipeline NVFP4", section 2 (absmax; MSE, which
 * tries several scales and keeps the one with the least reconstruction
 * error of the block; four-over-six, which lets each block map its largest
 * magnitude to 4 or to 6, whichever errs less).  Meant for weights, which
 * are quantized once; the GEMM consumes the result unchanged.
 *
 * g, the candidate arithmetic and the codes are exactly those of
 * nvfp4_quantize; only the stored scale byte of a block may differ:
 *   error(s) = sum over the block, in element order, of (x - v * d)^2 with
 *     d = s * g and v the signed E2M1 value of each code, every step an fp32
 *     operation with one rounding (no fused multiply-add);
 *   FOUR_OVER_SIX: candidates s6 = E4M3(fl32(fl32(amax_b / 6) / g)) and
 *     s4 = E4M3(fl32(fl32(amax_b / 4) / g)); s4 only if strictly better;
 *   MSE: the E4M3 codes c6, c6 - 1, c6 + 1, ..., c6 - 8, c6 + 8 (within
 *     1..0x7E), c6 being the absmax code; a later candidate only if
 *     strictly better.
 * The error under MSE is never above four-over-six's, which is never above
 * absmax's.  Unknown rules return NVFP4_ERR_INVALID_ARG.  All other
 * arguments and errors as nvfp4_quantize.
 */
nvfp4_status nvfp4_quantize_ex(const void* x_bf16, int64_t rows, int64_t cols,
                               uint8_t* codes, uint8_t* scales, float* global_scale,
                               int use_given_global_scale, int scale_rule, void* workspace,
                               void* stream);

/*
 * out[M, N] (bf16) = bf16_RNE( g_a * g_w * sum_k A[m, k] * W[n, k] )
 * where A[m, k] = E2M1(a code) * E4M3(a scale) and likewise for W: the
 * decoded activation times the decoded weight, transposed.  Passage: the
 * block-scaled matmul of "NVFP4 en difusión", section 2 (scale_a, scale_b,
 * bfloat16 output).  Each decoded product is exact; sums are fp32.
 * a_codes [M, K/2], a_scales [M, K/16], w_codes [N, K/2], w_scales
 * [N, K/16]; a_gscale and w_gscale are device fp32 pointers (no host sync).
 * K % 16 == 0.  M <= 16 runs the decode kernel that streams W once
 * (K % 128 == 0 and K <= 2^24; other K take the simple kernel).
 * K == 0 writes zeros (the packed operands may then be NULL).
 * out must not overlap any input.
 */
nvfp4_status nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                        const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale,
                        void* out_bf16, int64_t M, int64_t N, int64_t K, void* stream);

/* Kernel choice for nvfp4_gemm_ex / int4g_gemv_ex. */
typedef enum nvfp4_algo {
  NVFP4_ALGO_AUTO = 0,    /* what nvfp4_gemm / int4g_gemv pick */
  NVFP4_ALGO_TILED = 1,   /* the LDS-staged MFMA tile kernel (any M; nvfp4_gemm:
                             K % 128 == 0 and K < 2^24, int4g_gemv: K < 2^22;
                             else NVFP4_ERR_UNSUPPORTED) */
  NVFP4_ALGO_DECODE = 2,  /* the weight-streaming kernel (M <= 16, K % 128 == 0
                             and K <= 2^24 only; else NVFP4_ERR_UNSUPPORTED) */
  NVFP4_ALGO_SIMPLE = 3   /* one output per thread, fp32 FMA (any shape) */
} nvfp4_algo;

/* nvfp4_gemm with an explicit kernel choice (tests and benchmarks). */
nvfp4_status nvfp4_gemm_ex(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                           const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale,
                           void* out_bf16, int64_t M, int64_t N, int64_t K, int algo, void* stream);

/*
 * nvfp4_gemm_ex with a workspace.  The tiled kernel runs one 256 x 256
 * output tile per compute unit at a time; when the tile count is not a
 * multiple of the compute units, the leftover tiles of the last, partial
 * round are split along K into up to 8 parts that run side by side, and a
 * second kernel sums each tile's parts in order and rounds.  Only the
 * summation order of those tiles changes (the same fp32 products, the same
 * tolerance); the split depends only on M, N, K and the device's compute
 * unit count, so repeated calls give identical bits.
 * workspace: >= nvfp4_gemm_workspace_bytes(M, N, K) bytes of device memory
 * for the current device, 256-byte aligned, no initialization, not shared
 * with a concurrent call, not overlapping any argument.  The size is 0 when
 * no split applies (M <= 16, K % 128 != 0, K >= 2^24, whole rounds); with workspace
 * NULL or workspace_bytes below the size, the call runs as nvfp4_gemm_ex.
 */
size_t nvfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
nvfp4_status nvfp4_gemm_ws(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                           const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale,
                           void* out_bf16, int64_t M, int64_t N, int64_t K, int algo, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Quantize a bf16 activation and multiply it by an NVFP4 weight: the
 * forward of a linear layer whose activation is quantized on every call
 * ("NVFP4 en difusión", section 2).  Results are bit-identical to
 * nvfp4_quantize(x) (absmax rule, g from max|x|) followed by nvfp4_gemm on
 * its codes: out [M, N] bf16, and x's codes [M, K/2], scales [M, K/16] and
 * g (one fp32) in x_codes, x_scales, x_gscale, which the caller provides.
 * Decode steps run one kernel, which quantizes x itself with the
 * quantizer's arithmetic and also stores x_codes / x_scales / x_gscale:
 * 1 <= M <= 2 with K % 128 == 0 and K <= 8192 (the weight-streaming GEMV),
 * and 3 <= M <= 16 with K % 128 == 0 and M * K / 16 <= 3072 (the row-block
 * GEMM, each workgroup quantizing all of x into LDS first).  Other shapes
 * run the quantizer and then the GEMM.
 * K > 0, K % 16 == 0 (else NVFP4_ERR_SHAPE); M == 0 does nothing; N == 0
 * only quantizes x.  x, out, x_codes, x_scales: 16-byte aligned.
 * workspace: >= nvfp4_linear_workspace_bytes(M, N, K) bytes of device
 * memory, 256-byte aligned, no initialization, not shared with a concurrent
 * call (NULL when the size is 0, as for the one-kernel shapes).  No output
 * may overlap another argument.
 */
size_t nvfp4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);
nvfp4_status nvfp4_linear(const void* x_bf16, const uint8_t* w_codes, const uint8_t* w_scales,
                          const float* w_gscale, void* out_bf16, int64_t M, int64_t N, int64_t K,
                          uint8_t* x_codes, uint8_t* x_scales, float* x_gscale, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * nvfp4_gemm_ws (AUTO kernel choice) that also leaves the global amax of
 * its output ready for nvfp4_quantize_amax, so that quantizing the output
 * (the next layer's activation, quantized on every forward: "NVFP4 en
 * difusión", section 2) skips its own read of the output for max|out|.
 * amax_slots: >= nvfp4_gemm_amax_slots(M, N, K) uint32 of device memory,
 * 4-byte aligned, no initialization, not overlapping any argument.  Every
 * slot is written with a bf16 magnitude pattern (sign cleared) and the
 * largest of them is that of max|out[m, n]|: the tiled kernel (M > 16,
 * K % 128 == 0, K < 2^24) writes one slot per 256 x 256 output tile from its
 * epilogue; other shapes run a separate pass over out.  N % 16 == 0 (the
 * output is quantized along N); workspace as for nvfp4_gemm_ws.
 */
size_t nvfp4_gemm_amax_slots(int64_t M, int64_t N, int64_t K);
nvfp4_status nvfp4_gemm_amax(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                             const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale,
                             void* out_bf16, int64_t M, int64_t N, int64_t K, void* workspace,
                             size_t workspace_bytes, uint32_t* amax_slots, void* stream);

/*
 * nvfp4_quantize (absmax rule) with max|x| taken from nslots bf16 magnitude
 * patterns (1 <= nslots <= 2^28) instead of a pass over x: g = (largest
 * pattern as bf16) / 2688, written to *global_scale, then the codes and
 * scales of nvfp4_quantize.  With the slots nvfp4_gemm_amax wrote for x,
 * the result is bit-identical to nvfp4_quantize(x).  No workspace.
 */
nvfp4_status nvfp4_quantize_amax(const void* x_bf16, int64_t rows, int64_t cols, uint8_t* codes,
                                 uint8_t* scales, float* global_scale, const uint32_t* amax_slots,
                                 int64_t nslots, void* stream);

/*
 * Weight-only NVFP4 GEMM: out[M, N] (bf16) = bf16_RNE( g_w * sum_k x[m, k] *
 * W[n, k] ) with x a bf16 activation that is not quantized and W the NVFP4
 * weight of nvfp4_gemm.  Passages: the weight format of "NVFP4 en
 * difusión", section 2, and the remark in "Cuantización e inferencia
 * local" that weight-only methods keep activations in 16-bit to avoid
 * their outliers.
 * x [M, K] bf16 row-major; w_codes [N, K/2]; w_scales [N, K/16]; w_gscale
 * a device fp32 pointer.  K % 16 == 0; K == 0 writes zeros.
 * Exactness: W's decoded values are exact; the decode kernels (M <= 16,
 * K % 128 == 0, K <= 32768; each reads the weight once per call) feed the
 * matrix cores fp16, converting x after a power-of-two rescale that puts
 * the largest magnitude of each slice in [2^15, 2^16): per 2048-value slice
 * at M = 1, per row and slice of up to 768 values at 2 <= M <= 16 with
 * K <= 6144, per row and 512-value piece otherwise.  Elements within 2^32
 * of their slice's maximum are exact, smaller ones are truncated to the
 * fp16 subnormal grid.  Larger M (and decode-sized M the decode kernels do
 * not take) with K % 128 == 0 and K < 2^22 run MFMA tiles in bf16: x as
 * given and W decoded exactly to bf16, so every product is exact and only
 * the fp32 summation rounds.  Other shapes run a one-output-per-thread
 * kernel in fp32.
 * algo: NVFP4_ALGO_AUTO, _TILED, _DECODE or _SIMPLE (a kernel that cannot
 * take the shape returns NVFP4_ERR_UNSUPPORTED); other values return
 * NVFP4_ERR_INVALID_ARG.  out must not overlap any input.
 */
nvfp4_status nvfp4_gemm_w4a16(const void* x_bf16, const uint8_t* w_codes, const uint8_t* w_scales,
                              const float* w_gscale, void* out_bf16, int64_t M, int64_t N, int64_t K,
                              void* stream);
nvfp4_status nvfp4_gemm_w4a16_ex(const void* x_bf16, const uint8_t* w_codes, const uint8_t* w_scales,
                                 const float* w_gscale, void* out_bf16, int64_t M, int64_t N, int64_t K,
                                 int algo, void* stream);

/*
 * Symmetric INT4 per-group quantization of a bf16 weight w [N, K], groups
 * of `group` consecutive values along K (group == 128; K % 128 == 0).
 * Passage: the symmetric formula of "Cuantización e inferencia local"
 * (formula block) with b = 4 and one scale per group.
 *   s16 = fp16_RNE( fl32(max|w_group| / 7) );
 *   q   = clamp( rint_half_even( fl32(w / s16) ), -7, 7 ), 0 when s16 == 0.
 * Outputs: q [N, K/2] two's-complement nibbles; scales_fp16 [N, K/group].
 */
nvfp4_status int4g_quantize(const void* w_bf16, int64_t N, int64_t K, int64_t group,
                            uint8_t* q, void* scales_fp16, void* stream);

/*
 * W4A16: out[M, N] (bf16) = bf16_RNE( sum_g s16[n, g] * sum_{k in g}
 * x[m, k] * q[n, k] ), x bf16 [M, K], q / scales as int4g_quantize writes
 * them.  Passage: same formula block (x ~ s*q with a scale per group); the
 * weight-only GPU kernels of the same page's method chart.  Each group's
 * integer-weighted sum is taken in fp32, then scaled once by its s16.
 * Any M >= 1: M <= 16 streams the weight once (K <= 2^24; larger K take
 * the simple kernel); larger M runs MFMA tiles (K < 2^22; larger K take the
 * simple kernel, and NVFP4_ALGO_TILED returns NVFP4_ERR_UNSUPPORTED).
 */
nvfp4_status int4g_gemv(const void* x_bf16, const uint8_t* q, const void* scales_fp16,
                        void* out_bf16, int64_t M, int64_t N, int64_t K, int64_t group,
                        void* stream);

/* int4g_gemv with an explicit kernel choice (nvfp4_algo values). */
nvfp4_status int4g_gemv_ex(const void* x_bf16, const uint8_t* q, const void* scales_fp16,
                           void* out_bf16, int64_t M, int64_t N, int64_t K, int64_t group,
                           int algo, void* stream);

/* Static text of a status code. */
const char* nvfp4_status_string(nvfp4_status s);

/* Detail of the last error raised on the calling thread ("" if none). */
const char* nvfp4_last_error(void);

/*
 * Asymmetric (zero-point) INT4 per-group quantization of a bf16 weight
 * W [N, K] (group 128 along K, K % 128 == 0).  Passage: the asymmetric map
 * of "Cuantización e inferencia local", formula block: s = (x_max - x_min) /
 * (2^b - 1), z = round(-x_min / s), q = clamp(round(x / s) + z, 0, 2^b - 1),
 * x_hat = s (q - z), with b = 4 and one (s, z) per group.
 * The range is widened to contain 0 (lo = min(0, min w), hi = max(0, max w)),
 * so z is in [0, 15] and 0 is exact; s16 = fp16_RNE(fl32(fl32(hi - lo) /
 * 15)), z = clamp(rint(fl32(-lo / s16)), 0, 15), q = clamp(rint(fl32(w /
 * s16)) + z, 0, 15); q = z = 0 where s16 == 0.
 * Outputs: q [N, K/2] unsigned nibbles (element 2j in bits 0-3 of byte j),
 * scales [N, K/128] fp16, zeros [N, K/128] uint8.  group must be 128.
 */
nvfp4_status int4g_asym_quantize(const void* w_bf16, int64_t N, int64_t K, int64_t group,
                                 uint8_t* q, void* scales_fp16, uint8_t* zeros, void* stream);

/*
 * out[M, N] (bf16) = bf16_RNE( sum_k x[m, k] * s16[n, k/128] * (q[n, k] -
 * z[n, k/128]) ), x bf16 [M, K] (the same passage; weight-only).  M <= 2
 * (K <= 32768) runs the row-slot GEMV that streams q once; other shapes
 * with K < 2^22 the LDS-staged MFMA tile kernel (per group, s16 (sum x q -
 * z sum x), the group sums of x taken on the matrix cores), the rest a
 * one-output-per-thread kernel.  algo: NVFP4_ALGO_AUTO, _TILED (K < 2^22,
 * else NVFP4_ERR_UNSUPPORTED), _DECODE (M <= 2, K <= 32768) or _SIMPLE.
 */
nvfp4_status int4g_asym_gemv(const void* x_bf16, const uint8_t* q, const void* scales_fp16,
                             const uint8_t* zeros, void* out_bf16, int64_t M, int64_t N, int64_t K,
                             int64_t group, void* stream);
nvfp4_status int4g_asym_gemv_ex(const void* x_bf16, const uint8_t* q, const void* scales_fp16,
                                const uint8_t* zeros, void* out_bf16, int64_t M, int64_t N, int64_t K,
                                int64_t group, int algo, void* stream);

/*
 * Low-rank (LoRA) branch next to an NVFP4 layer.  Passage: "NVFP4 en
 * difusión", section 3 (fine-tuning a model already in 4 bits): a low-rank
 * correction cannot be folded into NVFP4 weights, so it runs at run time
 * beside the quantized product, and its down projection is computed in the
 * same pass that quantizes the activation.  The layer is
 *   y = bf16_RNE( g_a g_w A_hat W_hat^T + T L_up^T ),  T = X L_down^T,
 * with X the bf16 activation before quantization, L_down bf16 [r, cols]
 * and L_up bf16 [N, r] (nn.Linear layouts; a LoRA scale alpha / r is
 * folded into L_up by the caller).  Rank r: a multiple of 8 in [8, 128];
 * other values return NVFP4_ERR_UNSUPPORTED.
 *
 * nvfp4_quantize_lora: nvfp4_quantize (absmax rule) of x [rows, cols] plus
 * lora_t [rows, r] fp32 = X L_down^T, with X read once for the global
 * amax and the down projection.  Each bf16 product is exact in fp32, the
 * sums are fp32 in a fixed order (the same for every call with the same
 * shapes).  The workspace is always required, also with
 * use_given_global_scale: nvfp4_quantize_lora_workspace_bytes(rows, cols,
 * r) bytes, 4-byte aligned, no initialization (it holds partial maxima and,
 * when the down projection is split along K, partial products).  lora_down_bf16 and lora_t are 16-byte aligned
 * and must not overlap the outputs.  Other arguments and errors as
 * nvfp4_quantize.
 */
size_t nvfp4_quantize_lora_workspace_bytes(int64_t rows, int64_t cols, int64_t r);
nvfp4_status nvfp4_quantize_lora(const void* x_bf16, int64_t rows, int64_t cols, uint8_t* codes,
                                 uint8_t* scales, float* global_scale, int use_given_global_scale,
                                 const void* lora_down_bf16, int64_t r, float* lora_t, void* workspace,
                                 void* stream);

/*
 * nvfp4_gemm_lora: out[M, N] (bf16) = bf16_RNE( g_a g_w sum_k A[m, k] W[n, k]
 * + sum_j lora_t[m, j] L_up[n, j] ), A and W as nvfp4_gemm, lora_t fp32
 * [M, r] (as nvfp4_quantize_lora writes it), lora_up_bf16 [N, r].  The
 * branch is added in the GEMM epilogue before the single rounding (in the
 * tiled kernel on the matrix cores with T split into two bf16 parts, which
 * keeps about 16 bits of T).  Kernel choice as nvfp4_gemm(_ex).
 */
nvfp4_status nvfp4_gemm_lora(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                             const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale,
                             const float* lora_t, const void* lora_up_bf16, int64_t r, void* out_bf16,
                             int64_t M, int64_t N, int64_t K, void* stream);
nvfp4_status nvfp4_gemm_lora_ex(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                                const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale,
                                const float* lora_t, const void* lora_up_bf16, int64_t r, void* out_bf16,
                                int64_t M, int64_t N, int64_t K, int algo, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H_ */
