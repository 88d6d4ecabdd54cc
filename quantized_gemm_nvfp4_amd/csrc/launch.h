// Internal launchers behind the C ABI.  Arguments are validated by the
// caller (api.cpp) before any of these runs; each launcher only enqueues
// kernels on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4k {

// Partial maxima written by the global-amax pass of nvfp4_quantize (its
// workspace holds this many uint32).
constexpr int kAmaxPartials = 1024;

// Block-scale selection rules of the quantizer.
enum ScaleRule { kRuleAbsmax = 0, kRuleFourOverSix = 1, kRuleMse = 2 };

hipError_t launch_nvfp4_quantize(const void* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                 float* gscale, int use_given, int rule, uint32_t* workspace, hipStream_t stream);
// The first pass alone: partial maxima of |x| (bf16 patterns, sign cleared)
// over n bf16 values (n % 8 == 0), written to partial[0 .. amax_partial_count(n)).
int amax_partial_count(int64_t n);
hipError_t launch_amax_partials(const void* x, int64_t n, uint32_t* partial, hipStream_t stream);
// The second pass alone (codes and scales), reducing `npartial` partial
// maxima from workspace unless use_given.  With t_splits > 1 it also sums
// t_splits partial products t_part[s][t_n] into t_out[t_n], in order of s.
hipError_t launch_nvfp4_quantize_pass2(const void* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                       float* gscale, int use_given, int rule, int npartial, uint32_t* workspace,
                                       hipStream_t stream, const float* t_part = nullptr, int t_splits = 0,
                                       float* t_out = nullptr, int64_t t_n = 0);

// Low-rank branch: the quantizer with T = X L_down^T [rows, r] (fp32)
// computed in its first pass; r <= kLoraMaxRank.
constexpr int kLoraMaxRank = 128;
// The first pass runs on (row groups of 16) x (K slices) workgroups, at most
// kAmaxPartials in all; with more than one slice the slices' partial T go to
// the workspace after the partial maxima and the second pass sums them.
constexpr int kLoraSliceSteps = 8;        // at least 8 K steps of 32 per slice
inline int lora_row_blocks(int64_t rows) {
  const int64_t g = (rows + 15) / 16;
  return (int)(g < kAmaxPartials ? g : kAmaxPartials);
}
inline int lora_k_slices(int64_t rows, int64_t cols) {
  const int gx = lora_row_blocks(rows);
  const int64_t steps = (cols + 31) / 32;
  int64_t s = kAmaxPartials / (gx > 0 ? gx : 1);
  const int64_t smax = steps / kLoraSliceSteps;
  if (s > smax) s = smax;
  return (int)(s < 1 ? 1 : s);
}
inline int64_t lora_workspace_bytes(int64_t rows, int64_t cols, int64_t r) {
  const int s = lora_k_slices(rows, cols);
  return (int64_t)sizeof(uint32_t) * kAmaxPartials + (s > 1 ? (int64_t)s * rows * r * 4 : 0);
}
hipError_t launch_nvfp4_quantize_lora(const void* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                      float* gscale, int use_given, const void* l_down, int64_t r, float* t,
                                      uint32_t* workspace, hipStream_t stream);

hipError_t launch_int4g_quantize(const void* w, int64_t N, int64_t K, uint8_t* q, void* scales,
                                 hipStream_t stream);
// Device address of the quantizer's static scratch (kAmaxPartials uint32) on
// the device of `stream` (the current device for the null stream).
hipError_t quantize_scratch(hipStream_t stream, uint32_t** out);

// NVFP4 GEMM kernels; out[M, N] bf16 = g_a g_w * A . W^T.
// tiled: K % 128 == 0.  decode: M <= 16, K % 128 == 0.  simple: K % 16 == 0.
// Tiled GEMM with the leftover tiles of a partial last round split along K
// (fp32 parts in `workspace`, summed by a second kernel); without a large
// enough workspace every tile runs whole.
// With amax, amax[0 .. nvfp4_gemm_tiled_amax_slots(M, N)) receives each
// tile's largest |bf16| output pattern (for the global amax of out).
int64_t nvfp4_gemm_tiled_workspace_bytes(int64_t M, int64_t N, int64_t K);
int64_t nvfp4_gemm_tiled_amax_slots(int64_t M, int64_t N);
hipError_t launch_nvfp4_gemm_tiled_ws(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                      const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                      int64_t K, void* workspace, int64_t workspace_bytes, hipStream_t stream,
                                      uint32_t* amax = nullptr);
hipError_t launch_nvfp4_gemm_tiled(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                   const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N, int64_t K,
                                   hipStream_t stream);
hipError_t launch_nvfp4_gemm_decode(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                    const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                    int64_t K, hipStream_t stream);
hipError_t launch_nvfp4_gemm_simple(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                    const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                    int64_t K, hipStream_t stream);

// Quantize bf16 x and multiply in one launch (M <= 2: the streaming GEMV,
// each workgroup quantizing x in its prologue; 3 <= M <= 16 with M K / 16 <=
// 3072: the row-block GEMM, each workgroup quantizing x into LDS first);
// bit-identical to launch_nvfp4_quantize followed by the decode GEMM.
// q_codes / q_scales / q_g (optional) receive x's codes, scales and g.
// Needs nvfp4_linear_fused_supported(M, K).
bool nvfp4_linear_fused_supported(int64_t M, int64_t K);
hipError_t launch_nvfp4_linear_fused(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out,
                                     int64_t M, int64_t N, int64_t K, uint8_t* q_codes, uint8_t* q_scales,
                                     float* q_g, hipStream_t stream);

// Weight-only NVFP4: out[M, N] bf16 = g_w * x . dequant(W)^T, x bf16.
// decode: nvfp4_w4a16_decode_supported(M, K).  simple: K % 16 == 0.
bool nvfp4_w4a16_decode_supported(int64_t M, int64_t K);
hipError_t launch_nvfp4_w4a16_decode(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out,
                                     int64_t M, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_nvfp4_w4a16_simple(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out,
                                     int64_t M, int64_t N, int64_t K, hipStream_t stream);
// tiled (any M; K % 128 == 0, K < 2^22): the INT4 kernel's LDS-staged MFMA
// tiles with the NVFP4 weight decoded exactly to bf16.
hipError_t launch_nvfp4_w4a16_tiled(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out,
                                    int64_t M, int64_t N, int64_t K, hipStream_t stream);

// The same NVFP4 GEMMs plus the low-rank branch T L_up^T (T fp32 [M, r],
// L_up bf16 [N, r]) added before the bf16 rounding.
hipError_t launch_nvfp4_gemm_tiled_lora(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                        const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                        int64_t K, const float* lora_t, const void* lora_up, int64_t r,
                                        hipStream_t stream);
hipError_t launch_nvfp4_gemm_decode_lora(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                         const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                         int64_t K, const float* lora_t, const void* lora_up, int64_t r,
                                         hipStream_t stream);
hipError_t launch_nvfp4_gemm_simple_lora(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                         const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                         int64_t K, const float* lora_t, const void* lora_up, int64_t r,
                                         hipStream_t stream);

// INT4 per-group (128) W4A16 kernels; out[M, N] bf16 = x . dequant(q, s)^T.
// decode: M <= 16.  tiled: any M.  simple: any M.  All need K % 128 == 0.
// Compute units of the current device (cached per device; 256 if unknown).
int device_cus();
hipError_t launch_int4g_gemm_decode(const void* x, const uint8_t* q, const void* s, void* out, int64_t M,
                                    int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_int4g_gemm_tiled(const void* x, const uint8_t* q, const void* s, void* out, int64_t M,
                                   int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_int4g_gemm_simple(const void* x, const uint8_t* q, const void* s, void* out, int64_t M,
                                    int64_t N, int64_t K, hipStream_t stream);

// Asymmetric (zero-point) INT4 per-group (128): unsigned nibbles, fp16
// scales and uint8 zero points per group; out = x . (s16 (q - z))^T.
hipError_t launch_int4g_asym_quantize(const void* w, int64_t N, int64_t K, uint8_t* q, void* scales, uint8_t* zeros,
                                      hipStream_t stream);
bool int4g_asym_decode_supported(int64_t M, int64_t K);
hipError_t launch_int4g_asym_decode(const void* x, const uint8_t* q, const void* s, const uint8_t* z, void* out,
                                    int64_t M, int64_t N, int64_t K, hipStream_t stream);
// Zero-point INT4 on the LDS-staged MFMA tiles of the symmetric kernel (K < 2^22).
hipError_t launch_int4g_asym_tiled(const void* x, const uint8_t* q, const void* s, const uint8_t* z, void* out,
                                   int64_t M, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_int4g_asym_simple(const void* x, const uint8_t* q, const void* s, const uint8_t* z, void* out,
                                    int64_t M, int64_t N, int64_t K, hipStream_t stream);

}  // namespace nvfp4k
