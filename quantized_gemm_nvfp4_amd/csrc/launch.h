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

// rule: 0 absmax, 1 four-over-six, 2 MSE (block-scale selection).
hipError_t launch_nvfp4_quantize(const void* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                 float* gscale, int use_given, int rule, uint32_t* workspace, hipStream_t stream);

hipError_t launch_int4g_quantize(const void* w, int64_t N, int64_t K, uint8_t* q, void* scales,
                                 hipStream_t stream);

// NVFP4 GEMM kernels; out[M, N] bf16 = g_a g_w * A . W^T.
// tiled: K % 128 == 0.  decode: M <= 16, K % 128 == 0.  simple: K % 16 == 0.
hipError_t launch_nvfp4_gemm_tiled(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                   const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N, int64_t K,
                                   hipStream_t stream);
hipError_t launch_nvfp4_gemm_decode(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                    const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                    int64_t K, hipStream_t stream);
hipError_t launch_nvfp4_gemm_simple(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                    const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                    int64_t K, hipStream_t stream);

// Weight-only NVFP4: out[M, N] bf16 = g_w * x . dequant(W)^T, x bf16.
// decode: nvfp4_w4a16_decode_supported(M, K).  simple: K % 16 == 0.
bool nvfp4_w4a16_decode_supported(int64_t M, int64_t K);
hipError_t launch_nvfp4_w4a16_decode(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out,
                                     int64_t M, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_nvfp4_w4a16_simple(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out,
                                     int64_t M, int64_t N, int64_t K, hipStream_t stream);

// INT4 per-group (128) W4A16 kernels; out[M, N] bf16 = x . dequant(q, s)^T.
// decode: M <= 16.  tiled: any M.  simple: any M.  All need K % 128 == 0.
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
hipError_t launch_int4g_asym_simple(const void* x, const uint8_t* q, const void* s, const uint8_t* z, void* out,
                                    int64_t M, int64_t N, int64_t K, hipStream_t stream);

}  // namespace nvfp4k
