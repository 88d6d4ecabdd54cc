// One-output-per-thread GEMM kernels for shapes the tiled and decode kernels
// do not take (K not a multiple of 128).  Same products as those kernels:
//  - NVFP4: out = bf16_RNE(g_a g_w sum_b (s_a s_w) sum_{k in b} e_a e_w), the
//    block-scaled matmul of "NVFP4 en difusión ...", section 2.  Within a
//    16-block the E2M1 products are multiples of 1/4 below 36, so the block
//    sum and its product with s_a s_w are exact in fp32; only the sum over
//    blocks rounds.
//  - INT4: out = bf16_RNE(sum_g s16 sum_{k in g} x q), "Cuantización e
//    inferencia local", formula block.
#include "common.h"
#include "launch.h"

namespace nvfp4k {

namespace {
// E2M1 code (sign in bit 3) -> fp32 value.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  float v = (e == 0) ? 0.5f * (float)m : __uint_as_float(((e + 126u) << 23) | (m << 22));
  return (c & 8u) ? -v : v;
}
}  // namespace

__global__ __launch_bounds__(64) void nvfp4_gemm_simple_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const float* __restrict__ w_g,
    uint16_t* __restrict__ out, int M, int N, int K, const float* __restrict__ lora_t,
    const uint16_t* __restrict__ lora_up, int r) {
  const int n = blockIdx.x * 64 + threadIdx.x;
  if (n >= N) return;
  const int nb = K / 16;
  for (int m = blockIdx.y; m < M; m += gridDim.y) {
  const uint2* ar = (const uint2*)(a_codes + (int64_t)m * (K / 2));
  const uint2* wr = (const uint2*)(w_codes + (int64_t)n * (K / 2));
  const uint8_t* asr = a_scales + (int64_t)m * nb;
  const uint8_t* wsr = w_scales + (int64_t)n * nb;
  float acc = 0.0f;
  for (int b = 0; b < nb; ++b) {
    const uint2 av = ar[b], wv = wr[b];
    float bs = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t aw = e < 8 ? av.x : av.y, ww = e < 8 ? wv.x : wv.y;
      const int sh = 4 * (e & 7);
      bs += e2m1_value((aw >> sh) & 15u) * e2m1_value((ww >> sh) & 15u);
    }
    acc += (e4m3_to_f32(asr[b]) * e4m3_to_f32(wsr[b])) * bs;
  }
  float v = acc * ((*a_g) * (*w_g));
  if (lora_t != nullptr)        // low-rank branch: + sum_j T[m][j] L_up[n][j]
    for (int j = 0; j < r; ++j) v += lora_t[(int64_t)m * r + j] * bf16_bits_to_f32(lora_up[(int64_t)n * r + j]);
  out[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(v);
  }
}

// Weight-only NVFP4: out = bf16_RNE(g_w sum_b s_w sum_{k in b} x e_w); each
// x * e_w is exact in fp32 (8 x 2 significant bits), the block sums round.
__global__ __launch_bounds__(64) void nvfp4_w4a16_simple_kernel(const uint16_t* __restrict__ x,
                                                                const uint8_t* __restrict__ w_codes,
                                                                const uint8_t* __restrict__ w_scales,
                                                                const float* __restrict__ w_g,
                                                                uint16_t* __restrict__ out, int M, int N, int K) {
  const int n = blockIdx.x * 64 + threadIdx.x;
  if (n >= N) return;
  const int nb = K / 16;
  for (int m = blockIdx.y; m < M; m += gridDim.y) {
    const uint16_t* xr = x + (int64_t)m * K;
    const uint2* wr = (const uint2*)(w_codes + (int64_t)n * (K / 2));
    const uint8_t* wsr = w_scales + (int64_t)n * nb;
    float acc = 0.0f;
    for (int b = 0; b < nb; ++b) {
      const uint2 wv = wr[b];
      float bs = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t ww = e < 8 ? wv.x : wv.y;
        bs += bf16_bits_to_f32(xr[16 * b + e]) * e2m1_value((ww >> (4 * (e & 7))) & 15u);
      }
      acc += e4m3_to_f32(wsr[b]) * bs;
    }
    out[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(acc * (*w_g));
  }
}

__global__ __launch_bounds__(64) void int4g_gemm_simple_kernel(const uint16_t* __restrict__ x,
                                                               const uint8_t* __restrict__ q,
                                                               const uint16_t* __restrict__ s,
                                                               uint16_t* __restrict__ out, int M, int N, int K) {
  const int n = blockIdx.x * 64 + threadIdx.x;
  if (n >= N) return;
  const int ng = K / 128;
  for (int m = blockIdx.y; m < M; m += gridDim.y) {
  const uint16_t* xr = x + (int64_t)m * K;
  const uint32_t* qr = (const uint32_t*)(q + (int64_t)n * (K / 2));
  float acc = 0.0f;
  for (int g = 0; g < ng; ++g) {
    float gs = 0.0f;
    for (int d = 0; d < 16; ++d) {
      const uint32_t w = qr[g * 16 + d];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int qi = (int)(w << (28 - 4 * e)) >> 28;
        gs += bf16_bits_to_f32(xr[g * 128 + d * 8 + e]) * (float)qi;
      }
    }
    acc += f16_bits_to_f32(s[(int64_t)n * ng + g]) * gs;
  }
  out[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(acc);
  }
}

hipError_t launch_nvfp4_w4a16_simple(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out,
                                     int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  hipLaunchKernelGGL(nvfp4_w4a16_simple_kernel, dim3((unsigned)((N + 63) / 64), (unsigned)(M < 65535 ? M : 65535)),
                     dim3(64), 0, stream, (const uint16_t*)x, wc, ws, wg, (uint16_t*)out, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

hipError_t launch_nvfp4_gemm_simple_lora(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                         const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                         int64_t K, const float* lora_t, const void* lora_up, int64_t r,
                                         hipStream_t stream) {
  hipLaunchKernelGGL(nvfp4_gemm_simple_kernel, dim3((unsigned)((N + 63) / 64), (unsigned)(M < 65535 ? M : 65535)),
                     dim3(64), 0, stream, ac, as, ag, wc, ws, wg, (uint16_t*)out, (int)M, (int)N, (int)K, lora_t,
                     (const uint16_t*)lora_up, (int)r);
  return hipGetLastError();
}

hipError_t launch_nvfp4_gemm_simple(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                    const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                    int64_t K, hipStream_t stream) {
  return launch_nvfp4_gemm_simple_lora(ac, as, ag, wc, ws, wg, out, M, N, K, nullptr, nullptr, 0, stream);
}

hipError_t launch_int4g_gemm_simple(const void* x, const uint8_t* q, const void* s, void* out, int64_t M,
                                    int64_t N, int64_t K, hipStream_t stream) {
  hipLaunchKernelGGL(int4g_gemm_simple_kernel, dim3((unsigned)((N + 63) / 64), (unsigned)(M < 65535 ? M : 65535)), dim3(64), 0, stream,
                     (const uint16_t*)x, q, (const uint16_t*)s, (uint16_t*)out, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

}  // namespace nvfp4k
