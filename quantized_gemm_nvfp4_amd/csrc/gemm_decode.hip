// NVFP4 x NVFP4 -> bf16 GEMM for decode-sized M (M <= 16).
//
// Same product as the tiled kernel (the block-scaled matmul of "NVFP4 en
// difusión ...", section 2), shaped for the bandwidth-bound case: decode
// moves the whole packed weight once per call and does 2*M flops per weight,
// so the kernel's job is to stream W at HBM speed and keep the decoding
// (one VALU op per weight value) off the critical path.
//
//  - One workgroup per 16 weight rows; its 4 waves split K in 128-value
//    chunks (chunk c goes to wave c % 4) and are summed in LDS in a fixed
//    order, so results are deterministic.
//  - Per chunk a lane loads 16 bytes of codes (32 values) of one W row and
//    the 2 scale bytes of those values; each wave issues four chunks' loads
//    before decoding any of them.
//  - v_mfma_f32_16x16x32_f16 with W as the first operand: M <= 16 is padded
//    to the MFMA's 16 columns; the decoded fp16 operands are exact, as in the
//    tiled kernel.
//  - The activation operand: for M <= 2 the workgroup decodes the whole
//    activation once into LDS as fp16 (at most 2 x K x 2 bytes) and lanes of
//    rows >= M feed zeros, so per chunk only W is decoded.  For larger M each
//    wave decodes its chunk of the activation codes next to W's (the cost is
//    then shared by M useful columns).
#include "common.h"
#include "launch.h"

namespace nvfp4k {

namespace {
constexpr int kBatch = 4;            // chunks in flight per wave
constexpr int kLdsActRows = 2;       // activation rows decoded into LDS
constexpr int kLdsActMaxK = 16384;   // K limit of the LDS activation (64 KB)

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}
}  // namespace

template <bool kActInLds>
__global__ __launch_bounds__(256) void nvfp4_gemm_decode_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const float* __restrict__ w_g,
    uint16_t* __restrict__ out, int M, int N, int K) {
  extern __shared__ __attribute__((aligned(16))) _Float16 s_act[];   // [M][K] fp16 when kActInLds
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int r = lane & 15, grp = lane >> 4;
  const int64_t row_bytes = K / 2, row_scales = K / 16;
  const uint8_t* wrow = w_codes + (int64_t)min(n0 + r, N - 1) * row_bytes + 16 * grp;
  const uint8_t* wsrow = w_scales + (int64_t)min(n0 + r, N - 1) * row_scales + 2 * grp;
  const bool a_on = r < M;
  const uint8_t* arow = a_codes + (int64_t)(a_on ? r : 0) * row_bytes + 16 * grp;
  const uint8_t* asrow = a_scales + (int64_t)(a_on ? r : 0) * row_scales + 2 * grp;
  const int nchunks = K / 128;

  if (kActInLds) {
    // Decode the activation (M <= 2 rows) once: one 16-value block per
    // thread and iteration, written as 16 fp16 at [m][16 b].
    const int nblk = M * (K / 16);
    for (int b = threadIdx.x; b < nblk; b += 256) {
      const int m = b / (K / 16), kb = b - m * (K / 16);
      const uint2 c2 = *(const uint2*)(a_codes + (int64_t)m * row_bytes + 8 * kb);
      const half2v s2 = e4m3_to_f16x2(a_scales[(int64_t)m * row_scales + kb]);
      half8v* dst = (half8v*)(s_act + (int64_t)m * K + 16 * kb);
      dst[0] = dequant8_f16(c2.x, s2);
      dst[1] = dequant8_f16(c2.y, s2);
    }
    __syncthreads();
  }

  float4v acc = {0.f, 0.f, 0.f, 0.f};
  const half8v zero8 = {};
  for (int c0 = wave; c0 < nchunks; c0 += 4 * kBatch) {
    uint4 wc[kBatch], ac[kBatch];
    uint32_t ws[kBatch], as[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = c0 + 4 * u;
      wc[u] = make_uint4(0, 0, 0, 0);
      ws[u] = 0;
      ac[u] = make_uint4(0, 0, 0, 0);
      as[u] = 0;
      if (c < nchunks) {
        wc[u] = *(const uint4*)(wrow + (int64_t)c * 64);
        ws[u] = *(const uint16_t*)(wsrow + (int64_t)c * 8);
        if (!kActInLds && a_on) {
          ac[u] = *(const uint4*)(arow + (int64_t)c * 64);
          as[u] = *(const uint16_t*)(asrow + (int64_t)c * 8);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = c0 + 4 * u;
      if (c >= nchunks) break;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const half2v sw2 = e4m3_to_f16x2((ws[u] >> (8 * blk)) & 0xFFu);
        const half2v sa2 = e4m3_to_f16x2((as[u] >> (8 * blk)) & 0xFFu);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int jj = 2 * blk + t;
          const half8v wv = dequant8_f16(word_of(wc[u], jj), sw2);
          half8v av;
          if (kActInLds) {
            av = a_on ? *(const half8v*)(s_act + (int64_t)r * K + 128 * c + 32 * grp + 8 * jj) : zero8;
          } else {
            av = dequant8_f16(word_of(ac[u], jj), sa2);
          }
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, av, acc, 0, 0, 0);
        }
      }
    }
  }

  __shared__ float4v red[4][64];
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  const float4v s = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
  const float gg = (*a_g) * (*w_g);
  // D[n][m] (16 x 16): lane m + 16 (n / 4), register n % 4.
  const int m = lane & 15;
  const int n = n0 + 4 * (lane >> 4);
  if (m >= M) return;
  uint16_t* orow = out + (int64_t)m * N;
  const uint32_t b0 = f32_to_bf16_rne(s[0] * gg), b1 = f32_to_bf16_rne(s[1] * gg);
  const uint32_t b2 = f32_to_bf16_rne(s[2] * gg), b3 = f32_to_bf16_rne(s[3] * gg);
  if ((N & 3) == 0 && n + 3 < N) {
    *(uint2*)(orow + n) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
  } else {
    if (n + 0 < N) orow[n + 0] = (uint16_t)b0;
    if (n + 1 < N) orow[n + 1] = (uint16_t)b1;
    if (n + 2 < N) orow[n + 2] = (uint16_t)b2;
    if (n + 3 < N) orow[n + 3] = (uint16_t)b3;
  }
}

hipError_t launch_nvfp4_gemm_decode(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                    const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                    int64_t K, hipStream_t stream) {
  const unsigned grid = (unsigned)((N + 15) / 16);
  if (M <= kLdsActRows && K <= kLdsActMaxK) {
    const size_t lds = (size_t)M * K * 2;
    hipLaunchKernelGGL(nvfp4_gemm_decode_kernel<true>, dim3(grid), dim3(256), lds, stream, ac, as, ag, wc, ws, wg,
                       (uint16_t*)out, (int)M, (int)N, (int)K);
  } else {
    hipLaunchKernelGGL(nvfp4_gemm_decode_kernel<false>, dim3(grid), dim3(256), 0, stream, ac, as, ag, wc, ws, wg,
                       (uint16_t*)out, (int)M, (int)N, (int)K);
  }
  return hipGetLastError();
}

}  // namespace nvfp4k
