// Low-rank branch next to the NVFP4 product: the down projection, fused
// with the activation-quantization pass that reads x.
//
// "NVFP4 en difusión ...", section 3: a low-rank correction cannot be merged
// into NVFP4 weights, so it runs next to the quantized product, and the
// library the page cites computes it in the same pass that quantizes the
// activation.  Here the first pass of nvfp4_quantize (the global amax)
// becomes a row-blocked kernel that also computes T = X L_down^T [M, r] in
// fp32 from the bf16 activation, so X is read once for both; the second pass
// (codes and scales) is unchanged.  The up projection T L_up^T is added in
// the GEMM epilogues before the single bf16 rounding.
//
// Each bf16 x bf16 product is exact in fp32; the K sums are fp32
// (v_mfma_f32_16x16x32_bf16, four waves splitting K, summed in a fixed
// order).
#include "common.h"
#include "launch.h"

namespace nvfp4k {

namespace {
constexpr int kLoraMaxBlocks = kLoraMaxRank / 16;
}  // namespace

// Workgroup (bx, s) takes the row groups bx, bx + gridDim.x, ... (16 rows
// each) and K slice s (gridDim.y slices of whole 32-value steps); wave w
// takes the slice's steps w, w + 4, ..., two at a time so that two steps'
// loads are in flight.  Lane i + 16 g loads x[m0 + i][32 kb + 8 g .. + 8] as
// the MFMA's A operand and L_down[16 jb + j][32 kb + 8 g .. + 8]
// (j = lane & 15) as B, so D[i][j] = T[m0 + i][16 jb + j] over the slice.
// Rows past M, ranks past r and K past the end read as zero.  With one
// slice T goes to t, else slice s writes t_part[s][M][r].  The
// workgroup's largest |x| goes to partial[s * gridDim.x + bx].
__global__ __launch_bounds__(256) void amax_lora_down_kernel(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ l_down,
                                                             float* __restrict__ t, float* __restrict__ t_part,
                                                             uint32_t* __restrict__ partial, int M, int K, int r) {
  __shared__ float4v red[4][kLoraMaxBlocks][64];
  __shared__ uint32_t wmax[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int nkb = (K + 31) / 32;
  const int per = (nkb + gridDim.y - 1) / gridDim.y;
  const int kb0 = blockIdx.y * per, kb1 = min(nkb, kb0 + per);
  const int nrb = (r + 15) / 16;
  float* dst = gridDim.y == 1 ? t : t_part + (int64_t)blockIdx.y * M * r;
  const auto lr = buffer_of(l_down, (uint32_t)r * (uint32_t)K * 2u);
  uint32_t mx = 0;
  for (int m0 = blockIdx.x * 16; m0 < M; m0 += gridDim.x * 16) {
    const uint32_t rows = (uint32_t)min(16, M - m0);
    const auto xr = buffer_of(x + (int64_t)m0 * K, rows * (uint32_t)K * 2u);
    float4v acc[kLoraMaxBlocks];
#pragma unroll
    for (int jb = 0; jb < kLoraMaxBlocks; ++jb) acc[jb] = float4v{0.f, 0.f, 0.f, 0.f};
    for (int kb = kb0 + wave; kb < kb1; kb += 8) {
      // steps kb and kb + 4 (the second may lie past the slice: zeros)
      const uint32_t ka = 32u * kb + 8u * g, kc = ka + 128u;
      const bool ina = ka < (uint32_t)K, inc = kb + 4 < kb1 && kc < (uint32_t)K;
      const uint4 a = buffer_load16(xr, ina ? 2u * ((uint32_t)i * K + ka) : kBufferOob);
      const uint4 c = buffer_load16(xr, inc ? 2u * ((uint32_t)i * K + kc) : kBufferOob);
      uint4 ba[kLoraMaxBlocks], bc[kLoraMaxBlocks];
#pragma unroll
      for (int jb = 0; jb < kLoraMaxBlocks; ++jb) {
        if (jb >= nrb) break;
        const uint32_t row = 16u * jb + i;
        ba[jb] = buffer_load16(lr, ina && row < (uint32_t)r ? 2u * (row * K + ka) : kBufferOob);
        bc[jb] = buffer_load16(lr, inc && row < (uint32_t)r ? 2u * (row * K + kc) : kBufferOob);
      }
      mx = max(mx, max(max(bf16x2_absmax_bits(a.x), bf16x2_absmax_bits(a.y)),
                       max(bf16x2_absmax_bits(a.z), bf16x2_absmax_bits(a.w))));
      mx = max(mx, max(max(bf16x2_absmax_bits(c.x), bf16x2_absmax_bits(c.y)),
                       max(bf16x2_absmax_bits(c.z), bf16x2_absmax_bits(c.w))));
      const short8v av = __builtin_bit_cast(short8v, a), cv = __builtin_bit_cast(short8v, c);
#pragma unroll
      for (int jb = 0; jb < kLoraMaxBlocks; ++jb) {
        if (jb >= nrb) break;
        acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(short8v, ba[jb]), acc[jb], 0, 0, 0);
        acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cv, __builtin_bit_cast(short8v, bc[jb]), acc[jb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int jb = 0; jb < kLoraMaxBlocks; ++jb)
      if (jb < nrb) red[wave][jb][lane] = acc[jb];
    __syncthreads();
    // D[i][j] (16 x 16): lane j + 16 (i / 4), register i % 4.
    for (int e = threadIdx.x; e < nrb * 64; e += 256) {
      const int jb = e >> 6, ln = e & 63;
      const float4v s = ((red[0][jb][ln] + red[1][jb][ln]) + red[2][jb][ln]) + red[3][jb][ln];
      const int j = 16 * jb + (ln & 15);
      if (j < r) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = m0 + 4 * (ln >> 4) + q;
          if (m < M) dst[(int64_t)m * r + j] = s[q];
        }
      }
    }
    __syncthreads();
  }
  mx = wave_max_u32(mx);
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();
  if (threadIdx.x == 0)
    partial[blockIdx.y * gridDim.x + blockIdx.x] = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
}

hipError_t launch_nvfp4_quantize_lora(const void* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                      float* gscale, int use_given, const void* l_down, int64_t r, float* t,
                                      uint32_t* workspace, hipStream_t stream) {
  const int gx = lora_row_blocks(rows), gy = lora_k_slices(rows, cols);
  float* t_part = gy > 1 ? (float*)(workspace + kAmaxPartials) : nullptr;
  hipLaunchKernelGGL(amax_lora_down_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream,
                     (const uint16_t*)x, (const uint16_t*)l_down, t, t_part, workspace, (int)rows, (int)cols, (int)r);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_nvfp4_quantize_pass2(x, rows, cols, codes, scales, gscale, use_given, kRuleAbsmax, gx * gy,
                                     workspace, stream, t_part, gy, t, rows * r);
}

}  // namespace nvfp4k
