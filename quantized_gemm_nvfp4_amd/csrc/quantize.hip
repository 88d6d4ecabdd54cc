// NVFP4 and INT4 per-group quantization kernels for gfx950.
//
// NVFP4 ("Tu pipeline NVFP4 ...", section 2; "NVFP4 en difusión ...",
// section 2): each 16-value block along a row gets an E4M3 scale chosen from
// the block's largest magnitude, each value an E2M1 code, two codes per
// byte.  A per-tensor fp32 scale g = amax / (6 * 448) sits above the block
// scales.  The activation is quantized on every call, so g is computed on
// the device and never read back by the host.
//
// Two passes: (1) a grid of at most kAmaxPartials workgroups writes the
// largest bf16 magnitude each one saw (the max is order-independent, so the
// result is exact and deterministic); (2) every workgroup of the quantize
// kernel reduces those partials itself, derives g, and quantizes one 16-value
// block per thread.  No atomics, no memset, no host sync.
//
// INT4 ("Cuantización e inferencia local", formula block, b = 4): per row
// and group of 128 values, s = max|w| / 7 stored as fp16, q = clamp(rint(w /
// s), -7, 7) stored as two's-complement nibbles.
#include <mutex>

#include "common.h"
#include "launch.h"
#include "quant_block.h"

namespace nvfp4k {

namespace {
constexpr int64_t kSmallQuantBlocks = 8192;   // the single-launch kernel: up to 128K values
}  // namespace

// ---- pass 1: partial maxima of |x| over a bf16 tensor ---------------------
// x is read as 16-byte vectors (8 bf16); n_vec = elements / 8.
__global__ __launch_bounds__(256) void amax_partial_kernel(const uint4* __restrict__ x, int64_t n_vec,
                                                           uint32_t* __restrict__ partial) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n_vec; i += 4 * stride) {
    uint4 v0 = x[i], v1 = x[i + stride], v2 = x[i + 2 * stride], v3 = x[i + 3 * stride];
    uint32_t a = bf16x2_absmax_bits(v0.x), b = bf16x2_absmax_bits(v0.y);
    a = max(a, bf16x2_absmax_bits(v0.z)); b = max(b, bf16x2_absmax_bits(v0.w));
    a = max(a, bf16x2_absmax_bits(v1.x)); b = max(b, bf16x2_absmax_bits(v1.y));
    a = max(a, bf16x2_absmax_bits(v1.z)); b = max(b, bf16x2_absmax_bits(v1.w));
    a = max(a, bf16x2_absmax_bits(v2.x)); b = max(b, bf16x2_absmax_bits(v2.y));
    a = max(a, bf16x2_absmax_bits(v2.z)); b = max(b, bf16x2_absmax_bits(v2.w));
    a = max(a, bf16x2_absmax_bits(v3.x)); b = max(b, bf16x2_absmax_bits(v3.y));
    a = max(a, bf16x2_absmax_bits(v3.z)); b = max(b, bf16x2_absmax_bits(v3.w));
    m = max(m, max(a, b));
  }
  for (; i < n_vec; i += stride) {
    uint4 v = x[i];
    m = max(m, max(max(bf16x2_absmax_bits(v.x), bf16x2_absmax_bits(v.y)),
                   max(bf16x2_absmax_bits(v.z), bf16x2_absmax_bits(v.w))));
  }
  m = wave_max_u32(m);
  __shared__ uint32_t red[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

// ---- pass 2: one 16-value block per thread ---------------------------------
// Block-scale rules ("Tu pipeline NVFP4 ...", section 2, table of scale
// algorithms): absmax maps the block's largest magnitude to 6; four-over-six
// also tries mapping it to 4 and keeps whichever reconstructs the block with
// less error; MSE tries the E4M3 scales within one binade (8 codes) of the
// absmax scale, visited c6, c6 - 1, c6 + 1, ..., c6 + 8, and keeps the
// least error (a later candidate must be strictly better).  The error of a
// block under scale s is, in fp32 with one rounding per step and no fused
// multiply-add: d = s * g, x_hat = v * d (v the signed E2M1 value of the
// element's code), e = x - x_hat, err = sum of e * e in element order.
namespace {
// Signed E2M1 values of elements 2J and 2J + 1 of a code word (byte J),
// exact (the conversion's scale 1.0 leaves them unscaled).
template <int J>
__device__ __forceinline__ float2v e2m1x2_values(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, J);
}

// The block's codes under d come from encode_block, as when they are
// stored, and go back to their E2M1 values through the matching conversion.
template <bool kFast>
__device__ __forceinline__ float block_error_d(const uint32_t (&w)[8], float d, float r) {
#pragma clang fp contract(off)
  const uint2 c = encode_block<kFast>(w, d, r);
  const float2v v[8] = {e2m1x2_values<0>(c.x), e2m1x2_values<1>(c.x), e2m1x2_values<2>(c.x),
                        e2m1x2_values<3>(c.x), e2m1x2_values<0>(c.y), e2m1x2_values<1>(c.y),
                        e2m1x2_values<2>(c.y), e2m1x2_values<3>(c.y)};
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float x0 = __uint_as_float(w[i] << 16), x1 = __uint_as_float(w[i] & 0xFFFF0000u);
    const float h0 = v[i][0] * d, h1 = v[i][1] * d;
    const float e0 = x0 - h0, e1 = x1 - h1;
    const float s0 = e0 * e0, s1 = e1 * e1;
    acc = acc + s0;
    acc = acc + s1;
  }
  return acc;
}

__device__ __forceinline__ float block_error(const uint32_t (&w)[8], uint32_t sc, float g) {
#pragma clang fp contract(off)
  const float d = e4m3_to_f32(sc) * g;
  return quot_fast(d) ? block_error_d<true>(w, d, 1.0f / d) : block_error_d<false>(w, d, 0.0f);
}

}  // namespace

// One 16-value block b of x: its scale under rule kRule (given g) and its
// codes, stored at codes[b] and scales[b].
template <int kRule>
__device__ __forceinline__ void quantize_block_words(const uint4 v0, const uint4 v1, int64_t b, float g, float rg,
                                                     uint2* __restrict__ codes, uint8_t* __restrict__ scales) {
  const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax_bits = max(amax_bits, bf16x2_absmax_bits(w[i]));
  const float amax_b = bf16_bits_to_f32(amax_bits);
  uint32_t sc = scale_code(amax_b, 6.0f, g, rg);
  if (kRule != kRuleAbsmax) {
    float best = block_error(w, sc, g);
    if (kRule == kRuleFourOverSix) {
      const uint32_t c4 = scale_code(amax_b, 4.0f, g, rg);
      if (block_error(w, c4, g) < best) sc = c4;
    } else {
      const int c6 = (int)sc;
      for (int step = 1; step <= 8; ++step) {
#pragma unroll
        for (int sgn = 0; sgn < 2; ++sgn) {
          const int c = sgn ? c6 + step : c6 - step;
          if (c < 1 || c > 0x7E) continue;
          const float e = block_error(w, (uint32_t)c, g);
          if (e < best) {
            best = e;
            sc = (uint32_t)c;
          }
        }
      }
    }
  }
  const float d = e4m3_to_f32(sc) * g;
  codes[b] = quot_fast(d) ? encode_block<true>(w, d, 1.0f / d) : encode_block<false>(w, d, 0.0f);
  scales[b] = (uint8_t)sc;
}

template <int kRule>
__device__ __forceinline__ void quantize_block(const uint4* __restrict__ x, int64_t b, float g, float rg,
                                               uint2* __restrict__ codes, uint8_t* __restrict__ scales) {
  quantize_block_words<kRule>(x[2 * b], x[2 * b + 1], b, g, rg, codes, scales);
}

// x: bf16 [nblocks * 16]; codes: 8 bytes per block; scales: 1 byte per block.
template <int kRule>
__global__ __launch_bounds__(256) void nvfp4_quant_kernel(const uint4* __restrict__ x, int64_t nblocks,
                                                          uint2* __restrict__ codes, uint8_t* __restrict__ scales,
                                                          float* __restrict__ gscale,
                                                          const uint32_t* __restrict__ partial, int npartial,
                                                          int use_given, const float* __restrict__ t_part,
                                                          int t_splits, float* __restrict__ t_out, int64_t t_n) {
  __shared__ float s_g, s_rg;
  __shared__ uint32_t s_max[4];
  if (use_given) {
    if (threadIdx.x == 0) {
      s_g = *gscale;
      s_rg = scale_recip(s_g);
    }
  } else {
    // All 256 threads load their partials four at a time before using any,
    // so a workgroup waits for about one memory latency, not one per load.
    // (buffer loads: indices past npartial read as zero, no branches)
    const auto pr = buffer_of(partial, 4u * (uint32_t)npartial);
    uint32_t m = 0;
    for (int i = threadIdx.x; i < npartial; i += 1024) {
      uint32_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = buffer_load4(pr, 4u * (uint32_t)(i + 256 * u));
      m = max(m, max(max(v[0], v[1]), max(v[2], v[3])));
    }
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      m = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
      const float g = bf16_bits_to_f32(m) / 2688.0f;   // amax / (6 * 448)
      if (blockIdx.x == 0) *gscale = g;
      s_g = g;
      s_rg = scale_recip(g);
    }
  }
  __syncthreads();
  const float g = s_g, rg = s_rg;

  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // Side job for a split low-rank down projection: T = the sum of its K
  // slices' partial products, in slice order.
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t_splits > 1 && e < t_n; e += stride) {
    float v = t_part[e];
    for (int sp = 1; sp < t_splits; ++sp) v += t_part[(int64_t)sp * t_n + e];
    t_out[e] = v;
  }
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks; b += stride)
    quantize_block<kRule>(x, b, g, rg, codes, scales);
}

// Small tensors (decode activations, at most kSmallQuantBlocks blocks): a
// single launch of one workgroup per 1024 blocks, each of which takes the
// maximum over all of x itself (x is at most 256 KB and stays in L2) and
// then quantizes its own 1024 blocks.  The maximum is the same integer max
// of |bf16| patterns and the blocks go through the same quantize_block, so
// g, scales and codes equal the two-pass kernels'; workgroup 0 stores g.
template <int kRule>
__global__ __launch_bounds__(1024) void nvfp4_quant_small_kernel(const uint4* __restrict__ x, int64_t nblocks,
                                                                uint2* __restrict__ codes, uint8_t* __restrict__ scales,
                                                                float* __restrict__ gscale, int use_given) {
  __shared__ float s_g, s_rg;
  __shared__ uint32_t s_max[16];
  // the thread's own block, loaded once for the maximum and the codes
  // (offsets past x read zero)
  const int64_t b = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  const uint32_t nbytes = (uint32_t)nblocks * 32u;
  const auto xr = buffer_of(x, nbytes);
  const uint4 own0 = buffer_load16(xr, 32u * (uint32_t)b), own1 = buffer_load16(xr, 32u * (uint32_t)b + 16u);
  if (use_given) {
    if (threadIdx.x == 0) {
      s_g = *gscale;
      s_rg = scale_recip(s_g);
    }
  } else {
    // eight 16-byte loads per thread in flight (offsets past x read zero)
    uint32_t m = 0;
    for (uint32_t i = 16u * threadIdx.x; i < nbytes; i += 8u * 16384u) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = buffer_load16(xr, i + 16384u * u);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        m = max(m, max(max(bf16x2_absmax_bits(v[u].x), bf16x2_absmax_bits(v[u].y)),
                       max(bf16x2_absmax_bits(v[u].z), bf16x2_absmax_bits(v[u].w))));
    }
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
      for (int w = 1; w < 16; ++w) m = max(m, s_max[w]);
      const float g = bf16_bits_to_f32(m) / 2688.0f;   // amax / (6 * 448)
      if (blockIdx.x == 0) *gscale = g;
      s_g = g;
      s_rg = scale_recip(g);
    }
  }
  __syncthreads();
  const float g = s_g, rg = s_rg;
  if (b < nblocks) quantize_block_words<kRule>(own0, own1, b, g, rg, codes, scales);
}

// ---- INT4 per-group (128) quantization ------------------------------------
// 16 lanes per group, 8 values (16 bytes) per lane; a wave covers 4 groups.
__global__ __launch_bounds__(256) void int4g_quant_kernel(const uint4* __restrict__ w, int64_t ngroups,
                                                          uint32_t* __restrict__ q,
                                                          uint16_t* __restrict__ scales) {
  const int64_t gthreads = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < ngroups * 16;
       t += gthreads) {
    // t / 16 is the group; every lane of a 16-lane group runs the same trip
    // count (blockDim and the grid stride are multiples of 16), so the
    // shuffles below see full groups.
    const uint4 v = w[t];
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
    uint32_t m = max(max(bf16x2_absmax_bits(x[0]), bf16x2_absmax_bits(x[1])),
                     max(bf16x2_absmax_bits(x[2]), bf16x2_absmax_bits(x[3])));
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      uint32_t u = __shfl_xor(m, o, 16);
      m = max(m, u);
    }
    const float s32 = bf16_bits_to_f32(m) / 7.0f;
    const uint32_t s16 = f32_to_f16_rne(s32);
    const float s = f16_bits_to_f32(s16);
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t h = (x[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      int qi = 0;
      if (s != 0.0f) {
        float y = __builtin_rintf(bf16_bits_to_f32(h) / s);
        y = y > 7.0f ? 7.0f : (y < -7.0f ? -7.0f : y);
        qi = (int)y;
      }
      out |= ((uint32_t)qi & 0xFu) << (4 * i);
    }
    q[t] = out;
    if ((t & 15) == 0) scales[t >> 4] = (uint16_t)s16;
  }
}

// ---- launchers -------------------------------------------------------------
hipError_t launch_nvfp4_quantize_pass2(const void* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                       float* gscale, int use_given, int rule, int npartial, uint32_t* workspace,
                                       hipStream_t stream, const float* t_part, int t_splits, float* t_out,
                                       int64_t t_n) {
  const int64_t nblocks = rows * cols / kBlock;
  int64_t grid = (nblocks + 255) / 256;
  if (grid > 2048) grid = 2048;
  if (rule == kRuleFourOverSix) {
    hipLaunchKernelGGL(nvfp4_quant_kernel<kRuleFourOverSix>, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint4*)x, nblocks, (uint2*)codes, scales, gscale, (const uint32_t*)workspace, npartial,
                       use_given, t_part, t_splits, t_out, t_n);
  } else if (rule == kRuleMse) {
    hipLaunchKernelGGL(nvfp4_quant_kernel<kRuleMse>, dim3((unsigned)grid), dim3(256), 0, stream, (const uint4*)x,
                       nblocks, (uint2*)codes, scales, gscale, (const uint32_t*)workspace, npartial, use_given,
                       t_part, t_splits, t_out, t_n);
  } else {
    hipLaunchKernelGGL(nvfp4_quant_kernel<kRuleAbsmax>, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint4*)x, nblocks, (uint2*)codes, scales, gscale, (const uint32_t*)workspace, npartial,
                       use_given, t_part, t_splits, t_out, t_n);
  }
  return hipGetLastError();
}

int amax_partial_count(int64_t n) {
  const int64_t grid = (n / 8 + 255) / 256;
  return (int)(grid < 1 ? 1 : (grid > kAmaxPartials ? kAmaxPartials : grid));
}

hipError_t launch_amax_partials(const void* x, int64_t n, uint32_t* partial, hipStream_t stream) {
  hipLaunchKernelGGL(amax_partial_kernel, dim3((unsigned)amax_partial_count(n)), dim3(256), 0, stream,
                     (const uint4*)x, n / 8, partial);
  return hipGetLastError();
}

hipError_t launch_nvfp4_quantize(const void* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                 float* gscale, int use_given, int rule, uint32_t* workspace, hipStream_t stream) {
  const int64_t n = rows * cols;
  const int64_t nblocks = n / kBlock;
  if (nblocks <= kSmallQuantBlocks) {
    const dim3 grid((unsigned)((nblocks + 1023) / 1024)), block(1024);
    if (rule == kRuleFourOverSix)
      hipLaunchKernelGGL(nvfp4_quant_small_kernel<kRuleFourOverSix>, grid, block, 0, stream, (const uint4*)x, nblocks,
                         (uint2*)codes, scales, gscale, use_given);
    else if (rule == kRuleMse)
      hipLaunchKernelGGL(nvfp4_quant_small_kernel<kRuleMse>, grid, block, 0, stream, (const uint4*)x, nblocks,
                         (uint2*)codes, scales, gscale, use_given);
    else
      hipLaunchKernelGGL(nvfp4_quant_small_kernel<kRuleAbsmax>, grid, block, 0, stream, (const uint4*)x, nblocks,
                         (uint2*)codes, scales, gscale, use_given);
    return hipGetLastError();
  }
  int npartial = 0;
  if (!use_given) {
    npartial = amax_partial_count(n);
    hipError_t e = launch_amax_partials(x, n, workspace, stream);
    if (e != hipSuccess) return e;
  }
  return launch_nvfp4_quantize_pass2(x, rows, cols, codes, scales, gscale, use_given, rule, npartial, workspace,
                                     stream);
}

// ---- scratch for callers that cannot allocate ------------------------------
// nvfp4_quantize_noalloc keeps the first pass's partial maxima here instead
// of in a caller workspace.  Each GPU holds its own copy of the array until
// the process ends; host code never passes the array's name to a kernel (on
// the host it only stands for the symbol), but the device address that
// hipGetSymbolAddress returns for the device, looked up once per device with
// that device current.
static __device__ __align__(256) uint32_t scratch[kAmaxPartials];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
uint32_t* g_scratch_ptr[kScratchDevices] = {};
}  // namespace

hipError_t quantize_scratch(hipStream_t stream, uint32_t** out) {
  int cur = 0, dev = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = (uint32_t*)p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_int4g_quantize(const void* w, int64_t N, int64_t K, uint8_t* q, void* scales,
                                 hipStream_t stream) {
  const int64_t ngroups = N * (K / 128);
  int64_t grid = (ngroups * 16 + 255) / 256;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(int4g_quant_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (const uint4*)w, ngroups,
                     (uint32_t*)q, (uint16_t*)scales);
  return hipGetLastError();
}

}  // namespace nvfp4k
