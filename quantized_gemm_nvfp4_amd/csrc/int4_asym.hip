// Asymmetric (zero-point) INT4 per-group quantization and its W4A16 GEMV.
//
// The asymmetric map of "Cuantización e inferencia local" (formula block):
// s = (x_max - x_min) / (2^b - 1), z = round(-x_min / s),
// q = clamp(round(x / s) + z, 0, 2^b - 1), x_hat = s (q - z); here b = 4,
// one fp16 scale and one zero point per group of 128 values along K.  The
// range is widened to contain 0 (lo = min(0, min w), hi = max(0, max w)), so
// z is an integer in [0, 15] and zero is represented exactly.  Arithmetic:
// s16 = fp16_RNE(fl32(fl32(hi - lo) / 15)), z = clamp(rint(fl32(-lo / s16)),
// 0, 15), q = clamp(rint(fl32(w / s16)) + z, 0, 15); q = z = 0 where
// s16 == 0.  q is stored as unsigned nibbles (element 2j in bits 0-3 of byte
// j), s16 as fp16 [N, K/128], z as uint8 [N, K/128].
//
// GEMV: out[m, n] = bf16_RNE( sum_g s16 (sum_{k in g} x q - z sum_{k in g} x) ).
#include "common.h"
#include "launch.h"

namespace nvfp4k {

namespace {
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// 8 unsigned nibbles (dword w, element 2j in the low nibble of byte j) -> 8
// bf16 values q, exactly: a byte 0x00..0x0F read as E4M3 is q * 2^-9, and the
// conversion scales by 2^9 (it applies the exponent of its scale operand).
__device__ __forceinline__ short8v uint4x8_bf16(uint32_t w) {
  const uint32_t ev = w & 0x0F0F0F0Fu;          // elements 0, 2, 4, 6
  const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;   // elements 1, 3, 5, 7
  const uint32_t lo = __builtin_amdgcn_perm(od, ev, 0x05010400u);   // e0 e1 e2 e3
  const uint32_t hi = __builtin_amdgcn_perm(od, ev, 0x07030602u);   // e4 e5 e6 e7
  const bf16x2v p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, false);
  const bf16x2v p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, true);
  const bf16x2v p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, false);
  const bf16x2v p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, true);
  const short2v s0 = __builtin_bit_cast(short2v, p0), s1 = __builtin_bit_cast(short2v, p1);
  const short2v s2 = __builtin_bit_cast(short2v, p2), s3 = __builtin_bit_cast(short2v, p3);
  return short8v{s0.x, s0.y, s1.x, s1.y, s2.x, s2.y, s3.x, s3.y};
}

constexpr short kOneBf16 = (short)0x3F80;     // 1.0 in bf16

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}
__device__ __forceinline__ short8v as_short8(const uint4& v) { return __builtin_bit_cast(short8v, v); }
}  // namespace

// ---- quantize: 16 lanes per group of 128, 8 values (16 bytes) per lane ------
__global__ __launch_bounds__(256) void int4g_asym_quant_kernel(const uint4* __restrict__ w, int64_t ngroups,
                                                               uint32_t* __restrict__ q,
                                                               uint16_t* __restrict__ scales,
                                                               uint8_t* __restrict__ zeros) {
  const int64_t gthreads = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < ngroups * 16; t += gthreads) {
    // every lane of a 16-lane group runs the same trip count (blockDim and
    // the grid stride are multiples of 16), so the shuffles see full groups
    const uint4 v = w[t];
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float f = bf16_bits_to_f32((x[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
      lo = fminf(lo, f);
      hi = fmaxf(hi, f);
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      lo = fminf(lo, __shfl_xor(lo, o, 16));
      hi = fmaxf(hi, __shfl_xor(hi, o, 16));
    }
    const float s32 = (hi - lo) / 15.0f;
    const uint32_t s16 = f32_to_f16_rne(s32);
    const float s = f16_bits_to_f32(s16);
    float z = 0.0f;
    if (s != 0.0f) z = fminf(fmaxf(__builtin_rintf((-lo) / s), 0.0f), 15.0f);
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t qi = 0;
      if (s != 0.0f) {
        const float y = __builtin_rintf(bf16_bits_to_f32((x[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) / s) + z;
        qi = (uint32_t)fminf(fmaxf(y, 0.0f), 15.0f);
      }
      out |= qi << (4 * i);
    }
    q[t] = out;
    if ((t & 15) == 0) {
      scales[t >> 4] = (uint16_t)s16;
      zeros[t >> 4] = (uint8_t)z;
    }
  }
}

// ---- GEMV, M <= 2: row-slot layout (weight read in storage order) ----------
// As the symmetric INT4 row-slot kernel: lane i + 16 g of slot s loads the
// 16-byte piece 4 i + g (group i's quarter g), the MFMA's diagonal D[i][i]
// sums group i.  One extra MFMA chain per wave against a constant 1 gives
// the group sums of x; per row the diagonal lane of group i forms
// s16 (sum x q - z sum x).
template <int kM, int kR>
__global__ __launch_bounds__(1024) void int4g_asym_gemv_rowslot_kernel(const uint16_t* __restrict__ x,
                                                                       const uint8_t* __restrict__ q,
                                                                       const uint16_t* __restrict__ s,
                                                                       const uint8_t* __restrict__ zp,
                                                                       uint16_t* __restrict__ out, int M, int N,
                                                                       int K) {
  extern __shared__ __attribute__((aligned(16))) float4v s_diag[];   // [slots][kR][kM][16]
  const int lane = threadIdx.x & 63;
  const int slot = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nslots = blockDim.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const uint32_t row_bytes = (uint32_t)K / 2, row_groups = (uint32_t)K / 128;
  const int n0 = blockIdx.x * kR;
  const uint32_t nrows = (uint32_t)min(kR, N - n0);
  const auto qr = buffer_of(q + (int64_t)n0 * row_bytes, nrows * row_bytes);
  const auto sr = buffer_of(s + (int64_t)n0 * row_groups, nrows * row_groups * 2);
  const auto zr = buffer_of(zp + (int64_t)n0 * row_groups, nrows * row_groups);
  const auto xr = buffer_of(x, (uint32_t)M * K * 2);

  const uint32_t piece = 1024u * slot + 16u * (4 * i + g);
  const bool in = piece < row_bytes;
  const uint32_t qoff = in ? piece : kBufferOob;
  const uint32_t k0 = 2u * piece;
  const bool gin = 16u * slot + i < row_groups;
  const uint32_t goff = gin ? 16u * slot + i : kBufferOob;
  uint4 xv[kM][4];
#pragma unroll
  for (int m = 0; m < kM; ++m)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) xv[m][jj] = buffer_load16(xr, in ? 2u * (m * (uint32_t)K + k0 + 8u * jj) : kBufferOob);
  uint4 wq[kR];
  uint32_t ws[kR], wz[kR];
#pragma unroll
  for (int rho = 0; rho < kR; ++rho) {
    wq[rho] = buffer_load16<kCachePolicyNT>(qr, qoff + rho * row_bytes);
    ws[rho] = buffer_load2<kCachePolicyNT>(sr, gin ? 2u * (goff + rho * row_groups) : kBufferOob);
    wz[rho] = __builtin_amdgcn_raw_buffer_load_b8(zr, gin ? goff + rho * row_groups : kBufferOob, 0, kCachePolicyNT);
  }
  __builtin_amdgcn_sched_barrier(0);

  const short8v one8 = {kOneBf16, kOneBf16, kOneBf16, kOneBf16, kOneBf16, kOneBf16, kOneBf16, kOneBf16};
  float4v xsum[kM];                     // D[i][i] = sum of x over group i
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    xsum[m] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      xsum[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(one8, as_short8(xv[m][jj]), xsum[m], 0, 0, 0);
  }
  float4v tot[kR][kM];
#pragma unroll
  for (int rho = 0; rho < kR; ++rho) {
    const float sc = f16_bits_to_f32(ws[rho] & 0xFFFFu);
    const float zf = (float)(wz[rho] & 0xFFu);
#pragma unroll
    for (int m = 0; m < kM; ++m) tot[rho][m] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const short8v wv = uint4x8_bf16(word_of(wq[rho], jj));
#pragma unroll
      for (int m = 0; m < kM; ++m)
        tot[rho][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv, as_short8(xv[m][jj]), tot[rho][m], 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < kM; ++m) tot[rho][m] = (tot[rho][m] - zf * xsum[m]) * sc;
  }

  // D[i][i] sits at lane i + 16 (i / 4), register i % 4.
  if ((i >> 2) == g) {
#pragma unroll
    for (int rho = 0; rho < kR; ++rho)
#pragma unroll
      for (int m = 0; m < kM; ++m) s_diag[((slot * kR + rho) * kM + m) * 16 + i] = tot[rho][m];
  }
  __syncthreads();
  for (int t = threadIdx.x; t < 16 * kR * kM; t += blockDim.x) {
    const int pair = t >> 4, ii = t & 15;
    float v = 0.f;
    for (int w = 0; w < nslots; ++w) v += s_diag[(w * kR * kM + pair) * 16 + ii][ii & 3];
    v += __shfl_xor(v, 1, 16);
    v += __shfl_xor(v, 2, 16);
    v += __shfl_xor(v, 4, 16);
    v += __shfl_xor(v, 8, 16);
    const int rho = pair / kM, m = pair % kM;
    if (ii == 0 && m < M && n0 + rho < N) out[(int64_t)m * N + n0 + rho] = (uint16_t)f32_to_bf16_rne(v);
  }
}

// ---- GEMV/GEMM, any M: one output per thread ---------------------------------
__global__ __launch_bounds__(64) void int4g_asym_simple_kernel(const uint16_t* __restrict__ x,
                                                               const uint8_t* __restrict__ q,
                                                               const uint16_t* __restrict__ s,
                                                               const uint8_t* __restrict__ zp,
                                                               uint16_t* __restrict__ out, int M, int N, int K) {
  const int n = blockIdx.x * 64 + threadIdx.x;
  if (n >= N) return;
  const int ng = K / 128;
  for (int m = blockIdx.y; m < M; m += gridDim.y) {
    const uint16_t* xr = x + (int64_t)m * K;
    const uint32_t* qr = (const uint32_t*)(q + (int64_t)n * (K / 2));
    float acc = 0.0f;
    for (int gi = 0; gi < ng; ++gi) {
      const float zf = (float)zp[(int64_t)n * ng + gi];
      float gs = 0.0f;
      for (int d = 0; d < 16; ++d) {
        const uint32_t wd = qr[gi * 16 + d];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float qe = (float)((wd >> (4 * e)) & 15u) - zf;
          gs += bf16_bits_to_f32(xr[gi * 128 + d * 8 + e]) * qe;
        }
      }
      acc += f16_bits_to_f32(s[(int64_t)n * ng + gi]) * gs;
    }
    out[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(acc);
  }
}

// ---- launchers ----------------------------------------------------------------
hipError_t launch_int4g_asym_quantize(const void* w, int64_t N, int64_t K, uint8_t* q, void* scales, uint8_t* zeros,
                                      hipStream_t stream) {
  const int64_t ngroups = N * (K / 128);
  int64_t grid = (ngroups * 16 + 255) / 256;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(int4g_asym_quant_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (const uint4*)w, ngroups,
                     (uint32_t*)q, (uint16_t*)scales, zeros);
  return hipGetLastError();
}

namespace {
template <int kM, int kR>
void launch_asym_rowslot(const void* x, const uint8_t* q, const void* s, const uint8_t* z, void* out, int M, int N,
                         int K, hipStream_t stream) {
  const int nslots = (K / 2 + 1023) / 1024;
  const size_t lds = (size_t)nslots * kR * kM * 16 * sizeof(float4v);
  hipLaunchKernelGGL((int4g_asym_gemv_rowslot_kernel<kM, kR>), dim3((unsigned)((N + kR - 1) / kR)),
                     dim3(64 * nslots), lds, stream, (const uint16_t*)x, q, (const uint16_t*)s, z, (uint16_t*)out,
                     M, N, K);
}
}  // namespace

bool int4g_asym_decode_supported(int64_t M, int64_t K) {
  return M >= 1 && M <= 2 && K > 0 && K <= 16 * 2048 && M * K * 2 < (1ll << 31);
}

hipError_t launch_int4g_asym_decode(const void* x, const uint8_t* q, const void* s, const uint8_t* z, void* out,
                                    int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  // Rows per workgroup, interleaved runs on 28672 x 8192 (identical outputs):
  // M = 1: 8 rows 24.4 us, 4 rows 28.6 us; M = 2: 6 rows 34.1 us, 4 rows
  // 41.0 us, 8 rows 38.7 us (spills registers).
  if (M == 1) {
    launch_asym_rowslot<1, 8>(x, q, s, z, out, (int)M, (int)N, (int)K, stream);
  } else {
    launch_asym_rowslot<2, 6>(x, q, s, z, out, (int)M, (int)N, (int)K, stream);
  }
  return hipGetLastError();
}

hipError_t launch_int4g_asym_simple(const void* x, const uint8_t* q, const void* s, const uint8_t* z, void* out,
                                    int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  hipLaunchKernelGGL(int4g_asym_simple_kernel, dim3((unsigned)((N + 63) / 64), (unsigned)(M < 65535 ? M : 65535)),
                     dim3(64), 0, stream, (const uint16_t*)x, q, (const uint16_t*)s, z, (uint16_t*)out, (int)M,
                     (int)N, (int)K);
  return hipGetLastError();
}

}  // namespace nvfp4k
