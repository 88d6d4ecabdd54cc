// Roofline denominators measured on the device itself: a dense fp16 MFMA
// issue loop and an HBM read stream.  bench.py reports the path's fractions
// against these next to the published peaks (2.5 PFLOP/s dense fp16,
// 8 TB/s HBM3E).  Measurement code only: nothing in libnvfp4.so uses it.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kChains = 4;          // independent accumulators per wave
constexpr int kMfmaThreads = 256;   // 4 waves per workgroup
constexpr int kMfmaWgsPerCu = 2;    // 2 waves per SIMD
constexpr int kReadThreads = 256;
constexpr int kReadMaxWgsPerCu = 8;
constexpr int kReadDepth = 8;       // 16-byte loads per lane in flight

// Every wave issues kChains independent chains of v_mfma_f32_16x16x32_f16
// (16 x 16 x 32 x 2 = 16384 flops each), `iters` (a multiple of 4) times;
// one float per thread goes out so the loop is kept.
__global__ __launch_bounds__(kMfmaThreads) void peak_mfma_kernel(int iters, float* __restrict__ out) {
  const int t = blockIdx.x * kMfmaThreads + threadIdx.x;
  half8v a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(float)((t + i) & 7) * (_Float16)0.125f;
    b[i] = (_Float16)(float)((t * 3 + i) & 7) * (_Float16)0.0625f;
  }
  float4v acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = float4v{0.f, 0.f, 0.f, 0.f};
  // The MFMAs are written as one asm statement per trip (16 of them, four
  // per accumulator): written as builtins, the compiler rotated the
  // accumulators through other registers every trip, with moves the MFMAs
  // then waited for.  No memory access is inside.
  for (int it = 0; it < iters; it += 4) {
    asm volatile(
        "v_mfma_f32_16x16x32_f16 %0, %4, %5, %0\n\t"
        "v_mfma_f32_16x16x32_f16 %1, %4, %5, %1\n\t"
        "v_mfma_f32_16x16x32_f16 %2, %4, %5, %2\n\t"
        "v_mfma_f32_16x16x32_f16 %3, %4, %5, %3\n\t"
        "v_mfma_f32_16x16x32_f16 %0, %4, %5, %0\n\t"
        "v_mfma_f32_16x16x32_f16 %1, %4, %5, %1\n\t"
        "v_mfma_f32_16x16x32_f16 %2, %4, %5, %2\n\t"
        "v_mfma_f32_16x16x32_f16 %3, %4, %5, %3\n\t"
        "v_mfma_f32_16x16x32_f16 %0, %4, %5, %0\n\t"
        "v_mfma_f32_16x16x32_f16 %1, %4, %5, %1\n\t"
        "v_mfma_f32_16x16x32_f16 %2, %4, %5, %2\n\t"
        "v_mfma_f32_16x16x32_f16 %3, %4, %5, %3\n\t"
        "v_mfma_f32_16x16x32_f16 %0, %4, %5, %0\n\t"
        "v_mfma_f32_16x16x32_f16 %1, %4, %5, %1\n\t"
        "v_mfma_f32_16x16x32_f16 %2, %4, %5, %2\n\t"
        "v_mfma_f32_16x16x32_f16 %3, %4, %5, %3"
        : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3])
        : "v"(a), "v"(b));
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[t] = s;
}

__device__ __forceinline__ uint4 load_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);   // non-temporal
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Reads `bytes` (< 2^31) once: wave w takes the 1 KB chunks w, w + W,
// w + 2W, ... (W waves in the grid), 16 bytes per lane, with kReadDepth
// chunks in flight (each chunk's load is reissued for chunk + kReadDepth W as
// soon as it has been consumed); XOR of everything per lane goes out.
// Offsets past the end read zero.
__global__ __launch_bounds__(kReadThreads) void peak_read_kernel(const void* __restrict__ src, uint32_t bytes,
                                                                 uint32_t* __restrict__ out) {
  const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), 0, (int)bytes, 0x00020000);
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t w = blockIdx.x * (kReadThreads / 64) + (threadIdx.x >> 6);
  const uint32_t W = gridDim.x * (kReadThreads / 64);
  const uint32_t nch = (bytes + 1023u) / 1024u;
  uint4 v[kReadDepth];
#pragma unroll
  for (int d = 0; d < kReadDepth; ++d) {
    const uint32_t c = w + d * W;
    v[d] = load_nt(r, c < nch ? 1024u * c + 16u * lane : 0x80000000u);
  }
  uint32_t x = 0;
  for (uint32_t c0 = w; c0 < nch; c0 += kReadDepth * W) {
#pragma unroll
    for (int d = 0; d < kReadDepth; ++d) {
      x ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
      const uint32_t c = c0 + (d + kReadDepth) * W;
      v[d] = load_nt(r, c < nch ? 1024u * c + 16u * lane : 0x80000000u);
    }
  }
  out[blockIdx.x * kReadThreads + threadIdx.x] = x;
}

// The same stream of 1 KB chunks as peak_read_kernel, but each chunk goes
// to LDS by DMA (buffer_load_dwordx4 ... lds, as the GEMM kernels copy their
// operands): wave w keeps kReadDepth chunks in flight in a ring of
// kReadDepth 1 KB slots of its own, waiting (vmcnt) only for the oldest
// before reusing its slot.  Four waves per workgroup, one workgroup per CU
// (the ring takes 32 KB of LDS).  Offsets past the end read zero.
constexpr int kLdsWaves = 4;
__shared__ __attribute__((aligned(1024))) uint8_t g_read_ring[kLdsWaves * kReadDepth * 1024];
typedef __attribute__((address_space(3))) void* lds_void_t;
__device__ __forceinline__ void read_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, uint8_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t)dst, 16, off, 0, 0, 0);
}
__global__ __launch_bounds__(64 * kLdsWaves) void peak_read_lds_kernel(const void* __restrict__ src, uint32_t bytes,
                                                                        uint32_t* __restrict__ out) {
  const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), 0, (int)bytes, 0x00020000);
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t w = blockIdx.x * kLdsWaves + wave, W = gridDim.x * kLdsWaves;
  const uint32_t nch = (bytes + 1023u) / 1024u;
  uint8_t* ring = g_read_ring + wave * kReadDepth * 1024;
  uint32_t slot = 0;
  for (uint32_t c = w; c < nch; c += W) {
    read_to_lds(r, 1024u * c + 16u * lane, ring + slot * 1024);
    slot = slot + 1 == kReadDepth ? 0 : slot + 1;
    // vmcnt(kReadDepth - 1): the chunk issued kReadDepth chunks ago has
    // landed, so its slot may be written again
    __builtin_amdgcn_s_waitcnt(((kReadDepth - 1) & 0xF) | (((kReadDepth - 1) >> 4) << 14) | 0x70 | 0xF00);
  }
  __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);   // vmcnt(0): nothing lands after the workgroup ends
  __syncthreads();
  out[blockIdx.x * 64 * kLdsWaves + threadIdx.x] = ring[lane];
}

// The tiled GEMM's matrix instruction, v_mfma_f32_32x32x16_f16, at one
// wave per SIMD (one 4-wave workgroup per CU, as the GEMM runs), with
// operands that change every instruction: each wave holds four A and four B
// operands and issues 16 MFMAs per trip over four independent accumulators,
// each pairing a different (A, B).  The operand values are drawn in the
// prologue from a per-lane hash (no memory access inside the loop):
//   mode 0: zeros;
//   mode 1: E2M1 value x E4M3 scale products, the values the GEMM feeds the
//           matrix cores (signed codes from {0.5, 1, 1.5, 2, 3, 4, 6}, block
//           scales 2^[-4, 3] x (1 + j/8));
//   mode 2: random fp16 (random sign and 10-bit mantissa, exponent in
//           [-4, 3]).
// kV independent vector instructions (v_xor_b32 on registers no MFMA reads)
// follow every MFMA, so the loop measures what issuing vector work between
// the MFMAs costs.  The matrix cores' rate depends on the operand bits
// (power), which is why the three modes differ.
typedef float float16v __attribute__((ext_vector_type(16)));
constexpr int kMixThreads = 256;

__device__ __forceinline__ uint32_t mix_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__device__ __forceinline__ _Float16 mix_value(int mode, uint32_t h) {
  if (mode == 0) return (_Float16)0.0f;
  const float sign = (h & 1u) ? -1.0f : 1.0f;
  if (mode == 1) {
    const float e2m1[7] = {0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    const float c = e2m1[(h >> 1) % 7u];
    const float scale = __builtin_ldexpf(1.0f + 0.125f * (float)((h >> 4) & 7u), (int)((h >> 7) & 7u) - 4);
    return (_Float16)(sign * c * scale);
  }
  const float m = 1.0f + (float)((h >> 1) & 1023u) / 1024.0f;
  return (_Float16)(sign * __builtin_ldexpf(m, (int)((h >> 11) & 7u) - 4));
}

#define PK_MF(C, A, B) "v_mfma_f32_32x32x16_f16 %" #C ", %" #A ", %" #B ", %" #C "\n\t"
#define PK_VX(U) "v_xor_b32 %" #U ", %" #U ", %16\n\t"
// kP = 0: both operands change with every MFMA; kP = 1: the GEMM's order,
// the first operand (a weight fragment) held for eight MFMAs while the second
// (an activation fragment) changes with every one.
#define PK_BODY(V)                                                                                        \
  PK_MF(0, 8, 12) V PK_MF(1, 9, 13) V PK_MF(2, 10, 14) V PK_MF(3, 11, 15) V PK_MF(0, 9, 14) V              \
  PK_MF(1, 10, 15) V PK_MF(2, 11, 12) V PK_MF(3, 8, 13) V PK_MF(0, 10, 12) V PK_MF(1, 11, 13) V           \
  PK_MF(2, 8, 14) V PK_MF(3, 9, 15) V PK_MF(0, 11, 14) V PK_MF(1, 8, 15) V PK_MF(2, 9, 12) V              \
  PK_MF(3, 10, 13) V
#define PK_BODY_HOLD(V)                                                                                   \
  PK_MF(0, 8, 12) V PK_MF(1, 8, 13) V PK_MF(2, 8, 14) V PK_MF(3, 8, 15) V PK_MF(0, 8, 12) V                \
  PK_MF(1, 8, 13) V PK_MF(2, 8, 14) V PK_MF(3, 8, 15) V PK_MF(0, 9, 12) V PK_MF(1, 9, 13) V               \
  PK_MF(2, 9, 14) V PK_MF(3, 9, 15) V PK_MF(0, 9, 12) V PK_MF(1, 9, 13) V PK_MF(2, 9, 14) V               \
  PK_MF(3, 9, 15) V
#define PK_ASM(BODY)                                                                                     \
  asm volatile(BODY                                                                                      \
               : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+v"(u0), "+v"(u1), "+v"(u2), "+v"(u3) \
               : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]), "v"(k))

template <int kV, int kP>
__global__ __launch_bounds__(kMixThreads) void peak_mfma_mix_kernel(int iters, int mode, float* __restrict__ out) {
  const uint32_t t = blockIdx.x * kMixThreads + threadIdx.x;
  half8v a[4], b[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[r][i] = mix_value(mode, mix_hash(t * 64u + r * 8u + i));
      b[r][i] = mix_value(mode, mix_hash(t * 64u + 32u + r * 8u + i));
    }
  float16v acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  uint32_t u0 = t, u1 = t + 1u, u2 = t + 2u, u3 = t + 3u;
  const uint32_t k = mix_hash(t);
  for (int it = 0; it < iters; it += 16) {
    if (kP == 0) {
      if (kV == 0) PK_ASM(PK_BODY(""));
      else if (kV == 2) PK_ASM(PK_BODY(PK_VX(4) PK_VX(5)));
      else PK_ASM(PK_BODY(PK_VX(4) PK_VX(5) PK_VX(6) PK_VX(7)));
    } else {
      if (kV == 0) PK_ASM(PK_BODY_HOLD(""));
      else if (kV == 2) PK_ASM(PK_BODY_HOLD(PK_VX(4) PK_VX(5)));
      else PK_ASM(PK_BODY_HOLD(PK_VX(4) PK_VX(5) PK_VX(6) PK_VX(7)));
    }
  }
  float s = (float)(u0 ^ u1 ^ u2 ^ u3) * 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  out[t] = s;
}
#undef PK_ASM
#undef PK_BODY_HOLD
#undef PK_BODY
#undef PK_VX
#undef PK_MF

int cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess)
      n = 0;
  }
  return n;
}

}  // namespace

extern "C" {

// Threads of either kernel's largest grid: the length of `out` (floats / uint32).
int peak_out_elems(void) {
  const int a = cus() * kMfmaWgsPerCu * kMfmaThreads, b = cus() * kReadMaxWgsPerCu * kReadThreads;
  return a > b ? a : b;
}

// Launches the MFMA loop on `stream`; *flops receives the flops it performs.
// Returns a hipError_t value (0 = success).
int peak_mfma(int iters, float* out, double* flops, void* stream) {
  if (iters <= 0 || iters % 4 != 0 || out == nullptr || flops == nullptr || cus() <= 0)
    return (int)hipErrorInvalidValue;
  const int grid = cus() * kMfmaWgsPerCu;
  *flops = (double)grid * (kMfmaThreads / 64) * iters * kChains * 16384.0;
  hipLaunchKernelGGL(peak_mfma_kernel, dim3(grid), dim3(kMfmaThreads), 0, (hipStream_t)stream, iters, out);
  return (int)hipGetLastError();
}

// Launches the 32x32x16 MFMA loop (one 4-wave workgroup per CU) with
// operand data `mode` (0 zeros, 1 E2M1 x E4M3 products, 2 random fp16),
// `valu` (0, 2 or 4) vector instructions after every MFMA and operand order
// `hold` (0: both operands change every MFMA; 1: the first held for eight
// MFMAs, as in the GEMM); iters a multiple of 16.  *flops receives the flops
// it performs.  Returns a hipError_t value.
int peak_mfma_mix(int iters, int mode, int valu, int hold, float* out, double* flops, void* stream) {
  if (iters <= 0 || iters % 16 != 0 || mode < 0 || mode > 2 || (valu != 0 && valu != 2 && valu != 4) ||
      (hold != 0 && hold != 1) || out == nullptr || flops == nullptr || cus() <= 0)
    return (int)hipErrorInvalidValue;
  const int grid = cus();
  *flops = (double)grid * (kMixThreads / 64) * iters * 32768.0;
  const hipStream_t st = (hipStream_t)stream;
  const dim3 g(grid), b(kMixThreads);
  if (hold == 0) {
    if (valu == 0) hipLaunchKernelGGL((peak_mfma_mix_kernel<0, 0>), g, b, 0, st, iters, mode, out);
    else if (valu == 2) hipLaunchKernelGGL((peak_mfma_mix_kernel<2, 0>), g, b, 0, st, iters, mode, out);
    else hipLaunchKernelGGL((peak_mfma_mix_kernel<4, 0>), g, b, 0, st, iters, mode, out);
  } else {
    if (valu == 0) hipLaunchKernelGGL((peak_mfma_mix_kernel<0, 1>), g, b, 0, st, iters, mode, out);
    else if (valu == 2) hipLaunchKernelGGL((peak_mfma_mix_kernel<2, 1>), g, b, 0, st, iters, mode, out);
    else hipLaunchKernelGGL((peak_mfma_mix_kernel<4, 1>), g, b, 0, st, iters, mode, out);
  }
  return (int)hipGetLastError();
}

// Launches one read of `bytes` (0 < bytes < 2^31, 16-byte aligned src) on
// `stream`, with wgs_per_cu (1 .. 8) workgroups of 4 waves per compute unit.
// Returns a hipError_t value.
int peak_read(const void* src, int64_t bytes, int wgs_per_cu, uint32_t* out, void* stream) {
  if (src == nullptr || out == nullptr || bytes <= 0 || bytes >= (int64_t(1) << 31) || cus() <= 0 ||
      wgs_per_cu < 1 || wgs_per_cu > kReadMaxWgsPerCu || (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(peak_read_kernel, dim3(cus() * wgs_per_cu), dim3(kReadThreads), 0, (hipStream_t)stream, src,
                     (uint32_t)bytes, out);
  return (int)hipGetLastError();
}

// Launches one read of `bytes` (0 < bytes < 2^31, 16-byte aligned src)
// through LDS by DMA on `stream`, one workgroup of 4 waves per compute unit.
// Returns a hipError_t value.
int peak_read_lds(const void* src, int64_t bytes, uint32_t* out, void* stream) {
  if (src == nullptr || out == nullptr || bytes <= 0 || bytes >= (int64_t(1) << 31) || cus() <= 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(peak_read_lds_kernel, dim3(cus()), dim3(64 * kLdsWaves), 0, (hipStream_t)stream, src,
                     (uint32_t)bytes, out);
  return (int)hipGetLastError();
}

}  // extern "C"
