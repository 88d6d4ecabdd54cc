// Device helpers shared by the NVFP4 / INT4 kernels (gfx950, wave64).
//
// Number formats (pages cited by title and section):
//  - "Tu pipeline NVFP4 ...", section 2: E2M1 elements (1 sign, 2 exponent,
//    1 mantissa bit, largest magnitude 6), one FP8 E4M3 scale per 16 values.
//  - "NVFP4 en difusión ...", section 2: the scale type is float8_e4m3fn
//    (OCP "finite" variant: bias 7, largest finite 448, no infinities).
//
// The conversions below work on IEEE bit patterns: a round-to-nearest-even
// to n mantissa bits is "add half an ulp minus one, plus the kept LSB, then
// truncate", which also carries into the exponent when the mantissa
// overflows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace nvfp4k {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef short short2v __attribute__((ext_vector_type(2)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));

constexpr int kBlock = 16;        // values per NVFP4 scale block

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; overflow -> inf).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> two bf16 (round to nearest even) in one dword, a in the low
// half: v_cvt_pk_bf16_f32, bit-identical to f32_to_bf16_rne for every
// non-NaN input (checked on gfx950 over all 2^32 patterns).
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{a, b}, bf16x2v));
}

// E4M3 (fn) byte of a non-negative fp32, RNE, saturating to 448 (0x7E)
// above the largest finite value (and for +inf).
__device__ __forceinline__ uint32_t e4m3_from_f32_sat(float v) {
  if (!(v <= 448.0f)) return 0x7Eu;
  if (v < 0.015625f) {                       // below 2^-6: quantum 2^-9
    return (uint32_t)__builtin_rintf(v * 512.0f);   // 0..8; 8 is 2^-6
  }
  uint32_t b = __float_as_uint(v);
  uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;   // exp8:3 | man3
  return r - (120u << 3);                   // rebias 127 -> 7
}

// Value of a non-negative E4M3 byte (0x00..0x7E) as fp32, exact.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = c >> 3, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;          // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// fp32 -> fp16 bits, RNE, gradual underflow, overflow -> inf.
__device__ __forceinline__ uint32_t f32_to_f16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t sign = (u >> 16) & 0x8000u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x477FF000u) return sign | 0x7C00u;              // >= 65520
  if (a < 0x38800000u) {                                     // below 2^-14
    float t = __uint_as_float(a) * 16777216.0f;              // units of 2^-24
    return sign | (uint32_t)__builtin_rintf(t);
  }
  uint32_t r = (a + 0xFFFu + ((a >> 13) & 1u)) >> 13;
  return sign | (r - (112u << 10));
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  _Float16 x = __builtin_bit_cast(_Float16, (unsigned short)h);
  return (float)x;
}

// Raw buffer resources (gfx9 descriptor word 3 for an untyped buffer): the
// hardware range-checks every access against `bytes`, and loads past the end
// return zero, so callers can map tails to an offset past the end instead of
// branching (and keep every wave's load count the same).
constexpr uint32_t kBufferOob = 0x80000000u;     // an offset past every buffer's end
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kCachePolicyNT = 2;                // streamed once: non-temporal

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferWord3);
}

template <int kAux = 0>
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAux);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int kAux = 0>
__device__ __forceinline__ uint32_t buffer_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kAux);
}

template <int kAux = 0>
__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kAux);
}

// Largest bf16 magnitude pattern among the two bf16 in a dword.
__device__ __forceinline__ uint32_t bf16x2_absmax_bits(uint32_t w) {
  uint32_t lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
  return lo > hi ? lo : hi;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t t = __shfl_xor(v, o, 64);
    v = v > t ? v : t;
  }
  return v;
}

// Two E2M1 codes of byte `sel` of `w` -> two fp16 (element 2j low nibble in
// .x), exact.  The hardware conversion applies only the exponent of its fp32
// scale operand; with 1.0 it is a plain decode.
template <int sel>
__device__ __forceinline__ half2v e2m1x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, sel);
}

// Dequantize the 8 E2M1 codes in dword `w` and multiply by the block scale
// `s2` (the scale in both halves): every product has at most 6 significant
// bits and lies in [2^-10, 2688], so it is exact in fp16.
__device__ __forceinline__ half8v dequant8_f16(uint32_t w, half2v s2) {
  half2v p0 = e2m1x2_to_f16<0>(w) * s2;
  half2v p1 = e2m1x2_to_f16<1>(w) * s2;
  half2v p2 = e2m1x2_to_f16<2>(w) * s2;
  half2v p3 = e2m1x2_to_f16<3>(w) * s2;
  return half8v{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// E4M3 byte -> fp16 scale in both halves (exact: E4M3 values are fp16 normals).
__device__ __forceinline__ half2v e4m3_to_f16x2(uint32_t byte) {
  float f = __builtin_amdgcn_cvt_f32_fp8(byte, 0);
  _Float16 h = (_Float16)f;
  return half2v{h, h};
}

// Two E4M3 scale bytes (low half of `pair`) -> fp16 in both halves, each
// equal to the scale times 2^-8, exact: the E4M3 bit pattern shifted left by
// 7 is an fp16 pattern with the same mantissa and exponent bits, and the bias
// difference (15 - 7) divides by 2^8 (subnormal scales included).
__device__ __forceinline__ half2v e4m3x2_to_f16x2_div256(uint32_t pair) {
  const uint32_t spread = __builtin_amdgcn_perm(0u, pair, 0x0C010C00u);   // [b0, 0, b1, 0]
  return __builtin_bit_cast(half2v, spread << 7);
}

// Eight E2M1 codes of `w` times a block scale given as scale * 2^-8 (see
// e4m3x2_to_f16x2_div256): the conversion multiplies by 2^8 (a power of two,
// applied exactly), so every product equals code value * scale exactly.
__device__ __forceinline__ half8v dequant8_f16_div256(uint32_t w, half2v s2) {
  half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * s2;
  half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * s2;
  half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * s2;
  half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * s2;
  return half8v{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Signed INT4 nibble pair of byte `sel` -> two bf16 bit patterns in a dword
// (exact: |q| <= 8).
__device__ __forceinline__ uint32_t int4x2_to_bf16x2(uint32_t w, int sel) {
  int lo = (int)(w << (28 - 8 * sel)) >> 28;
  int hi = (int)(w << (24 - 8 * sel)) >> 28;
  uint32_t blo = __float_as_uint((float)lo) >> 16;
  uint32_t bhi = __float_as_uint((float)hi) & 0xFFFF0000u;
  return bhi | blo;
}

// ---- waits, barriers and LDS addresses for kernels that copy into LDS ----
typedef unsigned uint2v __attribute__((ext_vector_type(2)));
typedef unsigned uint4v __attribute__((ext_vector_type(4)));

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
// s_waitcnt lgkmcnt(0): this wave's LDS accesses are complete.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// A workgroup barrier without the memory fence of __syncthreads() (which
// would also wait for every copy in flight).
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Byte address in LDS of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

}  // namespace nvfp4k
