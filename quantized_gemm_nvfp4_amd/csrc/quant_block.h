// The absmax block quantizer of one 16-value NVFP4 block, shared by the
// quantize kernels and the decode kernel that quantizes its activation
// itself ("Tu pipeline NVFP4 ...", section 2: block scale from the block's
// largest magnitude, E2M1 codes; the per-tensor scale g above the block
// scales).  Every step is an fp32 operation with one rounding, in the order
// the format's definition gives, so the codes are bit-exact.
#pragma once

#include "common.h"

namespace nvfp4k {

// The element step divides |x| by the block's d with one rounding.  Per
// element that division is replaced by the block's reciprocal r = 1/d
// (correctly rounded, once per block) and Markstein's correction: q = x r
// lies within one ulp of the quotient, the remainder q d - x is exact in
// one fma, and q - (q d - x) r rounded once is the correctly rounded
// quotient.  Each step is odd in x under round-to-nearest-even, so taken on
// the signed x it gives the quotient of |x| with x's sign (-0 and +0
// included) and no separate sign step.  It equals the division for every
// bf16 significand, of either sign, against every fp32 significand
// (tests/quotient_check.c runs all 2^30 pairs) as long as no step under- or
// overflows, which holds for 2^-64 <= d < 2^100; blocks outside that range
// divide.
constexpr float kQuotLo = 0x1p-64f, kQuotHi = 0x1p100f;

__device__ __forceinline__ bool quot_fast(float d) { return d >= kQuotLo && d < kQuotHi; }

// |x| / d (one rounding: the element step above) carrying the sign of x,
// for x given as the fp32 pattern of a bf16 value.
template <bool kFast>
__device__ __forceinline__ float signed_quotient(uint32_t xbits, float d, float r) {
#pragma clang fp contract(off)
  if (kFast) {
    const float x = __uint_as_float(xbits);
    const float q = x * r;
    return __builtin_fmaf(-__builtin_fmaf(q, d, -x), r, q);
  }
  const float ax = __uint_as_float(xbits & 0x7FFFFFFFu);
  const float y = (d != 0.0f) ? ax / d : 0.0f;
  return __uint_as_float(__float_as_uint(y) | (xbits & 0x80000000u));
}

// Codes of a block under d, two per byte (element 2j in the low nibble).
// v_cvt_scalef32_pk_fp4_f32 (scale 1.0: no scaling) rounds two fp32 values
// to E2M1 codes, nearest even, saturating at 6, sign kept, into the byte
// its last operand selects: the code of element_code for every fp32 input
// (compared on gfx950 over all 2^32 patterns, NaN and infinities
// included), so the quotient's rounding is the only arithmetic step.
template <bool kFast>
__device__ __forceinline__ uint2 encode_block(const uint32_t (&w)[8], float d, float r) {
  float y[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    y[2 * i] = signed_quotient<kFast>(w[i] << 16, d, r);
    y[2 * i + 1] = signed_quotient<kFast>(w[i] & 0xFFFF0000u, d, r);
  }
  uint32_t p0 = 0u, p1 = 0u;
  p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, y[0], y[1], 1.0f, 0);
  p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, y[2], y[3], 1.0f, 1);
  p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, y[4], y[5], 1.0f, 2);
  p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, y[6], y[7], 1.0f, 3);
  p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, y[8], y[9], 1.0f, 0);
  p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, y[10], y[11], 1.0f, 1);
  p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, y[12], y[13], 1.0f, 2);
  p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, y[14], y[15], 1.0f, 3);
  return make_uint2(p0, p1);
}

// RN(a / b) from rb = RN(1 / b) by the same correction (a of either sign),
// valid while no step under- or overflows.
__device__ __forceinline__ float div_by_recip(float a, float b, float rb) {
#pragma clang fp contract(off)
  const float q = a * rb;
  return __builtin_fmaf(-__builtin_fmaf(q, b, -a), rb, q);
}

// RN(1 / g) for the block-scale step when 2^-60 <= g <= 2^60, else 0 (the
// step then divides).  Taken once per thread or workgroup, not per block.
__device__ __forceinline__ float scale_recip(float g) {
#pragma clang fp contract(off)
  return (g >= 0x1p-60f && g <= 0x1p60f) ? 1.0f / g : 0.0f;
}

// E4M3 code of (amax_b / top) / g, each division rounded once; top is 6 or
// 4 (a compile-time constant after inlining), rg = scale_recip(g).  With g
// in the range scale_recip accepts and amax_b zero or in [2^-60, 2^60],
// both quotients stay inside the normal fp32 range and come from the
// reciprocals; other values (NaN and infinities included) divide.
__device__ __forceinline__ uint32_t scale_code(float amax_b, float top, float g, float rg) {
#pragma clang fp contract(off)
  float s_raw;
  if (g == 0.0f) {
    s_raw = 0.0f;
  } else if (rg != 0.0f && amax_b <= 0x1p60f && !(amax_b > 0.0f && amax_b < 0x1p-60f)) {
    const float rtop = 1.0f / top;   // folded: RN(1/6) or exactly 1/4
    s_raw = div_by_recip(div_by_recip(amax_b, top, rtop), g, rg);
  } else {
    s_raw = (amax_b / top) / g;
  }
  return e4m3_from_f32_sat(s_raw);
}

// Scale byte and codes of the block of 16 bf16 values in w (element 2 i in
// the low and 2 i + 1 in the high half of w[i]) under the absmax rule and
// global scale g (rg = scale_recip(g)).
__device__ __forceinline__ uint2 absmax_block(const uint32_t (&w)[8], float g, float rg, uint32_t& sc) {
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax_bits = max(amax_bits, bf16x2_absmax_bits(w[i]));
  sc = scale_code(bf16_bits_to_f32(amax_bits), 6.0f, g, rg);
  const float d = e4m3_to_f32(sc) * g;
  return quot_fast(d) ? encode_block<true>(w, d, 1.0f / d) : encode_block<false>(w, d, 0.0f);
}

}  // namespace nvfp4k
