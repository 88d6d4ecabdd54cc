// INT4 per-group W4A16 GEMM / GEMV for gfx950.
//
// out[m, n] = bf16_RNE( sum_g s16[n, g] * sum_{k in g} x[m, k] * q[n, k] ),
// the symmetric per-group scheme of "Cuantización e inferencia local"
// (formula block, b = 4, one fp16 scale per group of 128 along K).
//
// Exact decode of the weight on the matrix cores:
//  - A two's-complement nibble u holds q in [-7, 7]; u ^ 8 = q + 8 in
//    [1, 15].  An E4M3 byte 0x00..0x0F is exactly (its value) * 2^-9 (the
//    subnormals continue linearly into the first normal binade), and
//    v_cvt_scalef32_pk_bf16_fp8 with scale 2^9 (the instruction uses only the
//    scale's exponent) returns q + 8 exactly as bf16.  Spreading 8 nibbles to
//    bytes takes 5 integer ops, so the decode costs about one op per value.
//  - The offset is removed with one more MFMA per step against a constant
//    -8 operand: sum x (q + 8) + sum x (-8) = sum x q, both sides exact
//    products, summed in fp32 (the offset is small, so the two sums do not
//    cancel catastrophically).  The tiled kernel, where that MFMA would be
//    a third of the matrix work, decodes q itself (sign-magnitude bytes).
//  - Each 128-value group is accumulated in its own fp32 tile, then scaled
//    once by its fp16 scale: q * s16 is not exact in bf16, so the scale is
//    kept out of the MFMA operands.
#include "common.h"
#include "launch.h"

namespace nvfp4k {

namespace {
typedef __attribute__((address_space(3))) void* lds_void_t;
typedef __attribute__((address_space(1))) void* gbl_void_t;

// 8 int4 codes (dword w, element 2j in the low nibble of byte j) -> 8 bf16
// values q + 8 in element order.
__device__ __forceinline__ short8v int4x8_offset_bf16(uint32_t w) {
  const uint32_t t = w ^ 0x88888888u;
  const uint32_t ev = t & 0x0F0F0F0Fu;          // elements 0, 2, 4, 6
  const uint32_t od = (t >> 4) & 0x0F0F0F0Fu;   // elements 1, 3, 5, 7
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

// 8 int4 codes -> 8 bf16 values q (signed) in element order: each nibble
// becomes a sign-magnitude E4M3 byte, sign in bit 7 and |q| * 2^-9 as its
// value (subnormals for |q| <= 7, the smallest normal for 8), which the
// conversion at scale 2^9 returns exactly.  Per nibble u (two's complement):
// |q| = u for u < 8, else 16 - u = ((u ^ 7) & 7) + 1; on all eight nibbles
// at once, mask = 7 where the sign is set and |q| = ((u ^ mask) & 7) + sign,
// which never carries into the next nibble (it is at most 8).  About twice
// the work of the offset form above, but no offset term to add.
__device__ __forceinline__ short8v int4x8_signed_bf16(uint32_t w) {
  const uint32_t sg = w & 0x88888888u;                      // sign bits
  const uint32_t one = sg >> 3;                             // 1 where negative
  const uint32_t mag = ((w ^ (sg - one)) & 0x77777777u) + one;
  const uint32_t ev = (mag & 0x0F0F0F0Fu) | ((sg << 4) & 0x80808080u);          // elements 0, 2, 4, 6
  const uint32_t od = ((mag >> 4) & 0x0F0F0F0Fu) | (sg & 0x80808080u);          // elements 1, 3, 5, 7
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

// 8 unsigned nibbles (the zero-point form) -> 8 bf16 values q in element
// order: a byte 0x00..0x0F read as E4M3 is exactly q * 2^-9.
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

constexpr short kMinus8Bf16 = (short)0xC100;    // -8.0 in bf16
constexpr short kOneBf16 = (short)0x3F80;       // 1.0 in bf16

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}
__device__ __forceinline__ short8v as_short8(const uint4& v) { return __builtin_bit_cast(short8v, v); }
}  // namespace

// ---- M <= 16: stream the weight once -------------------------------------
// (Serves 3 <= M <= 16 when K % 512 != 0 or K > 32768; other decode shapes
// take the activation-stationary kernel below or the row-slot GEMV.)
// A workgroup owns kI4Groups x 16 weight rows; its kI4Waves waves take steps
// of two 128-value groups (128 bytes of a row) in turn, step t going to wave
// t % kI4Waves, and are summed in LDS in a fixed order.
//  - Per step a lane (i, g) = i + 16 g loads 16 bytes at 16 g of both groups
//    of the step from row i of each row group (the wave reads both halves of
//    each 128-byte line back to back; half lines split across waves measured
//    ~40% slower), the rows' two group scales, and x row i at the same
//    positions.  All loads are unconditional buffer loads (rows past N or M
//    and groups past K read as zero) and issue before any decoding.
//  - v_mfma_f32_16x16x32_bf16 with x as the first operand (rows m) and the
//    weight as the second (columns n), so each lane's accumulators share one
//    column n and one group scale.  The -8 offset term of a group, sum x (-8),
//    does not depend on the weight row: it is computed once per group on the
//    matrix cores and starts each row group's accumulation, so every row
//    group costs four MFMAs per group.
//  - Bound by the loads: on 28672 x 8192 removing the decode or the MFMAs
//    changed nothing, removing the x loads saved 6 us at M = 3 and 15 us at
//    M = 16.
//  - Workgroups of 4 row groups (64 rows), or 7 (112 rows) from M = 8 when
//    N covers a workgroup per compute unit: the time follows the busiest
//    compute unit, and on 28672 x 8192 the 448 workgroups of 64 rows put
//    two on 192 CUs and one on the other 64, while 112 rows make exactly
//    one per CU.  Interleaved runs (us, 64 / 112 rows): M = 3 43.6 / 45.3,
//    M = 6 45.3 / 46.0, M = 8 47.0 / 46.2, M = 12 49.7 / 47.1, M = 16
//    53.0 / 48.3 (identical outputs).
namespace {
constexpr int kI4Waves = 8;
}  // namespace

template <int kI4Groups, int kI4Waves>
__global__ __launch_bounds__(64 * kI4Waves) void int4g_gemm_decode_kernel(const uint16_t* __restrict__ x,
                                                                         const uint8_t* __restrict__ q,
                                                                         const uint16_t* __restrict__ s,
                                                                         uint16_t* __restrict__ out, int M, int N,
                                                                         int K) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 16 * kI4Groups;
  const int i = lane & 15, g = lane >> 4;
  const uint32_t ng = (uint32_t)K / 128;
  const uint32_t row_bytes = (uint32_t)K / 2;
  const uint32_t nrows = (uint32_t)min(16 * kI4Groups, N - n0);
  const auto qr = buffer_of(q + (int64_t)n0 * row_bytes, nrows * row_bytes);
  const auto sr = buffer_of(s + (int64_t)n0 * ng, nrows * ng * 2u);
  const auto xr = buffer_of(x, (uint32_t)M * (uint32_t)K * 2u);
  const short8v c8 = {kMinus8Bf16, kMinus8Bf16, kMinus8Bf16, kMinus8Bf16,
                      kMinus8Bf16, kMinus8Bf16, kMinus8Bf16, kMinus8Bf16};
  const uint32_t nsteps = (ng + 1) / 2;

  float4v acc[kI4Groups];
#pragma unroll
  for (int rg = 0; rg < kI4Groups; ++rg) acc[rg] = float4v{0.f, 0.f, 0.f, 0.f};
  for (uint32_t t = wave; t < nsteps; t += kI4Waves) {
    uint4 wq[kI4Groups][2], xv[2][4];
    uint32_t sb[kI4Groups][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t grp = 2 * t + h;
      const bool in = grp < ng;
#pragma unroll
      for (int rg = 0; rg < kI4Groups; ++rg) {
        const uint32_t row = 16u * rg + i;
        wq[rg][h] = buffer_load16(qr, in ? row * row_bytes + 64u * grp + 16u * g : kBufferOob);
        sb[rg][h] = buffer_load2(sr, in ? (row * ng + grp) * 2u : kBufferOob);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        xv[h][jj] = buffer_load16(xr, in ? ((uint32_t)i * (uint32_t)K + 128u * grp + 32u * g + 8u * jj) * 2u : kBufferOob);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float4v off = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) off = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_short8(xv[h][jj]), c8, off, 0, 0, 0);
#pragma unroll
      for (int rg = 0; rg < kI4Groups; ++rg) {
        float4v tmp = off;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_short8(xv[h][jj]), int4x8_offset_bf16(word_of(wq[rg][h], jj)),
                                                        tmp, 0, 0, 0);
        acc[rg] += f16_bits_to_f32(sb[rg][h]) * tmp;
      }
    }
  }

  __shared__ float4v red[kI4Waves][kI4Groups][64];
#pragma unroll
  for (int rg = 0; rg < kI4Groups; ++rg) red[wave][rg][lane] = acc[rg];
  __syncthreads();
  for (int e = threadIdx.x; e < kI4Groups * 64; e += 64 * kI4Waves) {
    const int rg = e >> 6, ln = e & 63;
    float4v sum = red[0][rg][ln];
#pragma unroll
    for (int wv = 1; wv < kI4Waves; ++wv) sum += red[wv][rg][ln];
    // D[m][n] (16 x 16): lane n + 16 (m / 4), register m % 4.
    const int n = n0 + 16 * rg + (ln & 15);
    if (n >= N) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * (ln >> 4) + r;
      if (m < M) out[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(sum[r]);
    }
  }
}

// ---- 3 <= M <= 16: activation-stationary GEMM, weight through LDS ---------
// The decode kernel above loads the weight straight into the MFMA's operand
// layout, 16 rows x 64 bytes per instruction, and reloads its x slice for
// every 112 rows; both cost: a pure read of this layout ran at ~60% of the
// speed of contiguous rows, and the x reloads (x is four times the weight's
// bytes per K range at M = 16) were a third of its loads.  Here:
//  - Wave w of the workgroup owns the 512-value K piece p * kXsWaves + w of
//    every weight row in pass p; its slice of x (16 rows x 512 values) is
//    loaded once per pass into registers, in MFMA order, with the -8 offset
//    terms of its four groups.
//  - The weight arrives through LDS: per 16-row group the wave copies its
//    piece (16 rows x 256 bytes) with four LDS-DMA instructions, each 4 rows
//    x 256 contiguous bytes (global memory serves 4-row bands nearly as fast
//    as whole rows), and the 16 x 4 group scales with a fifth, into a
//    private ring of kXsDepth stage slots, kXsAhead stages ahead of the one
//    it multiplies, so no barrier is needed until the epilogue.  Lane 4 c + r of a code copy takes bytes [16 c, 16 c + 16) of
//    band row r, and each 1 KB copy region is padded by 64 bytes, so the
//    MFMA-order reads below hit 16 different banks.
//  - Lane (n, g) then reads row n's bytes [64 G + 16 g, +16) for group G:
//    the 32 values of MFMA steps (G, 0..3), whose K positions the x slice
//    was loaded to match.  Per group: its offset term, four MFMAs
//    (v_mfma_f32_16x16x32_bf16, x as A, the weight q + 8 as B), and one
//    multiply-add by the lane's column scale.
//  - The row groups are taken in batches of kRG; after each batch the ring
//    is drained and the waves' accumulators are added through it, in wave
//    order.
// Needs K % 512 == 0 (whole pieces; every 4-byte scale pair aligned).
namespace {
constexpr int kXsWaves = 8;
constexpr int kXsPiece = 512;                     // K values per wave per pass
constexpr int kXsPass = kXsWaves * kXsPiece;      // K values per pass
constexpr int kXsDepth = 4;                       // stage slots per wave (one LDS object each)
// Stages copied ahead.  Fewer copies in flight wait less: with the whole
// chip's waves each keeping 3 stages in flight (~23 MB) a copy took ~7 us to
// land and 28672 x 8192 at M = 4 / 16 took 34.9 / 42.0 us; 2 ahead: 33.0 /
// 40.2 us (3 ahead: 33.7 / 41.0).
constexpr int kXsAhead = 2;
constexpr int kXsRegion = 1024 + 64;              // one code copy (4 rows x 256 B) + bank padding
constexpr int kXsScaleOff = 4 * kXsRegion;        // 16 rows x 4 fp16 scales (256 B copied)
constexpr int kXsStage = kXsScaleOff + 256;
constexpr int kXsStageLoads = 5;                  // LDS-DMA instructions per stage

}  // namespace

// The four ring slots are distinct LDS objects and every slot index below is
// a compile-time constant (row group rg uses slot rg % 4; kRG is a multiple
// of 4), so the compiler can see that the copies in flight never alias the
// slot being read and waits only where the explicit counts say.
__shared__ __attribute__((aligned(1024))) uint8_t g_xs0[kXsWaves][kXsStage];
__shared__ __attribute__((aligned(1024))) uint8_t g_xs1[kXsWaves][kXsStage];
__shared__ __attribute__((aligned(1024))) uint8_t g_xs2[kXsWaves][kXsStage];
__shared__ __attribute__((aligned(1024))) uint8_t g_xs3[kXsWaves][kXsStage];

namespace {
template <int S>
__device__ __forceinline__ uint8_t* xs_slot(int wave) {
  return S == 0 ? g_xs0[wave] : (S == 1 ? g_xs1[wave] : (S == 2 ? g_xs2[wave] : g_xs3[wave]));
}

struct XsCtx {
  const uint8_t* q;
  const uint16_t* s;
  int r0, rows, bt, npass, nstages, wave;
  uint32_t row_bytes, ng, lane_q, lane_s;
};

// Copies of stage t (pass t / kRG, row group t % kRG of batch bt) into slot
// S.  The lane parts of the offsets are fixed; the stage's rows and piece go
// into the buffer resources (uniform), whose ranges end at the workgroup's
// last row, so rows past it and stages past the batch read zeros.
template <int kRG, int S>
__device__ __forceinline__ void xs_issue(const XsCtx& c, int t_in) {
  // (opaque to the compiler: folding t's known pattern let it hoist every
  // row group's lane offsets out of the pass loop)
  const int t = __builtin_amdgcn_readfirstlane(t_in);
  const int p = t / kRG, rg = t % kRG;
  const int row0 = (c.bt * kRG + rg) * 16;
  const int pc = p * kXsWaves + c.wave;                        // piece index
  const bool valid = t < c.nstages && pc * (kXsPiece / 2) < (int)c.row_bytes;
  uint8_t* dst = xs_slot<S>(c.wave);
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int left = valid ? min(max(c.rows - row0 - 4 * qq, 0), 4) : 0;
    const auto rq = buffer_of(c.q + (int64_t)(c.r0 + row0 + 4 * qq) * c.row_bytes + pc * (kXsPiece / 2),
                              (uint32_t)left * c.row_bytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void_t)(dst + qq * kXsRegion), 16, c.lane_q, 0, 0, 0);
  }
  const int sleft = valid ? min(max(c.rows - row0, 0), 16) : 0;
  const auto rs = buffer_of(c.s + (int64_t)(c.r0 + row0) * c.ng + pc * 4,
                            sleft > 0 ? (uint32_t)(sleft - 1) * c.ng * 2u + 8u : 0u);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t)(dst + kXsScaleOff), 4, c.lane_s, 0, 0, 0);
}

// Stage t from slot S into acc: wait for its copies, read the 16 rows' bytes
// in MFMA order and their scales, copy stage t + kXsAhead into its slot
// (read by stage t + kXsAhead - kXsDepth, long done), then four groups of
// (offset term + 4 MFMAs) * scale.
template <int kRG, int S>
__device__ __forceinline__ void xs_stage(const XsCtx& c, int t, int lane, const uint4 (&xv)[4][4],
                                         const float4v (&off)[4], float4v& acc) {
  const int n16 = lane & 15, g4 = lane >> 4;
  wait_vmcnt<(kXsAhead - 1) * kXsStageLoads>();   // later stages' copies may stay in flight
  const uint8_t* src = xs_slot<S>(c.wave);
  // The four code reads (groups G at +256 G) and the scale read, written as
  // one asm block that also waits for them: the compiler's own tracking of
  // LDS copies lost track of the slot after the first read and waited for
  // every copy in flight before the others.  (The wait inside the block
  // keeps no load in flight past it.)
  const uint32_t a_w = lds_addr(src + (n16 >> 2) * kXsRegion + 16 * (4 * g4 + (n16 & 3)));
  const uint32_t a_s = lds_addr(src + kXsScaleOff + 8 * n16);
  uint4v w0, w1, w2, w3;
  uint2v sbv;
  asm volatile(
      "ds_read_b128 %0, %5\n\t"
      "ds_read_b128 %1, %5 offset:256\n\t"
      "ds_read_b128 %2, %5 offset:512\n\t"
      "ds_read_b128 %3, %5 offset:768\n\t"
      "ds_read_b64 %4, %6\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3), "=&v"(sbv)
      : "v"(a_w), "v"(a_s)
      : "memory");
  const uint4 w[4] = {make_uint4(w0[0], w0[1], w0[2], w0[3]), make_uint4(w1[0], w1[1], w1[2], w1[3]),
                      make_uint4(w2[0], w2[1], w2[2], w2[3]), make_uint4(w3[0], w3[1], w3[2], w3[3])};
  const uint2 sb = make_uint2(sbv[0], sbv[1]);
  xs_issue<kRG, (S + kXsAhead) % kXsDepth>(c, t + kXsAhead);
  const float sc[4] = {f16_bits_to_f32(sb.x & 0xFFFFu), f16_bits_to_f32(sb.x >> 16), f16_bits_to_f32(sb.y & 0xFFFFu),
                       f16_bits_to_f32(sb.y >> 16)};
#pragma unroll
  for (int G = 0; G < 4; ++G) {
    float4v tmp = off[G];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_short8(xv[G][jj]), int4x8_offset_bf16(word_of(w[G], jj)), tmp,
                                                    0, 0, 0);
    acc += sc[G] * tmp;
  }
  // keep the unrolled row groups apart (hoisting the next group's reads and
  // decoding above this one's MFMAs only raised register pressure)
  __builtin_amdgcn_sched_barrier(0);
}
}  // namespace

template <int kRG>
__global__ __launch_bounds__(64 * kXsWaves) void int4g_gemm_xs_kernel(const uint16_t* __restrict__ x,
                                                                     const uint8_t* __restrict__ q,
                                                                     const uint16_t* __restrict__ s,
                                                                     uint16_t* __restrict__ out, int M, int N,
                                                                     int K) {
  static_assert(kRG % kXsDepth == 0, "row group rg uses slot rg % kXsDepth");
  static_assert(sizeof(float4v) * kXsWaves * kRG * 64 <= sizeof(g_xs0) * kXsDepth, "the reduction reuses the ring");
  float4v(*s_red)[kRG][64] = (float4v(*)[kRG][64])&g_xs0[0][0];     // [wave][rg][lane], after the drain
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, g4 = lane >> 4;          // MFMA column (weight row) / K quarter
  const int r0 = (int)((int64_t)blockIdx.x * N / gridDim.x), r1 = (int)((int64_t)(blockIdx.x + 1) * N / gridDim.x);
  const uint32_t row_bytes = (uint32_t)K / 2, ng = (uint32_t)K / 128;
  const auto xr = buffer_of(x, (uint32_t)M * (uint32_t)K * 2u);    // rows >= M read as zero
  const int npass = (K + kXsPass - 1) / kXsPass;
  const int nbatch = (r1 - r0 + 16 * kRG - 1) / (16 * kRG);
  const short8v c8 = {kMinus8Bf16, kMinus8Bf16, kMinus8Bf16, kMinus8Bf16,
                      kMinus8Bf16, kMinus8Bf16, kMinus8Bf16, kMinus8Bf16};
  XsCtx c;
  c.q = q;
  c.s = s;
  c.r0 = r0;
  c.rows = r1 - r0;
  c.npass = npass;
  c.nstages = npass * kRG;
  c.wave = wave;
  c.row_bytes = row_bytes;
  c.ng = ng;
  // copy lane 4 c + r: band row r, bytes [16 c, +16); scale lane 2 n + h
  // (< 32): row n, groups 2 h and 2 h + 1 of the piece
  c.lane_q = ((uint32_t)lane & 3u) * row_bytes + 16u * ((uint32_t)lane >> 2);
  c.lane_s = lane < 32 ? ((uint32_t)lane >> 1) * ng * 2u + 4u * ((uint32_t)lane & 1u) : kBufferOob;

  for (int bt = 0; bt < nbatch; ++bt) {
    c.bt = bt;
    static_assert(kXsAhead == 2 && kXsAhead < kXsDepth, "the prologue copies kXsAhead stages");
    xs_issue<kRG, 0>(c, 0);
    xs_issue<kRG, 1>(c, 1);
    float4v acc[kRG];
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) acc[rg] = float4v{0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < npass; ++p) {
      // x rows m = n16 (A rows), 8 values per MFMA step (G, jj) at K offset
      // 128 G + 32 g + 8 jj of this wave's piece
      const uint32_t k0 = (uint32_t)(p * kXsWaves + wave) * kXsPiece;
      uint4 xv[4][4];
#pragma unroll
      for (int G = 0; G < 4; ++G)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const uint32_t k = k0 + 128u * G + 32u * g4 + 8u * jj;
          xv[G][jj] = buffer_load16(xr, k < (uint32_t)K ? ((uint32_t)n16 * (uint32_t)K + k) * 2u : kBufferOob);
        }
      float4v off[4];
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        off[G] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          off[G] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_short8(xv[G][jj]), c8, off[G], 0, 0, 0);
      }
      const int t0 = p * kRG;
#pragma unroll
      for (int rg = 0; rg < kRG; rg += 4) {
        xs_stage<kRG, 0>(c, t0 + rg, lane, xv, off, acc[rg]);
        xs_stage<kRG, 1>(c, t0 + rg + 1, lane, xv, off, acc[rg + 1]);
        xs_stage<kRG, 2>(c, t0 + rg + 2, lane, xv, off, acc[rg + 2]);
        xs_stage<kRG, 3>(c, t0 + rg + 3, lane, xv, off, acc[rg + 3]);
      }
    }
    // drain the copies past the batch, then add the waves' partial sums in
    // wave order; D[m][n]: lane n + 16 (m / 4), register m % 4
    wait_vmcnt<0>();
    barrier_nofence();
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) s_red[wave][rg][lane] = acc[rg];
    wait_lgkm0();
    barrier_nofence();
    for (int e = threadIdx.x; e < kRG * 64; e += 64 * kXsWaves) {
      const int rg = e >> 6, ln = e & 63;
      float4v sum = s_red[0][rg][ln];
#pragma unroll
      for (int wv = 1; wv < kXsWaves; ++wv) sum += s_red[wv][rg][ln];
      const int row = (bt * kRG + rg) * 16 + (ln & 15);
      if (row >= r1 - r0) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * (ln >> 4) + r;
        if (m < M) out[(int64_t)m * N + r0 + row] = (uint16_t)f32_to_bf16_rne(sum[r]);
      }
    }
    wait_lgkm0();
    barrier_nofence();                // the ring is refilled by the next batch
  }
}

// ---- M <= 2: row-slot GEMV (the weight read in storage order) --------------
// As in the NVFP4 row-slot kernel: a weight row is cut into 1 KB slots (16
// groups of 128 values) and wave s of a workgroup owns slot s of the
// workgroup's kR consecutive rows, so each load instruction reads 1 KB of
// contiguous memory.  Within a slot, lane i + 16 g loads the 16-byte piece
// 4 i + g: the four lanes i, i + 16, i + 32, i + 48 hold the four quarters
// of group i.  With the weight (q + 8) as the MFMA's A operand and x at the
// same positions as B, D[i][i] = sum over group i of x (q + 8); the
// accumulator starts from D[i][i] = -8 sum over group i of x, computed once
// per wave, which removes the offset.  The diagonal lane of group i then
// multiplies by the group's fp16 scale (fp32 arithmetic), and the epilogue
// sums the diagonals over groups and slots in a fixed order.
template <int kM, int kR>
__global__ __launch_bounds__(1024) void int4g_gemv_rowslot_kernel(const uint16_t* __restrict__ x,
                                                                  const uint8_t* __restrict__ q,
                                                                  const uint16_t* __restrict__ s,
                                                                  uint16_t* __restrict__ out, int M, int N, int K) {
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
  const auto xr = buffer_of(x, (uint32_t)M * K * 2);                // rows >= M read as zero

  // Piece 4 i + g of the slot: 32 values starting at k0; group 16 slot + i.
  const uint32_t piece = 1024u * slot + 16u * (4 * i + g);
  const bool in = piece < row_bytes;
  const uint32_t qoff = in ? piece : kBufferOob;
  const uint32_t k0 = 2u * piece;
  const uint32_t soff = (16u * slot + i < row_groups) ? 2u * (16u * slot + i) : kBufferOob;
  uint4 xv[kM][4];
#pragma unroll
  for (int m = 0; m < kM; ++m)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) xv[m][jj] = buffer_load16(xr, in ? 2u * (m * (uint32_t)K + k0 + 8u * jj) : kBufferOob);
  uint4 wq[kR];
  uint32_t ws[kR];
#pragma unroll
  for (int rho = 0; rho < kR; ++rho) {
    wq[rho] = buffer_load16<kCachePolicyNT>(qr, qoff + rho * row_bytes);
    ws[rho] = buffer_load2<kCachePolicyNT>(sr, soff + rho * row_groups * 2);
  }
  __builtin_amdgcn_sched_barrier(0);

  const short8v c8 = {kMinus8Bf16, kMinus8Bf16, kMinus8Bf16, kMinus8Bf16,
                      kMinus8Bf16, kMinus8Bf16, kMinus8Bf16, kMinus8Bf16};
  float4v off8[kM];                     // D[i][i] = -8 * sum of x over group i
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    off8[m] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      off8[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c8, as_short8(xv[m][jj]), off8[m], 0, 0, 0);
  }
  float4v tot[kR][kM];
#pragma unroll
  for (int rho = 0; rho < kR; ++rho) {
    const float sc = f16_bits_to_f32(ws[rho] & 0xFFFFu);
#pragma unroll
    for (int m = 0; m < kM; ++m) tot[rho][m] = off8[m];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const short8v wv = int4x8_offset_bf16(word_of(wq[rho], jj));
#pragma unroll
      for (int m = 0; m < kM; ++m)
        tot[rho][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv, as_short8(xv[m][jj]), tot[rho][m], 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < kM; ++m) tot[rho][m] *= sc;
  }

  // D[i][i] sits at lane i + 16 (i / 4), register i % 4.
  if ((i >> 2) == g) {
#pragma unroll
    for (int rho = 0; rho < kR; ++rho)
#pragma unroll
      for (int m = 0; m < kM; ++m) s_diag[((slot * kR + rho) * kM + m) * 16 + i] = tot[rho][m];
  }
  __syncthreads();
  // Item t (< 16 kR kM, in strides of the block size): output (rho, m) =
  // t / 16, diagonal entry t % 16.  The slots are summed in order, then the
  // 16 entries by a fixed butterfly within each aligned group of 16 lanes
  // (the item count is a multiple of 16 and the block size of 64, so every
  // group is whole).
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

// ---- any M: LDS-staged MFMA tiles -----------------------------------------
// Workgroup tile 128 (m) x 256 (n), K stage = one 128-value group; 8 waves of
// 128 x 32 (4 x 1 tiles of 32 x 32), two per SIMD, so that while one wave
// scales a finished group into its accumulators the other keeps the matrix
// core busy (with one 64 x 128 wave per SIMD the scaling waited for the
// group's last MFMAs and the next group's MFMAs waited for the scaling),
// and each weight fragment is decoded by one wave only (the kernel is
// bound by vector work: 64 x 64 waves, each weight fragment decoded twice,
// took 1.29 ms at M = 2048 on 28672 x 8192 against 1.10-1.14 ms).  x fragments are stored in LDS in lane
// order (one 1 KB region per MFMA step), the packed weight likewise; both
// are copied with global_load_lds (16-byte transfers, which land at
// lane * 16 in LDS) into a ring of three stage slots, two stages ahead of
// the MFMAs.  Each stage waits only for its own copies (vmcnt counts the
// next stage's as still in flight) and one barrier, which also frees the
// slot the stage after next is copied into.  The slots are distinct LDS
// objects and the stage loop is unrolled by three, so the compiler sees that
// copies in flight never alias the slot being read.  Per group: tmp tiles
// start from zero, collect 8 steps, and are added to the accumulators times
// the lane's column scale (read from global memory with the stage's copies).
//
// The same tiles serve the weight-only NVFP4 GEMM (bf16 x times the NVFP4
// weight of nvfp4_gemm) at M > 16: the codes are copied the same way, and a
// lane reads its four E4M3 block scales of the stage (the 16-value blocks of
// its 64 K positions) with the stage's copies.  Each 8-value weight piece is
// decoded exactly to bf16 (E2M1 -> fp32, times the block's fp32 scale, both
// exact, an at most 6-bit product whose low 16 bits are zero, so the bf16 is
// its high half) and goes straight into the accumulators; g_w scales the
// stored result.
namespace {
constexpr int IT_M = 128, IT_N = 256, IT_K = 128;
constexpr int kXBytes = IT_M * IT_K * 2;        // 32 KB
constexpr int kQBytes = IT_N * IT_K / 2;        // 16 KB
constexpr int kIStage = kXBytes + kQBytes;
constexpr int kIRing = 3;
constexpr int kIWaves = 8;
constexpr int kIDma = 6;                        // LDS-DMA copies per wave per stage (4 of x, 2 of codes)
// Weight kinds of the tiled kernel.
constexpr int kWInt4 = 0, kWInt4Zp = 1, kWNvfp4 = 2;
// 32 x 32 tiles per wave along m and n: 4 x 1 for the symmetric and NVFP4
// kernels (every weight fragment decoded by one wave); 2 x 2 for the
// zero-point kernel, whose extra accumulators (the group sums of x) would
// not fit beside 4 x 1 at two waves per SIMD.
template <int kKind> struct I4Shape {
  static constexpr bool kAsym = kKind == kWInt4Zp;
  static constexpr int Fi = kAsym ? 2 : 4, Fj = kAsym ? 2 : 1;
  static constexpr int RegLoads = Fj * (kAsym ? 2 : 1);   // scales (and zero points) per stage
};

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
#define INT4_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x70 | 0xF00)

// A workgroup barrier without the memory fence of __syncthreads() (which
// would drain the copies in flight).
__device__ __forceinline__ void i4_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
}  // namespace

__shared__ __attribute__((aligned(1024))) uint8_t g_i4s0[kIStage];
__shared__ __attribute__((aligned(1024))) uint8_t g_i4s1[kIStage];
__shared__ __attribute__((aligned(1024))) uint8_t g_i4s2[kIStage];

namespace {
template <int B> __device__ __forceinline__ uint8_t* i4_slot() { return B == 0 ? g_i4s0 : (B == 1 ? g_i4s1 : g_i4s2); }

struct I4Ctx {
  // Copies go through buffer resources over the tile's rows of x and of the
  // codes (with a global_load_lds in flight the compiler waits for every
  // outstanding LDS access before using any LDS read; with the buffer form
  // it keeps exact counts).
  __amdgpu_buffer_rsrc_t rx, rq;
  uint32_t ox[4];          // x copy offsets of this lane
  int lds_x[4];
  uint32_t oq[2];          // weight copy offsets
  int lds_q[2];
  // (sized for the larger wave width, 2 columns of tiles; the symmetric
  // kernel uses the first)
  const uint16_t* gsc[2];     // group-scale rows of this lane's output columns
  const uint8_t* gzp[2];      // and their zero points (zero-point kernel)
  const uint8_t* gsb[2];      // NVFP4: this lane's block scales of stage 0
  uint32_t scr[kIRing][2];    // per ring slot: group scale (raw fp16) or 4 E4M3 block scales
  uint32_t zr[kIRing][2];     // zero points per ring slot
  int wm, wn, lane;
};

// Copies of stage (group) g into slot B (kIDma instructions per wave), then
// its group scales and zero points (I4Shape::RegLoads loads into registers).
template <int B, int kKind>
__device__ __forceinline__ void i4_issue(I4Ctx& c, int g) {
  constexpr bool kAsym = I4Shape<kKind>::kAsym;
  uint8_t* base = i4_slot<B>();
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rx, (lds_void_t)(base + c.lds_x[i]), 16, c.ox[i] + 256u * g, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rq, (lds_void_t)(base + c.lds_q[i]), 16, c.oq[i] + 64u * g, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < I4Shape<kKind>::Fj; ++j) {
    if (kKind == kWNvfp4) {
      c.scr[B][j] = *(const uint32_t*)(c.gsb[j] + 8 * g);
    } else {
      c.scr[B][j] = c.gsc[j][g];
      if (kAsym) c.zr[B][j] = c.gzp[j][g];
    }
  }
}

// 8 E2M1 codes (dword w, element 2j in the low nibble of byte j) times the
// block scale s -> 8 bf16 in element order, exact: each product has at most
// 6 significant bits, so its fp32 pattern ends in 16 zero bits.
__device__ __forceinline__ uint32_t e2m1x2_scaled_bf16(float2v f, float s) {
  return __builtin_amdgcn_perm(__float_as_uint(f[1] * s), __float_as_uint(f[0] * s), 0x07060302u);
}
__device__ __forceinline__ short8v e2m1x8_scaled_bf16(uint32_t w, float s) {
  const uint32_t o0 = e2m1x2_scaled_bf16(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0), s);
  const uint32_t o1 = e2m1x2_scaled_bf16(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1), s);
  const uint32_t o2 = e2m1x2_scaled_bf16(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2), s);
  const uint32_t o3 = e2m1x2_scaled_bf16(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3), s);
  return __builtin_bit_cast(short8v, make_uint4(o0, o1, o2, o3));
}

// Group g from slot B into acc.  Symmetric: q decoded signed, acc += s16
// sum x q.  Zero point: q decoded unsigned, and the group sums of x taken on
// the matrix cores against a constant 1: acc += s16 (sum x q - z sum x).
template <int B, int kKind>
__device__ __forceinline__ void i4_compute(I4Ctx& c,
                                           float16v (&acc)[I4Shape<kKind>::Fi][I4Shape<kKind>::Fj]) {
  constexpr bool kAsym = I4Shape<kKind>::kAsym;
  constexpr int Fi = I4Shape<kKind>::Fi, Fj = I4Shape<kKind>::Fj;
  const uint8_t* base = i4_slot<B>();
  const int lane = c.lane, wm = c.wm, wn = c.wn;
  if constexpr (kKind == kWNvfp4) {
    // NVFP4 weight: step jj holds K positions 64 (lane / 32) + 8 jj .. + 8 of
    // the stage, block 4 (lane / 32) + jj / 2, whose scale is byte jj / 2.
    float sb[Fj][4];
#pragma unroll
    for (int j = 0; j < Fj; ++j) {
      const float2v lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.scr[B][j], 1.0f, false);
      const float2v hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.scr[B][j], 1.0f, true);
      sb[j][0] = lo[0], sb[j][1] = lo[1], sb[j][2] = hi[0], sb[j][3] = hi[1];
    }
    uint4 cq[Fj][2];
#pragma unroll
    for (int j = 0; j < Fj; ++j)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
        cq[j][hs] = *(const uint4*)(base + kXBytes + ((Fj * wn + j) * 2 + hs) * 1024 + lane * 16);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      short8v xa[Fi], wb[Fj];
#pragma unroll
      for (int i = 0; i < Fi; ++i)
        xa[i] = as_short8(*(const uint4*)(base + ((Fi * wm + i) * 8 + jj) * 1024 + lane * 16));
#pragma unroll
      for (int j = 0; j < Fj; ++j) wb[j] = e2m1x8_scaled_bf16(word_of(cq[j][jj >> 2], jj & 3), sb[j][jj >> 1]);
#pragma unroll
      for (int i = 0; i < Fi; ++i)
#pragma unroll
        for (int j = 0; j < Fj; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[i], wb[j], acc[i][j], 0, 0, 0);
    }
    return;
  }
  float sc[Fj], sz[Fj];
#pragma unroll
  for (int j = 0; j < Fj; ++j) {
    sc[j] = f16_bits_to_f32(c.scr[B][j]);
    sz[j] = kAsym ? sc[j] * (float)c.zr[B][j] : 0.f;
  }
  uint4 cq[Fj][2];
#pragma unroll
  for (int j = 0; j < Fj; ++j)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs)
      cq[j][hs] = *(const uint4*)(base + kXBytes + ((Fj * wn + j) * 2 + hs) * 1024 + lane * 16);
  const short8v c1 = {kOneBf16, kOneBf16, kOneBf16, kOneBf16, kOneBf16, kOneBf16, kOneBf16, kOneBf16};
  float16v tmp[Fi][Fj], xs[kAsym ? Fi : 1];
#pragma unroll
  for (int i = 0; i < Fi; ++i) {
    if (kAsym) xs[i] = float16v{};
#pragma unroll
    for (int j = 0; j < Fj; ++j) tmp[i][j] = float16v{};
  }
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    short8v xa[Fi], wb[Fj];
#pragma unroll
    for (int i = 0; i < Fi; ++i)
      xa[i] = as_short8(*(const uint4*)(base + ((Fi * wm + i) * 8 + jj) * 1024 + lane * 16));
#pragma unroll
    for (int j = 0; j < Fj; ++j)
      wb[j] = kAsym ? uint4x8_bf16(word_of(cq[j][jj >> 2], jj & 3)) : int4x8_signed_bf16(word_of(cq[j][jj >> 2], jj & 3));
#pragma unroll
    for (int i = 0; i < Fi; ++i) {
      if (kAsym) xs[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[i], c1, xs[i], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < Fj; ++j)
        tmp[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[i], wb[j], tmp[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < Fi; ++i)
#pragma unroll
    for (int j = 0; j < Fj; ++j) {
      if (kAsym)
        acc[i][j] += sc[j] * tmp[i][j] - sz[j] * xs[i];
      else
        acc[i][j] += sc[j] * tmp[i][j];
    }
}

// Stage g in slot B.  kChecked: near the end, where stage g + 1 or g + 2
// may not exist (all conditions are uniform).
template <int B, bool kChecked, int kKind>
__device__ __forceinline__ void i4_stage(I4Ctx& c, int g, int ng,
                                         float16v (&acc)[I4Shape<kKind>::Fi][I4Shape<kKind>::Fj]) {
  // Newer than stage g's copies: its own register loads and all of stage
  // g + 1's, which may stay in flight.
  constexpr int kAfter = kIDma + 2 * I4Shape<kKind>::RegLoads;
  if (!kChecked || g + 1 < ng) {
    INT4_WAIT_VMCNT(kAfter);
  } else {
    INT4_WAIT_VMCNT(0);
  }
  i4_barrier();                   // stage g landed for every wave; slot (B + 2) % 3 is free
  if (!kChecked || g + 2 < ng) i4_issue<(B + 2) % kIRing, kKind>(c, g + 2);
  i4_compute<B, kKind>(c, acc);
}
}  // namespace

// s: the fp16 group scales (INT4) or the E4M3 block scales (NVFP4); zp: the
// zero points (kWInt4Zp); w_g: the NVFP4 weight's global scale.
template <int kKind>
__global__ __launch_bounds__(64 * kIWaves, 1) void int4g_gemm_tiled_kernel(const uint16_t* __restrict__ x,
                                                                  const uint8_t* __restrict__ q,
                                                                  const void* __restrict__ s,
                                                                  const uint8_t* __restrict__ zp,
                                                                  const float* __restrict__ w_g,
                                                                  uint16_t* __restrict__ out, int M, int N, int K,
                                                                  int tiles_m, int tiles_n) {
  constexpr bool kAsym = I4Shape<kKind>::kAsym;
  constexpr int kIFi = I4Shape<kKind>::Fi, kIFj = I4Shape<kKind>::Fj;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-aware order: each XCD gets a contiguous run of tiles, n fastest.
  const int total = tiles_m * tiles_n;
  int id = blockIdx.x;
  if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
  const int tile_m = id / tiles_n, tile_n = id % tiles_n;
  const int m0 = tile_m * IT_M, n0 = tile_n * IT_N;
  const int ng = K / 128;

  I4Ctx c;
  c.lane = lane;
  c.wm = wave / (IT_N / 32 / kIFj);     // waves along n first
  c.wn = wave % (IT_N / 32 / kIFj);
  // x: 4 fragments x 8 steps; wave w copies step w of every fragment.
  // Lane l of region (f, jj): row 32f + l%32, values 64(l/32) + 8jj .. +8.
  // Offsets are relative to the tile's first row (at most 128 x 2K bytes of
  // x and 256 x K/2 of codes: the host takes this kernel only for K < 2^22).
  // Rows past M or N re-read the last row.
  const int rows_x = min(IT_M, M - m0), rows_q = min(IT_N, N - n0);
  c.rx = buffer_of(x + (int64_t)m0 * K, (uint32_t)rows_x * (uint32_t)K * 2u);
  c.rq = buffer_of(q + (int64_t)n0 * (K / 2), (uint32_t)rows_q * (uint32_t)(K / 2));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = i, jj = wave;
    const int row = min(32 * f + (lane & 31), rows_x - 1);
    c.ox[i] = 2u * ((uint32_t)row * (uint32_t)K + 64u * (lane >> 5) + 8u * jj);
    c.lds_x[i] = (f * 8 + jj) * 1024;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int qd = 2 * wave + i, f = qd >> 1, hs = qd & 1;
    const int row = min(32 * f + (lane & 31), rows_q - 1);
    c.oq[i] = (uint32_t)row * (uint32_t)(K / 2) + 32u * (lane >> 5) + 16u * hs;
    c.lds_q[i] = kXBytes + qd * 1024;
  }
#pragma unroll
  for (int j = 0; j < kIFj; ++j) {
    const int64_t col = min(n0 + 32 * kIFj * c.wn + 32 * j + (lane & 31), N - 1);
    c.gsc[j] = (const uint16_t*)s + col * ng;
    c.gzp[j] = kAsym ? zp + col * ng : nullptr;
    // NVFP4: the row's 8 scale bytes per stage, of which this lane's four
    // start at 4 (lane / 32)
    c.gsb[j] = (const uint8_t*)s + col * (K / 16) + 4 * (lane >> 5);
  }

  float16v acc[kIFi][kIFj];
#pragma unroll
  for (int i = 0; i < kIFi; ++i)
#pragma unroll
    for (int j = 0; j < kIFj; ++j) acc[i][j] = float16v{};

  // Prologue: stages 0 and 1 in flight.  With a single group slot 1 gets
  // group 0 again (never read): no branch here, so the compiler's count of
  // copies in flight is the same on every path into the stage loop (a
  // branch made it wait for all copies before each group's first stage).
  i4_issue<0, kKind>(c, 0);
  i4_issue<1, kKind>(c, ng > 1 ? 1 : 0);
  int g = 0;
  // Whole groups of three stages while every wait and copy of the group is
  // in range (the last stage issued is g + 4).
  for (; g + 5 <= ng; g += 3) {
    i4_stage<0, false, kKind>(c, g, ng, acc);
    i4_stage<1, false, kKind>(c, g + 1, ng, acc);
    i4_stage<2, false, kKind>(c, g + 2, ng, acc);
  }
  // The last (up to 5) stages; g % 3 == 0 here.
  for (; g < ng; g += 3) {
    i4_stage<0, true, kKind>(c, g, ng, acc);
    if (g + 1 < ng) i4_stage<1, true, kKind>(c, g + 1, ng, acc);
    if (g + 2 < ng) i4_stage<2, true, kKind>(c, g + 2, ng, acc);
  }
  INT4_WAIT_VMCNT(0);      // no copy may land in LDS after the workgroup ends

  // D[m][n] of each 32 x 32 tile: lane n + 32((m/4)%2), register (m%4) + 4(m/8).
  const int wm = c.wm, wn = c.wn, h = lane >> 5, r32 = lane & 31;
  const float gw = kKind == kWNvfp4 ? *w_g : 1.0f;
#pragma unroll
  for (int j = 0; j < kIFj; ++j) {
    const int n = n0 + 32 * kIFj * wn + 32 * j + r32;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < kIFi; ++i) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int m = m0 + 32 * kIFi * wm + 32 * i + 8 * (rr >> 2) + 4 * h + (rr & 3);
        if (m < M) out[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(kKind == kWNvfp4 ? acc[i][j][rr] * gw : acc[i][j][rr]);
      }
    }
  }
}

namespace {
template <int kM, int kR>
void launch_int4_rowslot(const void* x, const uint8_t* q, const void* s, void* out, int M, int N, int K,
                         hipStream_t stream) {
  const int nslots = (K / 2 + 1023) / 1024;
  const size_t lds = (size_t)nslots * kR * kM * 16 * sizeof(float4v);
  hipLaunchKernelGGL((int4g_gemv_rowslot_kernel<kM, kR>), dim3((unsigned)((N + kR - 1) / kR)), dim3(64 * nslots),
                     lds, stream, (const uint16_t*)x, q, (const uint16_t*)s, (uint16_t*)out, M, N, K);
}
}  // namespace

hipError_t launch_int4g_gemm_decode(const void* x, const uint8_t* q, const void* s, void* out, int64_t M,
                                    int64_t N, int64_t K, hipStream_t stream) {
  // Row-slot: 8 rows per workgroup at M = 1 and 2 (28672 x 8192, M = 2:
  // 30.1 us against 39.5 us with 4 rows; M = 1: 23.0 against 27.8 us).
  if (K <= 16 * 2048 && (int64_t)M * K * 2 < (1ll << 31)) {
    if (M == 1) {
      launch_int4_rowslot<1, 8>(x, q, s, out, (int)M, (int)N, (int)K, stream);
      return hipGetLastError();
    }
    if (M == 2) {
      launch_int4_rowslot<2, 8>(x, q, s, out, (int)M, (int)N, (int)K, stream);
      return hipGetLastError();
    }
  }
  if (M >= 3 && K % kXsPiece == 0 && (int64_t)M * K * 2 < (1ll << 31)) {
    const int64_t cus = device_cus();
    // 8 row groups (128 rows) per batch and, where N allows, one batch per
    // workgroup; 4 row groups when N has fewer than 128 rows per CU
    const bool big = N >= 128 * cus / 2;
    const int64_t per = big ? 128 : 64;
    const int64_t grid = (N + per - 1) / per < cus ? (N + per - 1) / per : cus;
    const dim3 g3((unsigned)grid), b3(64 * kXsWaves);
    const uint16_t* xx = (const uint16_t*)x;
    const uint16_t* ss = (const uint16_t*)s;
    uint16_t* oo = (uint16_t*)out;
    if (big)
      hipLaunchKernelGGL(int4g_gemm_xs_kernel<8>, g3, b3, 0, stream, xx, q, ss, oo, (int)M, (int)N, (int)K);
    else
      hipLaunchKernelGGL(int4g_gemm_xs_kernel<4>, g3, b3, 0, stream, xx, q, ss, oo, (int)M, (int)N, (int)K);
    return hipGetLastError();
  }
  if (M >= 8 && N >= 112ll * device_cus())
    hipLaunchKernelGGL((int4g_gemm_decode_kernel<7, kI4Waves>), dim3((unsigned)((N + 111) / 112)), dim3(64 * kI4Waves), 0,
                       stream, (const uint16_t*)x, q, (const uint16_t*)s, (uint16_t*)out, (int)M, (int)N, (int)K);
  else
    hipLaunchKernelGGL((int4g_gemm_decode_kernel<4, kI4Waves>), dim3((unsigned)((N + 63) / 64)), dim3(64 * kI4Waves), 0,
                       stream, (const uint16_t*)x, q, (const uint16_t*)s, (uint16_t*)out, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

hipError_t launch_int4g_gemm_tiled(const void* x, const uint8_t* q, const void* s, void* out, int64_t M,
                                   int64_t N, int64_t K, hipStream_t stream) {
  const int tiles_m = (int)((M + IT_M - 1) / IT_M), tiles_n = (int)((N + IT_N - 1) / IT_N);
  hipLaunchKernelGGL(int4g_gemm_tiled_kernel<kWInt4>, dim3((unsigned)(tiles_m * tiles_n)), dim3(64 * kIWaves), 0,
                     stream, (const uint16_t*)x, q, s, (const uint8_t*)nullptr, (const float*)nullptr,
                     (uint16_t*)out, (int)M, (int)N, (int)K, tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_int4g_asym_tiled(const void* x, const uint8_t* q, const void* s, const uint8_t* z, void* out,
                                   int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int tiles_m = (int)((M + IT_M - 1) / IT_M), tiles_n = (int)((N + IT_N - 1) / IT_N);
  hipLaunchKernelGGL(int4g_gemm_tiled_kernel<kWInt4Zp>, dim3((unsigned)(tiles_m * tiles_n)), dim3(64 * kIWaves), 0,
                     stream, (const uint16_t*)x, q, s, z, (const float*)nullptr, (uint16_t*)out, (int)M, (int)N,
                     (int)K, tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_nvfp4_w4a16_tiled(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out,
                                    int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int tiles_m = (int)((M + IT_M - 1) / IT_M), tiles_n = (int)((N + IT_N - 1) / IT_N);
  hipLaunchKernelGGL(int4g_gemm_tiled_kernel<kWNvfp4>, dim3((unsigned)(tiles_m * tiles_n)), dim3(64 * kIWaves), 0,
                     stream, (const uint16_t*)x, wc, (const void*)ws, (const uint8_t*)nullptr, wg, (uint16_t*)out,
                     (int)M, (int)N, (int)K, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace nvfp4k
