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
//    cancel catastrophically).
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

constexpr short kMinus8Bf16 = (short)0xC100;    // -8.0 in bf16

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}
__device__ __forceinline__ short8v as_short8(const uint4& v) { return __builtin_bit_cast(short8v, v); }
}  // namespace

// ---- M <= 16: stream the weight once -------------------------------------
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
// Workgroup tile 128 (m) x 256 (n), K stage = one 128-value group; 4 waves of
// 64 x 128 (2 x 4 tiles of 32 x 32).  x fragments are stored in LDS in lane
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
namespace {
constexpr int IT_M = 128, IT_N = 256, IT_K = 128;
constexpr int kXBytes = IT_M * IT_K * 2;        // 32 KB
constexpr int kQBytes = IT_N * IT_K / 2;        // 16 KB
constexpr int kIStage = kXBytes + kQBytes;
constexpr int kIRing = 3;
constexpr int kILoads = 16;                     // vector memory instructions per wave per stage

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
  uint32_t ox[8];          // x copy offsets of this lane
  int lds_x[8];
  uint32_t oq[4];          // weight copy offsets
  int lds_q[4];
  const uint16_t* gsc[4];  // group-scale rows of this lane's 4 output columns
  uint32_t scr[kIRing][4]; // group scales per ring slot (raw fp16)
  int wm, wn, lane;
};

// Copies of stage (group) g into slot B, and its group scales: kILoads
// vector memory instructions per wave.
template <int B>
__device__ __forceinline__ void i4_issue(I4Ctx& c, int g) {
  uint8_t* base = i4_slot<B>();
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rx, (lds_void_t)(base + c.lds_x[i]), 16, c.ox[i] + 256u * g, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rq, (lds_void_t)(base + c.lds_q[i]), 16, c.oq[i] + 64u * g, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) c.scr[B][j] = c.gsc[j][g];
}

template <int B>
__device__ __forceinline__ void i4_compute(I4Ctx& c, float16v (&acc)[2][4]) {
  const uint8_t* base = i4_slot<B>();
  const int lane = c.lane, wm = c.wm, wn = c.wn;
  const short8v c8 = {kMinus8Bf16, kMinus8Bf16, kMinus8Bf16, kMinus8Bf16,
                      kMinus8Bf16, kMinus8Bf16, kMinus8Bf16, kMinus8Bf16};
  float sc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sc[j] = f16_bits_to_f32(c.scr[B][j]);
  uint4 cq[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs)
      cq[j][hs] = *(const uint4*)(base + kXBytes + ((4 * wn + j) * 2 + hs) * 1024 + lane * 16);
  float16v tmp[2][4], corr[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    corr[i] = float16v{};
#pragma unroll
    for (int j = 0; j < 4; ++j) tmp[i][j] = float16v{};
  }
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    short8v xa[2], wb[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) xa[i] = as_short8(*(const uint4*)(base + ((2 * wm + i) * 8 + jj) * 1024 + lane * 16));
#pragma unroll
    for (int j = 0; j < 4; ++j) wb[j] = int4x8_offset_bf16(word_of(cq[j][jj >> 2], jj & 3));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      corr[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[i], c8, corr[i], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        tmp[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[i], wb[j], tmp[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] += sc[j] * (tmp[i][j] + corr[i]);
}

// Stage g in slot B.  kChecked: near the end, where stage g + 1 or g + 2
// may not exist (all conditions are uniform).
template <int B, bool kChecked>
__device__ __forceinline__ void i4_stage(I4Ctx& c, int g, int ng, float16v (&acc)[2][4]) {
  if (!kChecked || g + 1 < ng) {
    INT4_WAIT_VMCNT(kILoads);     // stage g + 1's loads may stay in flight
  } else {
    INT4_WAIT_VMCNT(0);
  }
  i4_barrier();                   // stage g landed for every wave; slot (B + 2) % 3 is free
  if (!kChecked || g + 2 < ng) i4_issue<(B + 2) % kIRing>(c, g + 2);
  i4_compute<B>(c, acc);
}
}  // namespace

__global__ __launch_bounds__(256, 1) void int4g_gemm_tiled_kernel(const uint16_t* __restrict__ x,
                                                                  const uint8_t* __restrict__ q,
                                                                  const uint16_t* __restrict__ s,
                                                                  uint16_t* __restrict__ out, int M, int N, int K,
                                                                  int tiles_m, int tiles_n) {
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
  c.wm = wave >> 1;
  c.wn = wave & 1;
  // x: 4 fragments x 8 steps; wave w copies steps 2w, 2w+1 of every fragment.
  // Lane l of region (f, jj): row 32f + l%32, values 64(l/32) + 8jj .. +8.
  // Offsets are relative to the tile's first row (at most 128 x 2K bytes of
  // x and 256 x K/2 of codes: the host takes this kernel only for K < 2^22).
  // Rows past M or N re-read the last row.
  const int rows_x = min(IT_M, M - m0), rows_q = min(IT_N, N - n0);
  c.rx = buffer_of(x + (int64_t)m0 * K, (uint32_t)rows_x * (uint32_t)K * 2u);
  c.rq = buffer_of(q + (int64_t)n0 * (K / 2), (uint32_t)rows_q * (uint32_t)(K / 2));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int f = i >> 1, jj = 2 * wave + (i & 1);
    const int row = min(32 * f + (lane & 31), rows_x - 1);
    c.ox[i] = 2u * ((uint32_t)row * (uint32_t)K + 64u * (lane >> 5) + 8u * jj);
    c.lds_x[i] = (f * 8 + jj) * 1024;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qd = 4 * wave + i, f = qd >> 1, hs = qd & 1;
    const int row = min(32 * f + (lane & 31), rows_q - 1);
    c.oq[i] = (uint32_t)row * (uint32_t)(K / 2) + 32u * (lane >> 5) + 16u * hs;
    c.lds_q[i] = kXBytes + qd * 1024;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) c.gsc[j] = s + (int64_t)min(n0 + 128 * (wave & 1) + 32 * j + (lane & 31), N - 1) * ng;

  float16v acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float16v{};

  // Prologue: stages 0 and 1 in flight.  With a single group slot 1 gets
  // group 0 again (never read): no branch here, so the compiler's count of
  // copies in flight is the same on every path into the stage loop (a
  // branch made it wait for all copies before each group's first stage).
  i4_issue<0>(c, 0);
  i4_issue<1>(c, ng > 1 ? 1 : 0);
  int g = 0;
  // Whole groups of three stages while every wait and copy of the group is
  // in range (the last stage issued is g + 4).
  for (; g + 5 <= ng; g += 3) {
    i4_stage<0, false>(c, g, ng, acc);
    i4_stage<1, false>(c, g + 1, ng, acc);
    i4_stage<2, false>(c, g + 2, ng, acc);
  }
  // The last (up to 5) stages; g % 3 == 0 here.
  for (; g < ng; g += 3) {
    i4_stage<0, true>(c, g, ng, acc);
    if (g + 1 < ng) i4_stage<1, true>(c, g + 1, ng, acc);
    if (g + 2 < ng) i4_stage<2, true>(c, g + 2, ng, acc);
  }
  INT4_WAIT_VMCNT(0);      // no copy may land in LDS after the workgroup ends

  // D[m][n] of each 32 x 32 tile: lane n + 32((m/4)%2), register (m%4) + 4(m/8).
  const int wm = c.wm, wn = c.wn, h = lane >> 5, r32 = lane & 31;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 128 * wn + 32 * j + r32;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int m = m0 + 64 * wm + 32 * i + 8 * (rr >> 2) + 4 * h + (rr & 3);
        if (m < M) out[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(acc[i][j][rr]);
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
  hipLaunchKernelGGL(int4g_gemm_tiled_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, stream,
                     (const uint16_t*)x, q, (const uint16_t*)s, (uint16_t*)out, (int)M, (int)N, (int)K, tiles_m,
                     tiles_n);
  return hipGetLastError();
}

}  // namespace nvfp4k
