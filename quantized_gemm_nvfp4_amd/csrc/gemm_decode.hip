// NVFP4 x NVFP4 -> bf16 GEMM for decode-sized M (M <= 16).
//
// Same product as the tiled kernel (the block-scaled matmul of "NVFP4 en
// difusión ...", section 2), shaped for the bandwidth-bound case: decode
// moves the whole packed weight once per call and does 2*M flops per weight,
// so the kernels' job is to stream W at HBM speed and to keep the decoding
// (about one VALU op per weight value: the E2M1 conversion and the block
// scale multiply, two values per instruction each) from becoming the limit.
//
// Two kernels:
//  - row-slot GEMV (M <= 2): W is read in storage order, one contiguous
//    1 KB per load instruction; the MFMA reduces along each lane's own data
//    (diagonal trick below).
//  - row-block GEMM (3 <= M <= 16): 48 rows of W per workgroup, the
//    activation rows in the MFMA's columns, each decoded activation fragment
//    shared by three 16-row groups; the 16 lanes of a row read whole
//    128-byte lines.
#include "common.h"
#include "launch.h"

namespace nvfp4k {

namespace {
constexpr int kMaxSlots = 16;                   // row-slot kernel: K <= 16 * 2048
constexpr uint32_t kOob = kBufferOob;

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}
}  // namespace

// ---------------------------------------------------------------------------
// Row-slot GEMV (M <= 2).
//
// A row of W is cut into 1 KB slots (2048 values); wave s of a workgroup owns
// slot s of each of the workgroup's kR consecutive rows, so every load
// instruction reads 1 KB of contiguous memory and a workgroup reads kR whole
// rows (one contiguous region).  HBM serves this pattern markedly faster than
// 16 rows x 64 bytes per instruction.
//
// The product still runs on v_mfma_f32_16x16x32_f16 although the MFMA's row
// structure does not match the load pattern: lane L = i + 16 g feeds A with
// 8 of the W values at its own slot position and B with the activation values
// at the same position, so D[i][i] = sum over g of <W(i + 16 g), x(i + 16 g)>:
// the diagonal holds the slot's dot product in 16 pieces.  Each (row,
// activation row) pair has its own accumulator and only its diagonal is read;
// the matrix cores do 16x the useful work, which at M <= 2 still leaves them
// mostly idle.
//
// All of a wave's loads (its activation slot, then its slot of each of the
// kR rows) are issued before any decoding; the activation slot is decoded
// once into registers.  Block scales are converted with the exact 2^-8 bit
// trick of e4m3x2_to_f16x2_div256 (the E2M1 conversion multiplies by 2^8).
template <int kM, int kR, bool kLora>
__global__ __launch_bounds__(1024) void nvfp4_gemv_rowslot_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const float* __restrict__ w_g,
    uint16_t* __restrict__ out, int M, int N, int K, const float* __restrict__ lora_t,
    const uint16_t* __restrict__ lora_up, int r) {
  extern __shared__ __attribute__((aligned(16))) float4v s_diag[];   // [slots][kR][kM][16]
  const int lane = threadIdx.x & 63;
  const int slot = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nslots = blockDim.x >> 6;
  const uint32_t row_bytes = (uint32_t)K / 2, row_scales = (uint32_t)K / 16;
  const int n0 = blockIdx.x * kR;
  const uint32_t nrows = (uint32_t)min(kR, N - n0);
  const auto wr = buffer_of(w_codes + (int64_t)n0 * row_bytes, nrows * row_bytes);
  const auto wsr = buffer_of(w_scales + (int64_t)n0 * row_scales, nrows * row_scales);
  const auto ar = buffer_of(a_codes, (uint32_t)M * row_bytes);      // rows >= M read as zero
  const auto asr = buffer_of(a_scales, (uint32_t)M * row_scales);

  // This lane's 32 values of a row: 16 code bytes and 2 scale bytes.
  const uint32_t off = 1024u * slot + 16u * lane;
  const bool in = off < row_bytes;
  const uint32_t coff = in ? off : kOob;
  const uint32_t soff = in ? 128u * slot + 2u * lane : kOob;
  uint4 xc[kM];
  uint32_t xs[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    xc[m] = buffer_load16(ar, coff + m * row_bytes);
    xs[m] = buffer_load2(asr, soff + m * row_scales);
  }
  uint4 wc[kR];
  uint32_t ws[kR];
#pragma unroll
  for (int rho = 0; rho < kR; ++rho) {
    wc[rho] = buffer_load16<kCachePolicyNT>(wr, coff + rho * row_bytes);
    ws[rho] = buffer_load2<kCachePolicyNT>(wsr, soff + rho * row_scales);
  }
  __builtin_amdgcn_sched_barrier(0);

  half8v xv[kM][4];
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    const half2v s = e4m3x2_to_f16x2_div256(xs[m]);
    const half2v s0 = {s.x, s.x}, s1 = {s.y, s.y};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) xv[m][jj] = dequant8_f16_div256(word_of(xc[m], jj), jj < 2 ? s0 : s1);
  }
  float4v acc[kR][kM];
#pragma unroll
  for (int rho = 0; rho < kR; ++rho) {
    const half2v s = e4m3x2_to_f16x2_div256(ws[rho]);
    const half2v s0 = {s.x, s.x}, s1 = {s.y, s.y};
#pragma unroll
    for (int m = 0; m < kM; ++m) acc[rho][m] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const half8v wv = dequant8_f16_div256(word_of(wc[rho], jj), jj < 2 ? s0 : s1);
#pragma unroll
      for (int m = 0; m < kM; ++m)
        acc[rho][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, xv[m][jj], acc[rho][m], 0, 0, 0);
    }
  }

  // D[i][i] sits at lane i + 16 (i / 4), register i % 4: those 16 lanes store
  // their whole float4 and the reduction picks component i % 4.
  const int i = lane & 15;
  if ((i >> 2) == (lane >> 4)) {
#pragma unroll
    for (int rho = 0; rho < kR; ++rho)
#pragma unroll
      for (int m = 0; m < kM; ++m) s_diag[((slot * kR + rho) * kM + m) * 16 + i] = acc[rho][m];
  }
  __syncthreads();
  const float gg = (*a_g) * (*w_g);
  // Item t (< 16 kR kM, in strides of the block size): output (rho, m) =
  // t / 16, diagonal entry t % 16.  The slots are summed in order, then the
  // 16 entries by a fixed butterfly within each aligned group of 16 lanes
  // (the item count is a multiple of 16 and the block size of 64, so every
  // group is whole).  With the low-rank branch, entry ii also carries the
  // terms j = ii, ii + 16, ... of sum_j T[m][j] L_up[n][j] (not scaled by
  // g_a g_w).
  for (int t = threadIdx.x; t < 16 * kR * kM; t += blockDim.x) {
    const int pair = t >> 4, ii = t & 15;
    float v = 0.f;
    for (int w = 0; w < nslots; ++w) v += s_diag[(w * kR * kM + pair) * 16 + ii][ii & 3];
    if (kLora) {
      v *= gg;
      const int rho = pair / kM, m = pair % kM, n = n0 + rho;
      if (m < M && n < N)
        for (int j = ii; j < r; j += 16) v += lora_t[(int64_t)m * r + j] * bf16_bits_to_f32(lora_up[(int64_t)n * r + j]);
    }
    v += __shfl_xor(v, 1, 16);
    v += __shfl_xor(v, 2, 16);
    v += __shfl_xor(v, 4, 16);
    v += __shfl_xor(v, 8, 16);
    const int rho = pair / kM, m = pair % kM;
    if (ii == 0 && m < M && n0 + rho < N) out[(int64_t)m * N + n0 + rho] = (uint16_t)f32_to_bf16_rne(kLora ? v : v * gg);
  }
}

// ---------------------------------------------------------------------------
// Weight-only row-slot GEMV (M <= 2): bf16 activation x NVFP4 weight.
//
// The weight side is the row-slot GEMV above.  The activation is bf16 and is
// not quantized; the MFMA takes fp16, so each wave converts its slot of x to
// fp16 after multiplying by a power of two 2^-k chosen from the slot's
// largest magnitude (which lands in [2^15, 2^16)): every element within 2^32
// of that maximum converts exactly (bf16's 8 significant bits fit fp16's
// normal and upper subnormal range), smaller ones are truncated to the fp16
// subnormal grid.  The slot's partial sums are multiplied back by 2^k
// (exact) before the slots are added.
template <int kM, int kR>
__global__ __launch_bounds__(1024) void nvfp4_gemv_w4a16_rowslot_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
    const float* __restrict__ w_g, uint16_t* __restrict__ out, int M, int N, int K) {
  extern __shared__ __attribute__((aligned(16))) float4v s_diag[];   // [slots][kR][kM][16]
  const int lane = threadIdx.x & 63;
  const int slot = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nslots = blockDim.x >> 6;
  const uint32_t row_bytes = (uint32_t)K / 2, row_scales = (uint32_t)K / 16;
  const int n0 = blockIdx.x * kR;
  const uint32_t nrows = (uint32_t)min(kR, N - n0);
  const auto wr = buffer_of(w_codes + (int64_t)n0 * row_bytes, nrows * row_bytes);
  const auto wsr = buffer_of(w_scales + (int64_t)n0 * row_scales, nrows * row_scales);
  const auto xr = buffer_of(x, (uint32_t)M * (uint32_t)K * 2u);   // rows >= M read as zero

  // This lane's 32 values of a row: 16 code bytes, 2 scale bytes, and the
  // 32 bf16 activation values at the same K positions (64 bytes).
  const uint32_t off = 1024u * slot + 16u * lane;
  const bool in = off < row_bytes;
  const uint32_t coff = in ? off : kOob;
  const uint32_t soff = in ? 128u * slot + 2u * lane : kOob;
  uint4 xb[kM][4];
#pragma unroll
  for (int m = 0; m < kM; ++m)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      xb[m][jj] = buffer_load16(xr, in ? 2u * ((uint32_t)m * K + 2u * off + 8u * jj) : kOob);
  uint4 wc[kR];
  uint32_t ws[kR];
#pragma unroll
  for (int rho = 0; rho < kR; ++rho) {
    wc[rho] = buffer_load16<kCachePolicyNT>(wr, coff + rho * row_bytes);
    ws[rho] = buffer_load2<kCachePolicyNT>(wsr, soff + rho * row_scales);
  }
  __builtin_amdgcn_sched_barrier(0);

  half8v xv[kM][4];
  float unscale[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    uint32_t mx = 0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      mx = max(max(max(mx, bf16x2_absmax_bits(xb[m][jj].x)), bf16x2_absmax_bits(xb[m][jj].y)),
               max(bf16x2_absmax_bits(xb[m][jj].z), bf16x2_absmax_bits(xb[m][jj].w)));
    mx = wave_max_u32(mx);
    // k = (biased exponent of the max) - 127 - 15, kept where 2^-k and 2^k
    // are normal fp32 numbers.
    const int k = min(max((int)(mx >> 7) - 142, -126), 126);
    const float pre = __uint_as_float((uint32_t)(127 - k) << 23);
    unscale[m] = __uint_as_float((uint32_t)(127 + k) << 23);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t wv[4] = {xb[m][jj].x, xb[m][jj].y, xb[m][jj].z, xb[m][jj].w};
      half8v h;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float lo = __uint_as_float(wv[t] << 16) * pre;
        const float hi = __uint_as_float(wv[t] & 0xFFFF0000u) * pre;
        const half2v p = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(lo, hi));
        h[2 * t] = p.x;
        h[2 * t + 1] = p.y;
      }
      xv[m][jj] = h;
    }
  }
  float4v acc[kR][kM];
#pragma unroll
  for (int rho = 0; rho < kR; ++rho) {
    const half2v s = e4m3x2_to_f16x2_div256(ws[rho]);
    const half2v s0 = {s.x, s.x}, s1 = {s.y, s.y};
#pragma unroll
    for (int m = 0; m < kM; ++m) acc[rho][m] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const half8v wv = dequant8_f16_div256(word_of(wc[rho], jj), jj < 2 ? s0 : s1);
#pragma unroll
      for (int m = 0; m < kM; ++m)
        acc[rho][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, xv[m][jj], acc[rho][m], 0, 0, 0);
    }
  }

  const int i = lane & 15;
  if ((i >> 2) == (lane >> 4)) {
#pragma unroll
    for (int rho = 0; rho < kR; ++rho)
#pragma unroll
      for (int m = 0; m < kM; ++m) s_diag[((slot * kR + rho) * kM + m) * 16 + i] = acc[rho][m] * unscale[m];
  }
  __syncthreads();
  const float gw = *w_g;
  for (int t = threadIdx.x; t < 16 * kR * kM; t += blockDim.x) {
    const int pair = t >> 4, ii = t & 15;
    float v = 0.f;
    for (int w = 0; w < nslots; ++w) v += s_diag[(w * kR * kM + pair) * 16 + ii][ii & 3];
    v += __shfl_xor(v, 1, 16);
    v += __shfl_xor(v, 2, 16);
    v += __shfl_xor(v, 4, 16);
    v += __shfl_xor(v, 8, 16);
    const int rho = pair / kM, m = pair % kM;
    if (ii == 0 && m < M && n0 + rho < N) out[(int64_t)m * N + n0 + rho] = (uint16_t)f32_to_bf16_rne(v * gw);
  }
}

// ---------------------------------------------------------------------------
// Row-block GEMM (3 <= M <= 16).
//
//  - A workgroup owns kRbGroups x 16 rows of W; its kRbWaves waves split K
//    in steps of 256 values (128 bytes of a row), step t going to wave
//    t % kRbWaves, and are summed in LDS in a fixed order, so results are
//    deterministic.
//  - Per step a lane (i, g) = i + 16 g loads bytes [32 g, 32 g + 32) of the
//    step from row i of each row group and from activation row i, with their
//    4 scale bytes, so the 16 lanes of a row read one whole 128-byte line
//    per load pair.  Half lines (64 bytes of 16 rows per step) measured ~35%
//    slower; so did the non-temporal cache policy on this pattern.
//  - v_mfma_f32_16x16x32_f16 with W as the first operand and the activation
//    rows as the second (columns; rows >= M read as zero); each decoded
//    activation fragment feeds kRbGroups row groups.  The decoded operands
//    are exact, as in the tiled kernel.
//  - All loads are unconditional buffer loads: rows past N or M and steps
//    past K read as zero (K % 128 == 0, so a lane's 32 bytes are all in the
//    row or all past it).
namespace {
constexpr int kRbGroups = 3;   // 48 W rows per workgroup
constexpr int kRbWaves = 8;    // waves splitting K
}  // namespace

template <bool kLora>
__global__ __launch_bounds__(64 * kRbWaves) void nvfp4_gemm_rowblock_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const float* __restrict__ w_g,
    uint16_t* __restrict__ out, int M, int N, int K, const float* __restrict__ lora_t,
    const uint16_t* __restrict__ lora_up, int rank) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t row_bytes = (uint32_t)K / 2, row_scales = (uint32_t)K / 16;
  const int n0 = blockIdx.x * 16 * kRbGroups;
  const uint32_t nrows = (uint32_t)min(16 * kRbGroups, N - n0);
  const auto wr = buffer_of(w_codes + (int64_t)n0 * row_bytes, nrows * row_bytes);
  const auto wsr = buffer_of(w_scales + (int64_t)n0 * row_scales, nrows * row_scales);
  const auto ar = buffer_of(a_codes, (uint32_t)M * row_bytes);
  const auto asr = buffer_of(a_scales, (uint32_t)M * row_scales);
  const int i = lane & 15, g = lane >> 4;
  const uint32_t nsteps = (row_bytes + 127u) / 128u;

  float4v acc[kRbGroups];
#pragma unroll
  for (int rg = 0; rg < kRbGroups; ++rg) acc[rg] = float4v{0.f, 0.f, 0.f, 0.f};
  for (uint32_t t = wave; t < nsteps; t += kRbWaves) {
    const uint32_t off = 128u * t + 32u * g;   // byte offset in a row
    const bool in = off < row_bytes;
    uint4 wc[kRbGroups][2], xc[2];
    uint32_t ws[kRbGroups], xs;
#pragma unroll
    for (int rg = 0; rg < kRbGroups; ++rg) {
      const uint32_t row = 16u * rg + i;
      wc[rg][0] = buffer_load16(wr, in ? row * row_bytes + off : kOob);
      wc[rg][1] = buffer_load16(wr, in ? row * row_bytes + off + 16u : kOob);
      ws[rg] = buffer_load4(wsr, in ? row * row_scales + off / 8u : kOob);
    }
    xc[0] = buffer_load16(ar, in ? (uint32_t)i * row_bytes + off : kOob);
    xc[1] = buffer_load16(ar, in ? (uint32_t)i * row_bytes + off + 16u : kOob);
    xs = buffer_load4(asr, in ? (uint32_t)i * row_scales + off / 8u : kOob);
    // all of the step's loads issue before any decoding (left to itself the
    // compiler interleaves them with the math and waits earlier: ~18% slower)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < 2; ++p) {   // 16-byte piece p: 32 values, scale bytes 2p and 2p + 1
      const half2v xs2 = e4m3x2_to_f16x2_div256(xs >> (16 * p));
      const half2v x0 = {xs2.x, xs2.x}, x1 = {xs2.y, xs2.y};
      half8v xv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) xv[jj] = dequant8_f16_div256(word_of(xc[p], jj), jj < 2 ? x0 : x1);
#pragma unroll
      for (int rg = 0; rg < kRbGroups; ++rg) {
        const half2v ws2 = e4m3x2_to_f16x2_div256(ws[rg] >> (16 * p));
        const half2v w0 = {ws2.x, ws2.x}, w1 = {ws2.y, ws2.y};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant8_f16_div256(word_of(wc[rg][p], jj), jj < 2 ? w0 : w1),
                                                           xv[jj], acc[rg], 0, 0, 0);
      }
    }
  }

  __shared__ float4v red[kRbWaves][kRbGroups][64];
#pragma unroll
  for (int rg = 0; rg < kRbGroups; ++rg) red[wave][rg][lane] = acc[rg];
  __syncthreads();
  const float gg = (*a_g) * (*w_g);
  // D[n][m] (16 x 16) of row group rg: lane m + 16 (n / 4), register n % 4.
  for (int e = threadIdx.x; e < kRbGroups * 64; e += 64 * kRbWaves) {
    const int rg = e >> 6, ln = e & 63;
    float4v s = red[0][rg][ln];
#pragma unroll
    for (int wv = 1; wv < kRbWaves; ++wv) s += red[wv][rg][ln];
    const int m = ln & 15, n = n0 + 16 * rg + 4 * (ln >> 4);
    if (m >= M) continue;
    float v[4] = {s[0] * gg, s[1] * gg, s[2] * gg, s[3] * gg};
    if (kLora) {    // low-rank branch: + sum_j T[m][j] L_up[n][j]
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (n + q >= N) continue;
        float l = 0.f;
        for (int j = 0; j < rank; ++j)
          l += lora_t[(int64_t)m * rank + j] * bf16_bits_to_f32(lora_up[(int64_t)(n + q) * rank + j]);
        v[q] += l;
      }
    }
    uint16_t* orow = out + (int64_t)m * N;
    const uint32_t b01 = f32x2_to_bf16x2_rne(v[0], v[1]), b23 = f32x2_to_bf16x2_rne(v[2], v[3]);
    if ((N & 3) == 0 && n + 3 < N) {
      *(uint2*)(orow + n) = make_uint2(b01, b23);
    } else {
      if (n + 0 < N) orow[n + 0] = (uint16_t)b01;
      if (n + 1 < N) orow[n + 1] = (uint16_t)(b01 >> 16);
      if (n + 2 < N) orow[n + 2] = (uint16_t)b23;
      if (n + 3 < N) orow[n + 3] = (uint16_t)(b23 >> 16);
    }
  }
}

namespace {
template <int kM, int kR, bool kLora = false>
void launch_rowslot(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc, const uint8_t* ws,
                    const float* wg, void* out, int M, int N, int K, hipStream_t stream, const float* lora_t = nullptr,
                    const void* lora_up = nullptr, int r = 0) {
  const int nslots = (K / 2 + 1023) / 1024;
  const size_t lds = (size_t)nslots * kR * kM * 16 * sizeof(float4v);
  hipLaunchKernelGGL((nvfp4_gemv_rowslot_kernel<kM, kR, kLora>), dim3((unsigned)((N + kR - 1) / kR)),
                     dim3(64 * nslots), lds, stream, ac, as, ag, wc, ws, wg, (uint16_t*)out, M, N, K, lora_t,
                     (const uint16_t*)lora_up, r);
}
template <int kM, int kR>
void launch_w4a16_rowslot(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out, int M,
                          int N, int K, hipStream_t stream) {
  const int nslots = (K / 2 + 1023) / 1024;
  const size_t lds = (size_t)nslots * kR * kM * 16 * sizeof(float4v);
  hipLaunchKernelGGL((nvfp4_gemv_w4a16_rowslot_kernel<kM, kR>), dim3((unsigned)((N + kR - 1) / kR)),
                     dim3(64 * nslots), lds, stream, (const uint16_t*)x, wc, ws, wg, (uint16_t*)out, M, N, K);
}
}  // namespace

bool nvfp4_w4a16_decode_supported(int64_t M, int64_t K) {
  return M >= 1 && M <= 16 && K > 0 && K % 128 == 0 && K <= (int64_t)kMaxSlots * 2048;
}

hipError_t launch_nvfp4_w4a16_decode(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out,
                                     int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  // 8 rows per workgroup at M = 1 and 2: at M = 2 (21504 x 5376) 8 rows took
  // 19.4 us per call against 21.5 us for 4 and 20.5 us for 6; 12 and more
  // spill registers.
  // From M = 3 the kernel runs once per pair of activation rows (and once
  // more for an odd last row): each row's arithmetic is the M <= 2 kernel's,
  // and the weight is read ceil(M / 2) times (21504 x 5376, M = 16: about
  // 8 x 19 us, against ~1 ms for the one-output-per-thread kernel).
  for (int64_t m0 = 0; m0 < M; m0 += 2) {
    const uint16_t* xm = (const uint16_t*)x + m0 * K;
    uint16_t* om = (uint16_t*)out + m0 * N;
    if (M - m0 >= 2)
      launch_w4a16_rowslot<2, 8>(xm, wc, ws, wg, om, 2, (int)N, (int)K, stream);
    else
      launch_w4a16_rowslot<1, 8>(xm, wc, ws, wg, om, 1, (int)N, (int)K, stream);
  }
  return hipGetLastError();
}

hipError_t launch_nvfp4_gemm_decode_lora(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                         const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                         int64_t K, const float* lora_t, const void* lora_up, int64_t r,
                                         hipStream_t stream) {
  const bool rowslot_k = K <= (int64_t)kMaxSlots * 2048;
  const bool lora = lora_t != nullptr;
  if (M == 1 && rowslot_k) {
    if (lora)
      launch_rowslot<1, 4, true>(ac, as, ag, wc, ws, wg, out, (int)M, (int)N, (int)K, stream, lora_t, lora_up, (int)r);
    else
      launch_rowslot<1, 4>(ac, as, ag, wc, ws, wg, out, (int)M, (int)N, (int)K, stream);
  } else if (M == 2 && rowslot_k) {
    if (lora)
      launch_rowslot<2, 4, true>(ac, as, ag, wc, ws, wg, out, (int)M, (int)N, (int)K, stream, lora_t, lora_up, (int)r);
    else
      launch_rowslot<2, 4>(ac, as, ag, wc, ws, wg, out, (int)M, (int)N, (int)K, stream);
  } else {
    const dim3 grid((unsigned)((N + 16 * kRbGroups - 1) / (16 * kRbGroups))), block(64 * kRbWaves);
    const uint16_t* up = (const uint16_t*)lora_up;
    if (lora)
      hipLaunchKernelGGL(nvfp4_gemm_rowblock_kernel<true>, grid, block, 0, stream, ac, as, ag, wc, ws, wg, (uint16_t*)out, (int)M, (int)N, (int)K, lora_t, up, (int)r);
    else
      hipLaunchKernelGGL(nvfp4_gemm_rowblock_kernel<false>, grid, block, 0, stream, ac, as, ag, wc, ws, wg, (uint16_t*)out, (int)M, (int)N, (int)K, lora_t, up, (int)r);
  }
  return hipGetLastError();
}

hipError_t launch_nvfp4_gemm_decode(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                    const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                    int64_t K, hipStream_t stream) {
  return launch_nvfp4_gemm_decode_lora(ac, as, ag, wc, ws, wg, out, M, N, K, nullptr, nullptr, 0, stream);
}

}  // namespace nvfp4k
