// NVFP4 x NVFP4 -> bf16 GEMM for decode-sized M (M <= 16).
//
// Same product as the tiled kernel (the block-scaled matmul of "NVFP4 en
// difusión ...", section 2), shaped for the bandwidth-bound case: decode
// moves the whole packed weight once per call and does 2*M flops per weight,
// so the kernels' job is to stream W at HBM speed and to keep the decoding
// (about one VALU op per weight value: the E2M1 conversion and the block
// scale multiply, two values per instruction each) from becoming the limit.
//
// Three kernels:
//  - row-slot GEMV (M <= 2): W is read in storage order, one contiguous
//    1 KB per load instruction; the MFMA reduces along each lane's own data
//    (diagonal trick below).
//  - packed row-block GEMM (3 <= M <= 8): 16 rows of W per workgroup, the
//    MFMA's columns shared by P = 16 / Mp K-chunks of Mp activation rows, so
//    the activation decode is shared and each load reads R = 16 / P rows x
//    1024 / R contiguous bytes;
//  - row-block GEMM (9 <= M <= 16): 16 rows of W per workgroup, the
//    activation rows in the MFMA's columns; each load instruction reads 64
//    bytes of 16 rows, which HBM serves less efficiently.
#include "common.h"
#include "launch.h"

namespace nvfp4k {

namespace {
constexpr int kBatch = 4;                       // row-block kernel: chunks in flight per wave
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
// Packed row-block GEMM (3 <= M <= 8).
//
// A workgroup owns 16 rows of W; its 4 waves split K.  The product runs on
// v_mfma_f32_16x16x32_f16 with W in the rows and the activation in the
// columns, but the 16 columns carry P = 16 / Mp K-chunks of Mp activation
// rows (Mp >= M): A row c R + w holds W row rg R + w (R = 16 / P, row group
// rg) at chunk c, B column c Mp + m holds activation row m at the same
// chunk, so the useful outputs are the P diagonal blocks D[c R + w][c Mp + m],
// summed at the end.  Every W value enters exactly one MFMA, as with P = 1,
// but each decoded activation fragment serves all P row groups, so the
// activation decode (at P = 1 as much VALU work as the weight decode) drops
// by P; and one load instruction covers R rows x 1024 / R contiguous bytes
// (4 rows x 256 B at P = 4) instead of 16 rows x 64 B.  (P = 16 would be the
// diagonal trick of the row-slot GEMV.)
//
// Lane (i, g) = i + 16 g handles 16-byte piece p = g + 4 (c + P t) of its
// rows in iteration t (any assignment of K positions to lanes gives the same
// dot products as long as both operands use it).  Every wave issues the same
// unconditional buffer loads (pieces past K and rows past N or M read as
// zero), kU iterations at a time, before decoding them.  (With P = 1, i.e.
// 9 <= M <= 16, this layout measured slower than the row-block kernel
// below, which is used there.)
template <int P, bool kLora, int kU>
__global__ __launch_bounds__(256) void nvfp4_gemm_rowpack_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const float* __restrict__ w_g,
    uint16_t* __restrict__ out, int M, int N, int K, const float* __restrict__ lora_t,
    const uint16_t* __restrict__ lora_up, int rank) {
  constexpr int R = 16 / P;     // W rows per row group = A rows per chunk = activation rows per chunk
  // kU: iterations in flight per wave (P W loads each)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t row_bytes = (uint32_t)K / 2, row_scales = (uint32_t)K / 16;
  const int n0 = blockIdx.x * 16;
  const uint32_t nrows = (uint32_t)min(16, N - n0);
  const auto wr = buffer_of(w_codes + (int64_t)n0 * row_bytes, nrows * row_bytes);
  const auto wsr = buffer_of(w_scales + (int64_t)n0 * row_scales, nrows * row_scales);
  const auto ar = buffer_of(a_codes, (uint32_t)M * row_bytes);      // rows >= M read as zero
  const auto asr = buffer_of(a_scales, (uint32_t)M * row_scales);
  const int i = lane & 15, g = lane >> 4, w = i % R, c = i / R;
  const uint32_t pbase = (uint32_t)(g + 4 * c);                    // piece in iteration 0
  const uint32_t niter = (row_bytes + 64u * P - 1) / (64u * P);

  float4v acc[P];
#pragma unroll
  for (int rg = 0; rg < P; ++rg) acc[rg] = float4v{0.f, 0.f, 0.f, 0.f};
  for (uint32_t t0 = wave; t0 < niter; t0 += 4 * kU) {
    uint4 wc[kU][P], xc[kU];
    uint32_t ws[kU][P], xs[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t p = pbase + 4u * P * (t0 + 4u * u);
      const bool in = 16u * p < row_bytes && t0 + 4u * u < niter;
#pragma unroll
      for (int rg = 0; rg < P; ++rg) {
        const uint32_t row = (uint32_t)(rg * R + w);
        wc[u][rg] = buffer_load16<kCachePolicyNT>(wr, in ? row * row_bytes + 16u * p : kOob);
        ws[u][rg] = buffer_load2<kCachePolicyNT>(wsr, in ? row * row_scales + 2u * p : kOob);
      }
      xc[u] = buffer_load16(ar, in ? (uint32_t)w * row_bytes + 16u * p : kOob);
      xs[u] = buffer_load2(asr, in ? (uint32_t)w * row_scales + 2u * p : kOob);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const half2v xs2 = e4m3x2_to_f16x2_div256(xs[u]);
      const half2v x0 = {xs2.x, xs2.x}, x1 = {xs2.y, xs2.y};
      half8v xv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) xv[jj] = dequant8_f16_div256(word_of(xc[u], jj), jj < 2 ? x0 : x1);
#pragma unroll
      for (int rg = 0; rg < P; ++rg) {
        const half2v ws2 = e4m3x2_to_f16x2_div256(ws[u][rg]);
        const half2v w0 = {ws2.x, ws2.x}, w1 = {ws2.y, ws2.y};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant8_f16_div256(word_of(wc[u][rg], jj), jj < 2 ? w0 : w1),
                                                           xv[jj], acc[rg], 0, 0, 0);
      }
    }
  }

  // D[ii][jj] (16 x 16) sits at lane jj + 16 (ii / 4), register ii % 4.
  // Output (W row rg R + w, activation row m) sums, over the waves in order
  // and then the chunks c, D[c R + w][c R + m].
  __shared__ float4v red[4][P][64];
#pragma unroll
  for (int rg = 0; rg < P; ++rg) red[wave][rg][lane] = acc[rg];
  __syncthreads();
  const float gg = (*a_g) * (*w_g);
  for (int t = threadIdx.x; t < 16 * R; t += blockDim.x) {
    const int nrow = t / R, mm = t % R;
    const int n = n0 + nrow;
    if (mm >= M || n >= N) continue;
    const int rg = nrow / R, wr_ = nrow % R;
    float v = 0.f;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv)
#pragma unroll
      for (int cc = 0; cc < P; ++cc) {
        const int ii = cc * R + wr_, jj = cc * R + mm;
        v += red[wv][rg][jj + 16 * (ii >> 2)][ii & 3];
      }
    v *= gg;
    if (kLora)      // low-rank branch: + sum_j T[mm][j] L_up[n][j]
      for (int q = 0; q < rank; ++q)
        v += lora_t[(int64_t)mm * rank + q] * bf16_bits_to_f32(lora_up[(int64_t)n * rank + q]);
    out[(int64_t)mm * N + n] = (uint16_t)f32_to_bf16_rne(v);
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
// Row-block GEMM (M <= 16).
//
//  - One workgroup per 16 weight rows; its 4 waves split K in 128-value
//    chunks (chunk c goes to wave c % 4) and are summed in LDS in a fixed
//    order, so results are deterministic.
//  - Per chunk a lane loads 16 bytes of codes (32 values) of one W row and
//    the 2 scale bytes of those values, and the same for one activation row;
//    each wave issues kBatch chunks' loads before decoding any of them.
//  - v_mfma_f32_16x16x32_f16 with W as the first operand: M <= 16 is padded
//    to the MFMA's 16 columns (lanes of rows >= M feed zeros); the decoded
//    fp16 operands are exact, as in the tiled kernel.
__global__ __launch_bounds__(256) void nvfp4_gemm_rowblock_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const float* __restrict__ w_g,
    uint16_t* __restrict__ out, int M, int N, int K, const float* __restrict__ lora_t,
    const uint16_t* __restrict__ lora_up, int rank) {
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

  float4v acc = {0.f, 0.f, 0.f, 0.f};
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
        if (a_on) {
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
          const half8v av = dequant8_f16(word_of(ac[u], jj), sa2);
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
  float v[4] = {s[0] * gg, s[1] * gg, s[2] * gg, s[3] * gg};
  if (lora_t != nullptr) {      // low-rank branch: + sum_j T[m][j] L_up[n][j]
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (n + q >= N) continue;
      float l = 0.f;
      for (int j = 0; j < rank; ++j) l += lora_t[(int64_t)m * rank + j] * bf16_bits_to_f32(lora_up[(int64_t)(n + q) * rank + j]);
      v[q] += l;
    }
  }
  const uint32_t b0 = f32_to_bf16_rne(v[0]), b1 = f32_to_bf16_rne(v[1]);
  const uint32_t b2 = f32_to_bf16_rne(v[2]), b3 = f32_to_bf16_rne(v[3]);
  if ((N & 3) == 0 && n + 3 < N) {
    *(uint2*)(orow + n) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
  } else {
    if (n + 0 < N) orow[n + 0] = (uint16_t)b0;
    if (n + 1 < N) orow[n + 1] = (uint16_t)b1;
    if (n + 2 < N) orow[n + 2] = (uint16_t)b2;
    if (n + 3 < N) orow[n + 3] = (uint16_t)b3;
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
  return M >= 1 && M <= 2 && K > 0 && K % 128 == 0 && K <= (int64_t)kMaxSlots * 2048;
}

hipError_t launch_nvfp4_w4a16_decode(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out,
                                     int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (M == 1) {
    launch_w4a16_rowslot<1, 8>(x, wc, ws, wg, out, (int)M, (int)N, (int)K, stream);
  } else {
    launch_w4a16_rowslot<2, 4>(x, wc, ws, wg, out, (int)M, (int)N, (int)K, stream);
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
  } else if (M <= 8) {
    // packed row-block kernel: P = 4 chunks for M <= 4 (2 iterations in
    // flight per wave), P = 2 for M <= 8 (8 in flight); the fastest settings
    // measured on the 21504 x 5376 decode weight
    const dim3 grid((unsigned)((N + 15) / 16)), block(256);
    const uint16_t* up = (const uint16_t*)lora_up;
    const int ri = (int)r;
    if (M <= 4) {
      if (lora) hipLaunchKernelGGL((nvfp4_gemm_rowpack_kernel<4, true, 2>), grid, block, 0, stream, ac, as, ag, wc, ws, wg, (uint16_t*)out, (int)M, (int)N, (int)K, lora_t, up, ri);
      else hipLaunchKernelGGL((nvfp4_gemm_rowpack_kernel<4, false, 2>), grid, block, 0, stream, ac, as, ag, wc, ws, wg, (uint16_t*)out, (int)M, (int)N, (int)K, lora_t, up, ri);
    } else {
      if (lora) hipLaunchKernelGGL((nvfp4_gemm_rowpack_kernel<2, true, 8>), grid, block, 0, stream, ac, as, ag, wc, ws, wg, (uint16_t*)out, (int)M, (int)N, (int)K, lora_t, up, ri);
      else hipLaunchKernelGGL((nvfp4_gemm_rowpack_kernel<2, false, 8>), grid, block, 0, stream, ac, as, ag, wc, ws, wg, (uint16_t*)out, (int)M, (int)N, (int)K, lora_t, up, ri);
    }
  } else {
    hipLaunchKernelGGL(nvfp4_gemm_rowblock_kernel, dim3((unsigned)((N + 15) / 16)), dim3(256), 0, stream, ac, as,
                       ag, wc, ws, wg, (uint16_t*)out, (int)M, (int)N, (int)K, lora_t, (const uint16_t*)lora_up,
                       (int)r);
  }
  return hipGetLastError();
}

hipError_t launch_nvfp4_gemm_decode(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                    const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                    int64_t K, hipStream_t stream) {
  return launch_nvfp4_gemm_decode_lora(ac, as, ag, wc, ws, wg, out, M, N, K, nullptr, nullptr, 0, stream);
}

}  // namespace nvfp4k
