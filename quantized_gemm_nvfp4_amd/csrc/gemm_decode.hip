// NVFP4 x NVFP4 -> bf16 GEMM for decode-sized M (M <= 16).
//
// Same product as the tiled kernel (the block-scaled matmul of "NVFP4 en
// difusión ...", section 2), shaped for the bandwidth-bound case: decode
// moves the whole packed weight once per call and does 2*M flops per weight,
// so the kernels' job is to stream W at HBM speed and to keep the decoding
// (about one VALU op per weight value: the E2M1 conversion and the block
// scale multiply, two values per instruction each) from becoming the limit.
//
// Four kernels:
//  - streaming row GEMV (M <= 2, K <= 8192): a persistent grid in which each
//    wave reads whole rows of W, one contiguous 1 KB per load instruction,
//    with the next rows' loads in flight while it decodes; the MFMA reduces
//    along each lane's own data (diagonal trick below).  A second mode takes
//    the bf16 activation and quantizes it in the prologue (nvfp4_linear).
//  - row-slot GEMV (M <= 2, larger K, and the low-rank branch): the same
//    product, one workgroup per 4 rows.
//  - row-block GEMM (3 <= M <= 16): 48 rows of W per workgroup, the
//    activation rows in the MFMA's columns, each decoded activation fragment
//    shared by three 16-row groups; the 16 lanes of a row read whole
//    128-byte lines.
//  - weight-only GEMM (bf16 x, 3 <= M <= 16): activation-stationary, W
//    streamed through LDS by DMA, so W is read once for all M rows.
// The weight-only (bf16 x) forms of the row-slot and streaming GEMVs and a
// row-band kernel (2 <= M <= 16, K <= 6144) follow the same patterns.
#include "common.h"
#include "launch.h"
#include "quant_block.h"

namespace nvfp4k {

namespace {
typedef __attribute__((address_space(3))) void* lds_void_t;
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
// Streaming row GEMV (M <= 2, K <= kS * 2048).
//
// A persistent grid: wave gw of TW computes rows gw, gw + TW, gw + 2 TW, ...
// Each row is read whole by its wave, kS load instructions of up to 1 KB of
// contiguous codes each (slot s = bytes [1024 s, 1024 s + 1024) of the row),
// and kD rows are in flight per wave: the codes of slot s of row k + kD are
// requested as soon as slot s of row k has been decoded, so the memory
// system always holds about kD rows of every wave while the wave computes.
// Interleaving the rows over the grid keeps the chip's outstanding reads in
// one window of about kD TW consecutive rows that sweeps the weight once
// (on the 21504 x 5376 weight this pattern read as fast as flat streaming
// of the same bytes; deeper prefetch or more waves widened the window and
// read slower).
//
// The product is the row-slot kernel's diagonal MFMA: lane i + 16 g feeds A
// with 8 of its W values and B with the activation values at the same K
// positions, so D[i][i] holds 16 pieces of the row's dot product; even and
// odd K steps go to two accumulators (two independent MFMA chains), added at
// the end of the row.  The activation is decoded once per wave into
// registers (it is the same for every row).  Each finished row leaves its 16
// diagonal values in the wave's own LDS area; every kStreamBatch rows the
// wave sums them (lane = row, fixed order), scales by g_a g_w and stores.
namespace {
constexpr int kStreamBatch = 64;                // rows per wave between LDS flushes
constexpr int kStreamDepth = 2;                 // rows in flight per wave
constexpr int kStreamWaves = 4;                 // waves per workgroup
constexpr int kStreamWgsPerCu = 2;              // workgroups per compute unit
constexpr int kStreamMaxSlots = 4;              // K <= 8192
}  // namespace

// With kQ the activation arrives as bf16 x [M, K] and every workgroup
// quantizes all of it itself, the quantizer's steps in the same fp32
// arithmetic (the global amax of x by an integer max over all of x, then
// per 16-value block the absmax scale and codes), so its codes, scales and
// g equal nvfp4_quantize's and the output equals that of nvfp4_quantize
// followed by this kernel, bit for bit; workgroup 0 also stores them
// (q_codes, q_scales, q_g) when those are given.
template <int kM, int kS, bool kQ>
__global__ __launch_bounds__(64 * kStreamWaves) void nvfp4_gemv_stream_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const float* __restrict__ w_g,
    uint16_t* __restrict__ out, int M, int N, int K, const uint16_t* __restrict__ x_bf16,
    uint8_t* __restrict__ q_codes, uint8_t* __restrict__ q_scales, float* __restrict__ q_g) {
  constexpr int kD = kStreamDepth;
  __shared__ __attribute__((aligned(16))) float s_part[kStreamWaves][kStreamBatch * kM * 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * kStreamWaves + wave, TW = gridDim.x * kStreamWaves;
  const uint32_t row_bytes = (uint32_t)K / 2, row_scales = (uint32_t)K / 16;
  float* part = s_part[wave];

  // Row `row`'s codes and scales; a row past N gets an empty buffer range,
  // so its loads read zeros.  Lanes past the row's end read zeros too (their
  // offsets lie outside the row's range).
  auto row_codes = [&](int row) {
    const bool valid = row < N;
    return buffer_of(w_codes + (int64_t)(valid ? row : 0) * row_bytes, valid ? row_bytes : 0u);
  };
  auto row_scl = [&](int row) {
    const bool valid = row < N;
    return buffer_of(w_scales + (int64_t)(valid ? row : 0) * row_scales, valid ? row_scales : 0u);
  };
  // kQ: x's 16-value blocks t, t + 256, ... of thread t are requested
  // before the weight (the prologue below waits for them, and the weight
  // requests then stay in flight while it quantizes)
  constexpr int kQB = (kM * kS + 1) / 2;                   // blocks per thread
  const uint32_t x_bytes = (uint32_t)M * (uint32_t)K * 2u;   // <= 2 * 8192 * 2
  uint32_t xw[kQ ? kQB : 1][8];
  // codes path: the activation's codes and scales, likewise ahead of the weight
  uint4 xc[kQ ? 1 : kM][kQ ? 1 : kS];
  uint32_t xsc[kQ ? 1 : kM][kQ ? 1 : kS];
  if (!kQ) {
    const auto ar = buffer_of(a_codes, (uint32_t)M * row_bytes);      // rows >= M read as zero
    const auto asr = buffer_of(a_scales, (uint32_t)M * row_scales);
#pragma unroll
    for (int s = 0; s < kS; ++s)
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        const bool in = 1024u * s + 16u * lane < row_bytes;
        xc[kQ ? 0 : m][kQ ? 0 : s] = buffer_load16(ar, in ? 1024u * s + 16u * lane + m * row_bytes : kOob);
        xsc[kQ ? 0 : m][kQ ? 0 : s] = buffer_load2(asr, in ? 128u * s + 2u * lane + m * row_scales : kOob);
      }
  }
  if (kQ) {
    const auto xr = buffer_of(x_bf16, x_bytes);              // blocks past x read zero
#pragma unroll
    for (int u = 0; u < kQB; ++u) {
      const uint32_t b = threadIdx.x + 256u * u;
      const uint4 v0 = buffer_load16(xr, 32u * b), v1 = buffer_load16(xr, 32u * b + 16u);
      xw[u][0] = v0.x, xw[u][1] = v0.y, xw[u][2] = v0.z, xw[u][3] = v0.w;
      xw[u][4] = v1.x, xw[u][5] = v1.y, xw[u][6] = v1.z, xw[u][7] = v1.w;
    }
  }
  uint4 wc[kD][kS];
  uint32_t ws[kD][kS];
  // the first kD rows are requested before the activation is decoded
#pragma unroll
  for (int d = 0; d < kD; ++d) {
    const auto wr = row_codes(gw + d * TW), wsr = row_scl(gw + d * TW);
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      wc[d][s] = buffer_load16<kCachePolicyNT>(wr, 1024u * s + 16u * lane);
      ws[d][s] = buffer_load2<kCachePolicyNT>(wsr, 128u * s + 2u * lane);
    }
  }

  half8v xv[kM][kS][4];
  float gq = 0.f;
  if (kQ) {
    // The workgroup quantizes x together: thread t takes the blocks it
    // loaded above (for the amax and for the codes), the maximum meets in
    // LDS, and each thread leaves its blocks decoded (the same conversions
    // as the codes path below) in the workgroup's copy of x^.
    constexpr int kKS = kS * 2048;                         // x^ row stride
    __shared__ __attribute__((aligned(16))) _Float16 s_xhat[kQ ? kM * kKS : 8];
    __shared__ uint32_t s_mx[kStreamWaves];
    const uint32_t nblk = x_bytes / 32u;
    uint32_t mx = 0;
#pragma unroll
    for (int u = 0; u < kQB; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = max(mx, bf16x2_absmax_bits(xw[u][j]));
    mx = wave_max_u32(mx);
    if (lane == 0) s_mx[wave] = mx;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kStreamWaves; ++w) mx = max(mx, s_mx[w]);
    gq = bf16_bits_to_f32(mx) / 2688.0f;   // amax / (6 * 448)
    const float rq = scale_recip(gq);
    const bool store = blockIdx.x == 0;     // workgroup 0 also returns x's NVFP4 form
    if (store && q_g != nullptr && threadIdx.x == 0) *q_g = gq;
#pragma unroll
    for (int u = 0; u < kQB; ++u) {
      const uint32_t b = threadIdx.x + 256u * u;
      if (b < nblk) {
        uint32_t sc;
        const uint2 c = absmax_block(xw[u], gq, rq, sc);
        if (store && q_codes != nullptr) {
          *(uint2*)(q_codes + 8u * b) = c;
          q_scales[b] = (uint8_t)sc;
        }
        const half2v scl = e4m3x2_to_f16x2_div256(sc | (sc << 8));
        const uint32_t m = 16u * b / (uint32_t)K, k = 16u * b - m * (uint32_t)K;
        half8v* dst = (half8v*)(s_xhat + m * kKS + k);
        dst[0] = dequant8_f16_div256(c.x, scl);
        dst[1] = dequant8_f16_div256(c.y, scl);
      }
    }
    __syncthreads();
    // each wave's 32 values per lane and slot (zero past K, as the codes
    // path reads them)
#pragma unroll
    for (int s = 0; s < kS; ++s)
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        const bool in = 2048 * s + 32 * lane < K;
        const half8v* src = (const half8v*)(s_xhat + m * kKS + 2048 * s + 32 * lane);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) xv[m][s][jj] = in ? src[jj] : half8v{};
      }
  } else {
    // The activation's 32 values per lane and slot, decoded once.
#pragma unroll
    for (int s = 0; s < kS; ++s)
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        const half2v sc = e4m3x2_to_f16x2_div256(xsc[kQ ? 0 : m][kQ ? 0 : s]);
        const half2v s0 = {sc.x, sc.x}, s1 = {sc.y, sc.y};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          xv[m][s][jj] = dequant8_f16_div256(word_of(xc[kQ ? 0 : m][kQ ? 0 : s], jj), jj < 2 ? s0 : s1);
      }
  }

  const int i = lane & 15;
  const bool diag_lane = (i >> 2) == (lane >> 4);
  const float gg = (kQ ? gq : *a_g) * (*w_g);
  int nbat = 0;                 // rows of the current batch
  int row0 = gw;                // first row of the current batch
  auto flush = [&]() {
    // lane l < nbat: row row0 + l TW, the sum of its 16 diagonal values
    if (lane < nbat) {
      const int n = row0 + lane * TW;
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        const float4v* p = (const float4v*)(part + (lane * kM + m) * 16);
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4v t = p[q];
          v += t[0];
          v += t[1];
          v += t[2];
          v += t[3];
        }
        if (m < M) out[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(v * gg);
      }
    }
  };
  for (int row = gw; row < N; row += kD * TW) {
#pragma unroll
    for (int d = 0; d < kD; ++d) {
      const int r = row + d * TW;
      const auto wr = row_codes(r + kD * TW), wsr = row_scl(r + kD * TW);
      float4v acc[kM][2];
#pragma unroll
      for (int m = 0; m < kM; ++m) acc[m][0] = acc[m][1] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        half8v wv[4];
        const half2v sc = e4m3x2_to_f16x2_div256(ws[d][s]);
        const half2v s0 = {sc.x, sc.x}, s1 = {sc.y, sc.y};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) wv[jj] = dequant8_f16_div256(word_of(wc[d][s], jj), jj < 2 ? s0 : s1);
        // slot s of row r + kD TW into the registers just decoded
        wc[d][s] = buffer_load16<kCachePolicyNT>(wr, 1024u * s + 16u * lane);
        ws[d][s] = buffer_load2<kCachePolicyNT>(wsr, 128u * s + 2u * lane);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int m = 0; m < kM; ++m)
            acc[m][jj & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv[jj], xv[m][s][jj], acc[m][jj & 1], 0, 0, 0);
      }
      if (r < N) {
        if (diag_lane) {
#pragma unroll
          for (int m = 0; m < kM; ++m) {
            const float4v a = acc[m][0] + acc[m][1];
            const int c = i & 3;
            part[(nbat * kM + m) * 16 + i] = c == 0 ? a[0] : (c == 1 ? a[1] : (c == 2 ? a[2] : a[3]));
          }
        }
        if (++nbat == kStreamBatch) {
          flush();
          nbat = 0;
          row0 = r + TW;
        }
      }
    }
  }
  flush();
}

// ---------------------------------------------------------------------------
// Weight-only GEMM for 3 <= M <= 16 (bf16 activation x NVFP4 weight),
// activation-stationary with the weight through LDS: the structure of the
// INT4 kernel of the same name, so the weight is read once for all M rows.
//  - Each of the workgroup's nw waves owns the 512-value K piece p nw + w of
//    every weight row in pass p (nw and the pass count chosen so the pieces
//    fill the passes; the last piece of a row may be partial).  Its slice of
//    the activation (16 rows x 512 values) sits in registers for the pass in
//    MFMA order, bf16 converted to fp16 after a per-row power of two that
//    puts the row's largest magnitude in the slice in [2^15, 2^16) (exact
//    for values within 2^32 of it); the partial sums are multiplied back
//    before they are added.
//  - Per 16-row group the wave copies its piece of the codes (4 rows x 256
//    contiguous bytes per LDS-DMA) and of the scales (2 x 8 rows x 32 bytes)
//    into a private ring of four stages, each a distinct LDS object, so
//    only the explicit counts wait; the slot is read by one asm block that
//    also waits for its reads.
//  - Lane (n, g) decodes row n's bytes [64 G + 16 g, +16) (group G of the
//    piece: 32 values, two blocks) with their two scales, and v_mfma_f32_
//    16x16x32_f16 takes the activation as A (rows m) and the weight as B
//    (columns n).  The decoded weight is exact in fp16, as elsewhere.
//  - Row groups go in batches of kRG; after a batch the ring is drained and
//    the waves' sums are added through it in wave order, then scaled by g_w
//    and rounded.
namespace {
constexpr int kNxWaves = 8;
constexpr int kNxPiece = 512;                     // K values per wave per pass
constexpr int kNxDepth = 4;                       // stage slots per wave (one LDS object each)
constexpr int kNxAhead = 2;                       // stages copied ahead (as in the INT4 kernel)
constexpr int kNxRegion = 1024 + 64;              // one code copy (4 rows x 256 B) + bank padding
constexpr int kNxScaleOff = 4 * kNxRegion;        // 16 rows x 32 scale bytes
constexpr int kNxStage = kNxScaleOff + 512;
constexpr int kNxStageLoads = 6;                  // LDS-DMA instructions per stage
}  // namespace

__shared__ __attribute__((aligned(1024))) uint8_t g_nx0[kNxWaves][kNxStage];
__shared__ __attribute__((aligned(1024))) uint8_t g_nx1[kNxWaves][kNxStage];
__shared__ __attribute__((aligned(1024))) uint8_t g_nx2[kNxWaves][kNxStage];
__shared__ __attribute__((aligned(1024))) uint8_t g_nx3[kNxWaves][kNxStage];

namespace {
template <int S>
__device__ __forceinline__ uint8_t* nx_slot(int wave) {
  return S == 0 ? g_nx0[wave] : (S == 1 ? g_nx1[wave] : (S == 2 ? g_nx2[wave] : g_nx3[wave]));
}

struct NxCtx {
  const uint8_t* wc;
  const uint8_t* ws;
  int r0, rows, bt, nstages, wave, nw;
  uint32_t row_bytes, row_scales, lane_q, lane_s, lane_col, lane_scol;
};

// Copies of stage t (pass t / kRG, row group t % kRG of batch bt) into slot
// S; the stage's rows and piece go into the (uniform) buffer resources,
// whose ranges end at the workgroup's last row.
template <int kRG, int S>
__device__ __forceinline__ void nx_issue(const NxCtx& c, int t_in) {
  const int t = __builtin_amdgcn_readfirstlane(t_in);     // (keeps lane offsets from being hoisted per stage)
  const int p = t / kRG, rg = t % kRG;
  const int row0 = (c.bt * kRG + rg) * 16;
  const int pc = p * c.nw + c.wave;
  const bool valid = t < c.nstages && pc * (kNxPiece / 2) < (int)c.row_bytes;
  // the last piece of a row may be partial (K % 512 == 128, 256 or 384):
  // its lanes past the row's end read zeros instead of the next row
  const int vbytes = valid ? min((int)c.row_bytes - pc * (kNxPiece / 2), kNxPiece / 2) : 0;
  const uint32_t lq = c.lane_col < (uint32_t)vbytes ? c.lane_q : kOob;
  const uint32_t ls = c.lane_scol < (uint32_t)(vbytes / 8) ? c.lane_s : kOob;
  uint8_t* dst = nx_slot<S>(c.wave);
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int left = valid ? min(max(c.rows - row0 - 4 * qq, 0), 4) : 0;
    const auto rq = buffer_of(c.wc + (int64_t)(c.r0 + row0 + 4 * qq) * c.row_bytes + pc * (kNxPiece / 2),
                              (uint32_t)left * c.row_bytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void_t)(dst + qq * kNxRegion), 16, lq, 0, 0, 0);
  }
  // scales: two copies of 8 rows x 32 bytes (4 bytes per lane)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int sleft = valid ? min(max(c.rows - row0 - 8 * h, 0), 8) : 0;
    const auto rs = buffer_of(c.ws + (int64_t)(c.r0 + row0 + 8 * h) * c.row_scales + pc * (kNxPiece / 16),
                              sleft > 0 ? (uint32_t)(sleft - 1) * c.row_scales + 32u : 0u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t)(dst + kNxScaleOff + 256 * h), 4, ls, 0, 0, 0);
  }
}

// Stage t from slot S: wait for its copies, read and decode the 16 rows'
// piece in MFMA order, copy stage t + kNxAhead into its slot, 16 MFMAs.
template <int kRG, int S>
__device__ __forceinline__ void nx_stage(const NxCtx& c, int t, int lane, const half8v (&xv)[4][4],
                                         const float4v& unscale, float4v& acc) {
  const int n16 = lane & 15, g4 = lane >> 4;
  wait_vmcnt<(kNxAhead - 1) * kNxStageLoads>();   // later stages' copies may stay in flight
  const uint8_t* src = nx_slot<S>(c.wave);
  const uint32_t a_w = lds_addr(src + (n16 >> 2) * kNxRegion + 16 * (4 * g4 + (n16 & 3)));
  const uint32_t a_s = lds_addr(src + kNxScaleOff + 32 * n16 + 2 * g4);
  uint4v w0, w1, w2, w3;
  uint32_t s0, s1, s2, s3;
  // one asm block with its own wait (the compiler's tracking of the copies
  // would wait for every copy in flight before the second read)
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:256\n\t"
      "ds_read_b128 %2, %8 offset:512\n\t"
      "ds_read_b128 %3, %8 offset:768\n\t"
      "ds_read_u16 %4, %9\n\t"
      "ds_read_u16 %5, %9 offset:8\n\t"
      "ds_read_u16 %6, %9 offset:16\n\t"
      "ds_read_u16 %7, %9 offset:24\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3), "=&v"(s0), "=&v"(s1), "=&v"(s2), "=&v"(s3)
      : "v"(a_w), "v"(a_s)
      : "memory");
  nx_issue<kRG, (S + kNxAhead) % kNxDepth>(c, t + kNxAhead);   // read by stage t + kNxAhead - kNxDepth
  const uint4 w[4] = {make_uint4(w0[0], w0[1], w0[2], w0[3]), make_uint4(w1[0], w1[1], w1[2], w1[3]),
                      make_uint4(w2[0], w2[1], w2[2], w2[3]), make_uint4(w3[0], w3[1], w3[2], w3[3])};
  const uint32_t sb[4] = {s0, s1, s2, s3};
  float4v tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int G = 0; G < 4; ++G) {
    const half2v sc = e4m3x2_to_f16x2_div256(sb[G]);
    const half2v lo = {sc.x, sc.x}, hi = {sc.y, sc.y};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      tmp = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv[G][jj], dequant8_f16_div256(word_of(w[G], jj), jj < 2 ? lo : hi),
                                                   tmp, 0, 0, 0);
  }
  acc += tmp * unscale;
  __builtin_amdgcn_sched_barrier(0);
}
}  // namespace

template <int kRG>
__global__ __launch_bounds__(64 * kNxWaves) void nvfp4_w4a16_xs_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
    const float* __restrict__ w_g, uint16_t* __restrict__ out, int M, int N, int K) {
  static_assert(kRG % kNxDepth == 0, "row group rg uses slot rg % kNxDepth");
  static_assert(sizeof(float4v) * kNxWaves * kRG * 64 <= sizeof(g_nx0) * kNxDepth, "the reduction reuses the ring");
  float4v(*s_red)[kRG][64] = (float4v(*)[kRG][64])&g_nx0[0][0];     // [wave][rg][lane], after the drain
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, g4 = lane >> 4;
  const int r0 = (int)((int64_t)blockIdx.x * N / gridDim.x), r1 = (int)((int64_t)(blockIdx.x + 1) * N / gridDim.x);
  const uint32_t row_bytes = (uint32_t)K / 2, row_scales = (uint32_t)K / 16;
  const int nw = blockDim.x >> 6;                     // waves (<= kNxWaves), one K piece each per pass
  const int npass = (K + nw * kNxPiece - 1) / (nw * kNxPiece);
  const int nbatch = (r1 - r0 + 16 * kRG - 1) / (16 * kRG);
  NxCtx c;
  c.wc = w_codes;
  c.ws = w_scales;
  c.r0 = r0;
  c.rows = r1 - r0;
  c.nstages = npass * kRG;
  c.wave = wave;
  c.nw = nw;
  c.row_bytes = row_bytes;
  c.row_scales = row_scales;
  // code copy lane 4 c + r: band row r, bytes [16 c, +16); scale copy lane
  // 8 n + b: row n (of 8), scale bytes [4 b, +4) of the piece
  c.lane_q = ((uint32_t)lane & 3u) * row_bytes + 16u * ((uint32_t)lane >> 2);
  c.lane_s = ((uint32_t)lane >> 3) * row_scales + 4u * ((uint32_t)lane & 7u);
  c.lane_col = 16u * ((uint32_t)lane >> 2);       // the lane's byte column in a piece (codes)
  c.lane_scol = 4u * ((uint32_t)lane & 7u);       // and in the piece's scales

  for (int bt = 0; bt < nbatch; ++bt) {
    c.bt = bt;
    static_assert(kNxAhead == 2 && kNxAhead < kNxDepth, "the prologue copies kNxAhead stages");
    nx_issue<kRG, 0>(c, 0);
    nx_issue<kRG, 1>(c, 1);
    float4v acc[kRG];
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) acc[rg] = float4v{0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < npass; ++p) {
      // activation row m = n16, MFMA step (G, jj): K offset 128 G + 32 g + 8 jj of the piece
      const uint32_t k0 = (uint32_t)(p * nw + wave) * kNxPiece;
      half8v xv[4][4];
      float4v unscale = {1.f, 1.f, 1.f, 1.f};
      {
        const auto xr = buffer_of(x, (uint32_t)M * (uint32_t)K * 2u);   // rows >= M read as zero
        uint4 xb[4][4];
        uint32_t mx = 0;
#pragma unroll
        for (int G = 0; G < 4; ++G)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const uint32_t k = k0 + 128u * G + 32u * g4 + 8u * jj;
            xb[G][jj] = buffer_load16(xr, k < (uint32_t)K ? ((uint32_t)n16 * (uint32_t)K + k) * 2u : kOob);
            mx = max(max(max(mx, bf16x2_absmax_bits(xb[G][jj].x)), bf16x2_absmax_bits(xb[G][jj].y)),
                     max(bf16x2_absmax_bits(xb[G][jj].z), bf16x2_absmax_bits(xb[G][jj].w)));
          }
        // the row's maximum over its four lanes (lanes n16 + 16 g)
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));
        // k = (biased exponent of the max) - 127 - 15, kept where 2^-k and
        // 2^k are normal fp32 numbers
        const int kexp = min(max((int)(mx >> 7) - 142, -126), 126);
        const float pre = __uint_as_float((uint32_t)(127 - kexp) << 23);
        const float post = __uint_as_float((uint32_t)(127 + kexp) << 23);
#pragma unroll
        for (int G = 0; G < 4; ++G)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const uint32_t wv[4] = {xb[G][jj].x, xb[G][jj].y, xb[G][jj].z, xb[G][jj].w};
            half8v h;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const half2v pr = __builtin_bit_cast(
                  half2v, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(wv[u] << 16) * pre,
                                                     __uint_as_float(wv[u] & 0xFFFF0000u) * pre));
              h[2 * u] = pr.x;
              h[2 * u + 1] = pr.y;
            }
            xv[G][jj] = h;
          }
        // D row m = 4 (lane / 16) + r takes row m's factor
        const int src = 4 * (lane >> 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) unscale[r] = __shfl(post, src + r);
      }
      const int t0 = p * kRG;
#pragma unroll
      for (int rg = 0; rg < kRG; rg += 4) {
        nx_stage<kRG, 0>(c, t0 + rg, lane, xv, unscale, acc[rg]);
        nx_stage<kRG, 1>(c, t0 + rg + 1, lane, xv, unscale, acc[rg + 1]);
        nx_stage<kRG, 2>(c, t0 + rg + 2, lane, xv, unscale, acc[rg + 2]);
        nx_stage<kRG, 3>(c, t0 + rg + 3, lane, xv, unscale, acc[rg + 3]);
      }
    }
    // drain the copies past the batch, then add the waves' sums in wave
    // order; D[m][n]: lane n + 16 (m / 4), register m % 4
    wait_vmcnt<0>();
    barrier_nofence();
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) s_red[wave][rg][lane] = acc[rg];
    wait_lgkm0();
    barrier_nofence();
    const float gg = *w_g;
    for (int e = threadIdx.x; e < kRG * 64; e += 64 * nw) {
      const int rg = e >> 6, ln = e & 63;
      float4v sum = s_red[0][rg][ln];
      for (int wv = 1; wv < nw; ++wv) sum += s_red[wv][rg][ln];
      const int row = (bt * kRG + rg) * 16 + (ln & 15);
      if (row >= r1 - r0) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * (ln >> 4) + r;
        if (m < M) out[(int64_t)m * N + r0 + row] = (uint16_t)f32_to_bf16_rne(sum[r] * gg);
      }
    }
    wait_lgkm0();
    barrier_nofence();                // the ring is refilled by the next batch
  }
}

// ---------------------------------------------------------------------------
// Weight-only row-band GEMM for 2 <= M <= 16, K <= 6144 (bf16 activation x
// NVFP4 weight).
//
// The stationary kernel above streams the weight through LDS by DMA and, as
// it turned out, runs at the same time per workgroup whatever the grid (a
// per-CU limit); here the weight goes straight into registers in the
// row-block kernel's pattern, which reads at HBM speed:
//  - A persistent grid of one 8-wave workgroup per CU; workgroup b takes a
//    contiguous band of the weight's 16-row groups (5 or 6 on the 21504-row
//    decode weight).
//  - Wave w owns K steps [w S / 8, (w + 1) S / 8) of the S steps of 256
//    values (at most kSt).  Its slice of x (16 rows, lanes i + 16 g: values
//    [256 t + 64 g, +64) of row i) is loaded once, scaled per row by the power
//    of two that puts the row's largest magnitude in the wave's slice in
//    [2^15, 2^16) (exact for values within 2^32 of it), and kept in registers
//    as fp16, in MFMA order.
//  - Per row group the wave loads its steps of the 16 rows (lane (i, g): 32
//    bytes of row i at byte 128 t + 32 g, the 16 lanes of a row one whole
//    128-byte line, and 4 scale bytes), the next group's loads in flight
//    while it decodes; v_mfma_f32_16x16x32_f16 with the weight as A and x as
//    B, so D[n][m] sits in lane m + 16 (n / 4) and the lane's own row factor
//    undoes the scaling.
//  - The waves' sums of each group meet in LDS and are added in wave order
//    (deterministic), scaled by g_w and rounded.
namespace {
constexpr int kBandWaves = 8;
constexpr int kBandMaxGroups = 8;   // row groups per pass through the band
constexpr int kBandMaxK = 6144;     // three 256-value steps per wave
}  // namespace

template <int kSt>
__global__ __launch_bounds__(64 * kBandWaves) void nvfp4_w4a16_band_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
    const float* __restrict__ w_g, uint16_t* __restrict__ out, int M, int N, int K) {
  __shared__ float4v s_red[kBandWaves][kBandMaxGroups][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, g = lane >> 4;
  const uint32_t row_bytes = (uint32_t)K / 2, row_scales = (uint32_t)K / 16;
  const int nsteps = (K + 255) / 256;
  const int t0 = wave * nsteps / kBandWaves, t1 = (wave + 1) * nsteps / kBandWaves;   // t1 - t0 <= kSt
  const int ngroups = (N + 15) / 16;
  const int gb0 = (int)((int64_t)blockIdx.x * ngroups / gridDim.x);
  const int gb1 = (int)((int64_t)(blockIdx.x + 1) * ngroups / gridDim.x);

  // Chunk c0 of the band: up to kBandMaxGroups row groups from group c0;
  // its buffer resources end at its last row, so rows past it read zero.
  int c0 = gb0, nc = 0, r0 = 0;
  __amdgpu_buffer_rsrc_t wr, wsr;
  auto set_chunk = [&]() {
    nc = min(kBandMaxGroups, gb1 - c0);
    r0 = 16 * c0;
    const uint32_t nrows = nc > 0 ? (uint32_t)min(16 * nc, N - r0) : 0u;
    wr = buffer_of(w_codes + (int64_t)r0 * row_bytes, nrows * row_bytes);
    wsr = buffer_of(w_scales + (int64_t)r0 * row_scales, nrows * row_scales);
  };
  uint4 wc[2][kSt][2];
  uint32_t wsc[2][kSt];
  // the wave's steps of row group c of the chunk into buffer b (nothing is
  // read past the chunk's groups: those offsets lie outside the range)
  auto issue = [&](int c, int b) {
#pragma unroll
    for (int s = 0; s < kSt; ++s) {
      const uint32_t off = 128u * (uint32_t)(t0 + s) + 32u * (uint32_t)g;
      const bool in = c < nc && t0 + s < t1 && off < row_bytes;
      const uint32_t row = 16u * (uint32_t)c + (uint32_t)i;
      wc[b][s][0] = buffer_load16(wr, in ? row * row_bytes + off : kOob);
      wc[b][s][1] = buffer_load16(wr, in ? row * row_bytes + off + 16u : kOob);
      wsc[b][s] = buffer_load4(wsr, in ? row * row_scales + off / 8u : kOob);
    }
  };
  // the first group's weight is requested with the x slice, so both are in
  // flight together
  set_chunk();
  issue(0, 0);

  // x slice, scaled and converted once
  half8v xv[kSt][2][4];
  float post;
  {
    const auto xr = buffer_of(x, (uint32_t)M * (uint32_t)K * 2u);   // rows >= M read as zero
    uint4 xb[kSt][8];
    uint32_t mx = 0;
#pragma unroll
    for (int s = 0; s < kSt; ++s) {
      const uint32_t k = 256u * (uint32_t)(t0 + s) + 64u * (uint32_t)g;
      const bool in = t0 + s < t1 && k < (uint32_t)K;
#pragma unroll
      for (int u = 0; u < 8; ++u) xb[s][u] = buffer_load16(xr, in ? ((uint32_t)i * (uint32_t)K + k) * 2u + 16u * u : kOob);
    }
#pragma unroll
    for (int s = 0; s < kSt; ++s)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        mx = max(max(max(mx, bf16x2_absmax_bits(xb[s][u].x)), bf16x2_absmax_bits(xb[s][u].y)),
                 max(bf16x2_absmax_bits(xb[s][u].z), bf16x2_absmax_bits(xb[s][u].w)));
    // the row's maximum over its four lanes (i + 16 g)
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));
    const int kexp = min(max((int)(mx >> 7) - 142, -126), 126);
    const float pre = __uint_as_float((uint32_t)(127 - kexp) << 23);
    post = __uint_as_float((uint32_t)(127 + kexp) << 23);
#pragma unroll
    for (int s = 0; s < kSt; ++s)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t wv[4] = {xb[s][u].x, xb[s][u].y, xb[s][u].z, xb[s][u].w};
        half8v h;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const half2v pr = __builtin_bit_cast(
              half2v, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(wv[v] << 16) * pre,
                                                 __uint_as_float(wv[v] & 0xFFFF0000u) * pre));
          h[2 * v] = pr.x;
          h[2 * v + 1] = pr.y;
        }
        xv[s][u >> 2][u & 3] = h;
      }
  }

  const float gw = *w_g;
  while (nc > 0) {
    float4v acc[kBandMaxGroups];
#pragma unroll
    for (int c = 0; c < kBandMaxGroups; ++c) acc[c] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kBandMaxGroups; ++c) {
      if (c >= nc) break;
      const int b = c & 1;
      issue(c + 1, b ^ 1);          // past nc: reads nothing
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < kSt; ++s)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const half2v ws2 = e4m3x2_to_f16x2_div256(wsc[b][s] >> (16 * p));
          const half2v w0 = {ws2.x, ws2.x}, w1 = {ws2.y, ws2.y};
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant8_f16_div256(word_of(wc[b][s][p], jj), jj < 2 ? w0 : w1),
                                                            xv[s][p][jj], acc[c], 0, 0, 0);
        }
    }
    // D[n][m]: lane m + 16 (n / 4), register n % 4; m = i, whose factor is post
#pragma unroll
    for (int c = 0; c < kBandMaxGroups; ++c)
      if (c < nc) s_red[wave][c][lane] = acc[c] * post;
    __syncthreads();
    for (int e = threadIdx.x; e < nc * 64; e += 64 * kBandWaves) {
      const int c = e >> 6, ln = e & 63;
      float4v sum = s_red[0][c][ln];
#pragma unroll
      for (int wv = 1; wv < kBandWaves; ++wv) sum += s_red[wv][c][ln];
      const int m = ln & 15, n = r0 + 16 * c + 4 * (ln >> 4);
      if (m >= M) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) out[(int64_t)m * N + n + r] = (uint16_t)f32_to_bf16_rne(sum[r] * gw);
    }
    __syncthreads();                // s_red is reused by the next chunk
    c0 += kBandMaxGroups;
    set_chunk();
    issue(0, 0);                    // nc == 0: reads nothing
  }
}

namespace {
template <int kSt>
void launch_w4a16_band_st(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out, int M,
                          int N, int K, hipStream_t stream) {
  const int64_t cus = device_cus(), ngroups = ((int64_t)N + 15) / 16;
  const unsigned grid = (unsigned)(ngroups < cus ? ngroups : cus);
  hipLaunchKernelGGL(nvfp4_w4a16_band_kernel<kSt>, dim3(grid), dim3(64 * kBandWaves), 0, stream,
                     (const uint16_t*)x, wc, ws, wg, (uint16_t*)out, M, N, K);
}
// The row-band kernel for M <= 16, K % 128 == 0, K <= 6144 (at most three
// steps per wave: four spill registers); false if the shape is outside that
// range.
bool launch_w4a16_band(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out, int64_t M,
                       int64_t N, int64_t K, hipStream_t stream) {
  if (M < 1 || M > 16 || K % 128 != 0 || K <= 0 || K > kBandMaxK) return false;
  const int nsteps = (int)((K + 255) / 256), st = (nsteps + kBandWaves - 1) / kBandWaves;
  switch (st) {
    case 1: launch_w4a16_band_st<1>(x, wc, ws, wg, out, (int)M, (int)N, (int)K, stream); return true;
    case 2: launch_w4a16_band_st<2>(x, wc, ws, wg, out, (int)M, (int)N, (int)K, stream); return true;
    case 3: launch_w4a16_band_st<3>(x, wc, ws, wg, out, (int)M, (int)N, (int)K, stream); return true;
    default: return false;
  }
}
}  // namespace

namespace {
// The weight-only GEMM for 3 <= M <= 16; false if the shape is outside its
// range.  Waves per workgroup and passes: P = ceil(pieces / 8) passes of
// ceil(pieces / P) waves, so few pieces of the last pass are empty (the
// 5376-value rows of the decode weight: 11 pieces, 2 passes of 6).
bool launch_w4a16_xs(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out, int64_t M,
                     int64_t N, int64_t K, hipStream_t stream) {
  if (M < 3 || M > 16 || K % 128 != 0 || K <= 0 || K > (1 << 24) || M * K * 2 >= (1ll << 31)) return false;
  const int64_t pieces = (K + kNxPiece - 1) / kNxPiece;
  const int64_t passes = (pieces + kNxWaves - 1) / kNxWaves;
  const int nw = (int)((pieces + passes - 1) / passes);
  const int64_t cus = device_cus();
  // 8 row groups (128 rows) per batch and, where N allows, one batch per
  // workgroup; 4 row groups when N has fewer than 64 rows per CU
  const bool big = N >= 64 * cus;
  const int64_t per = big ? 128 : 64;
  const int64_t grid = (N + per - 1) / per < cus ? (N + per - 1) / per : cus;
  const dim3 g3((unsigned)grid), b3(64 * nw);
  const uint16_t* xx = (const uint16_t*)x;
  uint16_t* o = (uint16_t*)out;
  if (big)
    hipLaunchKernelGGL(nvfp4_w4a16_xs_kernel<8>, g3, b3, 0, stream, xx, wc, ws, wg, o, (int)M, (int)N, (int)K);
  else
    hipLaunchKernelGGL(nvfp4_w4a16_xs_kernel<4>, g3, b3, 0, stream, xx, wc, ws, wg, o, (int)M, (int)N, (int)K);
  return true;
}
}  // namespace

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
// Weight-only streaming GEMV (bf16 x, M = 1, K <= 8192; the template also
// takes M = 2 with K <= 6144, which measured no faster than the row band).
//
// The streaming GEMV's schedule (a persistent grid, whole rows per wave, the
// next kStreamDepth rows in flight) with the weight-only row-slot kernel's
// arithmetic: each wave converts x once, slot by slot, to fp16 after the
// slot's power of two (the row-slot kernel converted it once per workgroup
// of 8 rows); per row, slot s's MFMA chain is multiplied back by 2^k_s and
// the slots are added in order, and every kStreamBatch rows the wave adds
// each row's 16 diagonal entries in the row-slot kernel's pairwise order.
// Every step repeats the row-slot kernel's, in the same order, so the
// outputs are the same bit for bit.
template <int kM, int kS>
__global__ __launch_bounds__(64 * kStreamWaves) void nvfp4_w4a16_stream_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
    const float* __restrict__ w_g, uint16_t* __restrict__ out, int M, int N, int K) {
#pragma clang fp contract(off)
  constexpr int kD = kStreamDepth;
  __shared__ __attribute__((aligned(16))) float s_part[kStreamWaves][kStreamBatch * kM * 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * kStreamWaves + wave, TW = gridDim.x * kStreamWaves;
  const uint32_t row_bytes = (uint32_t)K / 2, row_scales = (uint32_t)K / 16;
  float* part = s_part[wave];
  auto row_codes = [&](int row) {
    const bool valid = row < N;
    return buffer_of(w_codes + (int64_t)(valid ? row : 0) * row_bytes, valid ? row_bytes : 0u);
  };
  auto row_scl = [&](int row) {
    const bool valid = row < N;
    return buffer_of(w_scales + (int64_t)(valid ? row : 0) * row_scales, valid ? row_scales : 0u);
  };
  // the lane's 32 values of each slot (rows >= M read as zero): x first,
  // then the first kD rows
  const auto xr = buffer_of(x, (uint32_t)M * (uint32_t)K * 2u);
  uint4 xb[kM][kS][4];
#pragma unroll
  for (int m = 0; m < kM; ++m)
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      const uint32_t off = 1024u * s + 16u * lane;
      const bool in = off < row_bytes;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        xb[m][s][jj] = buffer_load16(xr, in ? 2u * ((uint32_t)m * K + 2u * off + 8u * jj) : kOob);
    }
  uint4 wc[kD][kS];
  uint32_t ws[kD][kS];
#pragma unroll
  for (int d = 0; d < kD; ++d) {
    const auto wr = row_codes(gw + d * TW), wsr = row_scl(gw + d * TW);
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      wc[d][s] = buffer_load16<kCachePolicyNT>(wr, 1024u * s + 16u * lane);
      ws[d][s] = buffer_load2<kCachePolicyNT>(wsr, 128u * s + 2u * lane);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // slot s of x in fp16 after 2^-k_s, k_s = (biased exponent of the slot's
  // largest magnitude) - 127 - 15, kept where 2^-k and 2^k are normal
  half8v xv[kM][kS][4];
  float unscale[kM][kS];
#pragma unroll
  for (int m = 0; m < kM; ++m)
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      uint32_t mx = 0;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        mx = max(max(max(mx, bf16x2_absmax_bits(xb[m][s][jj].x)), bf16x2_absmax_bits(xb[m][s][jj].y)),
                 max(bf16x2_absmax_bits(xb[m][s][jj].z), bf16x2_absmax_bits(xb[m][s][jj].w)));
      mx = wave_max_u32(mx);
      const int k = min(max((int)(mx >> 7) - 142, -126), 126);
      const float pre = __uint_as_float((uint32_t)(127 - k) << 23);
      unscale[m][s] = __uint_as_float((uint32_t)(127 + k) << 23);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint32_t wv[4] = {xb[m][s][jj].x, xb[m][s][jj].y, xb[m][s][jj].z, xb[m][s][jj].w};
        half8v h;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float lo = __uint_as_float(wv[t] << 16) * pre;
          const float hi = __uint_as_float(wv[t] & 0xFFFF0000u) * pre;
          const half2v p = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(lo, hi));
          h[2 * t] = p.x;
          h[2 * t + 1] = p.y;
        }
        xv[m][s][jj] = h;
      }
    }

  const int i = lane & 15;
  const bool diag_lane = (i >> 2) == (lane >> 4);
  const float gwt = *w_g;
  int nbat = 0;                 // rows of the current batch
  int row0 = gw;                // first row of the current batch
  auto flush = [&]() {
    // lane l < nbat: row row0 + l TW, its 16 diagonal entries added pairwise
    if (lane < nbat) {
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        const float4v* p = (const float4v*)(part + (lane * kM + m) * 16);
        const float4v a = p[0], b = p[1], c = p[2], e = p[3];
        const float t0 = (a[0] + a[1]) + (a[2] + a[3]), t1 = (b[0] + b[1]) + (b[2] + b[3]);
        const float t2 = (c[0] + c[1]) + (c[2] + c[3]), t3 = (e[0] + e[1]) + (e[2] + e[3]);
        if (m < M) out[(int64_t)m * N + row0 + lane * TW] = (uint16_t)f32_to_bf16_rne(((t0 + t1) + (t2 + t3)) * gwt);
      }
    }
  };
  for (int row = gw; row < N; row += kD * TW) {
#pragma unroll
    for (int d = 0; d < kD; ++d) {
      const int r = row + d * TW;
      const auto wr = row_codes(r + kD * TW), wsr = row_scl(r + kD * TW);
      float4v dsum[kM];
#pragma unroll
      for (int m = 0; m < kM; ++m) dsum[m] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        half8v wv[4];
        const half2v sc = e4m3x2_to_f16x2_div256(ws[d][s]);
        const half2v s0 = {sc.x, sc.x}, s1 = {sc.y, sc.y};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) wv[jj] = dequant8_f16_div256(word_of(wc[d][s], jj), jj < 2 ? s0 : s1);
        // slot s of row r + kD TW into the registers just decoded
        wc[d][s] = buffer_load16<kCachePolicyNT>(wr, 1024u * s + 16u * lane);
        ws[d][s] = buffer_load2<kCachePolicyNT>(wsr, 128u * s + 2u * lane);
#pragma unroll
        for (int m = 0; m < kM; ++m) {
          float4v acc = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv[jj], xv[m][s][jj], acc, 0, 0, 0);
          const float4v ps = acc * unscale[m][s];
          dsum[m] = dsum[m] + ps;
        }
      }
      if (r < N) {
        if (diag_lane) {
          const int c = i & 3;
#pragma unroll
          for (int m = 0; m < kM; ++m)
            part[(nbat * kM + m) * 16 + i] =
                c == 0 ? dsum[m][0] : (c == 1 ? dsum[m][1] : (c == 2 ? dsum[m][2] : dsum[m][3]));
        }
        if (++nbat == kStreamBatch) {
          flush();
          nbat = 0;
          row0 = r + TW;
        }
      }
    }
  }
  flush();
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
constexpr int kRbPad = 16;     // bytes after each activation row in LDS (kQ)
}  // namespace

// With kQ (nvfp4_linear, 3 <= M <= 16 with at most 512 kQB blocks of x) the
// activation arrives as bf16 x [M, K] and every workgroup quantizes all of
// it into LDS first, as the streaming GEMV's prologue does: thread t loads
// blocks t + 512 u (u < kQB) into registers, the workgroup's integer max of
// the |bf16| patterns is the quantizer's global amax, and each block then
// goes through the quantizer's own per-block function (csrc/quant_block.h),
// so codes, scales and g, and with them the output, equal those of
// nvfp4_quantize followed by this kernel; workgroup 0 also stores them
// (q_codes, q_scales, q_g).  The main loop then reads the activation's
// codes and scales from LDS (rows K/2 + kRbPad and K/16 + kRbPad bytes)
// instead of from global memory.
template <bool kLora, int kQB = 0>
__global__ __launch_bounds__(64 * kRbWaves) void nvfp4_gemm_rowblock_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const float* __restrict__ w_g,
    uint16_t* __restrict__ out, int M, int N, int K, const float* __restrict__ lora_t,
    const uint16_t* __restrict__ lora_up, int rank, const uint16_t* __restrict__ x_bf16 = nullptr,
    uint8_t* __restrict__ q_codes = nullptr, uint8_t* __restrict__ q_scales = nullptr,
    float* __restrict__ q_g = nullptr) {
  constexpr bool kQ = kQB > 0;
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
  extern __shared__ __attribute__((aligned(16))) uint8_t s_xq[];   // kQ: [M][K/2 + pad] codes, [M][K/16 + pad] scales
  const uint32_t xq_row = row_bytes + kRbPad, xq_srow = row_scales + kRbPad;
  uint8_t* const s_xs = s_xq + (uint32_t)M * xq_row;
  float gq = 0.f;
  if (kQ) {
    __shared__ uint32_t s_mx[kRbWaves];
    const uint32_t nblk = (uint32_t)M * row_scales;
    const auto xr = buffer_of(x_bf16, nblk * 32u);          // blocks past x read zero
    uint32_t xw[kQ ? kQB : 1][8];
#pragma unroll
    for (int u = 0; u < kQB; ++u) {
      const uint32_t b = threadIdx.x + 64u * kRbWaves * u;
      const uint4 v0 = buffer_load16(xr, 32u * b), v1 = buffer_load16(xr, 32u * b + 16u);
      xw[u][0] = v0.x, xw[u][1] = v0.y, xw[u][2] = v0.z, xw[u][3] = v0.w;
      xw[u][4] = v1.x, xw[u][5] = v1.y, xw[u][6] = v1.z, xw[u][7] = v1.w;
    }
    uint32_t mx = 0;
#pragma unroll
    for (int u = 0; u < kQB; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = max(mx, bf16x2_absmax_bits(xw[u][j]));
    mx = wave_max_u32(mx);
    if (lane == 0) s_mx[wave] = mx;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kRbWaves; ++w) mx = max(mx, s_mx[w]);
    gq = bf16_bits_to_f32(mx) / 2688.0f;   // amax / (6 * 448)
    const float rq = scale_recip(gq);
    const bool store = blockIdx.x == 0;    // workgroup 0 also returns x's NVFP4 form
    if (store && q_g != nullptr && threadIdx.x == 0) *q_g = gq;
#pragma unroll
    for (int u = 0; u < kQB; ++u) {
      const uint32_t b = threadIdx.x + 64u * kRbWaves * u;
      if (b < nblk) {
        uint32_t sc;
        const uint2 c = absmax_block(xw[u], gq, rq, sc);
        if (store && q_codes != nullptr) {
          *(uint2*)(q_codes + 8u * b) = c;
          q_scales[b] = (uint8_t)sc;
        }
        const uint32_t m = b / row_scales, kb = b - m * row_scales;
        *(uint2*)(s_xq + m * xq_row + 8u * kb) = c;
        s_xs[m * xq_srow + kb] = (uint8_t)sc;
      }
    }
    __syncthreads();
  }

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
    if (kQ) {
      // from the workgroup's quantized copy (rows past M and steps past K: zero)
      const bool xin = in && i < M;
      const uint8_t* xrow = s_xq + (uint32_t)(xin ? i : 0) * xq_row + (xin ? off : 0u);
      xc[0] = xin ? *(const uint4*)xrow : make_uint4(0u, 0u, 0u, 0u);
      xc[1] = xin ? *(const uint4*)(xrow + 16) : make_uint4(0u, 0u, 0u, 0u);
      xs = xin ? *(const uint32_t*)(s_xs + (uint32_t)i * xq_srow + off / 8u) : 0u;
    } else {
      xc[0] = buffer_load16(ar, in ? (uint32_t)i * row_bytes + off : kOob);
      xc[1] = buffer_load16(ar, in ? (uint32_t)i * row_bytes + off + 16u : kOob);
      xs = buffer_load4(asr, in ? (uint32_t)i * row_scales + off / 8u : kOob);
    }
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
  const float gg = (kQ ? gq : *a_g) * (*w_g);
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

namespace {
// Activation operands of the streaming GEMV: NVFP4 codes, or (kQ) bf16 x
// with optional outputs for its codes, scales and g.
struct StreamX {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* g;
  const uint16_t* x;
  uint8_t* q_codes;
  uint8_t* q_scales;
  float* q_g;
};
template <int kM, int kS, bool kQ>
void launch_stream(const StreamX& a, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out, int M, int N,
                   int K, hipStream_t stream) {
  const int64_t cap = (int64_t)device_cus() * kStreamWgsPerCu;
  const int64_t need = ((int64_t)N + kStreamWaves - 1) / kStreamWaves;
  const unsigned grid = (unsigned)(need < cap ? need : cap);
  hipLaunchKernelGGL((nvfp4_gemv_stream_kernel<kM, kS, kQ>), dim3(grid), dim3(64 * kStreamWaves), 0, stream, a.codes,
                     a.scales, a.g, wc, ws, wg, (uint16_t*)out, M, N, K, a.x, a.q_codes, a.q_scales, a.q_g);
}
template <int kM, int kS>
void launch_w4a16_stream(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out, int M, int N,
                         int K, hipStream_t stream) {
  const int64_t cap = (int64_t)device_cus() * kStreamWgsPerCu;
  const int64_t need = ((int64_t)N + kStreamWaves - 1) / kStreamWaves;
  const unsigned grid = (unsigned)(need < cap ? need : cap);
  hipLaunchKernelGGL((nvfp4_w4a16_stream_kernel<kM, kS>), dim3(grid), dim3(64 * kStreamWaves), 0, stream,
                     (const uint16_t*)x, wc, ws, wg, (uint16_t*)out, M, N, K);
}
// The weight-only streaming GEMV for M = 1 and K <= 8192 (kM = 2: K <= 6144,
// since four slots of two rows need more registers than two waves per SIMD
// allow); false otherwise.
template <int kM>
bool launch_w4a16_stream_k(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out, int M,
                           int N, int K, hipStream_t stream) {
  switch ((K + 2047) / 2048) {
    case 1: launch_w4a16_stream<kM, 1>(x, wc, ws, wg, out, M, N, K, stream); return true;
    case 2: launch_w4a16_stream<kM, 2>(x, wc, ws, wg, out, M, N, K, stream); return true;
    case 3: launch_w4a16_stream<kM, 3>(x, wc, ws, wg, out, M, N, K, stream); return true;
    case 4:
      if (kM > 1) return false;
      launch_w4a16_stream<1, 4>(x, wc, ws, wg, out, M, N, K, stream);
      return true;
    default: return false;
  }
}
// Launches the streaming GEMV for M <= 2 and K <= kStreamMaxSlots * 2048;
// false if the shape is outside that range.
template <int kM, bool kQ>
bool launch_stream_k(const StreamX& a, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out, int M, int N,
                     int K, hipStream_t stream) {
  switch ((K + 2047) / 2048) {
    case 1: launch_stream<kM, 1, kQ>(a, wc, ws, wg, out, M, N, K, stream); return true;
    case 2: launch_stream<kM, 2, kQ>(a, wc, ws, wg, out, M, N, K, stream); return true;
    case 3: launch_stream<kM, 3, kQ>(a, wc, ws, wg, out, M, N, K, stream); return true;
    case 4: launch_stream<kM, 4, kQ>(a, wc, ws, wg, out, M, N, K, stream); return true;
    default: return false;
  }
}
}  // namespace

bool nvfp4_w4a16_decode_supported(int64_t M, int64_t K) {
  return M >= 1 && M <= 16 && K > 0 && K % 128 == 0 && K <= (int64_t)kMaxSlots * 2048;
}

hipError_t launch_nvfp4_w4a16_decode(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out,
                                     int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  // 2 <= M <= 16 and K <= 6144: the row-band kernel (on 21504 x 5376 it
  // took 18.3 us at M = 3 against 21.5 us for the row-slot GEMV at M = 2).
  // 3 <= M <= 16, larger K: the activation-stationary kernel.  Both read the
  // weight once for all rows.  M = 1 and the remaining M = 2: the row-slot
  // GEMV, 8 rows per workgroup (at M = 2, 8 rows took 19.4 us per call
  // against 21.5 us for 4 and 20.5 us for 6; 12 and more spill registers).
  // M = 1, K <= 8192: the streaming GEMV (at M = 2 it measured no faster
  // than the row band: 19.9-20.2 against 20.1-20.2 us, alternating runs).
  if (M == 1 && launch_w4a16_stream_k<1>(x, wc, ws, wg, out, 1, (int)N, (int)K, stream)) return hipGetLastError();
  if (M >= 2 && launch_w4a16_band(x, wc, ws, wg, out, M, N, K, stream)) return hipGetLastError();
  if (M >= 3) {
    if (!launch_w4a16_xs(x, wc, ws, wg, out, M, N, K, stream)) return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (M == 2)
    launch_w4a16_rowslot<2, 8>(x, wc, ws, wg, out, 2, (int)N, (int)K, stream);
  else
    launch_w4a16_rowslot<1, 8>(x, wc, ws, wg, out, 1, (int)N, (int)K, stream);
  return hipGetLastError();
}

hipError_t launch_nvfp4_gemm_decode_lora(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                         const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                         int64_t K, const float* lora_t, const void* lora_up, int64_t r,
                                         hipStream_t stream) {
  const bool rowslot_k = K <= (int64_t)kMaxSlots * 2048;
  const bool lora = lora_t != nullptr;
  if (M <= 2 && !lora) {
    const StreamX a = {ac, as, ag, nullptr, nullptr, nullptr, nullptr};
    const bool done = M == 1 ? launch_stream_k<1, false>(a, wc, ws, wg, out, (int)M, (int)N, (int)K, stream)
                             : launch_stream_k<2, false>(a, wc, ws, wg, out, (int)M, (int)N, (int)K, stream);
    if (done) return hipGetLastError();
  }
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

namespace {
// 3 <= M <= 16: x's blocks in registers, at most 6 per thread of the
// row-block kernel's 512 (and its codes in at most 3072 * 9 = 27 KB of LDS).
constexpr int kRbQMaxPerThread = 6;
constexpr int64_t kRbQMaxBlocks = (int64_t)kRbQMaxPerThread * 64 * kRbWaves;

template <int kQB>
void launch_rowblock_q(const uint16_t* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out, int M,
                       int N, int K, uint8_t* q_codes, uint8_t* q_scales, float* q_g, hipStream_t stream) {
  const dim3 grid((unsigned)((N + 16 * kRbGroups - 1) / (16 * kRbGroups))), block(64 * kRbWaves);
  const size_t lds = (size_t)M * ((size_t)K / 2 + kRbPad + (size_t)K / 16 + kRbPad);
  hipLaunchKernelGGL((nvfp4_gemm_rowblock_kernel<false, kQB>), grid, block, lds, stream, (const uint8_t*)nullptr,
                     (const uint8_t*)nullptr, (const float*)nullptr, wc, ws, wg, (uint16_t*)out, M, N, K,
                     (const float*)nullptr, (const uint16_t*)nullptr, 0, x, q_codes, q_scales, q_g);
}
}  // namespace

bool nvfp4_linear_fused_supported(int64_t M, int64_t K) {
  if (K <= 0 || K % 128 != 0) return false;
  if (M >= 1 && M <= 2) return K <= (int64_t)kStreamMaxSlots * 2048;
  return M >= 3 && M <= 16 && M * (K / 16) <= kRbQMaxBlocks;
}

hipError_t launch_nvfp4_linear_fused(const void* x, const uint8_t* wc, const uint8_t* ws, const float* wg, void* out,
                                     int64_t M, int64_t N, int64_t K, uint8_t* q_codes, uint8_t* q_scales,
                                     float* q_g, hipStream_t stream) {
  if (M <= 2) {
    const StreamX a = {nullptr, nullptr, nullptr, (const uint16_t*)x, q_codes, q_scales, q_g};
    const bool done = M == 1 ? launch_stream_k<1, true>(a, wc, ws, wg, out, (int)M, (int)N, (int)K, stream)
                             : launch_stream_k<2, true>(a, wc, ws, wg, out, (int)M, (int)N, (int)K, stream);
    return done ? hipGetLastError() : hipErrorInvalidValue;
  }
  const int64_t per = (M * (K / 16) + 64 * kRbWaves - 1) / (64 * kRbWaves);   // blocks per thread
  const uint16_t* xb = (const uint16_t*)x;
  if (per <= 1)
    launch_rowblock_q<1>(xb, wc, ws, wg, out, (int)M, (int)N, (int)K, q_codes, q_scales, q_g, stream);
  else if (per <= 2)
    launch_rowblock_q<2>(xb, wc, ws, wg, out, (int)M, (int)N, (int)K, q_codes, q_scales, q_g, stream);
  else if (per <= 3)
    launch_rowblock_q<3>(xb, wc, ws, wg, out, (int)M, (int)N, (int)K, q_codes, q_scales, q_g, stream);
  else if (per <= 4)
    launch_rowblock_q<4>(xb, wc, ws, wg, out, (int)M, (int)N, (int)K, q_codes, q_scales, q_g, stream);
  else if (per <= kRbQMaxPerThread)
    launch_rowblock_q<kRbQMaxPerThread>(xb, wc, ws, wg, out, (int)M, (int)N, (int)K, q_codes, q_scales, q_g, stream);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_nvfp4_gemm_decode(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                    const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                    int64_t K, hipStream_t stream) {
  return launch_nvfp4_gemm_decode_lora(ac, as, ag, wc, ws, wg, out, M, N, K, nullptr, nullptr, 0, stream);
}

}  // namespace nvfp4k
