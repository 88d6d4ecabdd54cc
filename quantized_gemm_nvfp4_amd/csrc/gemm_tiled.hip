// NVFP4 x NVFP4 -> bf16 GEMM on the gfx950 matrix cores (large M).
//
// Computes out[m, n] = bf16_RNE(g_a * g_w * sum_k A[m, k] * W[n, k]) where
// A[m, k] = E2M1(code) * E4M3(block scale), the block-scaled product of
// "NVFP4 en difusión ...", section 2 (scale_a, scale_b, bfloat16 output).
//
// Every E2M1 x E4M3 product has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in fp16: the kernel decodes both operands to
// fp16 and runs v_mfma_f32_32x32x16_f16 with fp32 accumulation, which sees
// exactly the decoded values.  Decoding is v_cvt_scalef32_pk_f16_fp4 (two
// codes; the instruction applies only the exponent of its scale operand, so
// it is given 1.0) and one packed fp16 multiply by the block scale.
//
// Design for CDNA4:
//  - Workgroup tile 256 x 256, K stage of 64 values, 8 waves of 128 (m) x 64
//    (n); two waves share each SIMD so one wave's decoding (VALU) issues
//    while the other's MFMAs run.
//  - The packed operands (codes and scale bytes) are copied global -> LDS with
//    global_load_lds into a ring of four stage slots, three stages ahead of
//    the MFMAs.  Each code copy instruction reads 32 rows x 32 contiguous
//    bytes.  The slots are distinct LDS objects and the stage loop is
//    unrolled by four, so the compiler sees that copies in flight never alias
//    what is being read; every stage issues exactly three copies per wave and
//    one wait per stage leaves the newest stage's copies in flight.
//  - With copies in flight the compiler waits for all outstanding LDS reads
//    before consuming any, so within a step single MFMAs are interleaved with
//    the next step's LDS reads and the decoding (explicit scheduling groups):
//    the reads are issued early and have completed by the next step.
//  - A is decoded once per workgroup, one stage ahead, into a double-buffered
//    fp16 tile in LDS (32 values per thread per stage); the MFMA reads it
//    with one ds_read_b128 per fragment and step.  W stays packed in LDS and
//    each wave decodes its two W fragments in registers.  Decoding A per wave
//    instead would repeat it for all four waves that share an A fragment.
//  - The MFMA sums 16 values of K per lane-half; which physical K a lane
//    feeds does not change the sum as long as both operands use the same
//    assignment.  Lane-half h takes K [32h, 32h + 32) of the stage, 8 per
//    step, so a lane's W codes for the whole stage are one 16-byte piece.
//    In LDS the two 16-byte pieces of a row's stage segment sit at slot
//    2*row + (piece ^ ((row >> 3) & 1)): the copy writes them in order, and
//    16 readers of 16 consecutive rows hit 16 distinct bank groups.  The
//    fp16 A tile is stored in MFMA lane order (conflict-free reads).
//  - The W fragment is the MFMA's first operand, so each lane's accumulators
//    hold 4 consecutive output columns n: 8-byte bf16 stores.
//  - Workgroups are dispatched round-robin over the 8 XCDs; the tile order
//    gives each XCD a contiguous range of tiles, grouped 4 tile-rows at a
//    time, so tiles running together on one XCD share A and W in its L2.
#include "common.h"
#include "launch.h"

namespace nvfp4k {

namespace {
constexpr int TM = 256, TN = 256, TK = 64;
constexpr int kRowBytes = TK / 2;                    // 32 code bytes per row per stage
constexpr int kCodeBytes = TM * kRowBytes;           // 8 KB per operand per stage
constexpr int kScaleRow = TK / 16;                   // 4 scale bytes per row per stage
constexpr int kScaleBytes = TM * kScaleRow;          // 1 KB per operand per stage
constexpr int kAf16Bytes = TM * TK * 2;              // 32 KB decoded A per stage
constexpr int kRing = 4;                             // packed stage slots
constexpr int kCopies = 3;                           // copy instructions per wave per stage
constexpr int kGroupM = 4;

typedef __attribute__((address_space(3))) void* lds_void_t;
typedef __attribute__((address_space(1))) void* gbl_void_t;

__device__ __forceinline__ void g2lds16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((gbl_void_t)g, (lds_void_t)l, 16, 0, 0);
}
__device__ __forceinline__ void g2lds4(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((gbl_void_t)g, (lds_void_t)l, 4, 0, 0);
}


__device__ __forceinline__ void map_tile(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  int id = bid;
  if ((total & 7) == 0) id = (bid & 7) * (total >> 3) + (bid >> 3);
  const int per_group = kGroupM * tiles_n;
  const int grp = id / per_group;
  const int first_m = grp * kGroupM;
  const int gsize = min(kGroupM, tiles_m - first_m);
  const int in = id - grp * per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding), as
// a builtin so the compiler's own wait insertion accounts for it.
#define NVFP4_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x70 | 0xF00)

// A workgroup barrier without the memory fence of __syncthreads() (which
// would drain the copies in flight); the empty asm statements keep the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS slot (in 16-byte units) of piece p of row r's stage segment.  The
// XOR term makes one piece of any 8 consecutive rows land in 8 distinct
// 16-byte bank groups of a 128-byte window, and of any 16 consecutive rows
// in 16 distinct groups of a 256-byte window.
__device__ __forceinline__ int piece_swz(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }
__device__ __forceinline__ int piece_slot(int r, int p) { return 2 * r + (p ^ piece_swz(r)); }
}  // namespace

// Packed stage slots (A codes, W codes, A+W scales) and the decoded A tiles,
// each its own LDS object.
__shared__ __attribute__((aligned(1024))) uint8_t g_ac0[kCodeBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_ac1[kCodeBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_ac2[kCodeBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_ac3[kCodeBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_wc0[kCodeBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_wc1[kCodeBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_wc2[kCodeBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_wc3[kCodeBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_sc0[2 * kScaleBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_sc1[2 * kScaleBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_sc2[2 * kScaleBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_sc3[2 * kScaleBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_af0[kAf16Bytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_af1[kAf16Bytes];

template <int B> __device__ __forceinline__ uint8_t* a_slot() {
  return B == 0 ? g_ac0 : (B == 1 ? g_ac1 : (B == 2 ? g_ac2 : g_ac3));
}
template <int B> __device__ __forceinline__ uint8_t* w_slot() {
  return B == 0 ? g_wc0 : (B == 1 ? g_wc1 : (B == 2 ? g_wc2 : g_wc3));
}
template <int B> __device__ __forceinline__ uint8_t* s_slot() {
  return B == 0 ? g_sc0 : (B == 1 ? g_sc1 : (B == 2 ? g_sc2 : g_sc3));
}
template <int F> __device__ __forceinline__ uint8_t* af_buf() { return F == 0 ? g_af0 : g_af1; }

// Per-thread state of the tiled kernel.
struct TiledCtx {
  const uint8_t* ga;    // A code copy source (row, piece) of this lane
  const uint8_t* gw;    // W code copy source
  const uint8_t* gs;    // scale copy source (A for waves 0-3, W for 4-7)
  int wave, lane, wm, wn, h, r32, nst;
};

// Copies of stage `st` into ring slot B: 3 load instructions per wave.
template <int B>
__device__ __forceinline__ void tiled_issue(const TiledCtx& c, int st) {
  g2lds16(c.ga + st * kRowBytes, a_slot<B>() + c.wave * 1024);
  g2lds16(c.gw + st * kRowBytes, w_slot<B>() + c.wave * 1024);
  g2lds4(c.gs + st * kScaleRow, s_slot<B>() + (c.wave >> 2) * kScaleBytes + (c.wave & 3) * 256);
}

// The 32 A values a thread decodes per stage: wave w handles fragment w;
// lane l takes row 32w + l%32 and K [32 (l/32), +32) of the stage in slot B
// (one 16-byte code piece and the scale bytes of its two blocks), and
// writes them to the fp16 tile in MFMA lane order: region (w, step jj) of
// 1 KB, lane slot l (so a wave's writes are one contiguous 1 KB).
struct ADecode {
  uint4 codes;
  half2v s2;
  int dst;    // byte offset of this thread's lane slot in step 0's region
};

template <int B>
__device__ __forceinline__ ADecode decode_a_load(int wave, int lane) {
  const int r = 32 * wave + (lane & 31), hh = lane >> 5;
  ADecode d;
  d.codes = *(const uint4*)(a_slot<B>() + piece_slot(r, hh) * 16);
  const uint32_t sb = *(const uint16_t*)(s_slot<B>() + r * kScaleRow + 2 * hh);
  d.s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false);
  d.dst = wave * 4096 + lane * 16;
  return d;
}

// Decode step jj (8 values, block jj/2 of the thread's two) into tile F.
template <int F>
__device__ __forceinline__ void decode_a_step(const ADecode& d, int jj) {
  *(half8v*)(af_buf<F>() + d.dst + jj * 1024) = dequant8_f16(word_of(d.codes, jj), jj < 2 ? d.s2.xx : d.s2.yy);
}

// One K stage: B = st % 4 (ring slot), st % 2 = B % 2 (decoded A buffer).
// Wait for stage st + 1's copies, barrier, start the copies of stage st + 3
// into slot (B + 3) % 4 (free since the barrier), then multiply stage st
// while decoding A of stage st + 1.  Past the last stage the copies repeat
// the last stage (every stage issues the same number of copies) and the
// stage does nothing else; at the last stage the decode writes a tile
// nobody reads.
template <int B>
__device__ __forceinline__ void tiled_stage(const TiledCtx& c, int st, float16v (&acc)[2][4]) {
  NVFP4_WAIT_VMCNT(kCopies);
  stage_barrier();
  tiled_issue<(B + 3) % kRing>(c, min(st + 3, c.nst - 1));
  if (st >= c.nst) return;

  const int h = c.h, r32 = c.r32, lane = c.lane, wm = c.wm, wn = c.wn;
  const ADecode dec = decode_a_load<(B + 1) % kRing>(c.wave, lane);
  const uint8_t* af = af_buf<B & 1>();
  // W: this lane's code piece h of rows 32 (2 wn + j) + r32, and the two
  // scale bytes of its blocks 2h, 2h + 1.
  uint4 cw[2];
  half2v sw[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 32 * (2 * wn + j) + r32;
    cw[j] = *(const uint4*)(w_slot<B>() + piece_slot(row, h) * 16);
    const uint32_t sb = *(const uint16_t*)(s_slot<B>() + kScaleBytes + row * kScaleRow + 2 * h);
    sw[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false);
  }
  // Step jj's 8 MFMAs are interleaved one at a time with the LDS reads and W
  // decoding of step jj + 1 and step jj's share of the A decode; each MFMA
  // occupies the matrix core for several cycles, during which the wave
  // issues the other work.
  half8v av[2][4], wv[2][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) av[0][i] = *(const half8v*)(af + ((4 * wm + i) * 4 + 0) * 1024 + lane * 16);
#pragma unroll
  for (int j = 0; j < 2; ++j) wv[0][j] = dequant8_f16(word_of(cw[j], 0), sw[j].xx);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int cur = jj & 1, nxt = cur ^ 1;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wv[cur][j], av[cur][i], acc[j][i], 0, 0, 0);
    if (jj + 1 < 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        av[nxt][i] = *(const half8v*)(af + ((4 * wm + i) * 4 + jj + 1) * 1024 + lane * 16);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        wv[nxt][j] = dequant8_f16(word_of(cw[j], jj + 1), jj + 1 < 2 ? sw[j].xx : sw[j].yy);
    }
    decode_a_step<(B + 1) & 1>(dec, jj);
    // MFMA, read, 2 VALU (x4); MFMA, 4 VALU (x3); MFMA, write
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
#pragma unroll
    for (int g = 0; g < 3; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// kLora: add the low-rank branch T L_up^T (T fp32 [M, r], L_up bf16 [N, r])
// to each output before the bf16 rounding (see the epilogue).
template <bool kLora>
__global__ __launch_bounds__(512, 1) void nvfp4_gemm_tiled_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const float* __restrict__ w_g,
    uint16_t* __restrict__ out, int M, int N, int K, int tiles_m, int tiles_n, const float* __restrict__ lora_t,
    const uint16_t* __restrict__ lora_up, int r) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tile_m, tile_n;
  map_tile(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
  const int m0 = tile_m * TM, n0 = tile_n * TN;
  const int64_t row_bytes = K / 2, row_scales = K / 16;

  TiledCtx c;
  c.wave = wave;
  c.lane = lane;
  c.wm = wave >> 2;                 // wave's A rows 128 wm ..
  c.wn = wave & 3;                  // wave's W rows 64 wn ..
  c.h = lane >> 5;
  c.r32 = lane & 31;
  c.nst = K / TK;
  {
    // Code copies: wave w copies rows 32w..32w+31 of each operand's stage;
    // lane l holds row 32w + l/2 and piece (l%2) ^ piece_swz(row), so it
    // lands at piece_slot(row, piece).  Rows past M or N re-read the last
    // row: those results are never stored.
    const int r = 32 * wave + (lane >> 1);
    const int piece = (lane & 1) ^ piece_swz(r);
    c.ga = a_codes + (int64_t)min(m0 + r, M - 1) * row_bytes + 16 * piece;
    c.gw = w_codes + (int64_t)min(n0 + r, N - 1) * row_bytes + 16 * piece;
    // Scale copies: waves 0-3 copy A's rows 64 (w%4) + lane, 4-7 W's; laid
    // out [operand][row][4 bytes].
    const int sr = 64 * (wave & 3) + lane;
    c.gs = wave < 4 ? a_scales + (int64_t)min(m0 + sr, M - 1) * row_scales
                    : w_scales + (int64_t)min(n0 + sr, N - 1) * row_scales;
  }

  float16v acc[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = float16v{};

  // Prologue: stages 0-2 in flight, stage 0's A decoded.
  tiled_issue<0>(c, 0);
  tiled_issue<1>(c, min(1, c.nst - 1));
  tiled_issue<2>(c, min(2, c.nst - 1));
  NVFP4_WAIT_VMCNT(2 * kCopies);
  stage_barrier();
  {
    const ADecode d = decode_a_load<0>(wave, lane);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) decode_a_step<0>(d, jj);
  }
  for (int st = 0; st < c.nst; st += 4) {
    tiled_stage<0>(c, st, acc);
    tiled_stage<1>(c, st + 1, acc);
    tiled_stage<2>(c, st + 2, acc);
    tiled_stage<3>(c, st + 3, acc);
  }
  NVFP4_WAIT_VMCNT(0);      // no copy may land in LDS after the workgroup ends

  const int h = c.h, r32 = c.r32, wm = c.wm, wn = c.wn;
  // Epilogue: D[n][m] of each 32 x 32 tile sits at lane m + 32((n/4)%2),
  // register (n%4) + 4(n/8): four consecutive n per register quad.
  const float gg = (*a_g) * (*w_g);
  const bool vec_ok = (N & 3) == 0;
  if (kLora) {
    // Low-rank branch: D = L_up T^T on the same 32 x 32 fragments (L_up rows
    // n as the first operand, T rows m as the second), accumulated straight
    // into acc after acc is scaled by gg; the store below then multiplies by
    // 1.  T is split into bf16 hi + lo parts (T - hi is exact in fp32 and
    // its bf16 rounding leaves ~2^-17 of T), so the branch keeps near-fp32
    // precision.  Ranks go 32 at a time through LDS (the decoded-A buffers,
    // free once the main loop is done): all 512 threads load the tile's T
    // rows and L_up rows for the chunk at once, so the epilogue pays one
    // memory latency per chunk.  LDS rows hold 16-byte pieces, XOR-swizzled
    // by the row: T row (128 B) piece (2 kk + h) * 2 + {hi, lo}, L_up row
    // (64 B) piece 2 kk + h, where lane half h covers ranks 8h..8h+7 of the
    // 16-rank step kk.
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] = acc[j][i] * gg;
    const auto tr = buffer_of(lora_t, (uint32_t)M * (uint32_t)r * 4u);
    const auto ur = buffer_of(lora_up, (uint32_t)N * (uint32_t)r * 2u);
    uint4* st = (uint4*)g_af0;      // [256 rows][8 pieces]
    uint4* su = (uint4*)g_af1;      // [256 rows][4 pieces]
    const int srow = tid >> 1, shalf = tid & 1;
    for (int c0 = 0; c0 < r; c0 += 32) {
      __syncthreads();              // previous users of the buffers are done
      {
        const uint32_t m = (uint32_t)(m0 + srow), n = (uint32_t)(n0 + srow);
        uint4 tv[4], uv[2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t k = (uint32_t)(c0 + 16 * shalf + 4 * q);
          tv[q] = buffer_load16(tr, m < (uint32_t)M && k < (uint32_t)r ? 4u * (m * r + k) : kBufferOob);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t k = (uint32_t)(c0 + 16 * shalf + 8 * q);
          uv[q] = buffer_load16(ur, n < (uint32_t)N && k < (uint32_t)r ? 2u * (n * r + k) : kBufferOob);
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint4 t0 = tv[2 * hh], t1 = tv[2 * hh + 1];
          const float f[8] = {__uint_as_float(t0.x), __uint_as_float(t0.y), __uint_as_float(t0.z),
                              __uint_as_float(t0.w), __uint_as_float(t1.x), __uint_as_float(t1.y),
                              __uint_as_float(t1.z), __uint_as_float(t1.w)};
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t h0 = f32_to_bf16_rne(f[2 * e]), h1 = f32_to_bf16_rne(f[2 * e + 1]);
            const uint32_t l0 = f32_to_bf16_rne(f[2 * e] - bf16_bits_to_f32(h0));
            const uint32_t l1 = f32_to_bf16_rne(f[2 * e + 1] - bf16_bits_to_f32(h1));
            hi[e] = h0 | (h1 << 16);
            lo[e] = l0 | (l1 << 16);
          }
          const int p = (2 * shalf + hh) * 2;
          st[srow * 8 + (p ^ (srow & 7))] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
          st[srow * 8 + ((p + 1) ^ (srow & 7))] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
          su[srow * 4 + ((2 * shalf + hh) ^ (srow & 3))] = uv[hh];
        }
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (c0 + 16 * kk >= r) break;
        const int pt = (2 * kk + h) * 2, pu = 2 * kk + h;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 128 * wm + 32 * i + r32;
          const short8v hi = __builtin_bit_cast(short8v, st[row * 8 + (pt ^ (row & 7))]);
          const short8v lo = __builtin_bit_cast(short8v, st[row * 8 + ((pt + 1) ^ (row & 7))]);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int col = 64 * wn + 32 * j + r32;
            const short8v up = __builtin_bit_cast(short8v, su[col * 4 + (pu ^ (col & 3))]);
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(up, hi, acc[j][i], 0, 0, 0);
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(up, lo, acc[j][i], 0, 0, 0);
          }
        }
      }
    }
  }
  const float gmul = kLora ? 1.0f : gg;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 128 * wm + 32 * i + r32;
    if (m >= M) continue;
    uint16_t* orow = out + (int64_t)m * N;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int n = n0 + 64 * wn + 32 * j + 8 * rq + 4 * h;
        const uint32_t b0 = f32_to_bf16_rne(acc[j][i][4 * rq + 0] * gmul);
        const uint32_t b1 = f32_to_bf16_rne(acc[j][i][4 * rq + 1] * gmul);
        const uint32_t b2 = f32_to_bf16_rne(acc[j][i][4 * rq + 2] * gmul);
        const uint32_t b3 = f32_to_bf16_rne(acc[j][i][4 * rq + 3] * gmul);
        if (vec_ok && n + 3 < N) {
          *(uint2*)(orow + n) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
        } else {
          if (n + 0 < N) orow[n + 0] = (uint16_t)b0;
          if (n + 1 < N) orow[n + 1] = (uint16_t)b1;
          if (n + 2 < N) orow[n + 2] = (uint16_t)b2;
          if (n + 3 < N) orow[n + 3] = (uint16_t)b3;
        }
      }
    }
  }
}

hipError_t launch_nvfp4_gemm_tiled(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                   const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N, int64_t K,
                                   hipStream_t stream) {
  const int tiles_m = (int)((M + TM - 1) / TM), tiles_n = (int)((N + TN - 1) / TN);
  hipLaunchKernelGGL(nvfp4_gemm_tiled_kernel<false>, dim3((unsigned)(tiles_m * tiles_n)), dim3(512), 0, stream,
                     ac, as, ag, wc, ws, wg, (uint16_t*)out, (int)M, (int)N, (int)K, tiles_m, tiles_n, nullptr,
                     nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_nvfp4_gemm_tiled_lora(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                        const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                        int64_t K, const float* lora_t, const void* lora_up, int64_t r,
                                        hipStream_t stream) {
  const int tiles_m = (int)((M + TM - 1) / TM), tiles_n = (int)((N + TN - 1) / TN);
  hipLaunchKernelGGL(nvfp4_gemm_tiled_kernel<true>, dim3((unsigned)(tiles_m * tiles_n)), dim3(512), 0, stream,
                     ac, as, ag, wc, ws, wg, (uint16_t*)out, (int)M, (int)N, (int)K, tiles_m, tiles_n, lora_t,
                     (const uint16_t*)lora_up, (int)r);
  return hipGetLastError();
}

}  // namespace nvfp4k
