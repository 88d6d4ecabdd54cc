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
//  - Workgroup tile 256 x 256, K stage of 64 values, 4 waves, one per SIMD;
//    a wave's 16 accumulator fragments (256 registers) live in the
//    accumulation register file.  With scale groups (below) each wave
//    covers 256 (m) x 64 (n): it reads all eight A fragments from LDS (each
//    feeding 2 MFMAs) and decodes only its own two W fragments, so every
//    value of both operands is decoded once per workgroup (2 decode
//    instructions per MFMA).  Otherwise a wave covers 128 x 128 (each A
//    fragment feeds 4 MFMAs, and two waves decode each W fragment: 3 per
//    MFMA).  A low-rank branch runs on the scale-group kernel before the
//    product (lora_branch_n64); otherwise, and for small grids, on 8 waves
//    of 128 x 64 (two per SIMD, accumulators in ordinary registers), whose
//    epilogue scales and extends the accumulators with vector instructions.
//  - The packed operands (codes and scale bytes) are copied global -> LDS
//    (LDS DMA through buffer resources) three stages ahead of the MFMAs,
//    into a ring of single stages (each code copy instruction 32 rows x 32
//    contiguous bytes) or, on the scale-group path, of stage pairs.  The
//    slots are distinct LDS objects and the stage loop is unrolled, so the
//    compiler sees that copies in flight never alias what is being read;
//    one wait per stage leaves the newest stage's copies in flight.
//  - A copy instruction costs about one cache-line lookup per row it
//    touches, and a stage holds only 32 code and 4 scale bytes per row.
//    When K is a multiple of 256 the 4-wave kernel copies the codes of two
//    stages at once (64 bytes per row, 16 rows per instruction) into two
//    pair slots, and the scales of four stages at once (16 bytes per row,
//    one lane per row) into two group buffers: half the lines of the code
//    copies, a quarter of the scale copy instructions.
//  - Within a step single MFMAs are interleaved with the next step's LDS
//    reads and the decoding (explicit scheduling groups): the reads are
//    issued early and have completed by the next step, and each MFMA waits
//    only for its own operand.
//  - A is decoded once per workgroup, one stage ahead, into a double-buffered
//    fp16 tile in LDS (16384 values per stage); the MFMA reads it with one
//    ds_read_b128 per fragment and step.  W stays packed in LDS and each
//    wave decodes its W fragments in registers.
//  - The MFMA sums 16 values of K per lane-half; which physical K a lane
//    feeds does not change the sum as long as both operands use the same
//    assignment.  Lane-half h takes K [32h, 32h + 32) of the stage, 8 per
//    step, so a lane's W codes for the whole stage are one 16-byte piece.
//    In LDS the 16-byte pieces of a row's segment (two per stage, four per
//    stage pair) sit XOR-swizzled by the row (piece_slot, pair_piece_slot):
//    the copy writes them in order, and 16 readers of 16 consecutive rows
//    hit 16 distinct bank groups.  The fp16 A tile is stored in MFMA lane
//    order (conflict-free reads).
//  - The W fragment is the MFMA's first operand, so each lane's accumulators
//    hold 4 consecutive output columns n: 8-byte bf16 stores.
//  - One workgroup fills a CU (LDS), so a grid of T tiles runs in
//    ceil(T / CUs) rounds.  With a workspace, the tiles of the last, partial
//    round are split along K into S parts (S = CUs / leftover tiles, at most
//    8) that run side by side; each part stores its fp32 accumulators and a
//    second kernel sums the parts in order and rounds.  The split depends
//    only on the shape and the CU count, so results are reproducible.
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
constexpr int kGroupM = 4;
constexpr int kMaxSplit = 8;
constexpr int kMinPartStages = 4;
constexpr int kGroupStages = 4;                      // stages per scale group
constexpr int kGroupRow = kGroupStages * kScaleRow;  // 16 scale bytes per row per group
constexpr int kGroupBytes = TM * kGroupRow;          // 4 KB per operand per group
static_assert(kMinPartStages >= kGroupStages, "every split part must hold a whole scale group");
constexpr int64_t kPartFloats = (int64_t)TM * TN;    // one tile's fp32 accumulators

typedef __attribute__((address_space(3))) void* lds_void_t;

// Global -> LDS copies (LDS DMA) through buffer resources: lane i's 16 (4)
// bytes at offset off land at l + 16 i (4 i).  The buffer form, not
// global_load_lds: while a global_load_lds is in flight the compiler waits
// for every outstanding LDS access before using any LDS read (it counts the
// copy as a possible LDS access); with the buffer form it keeps exact
// counts, so an MFMA waits only for its own operand.
__device__ __forceinline__ void b2lds16(__amdgpu_buffer_rsrc_t r, uint32_t off, void* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t)l, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void b2lds4(__amdgpu_buffer_rsrc_t r, uint32_t off, void* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t)l, 4, off, 0, 0, 0);
}

// Tile (tm, tn) of tile index id: groups of kGroupM tile-rows, column-major
// within a group.
__device__ __forceinline__ void tile_of(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
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
// s_waitcnt lgkmcnt(0): this wave's LDS accesses are complete.
#define NVFP4_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

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
// The same for rows of two stages (four 16-byte pieces, 64 bytes): piece p
// of row r at slot 4 r + (p ^ pair_swz(r)); one piece of any 8 consecutive
// rows lands in 8 distinct 16-byte groups of a 128-byte window, and of any
// 16 in 16 distinct groups of a 256-byte window.
__device__ __forceinline__ int pair_swz(int r) { return 2 * ((r >> 2) & 1) + (((r >> 1) ^ (r >> 3)) & 1); }
__device__ __forceinline__ int pair_piece_slot(int r, int p) { return 4 * r + (p ^ pair_swz(r)); }
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
__shared__ __attribute__((aligned(1024))) uint8_t g_ap0[2 * kCodeBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_ap1[2 * kCodeBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_wp0[2 * kCodeBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_wp1[2 * kCodeBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_sg0[2 * kGroupBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_sg1[2 * kGroupBytes];
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
template <int P> __device__ __forceinline__ uint8_t* sg_buf() { return P == 0 ? g_sg0 : g_sg1; }
template <int S> __device__ __forceinline__ uint8_t* ap_slot() { return S == 0 ? g_ap0 : g_ap1; }
template <int S> __device__ __forceinline__ uint8_t* wp_slot() { return S == 0 ? g_wp0 : g_wp1; }
template <int F> __device__ __forceinline__ uint8_t* af_buf() { return F == 0 ? g_af0 : g_af1; }

// Per-thread state of the tiled kernel with kW waves.  The stage copies are
// 8 "copy slots" of 32 code rows of each operand and 64 scale rows of one
// operand; wave w moves slots kFr w .. kFr w + kFr - 1 (kFr = 8 / kW).
template <int kW>
struct TiledCtx {
  static constexpr int kFr = 8 / kW;       // copy slots and A fragments per wave
  static constexpr int kJ = kW == 4 ? 4 : 2;  // W fragments per wave
  static constexpr int kCopies = 3 * kFr;  // copy instructions per wave per stage
  // Buffer resources over the tile's rows of the A and W codes, and of the
  // scales each copy slot moves (A for copy slots 0-3, W for 4-7).
  __amdgpu_buffer_rsrc_t rca, rcw, rsq[kFr];
  uint32_t oa[kFr], ow[kFr], os[kFr];   // per-stage path: this lane's copy offsets
  uint32_t opa[4], opw[4];               // scale-group path: pair copy offsets
  int wave, lane, wm, wn, h, r32;
  int st0, nst;            // first K stage and number of stages of this workgroup
};

// Copies of local stage ls into ring slot B.  Past the last stage the
// copies repeat the last stage, so every stage issues the same number of
// copies.
template <int B, int kW>
__device__ __forceinline__ void tiled_issue(const TiledCtx<kW>& c, int ls) {
  constexpr int kFr = TiledCtx<kW>::kFr;
  const int st = c.st0 + min(ls, c.nst - 1);
#pragma unroll
  for (int q = 0; q < kFr; ++q) {
    const int vw = kFr * c.wave + q;
    b2lds16(c.rca, c.oa[q] + st * kRowBytes, a_slot<B>() + vw * 1024);
    b2lds16(c.rcw, c.ow[q] + st * kRowBytes, w_slot<B>() + vw * 1024);
    b2lds4(c.rsq[q], c.os[q] + st * kScaleRow, s_slot<B>() + (vw >> 2) * kScaleBytes + (vw & 3) * 256);
  }
}

// The 32 A values of fragment f (32 rows) a thread decodes per stage: lane
// l takes row 32f + l%32 and K [32 (l/32), +32) of the stage in slot B (one
// 16-byte code piece and the scale bytes of its two blocks), and writes them
// to the fp16 tile in MFMA lane order: region (f, step jj) of 1 KB, lane
// slot l.  Wave w decodes fragments kFr w .. kFr w + kFr - 1.
struct ADecode {
  uint4 codes;
  half2v s2;
  int dst;    // byte offset of this thread's lane slot in step 0's region
};

template <int B>
__device__ __forceinline__ ADecode decode_a_load(int f, int lane) {
  const int r = 32 * f + (lane & 31), hh = lane >> 5;
  ADecode d;
  d.codes = *(const uint4*)(a_slot<B>() + piece_slot(r, hh) * 16);
  const uint32_t sb = *(const uint16_t*)(s_slot<B>() + r * kScaleRow + 2 * hh);
  d.s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false);
  d.dst = f * 4096 + lane * 16;
  return d;
}

// Decode step jj (8 values, block jj/2 of the thread's two) into tile F.
template <int F>
__device__ __forceinline__ void decode_a_step(const ADecode& d, int jj) {
  *(half8v*)(af_buf<F>() + d.dst + jj * 1024) = dequant8_f16(word_of(d.codes, jj), jj < 2 ? d.s2.xx : d.s2.yy);
}

// One K stage: B = ls % 4 (ring slot), ls % 2 = B % 2 (decoded A buffer).
// Wait for stage ls + 1's copies, barrier, start the copies of stage ls + 3
// into slot (B + 3) % 4 (free since the barrier), then multiply stage ls
// while decoding A of stage ls + 1.  Past the last stage the stage does
// nothing but its copies; at the last stage the decode writes a tile nobody
// reads.
template <int B, int kW>
__device__ __forceinline__ void tiled_stage(const TiledCtx<kW>& c, int ls, float16v (&acc)[TiledCtx<kW>::kJ][4]) {
  constexpr int kFr = TiledCtx<kW>::kFr, kJ = TiledCtx<kW>::kJ;
  NVFP4_WAIT_VMCNT(TiledCtx<kW>::kCopies);
  stage_barrier();
  tiled_issue<(B + 3) % kRing>(c, ls + 3);
  if (ls >= c.nst) return;

  const int h = c.h, r32 = c.r32, lane = c.lane, wm = c.wm, wn = c.wn;
  ADecode dec[kFr];
#pragma unroll
  for (int q = 0; q < kFr; ++q) dec[q] = decode_a_load<(B + 1) % kRing>(kFr * c.wave + q, lane);
  const uint8_t* af = af_buf<B & 1>();
  // W: this lane's code piece h of rows 32 (kJ wn + j) + r32, and the two
  // scale bytes of its blocks 2h, 2h + 1.
  uint4 cw[kJ];
  half2v sw[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int row = 32 * (kJ * wn + j) + r32;
    cw[j] = *(const uint4*)(w_slot<B>() + piece_slot(row, h) * 16);
    const uint32_t sb = *(const uint16_t*)(s_slot<B>() + kScaleBytes + row * kScaleRow + 2 * h);
    sw[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false);
  }
  // Step jj's 4 kJ MFMAs are interleaved one at a time with the LDS reads
  // and W decoding of step jj + 1 and step jj's share of the A decode; each
  // MFMA occupies the matrix core for several cycles, during which the wave
  // issues the other work.
  half8v av[2][4], wv[2][kJ];
#pragma unroll
  for (int i = 0; i < 4; ++i) av[0][i] = *(const half8v*)(af + ((4 * wm + i) * 4 + 0) * 1024 + lane * 16);
#pragma unroll
  for (int j = 0; j < kJ; ++j) wv[0][j] = dequant8_f16(word_of(cw[j], 0), sw[j].xx);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int cur = jj & 1, nxt = cur ^ 1;
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wv[cur][j], av[cur][i], acc[j][i], 0, 0, 0);
    if (jj + 1 < 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        av[nxt][i] = *(const half8v*)(af + ((4 * wm + i) * 4 + jj + 1) * 1024 + lane * 16);
#pragma unroll
      for (int j = 0; j < kJ; ++j)
        wv[nxt][j] = dequant8_f16(word_of(cw[j], jj + 1), jj + 1 < 2 ? sw[j].xx : sw[j].yy);
    }
#pragma unroll
    for (int q = 0; q < kFr; ++q) decode_a_step<(B + 1) & 1>(dec[q], jj);
    if (kW == 4) {
      // MFMA, read, 3 VALU (x4); MFMA, 3 VALU (x10); MFMA, write (x2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
#pragma unroll
      for (int g = 0; g < 10; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      }
    } else {
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
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Four-wave stage with the work spread over the MFMAs.  A single wave per
// SIMD stalls its MFMA stream whenever an instruction cannot issue, so
// (a) the six copy instructions of stage ls + 3 are issued two per step in
// steps 0-2, between MFMAs, instead of back to back after the barrier, and
// (b) the W codes and scale bytes of stage ls + 1 are read into registers
// during step 3 (slot (B + 1) % 4 is complete and visible since this
// stage's barrier), so after the next barrier only the A fragment reads
// stand before the first MFMA.
struct WPre {
  uint4 cw[4];
  uint32_t sb[4];
};

template <int B>
__device__ __forceinline__ void w_prefetch(const TiledCtx<4>& c, WPre& p) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 32 * (4 * c.wn + j) + c.r32;
    p.cw[j] = *(const uint4*)(w_slot<B>() + piece_slot(row, c.h) * 16);
    p.sb[j] = *(const uint16_t*)(s_slot<B>() + kScaleBytes + row * kScaleRow + 2 * c.h);
  }
}

// Copy instructions 2 part, 2 part + 1 of the list (A, W, scales of copy
// slot 2w, then of slot 2w + 1) for local stage ls into ring slot B.
template <int B>
__device__ __forceinline__ void tiled_copy_part(const TiledCtx<4>& c, int ls, int part) {
  const int st = c.st0 + min(ls, c.nst - 1);
#pragma unroll
  for (int e = 2 * part; e < 2 * part + 2; ++e) {
    const int q = e / 3, kind = e % 3, vw = 2 * c.wave + q;
    if (kind == 0) b2lds16(c.rca, c.oa[q] + st * kRowBytes, a_slot<B>() + vw * 1024);
    else if (kind == 1) b2lds16(c.rcw, c.ow[q] + st * kRowBytes, w_slot<B>() + vw * 1024);
    else b2lds4(c.rsq[q], c.os[q] + st * kScaleRow, s_slot<B>() + (vw >> 2) * kScaleBytes + (vw & 3) * 256);
  }
}

// kChecked: the stage may lie past the last one (then it only issues its
// copies).  Whole groups of four stages run unchecked, with no branch in
// the stage, so the compiler's tracking of which LDS slots the copies in
// flight write stays exact and it does not wait for all of them before
// the next stage's LDS reads.
template <int B, bool kChecked>
__device__ __forceinline__ void tiled_stage4(const TiledCtx<4>& c, int ls, float16v (&acc)[4][4], WPre (&pw)[2]) {
  NVFP4_WAIT_VMCNT(TiledCtx<4>::kCopies);
  stage_barrier();
  if (kChecked && ls >= c.nst) {
    tiled_issue<(B + 3) % kRing>(c, ls + 3);
    return;
  }
  const int lane = c.lane, wm = c.wm;
  // The step-0 A fragments are the only LDS reads the first MFMA waits for:
  // issue them first (LDS reads complete in order), then the A-decode reads,
  // while the step-0 W fragments are decoded from registers.
  const uint8_t* af = af_buf<B & 1>();
  half8v av[2][4], wv[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) av[0][i] = *(const half8v*)(af + ((4 * wm + i) * 4 + 0) * 1024 + lane * 16);
  __builtin_amdgcn_sched_barrier(0);
  const ADecode dec0 = decode_a_load<(B + 1) % kRing>(2 * c.wave, lane);
  const ADecode dec1 = decode_a_load<(B + 1) % kRing>(2 * c.wave + 1, lane);
  __builtin_amdgcn_sched_barrier(0);
  const WPre& cur = pw[B & 1];
  half2v sw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sw[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur.sb[j], 1.0f, false);
#pragma unroll
  for (int j = 0; j < 4; ++j) wv[0][j] = dequant8_f16(word_of(cur.cw[j], 0), sw[j].xx);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int cu = jj & 1, nx = cu ^ 1;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wv[cu][j], av[cu][i], acc[j][i], 0, 0, 0);
    if (jj < 3) tiled_copy_part<(B + 3) % kRing>(c, ls + 3, jj);
    if (jj + 1 < 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        av[nx][i] = *(const half8v*)(af + ((4 * wm + i) * 4 + jj + 1) * 1024 + lane * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wv[nx][j] = dequant8_f16(word_of(cur.cw[j], jj + 1), jj + 1 < 2 ? sw[j].xx : sw[j].yy);
    } else {
      w_prefetch<(B + 1) % kRing>(c, pw[(B + 1) & 1]);
    }
    decode_a_step<(B + 1) & 1>(dec0, jj);
    decode_a_step<(B + 1) & 1>(dec1, jj);
    // MFMA, copy, 2 VALU (x2); MFMA, read, 3 VALU (x8); MFMA, 3 VALU (x4);
    // MFMA, write (x2)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Prologue of the per-stage paths: stages 0-2 in flight, stage 0's A
// decoded.
template <int kW>
__device__ __forceinline__ void tiled_prologue(const TiledCtx<kW>& c) {
  constexpr int kFr = TiledCtx<kW>::kFr;
  tiled_issue<0>(c, 0);
  tiled_issue<1>(c, 1);
  tiled_issue<2>(c, 2);
  NVFP4_WAIT_VMCNT(2 * TiledCtx<kW>::kCopies);
  stage_barrier();
#pragma unroll
  for (int q = 0; q < kFr; ++q) {
    const ADecode d = decode_a_load<0>(kFr * c.wave + q, c.lane);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) decode_a_step<0>(d, jj);
  }
}

// Scale-group path (K a multiple of 256, 4-wave kernel).
//
// Scale groups: group lg holds the scale bytes of local stages 4 lg ..
// 4 lg + 3 in group buffer lg % 2, laid out [operand][row][stage][4 bytes];
// copy slot vw (the same rows as the per-stage scale copies) moves rows
// 64 (vw % 4) + lane of operand vw / 4 with one 16-byte copy per lane.
// Past the last group the copies repeat it.  The part's first stage is a
// multiple of 4 and a scale row holds K/16 bytes, so every copy source is
// 16-byte aligned.
template <int P>
__device__ __forceinline__ void group_copy(const TiledCtx<4>& c, int lg) {
  const int st = c.st0 + kGroupStages * min(lg, c.nst / kGroupStages - 1);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int vw = 2 * c.wave + q;
    b2lds16(c.rsq[q], c.os[q] + st * kScaleRow, sg_buf<P>() + (vw >> 2) * kGroupBytes + (vw & 3) * 1024);
  }
}

// Code pairs: the codes of stages 2 lq and 2 lq + 1 (64 bytes per row) go
// to pair slot lq % 2 ([row][4 pieces], pair_piece_slot), one instruction
// per 16 rows (4 lanes per row): a copy touches 16 cache lines instead of
// 32.  Wave w copies rows 64 w .. 64 w + 63 of both operands; part 0-1: A,
// 2-3: W, two instructions each.  Past the last pair the copies repeat it.
template <int S>
__device__ __forceinline__ void pair_copy_part(const TiledCtx<4>& c, int lq, int part) {
  const int st = c.st0 + 2 * min(lq, c.nst / 2 - 1);
#pragma unroll
  for (int k = 2 * (part & 1); k < 2 * (part & 1) + 2; ++k) {
    if (part < 2) b2lds16(c.rca, c.opa[k] + st * kRowBytes, ap_slot<S>() + (4 * c.wave + k) * 1024);
    else b2lds16(c.rcw, c.opw[k] + st * kRowBytes, wp_slot<S>() + (4 * c.wave + k) * 1024);
  }
}

// decode_a_load from pair slot S (stage TH of the pair) and group buffer P
// (stage T of the group).  The scale bytes stay raw until the first decode
// step, so that nothing before the stage's first MFMA waits for these
// reads (they are issued after that MFMA's operands).
struct ADecodeRaw {
  uint4 codes;
  uint32_t sb;
  int dst;
};

template <int S, int TH, int P, int T>
__device__ __forceinline__ ADecodeRaw decode_a_load_p(int f, int lane) {
  const int r = 32 * f + (lane & 31), hh = lane >> 5;
  ADecodeRaw d;
  d.codes = *(const uint4*)(ap_slot<S>() + pair_piece_slot(r, 2 * TH + hh) * 16);
  d.sb = *(const uint16_t*)(sg_buf<P>() + r * kGroupRow + T * kScaleRow + 2 * hh);
  d.dst = f * 4096 + lane * 16;
  return d;
}

template <int F>
__device__ __forceinline__ void decode_a_step_raw(const ADecodeRaw& d, int jj) {
  const half2v s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d.sb, 1.0f, false);
  *(half8v*)(af_buf<F>() + d.dst + jj * 1024) = dequant8_f16(word_of(d.codes, jj), jj < 2 ? s2.xx : s2.yy);
}

// Wave tile 256 (m) x 64 (n): every wave multiplies all eight 32-row A
// fragments of the workgroup's fp16 A tile with its own two W fragments
// (rows 64 w .. 64 w + 63 of the W tile), so each W fragment is decoded by
// one wave only (with 128 x 128 wave tiles two waves decode each).  Per
// lane and stage that is 64 W and 64 A values decoded for 64 MFMAs,
// against 128 + 64; each A fragment read from LDS feeds two MFMAs instead
// of four.
struct WPre2 {
  uint4 cw[2];
  uint32_t sb[2];
};

template <int S, int TH, int P, int T>
__device__ __forceinline__ void w_prefetch_p(const TiledCtx<4>& c, WPre2& p) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 64 * c.wave + 32 * j + c.r32;
    p.cw[j] = *(const uint4*)(wp_slot<S>() + pair_piece_slot(row, 2 * TH + c.h) * 16);
    p.sb[j] = *(const uint16_t*)(sg_buf<P>() + kGroupBytes + row * kGroupRow + T * kScaleRow + 2 * c.h);
  }
}

// One K stage of the scale-group path; B8 = ls % 8, acc[j][i]: W fragment
// j, A fragment i.  As in tiled_stage4, the stage multiplies stage ls while
// decoding A of stage ls + 1 and reading its W into registers.  Copies:
// an odd stage copies code pair (ls + 3) / 2 (stages ls + 3, ls + 4; eight
// instructions per wave, two per step) into the slot of the pair holding
// stages ls - 1 and ls, whose last readers ran in stage ls - 1: each wave
// first waits for its own LDS reads, so after the barrier none is still in
// flight.  The first stage of group lg (B8 % 4 == 0) copies the scales of
// group lg + 1 (two instructions, step 2) into the buffer group lg - 1
// used.  Each stage waits until only the previous stage's copies are in
// flight: 8 after an odd stage, 2 after a group's first stage, else none.
// A pair is first read two stages after it is issued, a group three.
template <int B8>
__device__ __forceinline__ void tiled_stage_n64(const TiledCtx<4>& c, int ls, float16v (&acc)[2][8],
                                                WPre2 (&pw)[2]) {
  constexpr int S1 = ((B8 + 1) >> 1) & 1;   // pair slot of stage ls + 1
  constexpr int TH1 = (B8 + 1) & 1;         // its place in the pair
  constexpr int P1 = ((B8 + 1) >> 2) & 1;   // its group buffer
  constexpr int T1 = (B8 + 1) & 3;          // its place in the group
  constexpr int SN = ((B8 + 3) >> 1) & 1;   // slot of the pair copied here (odd B8)
  constexpr int PN = ((B8 >> 2) + 1) & 1;   // buffer of the group copied here (B8 % 4 == 0)
  constexpr int kPrev = (B8 & 1) ? ((B8 & 2) ? 0 : 2) : 8;
  if (B8 & 1) NVFP4_WAIT_LGKM0();
  NVFP4_WAIT_VMCNT(kPrev);
  stage_barrier();
  const int lane = c.lane;
  const uint8_t* af = af_buf<B8 & 1>();
  half8v av[2][8], wv[2][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) av[0][i] = *(const half8v*)(af + (i * 4 + 0) * 1024 + lane * 16);
  __builtin_amdgcn_sched_barrier(0);
  const ADecodeRaw dec0 = decode_a_load_p<S1, TH1, P1, T1>(2 * c.wave, lane);
  const ADecodeRaw dec1 = decode_a_load_p<S1, TH1, P1, T1>(2 * c.wave + 1, lane);
  __builtin_amdgcn_sched_barrier(0);
  const WPre2& cur = pw[B8 & 1];
  half2v sw[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) sw[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur.sb[j], 1.0f, false);
#pragma unroll
  for (int j = 0; j < 2; ++j) wv[0][j] = dequant8_f16(word_of(cur.cw[j], 0), sw[j].xx);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int cu = jj & 1, nx = cu ^ 1;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wv[cu][j], av[cu][i], acc[j][i], 0, 0, 0);
    if (B8 & 1) pair_copy_part<SN>(c, (ls + 3) >> 1, jj);
    if ((B8 & 3) == 0 && jj == 2) group_copy<PN>(c, ls / kGroupStages + 1);
    if (jj + 1 < 4) {
#pragma unroll
      for (int i = 0; i < 8; ++i) av[nx][i] = *(const half8v*)(af + (i * 4 + jj + 1) * 1024 + lane * 16);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        wv[nx][j] = dequant8_f16(word_of(cur.cw[j], jj + 1), jj + 1 < 2 ? sw[j].xx : sw[j].yy);
    } else {
      w_prefetch_p<S1, TH1, P1, T1>(c, pw[(B8 + 1) & 1]);
    }
    decode_a_step_raw<(B8 + 1) & 1>(dec0, jj);
    decode_a_step_raw<(B8 + 1) & 1>(dec1, jj);
    // MFMA, copy, 2 VALU (x2); MFMA, read, 2 VALU (x8); MFMA, 3 VALU (x4);
    // MFMA, write (x2)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// bf16 stores of one 32 x 32 fragment times gmul, row m.  D[n][m] of a
// fragment sits at lane m + 32((n/4)%2), register (n%4) + 4(n/8): four
// consecutive n per register quad.  With N % 8 == 0 and the fragment's 32
// columns inside N, lanes m and m + 32 swap halves (v_permlane32_swap) and
// each stores 8 consecutive columns nb + 16 k + 8 h .. + 7 (k = 0, 1) as
// 16 bytes; otherwise each lane stores columns nb + 8 rq + 4 h + (0..3)
// from registers 4 rq .. 4 rq + 3.  Returns the largest |bf16| bit pattern
// (sign cleared) among the values stored (0 if none).
__device__ __forceinline__ uint32_t store_frag(const float16v& a, float gmul, uint16_t* __restrict__ out, int M,
                                               int N, int m, int nb, int h) {
  if (m >= M) return 0u;
  uint16_t* orow = out + (int64_t)m * N;
  uint32_t mx = 0u;
  if ((N & 7) == 0 && nb + 31 < N) {
    // 16 bytes per lane: lanes m and m + 32 (the same row) swap halves so
    // that each holds 8 consecutive columns, nb + 16 k + 8 h .. + 7.
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t a01 = f32x2_to_bf16x2_rne(a[8 * k + 0] * gmul, a[8 * k + 1] * gmul);
      const uint32_t a23 = f32x2_to_bf16x2_rne(a[8 * k + 2] * gmul, a[8 * k + 3] * gmul);
      const uint32_t b01 = f32x2_to_bf16x2_rne(a[8 * k + 4] * gmul, a[8 * k + 5] * gmul);
      const uint32_t b23 = f32x2_to_bf16x2_rne(a[8 * k + 6] * gmul, a[8 * k + 7] * gmul);
      mx = max(mx, max(max(bf16x2_absmax_bits(a01), bf16x2_absmax_bits(a23)),
                       max(bf16x2_absmax_bits(b01), bf16x2_absmax_bits(b23))));
      // lanes 32..63 of the first operand trade with lanes 0..31 of the second
      const auto s01 = __builtin_amdgcn_permlane32_swap(a01, b01, false, false);
      const auto s23 = __builtin_amdgcn_permlane32_swap(a23, b23, false, false);
      *(uint4*)(orow + nb + 16 * k + 8 * h) = make_uint4(s01[0], s23[0], s01[1], s23[1]);
    }
    return mx;
  }
  const bool vec_ok = (N & 3) == 0;
#pragma unroll
  for (int rq = 0; rq < 4; ++rq) {
    const int n = nb + 8 * rq + 4 * h;
    const uint32_t b01 = f32x2_to_bf16x2_rne(a[4 * rq + 0] * gmul, a[4 * rq + 1] * gmul);
    const uint32_t b23 = f32x2_to_bf16x2_rne(a[4 * rq + 2] * gmul, a[4 * rq + 3] * gmul);
    if (vec_ok && n + 3 < N) {
      *(uint2*)(orow + n) = make_uint2(b01, b23);
      mx = max(mx, max(bf16x2_absmax_bits(b01), bf16x2_absmax_bits(b23)));
    } else {
      if (n + 0 < N) orow[n + 0] = (uint16_t)b01, mx = max(mx, b01 & 0x7FFFu);
      if (n + 1 < N) orow[n + 1] = (uint16_t)(b01 >> 16), mx = max(mx, (b01 >> 16) & 0x7FFFu);
      if (n + 2 < N) orow[n + 2] = (uint16_t)b23, mx = max(mx, b23 & 0x7FFFu);
      if (n + 3 < N) orow[n + 3] = (uint16_t)(b23 >> 16), mx = max(mx, (b23 >> 16) & 0x7FFFu);
    }
  }
  return mx;
}

// Adds the low-rank branch sum_k T[m][k] L_up[n][k] (fp32, plain loops) to
// the bf16 values of one stored 32 x 32 fragment: out = bf16(out + branch),
// for the elements this lane stored (store_frag's layout).
__device__ __noinline__ void add_branch_frag(const float* __restrict__ lora_t, const uint16_t* __restrict__ lora_up,
                                             int r, uint16_t* __restrict__ out, int M, int N, int m, int nb, int h) {
  if (m >= M) return;
  uint16_t* orow = out + (int64_t)m * N;
  const float* trow = lora_t + (int64_t)m * r;
  // the columns this lane stored (store_frag's two layouts)
  const bool swapped = (N & 7) == 0 && nb + 31 < N;
#pragma unroll 1
  for (int q = 0; q < 16; ++q) {
    const int n = swapped ? nb + 16 * (q >> 3) + 8 * h + (q & 7) : nb + 8 * (q >> 2) + 4 * h + (q & 3);
    if (n >= N) continue;
    const uint16_t* urow = lora_up + (int64_t)n * r;
    float v = 0.f;
#pragma unroll 1
    for (int k = 0; k < r; ++k) v += trow[k] * bf16_bits_to_f32(urow[k]);
    orow[n] = (uint16_t)f32_to_bf16_rne(bf16_bits_to_f32(orow[n]) + v);
  }
}

// A wave's 4 kJ fragments: fragment (j, i) covers rows m0 + 128 wm + 32 i
// and columns n0 + 32 kJ wn + 32 j.  Returns the lane's largest |bf16|
// pattern stored.
template <int kJ>
__device__ __forceinline__ uint32_t store_tile(const float16v (&acc)[kJ][4], float gmul, uint16_t* __restrict__ out,
                                               int M, int N, int m0, int n0, int wm, int wn, int h, int r32) {
  uint32_t mx = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kJ; ++j)
      mx = max(mx, store_frag(acc[j][i], gmul, out, M, N, m0 + 128 * wm + 32 * i + r32, n0 + 32 * kJ * wn + 32 * j, h));
  return mx;
}

// Largest of v over the workgroup's kW waves, valid in thread 0 (red: kW
// words of LDS; the caller's threads all take part).
template <int kW>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t m = 0u;
  if (threadIdx.x == 0)
#pragma unroll
    for (int w = 0; w < kW; ++w) m = max(m, red[w]);
  return m;
}

// Low-rank branch: D = L_up T^T on the same 32 x 32 fragments (L_up rows n
// as the first operand, T rows m as the second), accumulated straight into
// acc after acc is scaled by g_a g_w.  T is split into bf16 hi + lo parts
// (T - hi is exact in fp32 and its bf16 rounding leaves ~2^-17 of T), so
// the branch keeps near-fp32 precision.  Ranks go 32 at a time through LDS
// (the decoded-A buffers, free once the main loop is done): the threads
// load the tile's T rows and L_up rows of the chunk together (kW / 4
// threads per row), so the epilogue pays one memory latency per chunk.  LDS
// rows hold 16-byte pieces, XOR-swizzled by the row: T row (128 B) piece
// 2q + {hi, lo} and L_up row (64 B) piece q for the ranks 8q .. 8q + 7 of
// the chunk (q = 2 kk + h: lane half h of 16-rank step kk).
template <int kW>
__device__ __forceinline__ void lora_epilogue(float16v (&acc)[TiledCtx<kW>::kJ][4], float gg,
                                              const float* __restrict__ lora_t, const uint16_t* __restrict__ lora_up,
                                              int r, int M, int N, int m0, int n0, int wm, int wn, int h, int r32) {
  constexpr int kJ = TiledCtx<kW>::kJ;
  constexpr int kTpr = kW / 4;            // threads per staged row
  constexpr int kNq = 4 / kTpr;           // 8-rank groups per thread
#pragma unroll
  for (int j = 0; j < kJ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = acc[j][i] * gg;
  const auto tr = buffer_of(lora_t, (uint32_t)M * (uint32_t)r * 4u);
  const auto ur = buffer_of(lora_up, (uint32_t)N * (uint32_t)r * 2u);
  uint4* st = (uint4*)g_af0;      // [256 rows][8 pieces]
  uint4* su = (uint4*)g_af1;      // [256 rows][4 pieces]
  const int srow = threadIdx.x / kTpr, q0 = (threadIdx.x % kTpr) * kNq;
  for (int c0 = 0; c0 < r; c0 += 32) {
    __syncthreads();              // previous users of the buffers are done
    {
      const uint32_t m = (uint32_t)(m0 + srow), n = (uint32_t)(n0 + srow);
      uint4 tv[2 * kNq], uv[kNq];
#pragma unroll
      for (int e = 0; e < 2 * kNq; ++e) {
        const uint32_t k = (uint32_t)(c0 + 8 * q0 + 4 * e);
        tv[e] = buffer_load16(tr, m < (uint32_t)M && k < (uint32_t)r ? 4u * (m * r + k) : kBufferOob);
      }
#pragma unroll
      for (int e = 0; e < kNq; ++e) {
        const uint32_t k = (uint32_t)(c0 + 8 * (q0 + e));
        uv[e] = buffer_load16(ur, n < (uint32_t)N && k < (uint32_t)r ? 2u * (n * r + k) : kBufferOob);
      }
#pragma unroll
      for (int e = 0; e < kNq; ++e) {
        const int q = q0 + e;
        const uint4 t0 = tv[2 * e], t1 = tv[2 * e + 1];
        const float f[8] = {__uint_as_float(t0.x), __uint_as_float(t0.y), __uint_as_float(t0.z),
                            __uint_as_float(t0.w), __uint_as_float(t1.x), __uint_as_float(t1.y),
                            __uint_as_float(t1.z), __uint_as_float(t1.w)};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const uint32_t h0 = f32_to_bf16_rne(f[2 * x]), h1 = f32_to_bf16_rne(f[2 * x + 1]);
          const uint32_t l0 = f32_to_bf16_rne(f[2 * x] - bf16_bits_to_f32(h0));
          const uint32_t l1 = f32_to_bf16_rne(f[2 * x + 1] - bf16_bits_to_f32(h1));
          hi[x] = h0 | (h1 << 16);
          lo[x] = l0 | (l1 << 16);
        }
        st[srow * 8 + ((2 * q) ^ (srow & 7))] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        st[srow * 8 + ((2 * q + 1) ^ (srow & 7))] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        su[srow * 4 + (q ^ (srow & 3))] = uv[e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if (c0 + 16 * kk >= r) break;
      const int q = 2 * kk + h;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 128 * wm + 32 * i + r32;
        const short8v hi = __builtin_bit_cast(short8v, st[row * 8 + ((2 * q) ^ (row & 7))]);
        const short8v lo = __builtin_bit_cast(short8v, st[row * 8 + ((2 * q + 1) ^ (row & 7))]);
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
          const int col = 32 * kJ * wn + 32 * j + r32;
          const short8v up = __builtin_bit_cast(short8v, su[col * 4 + (q ^ (col & 3))]);
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(up, hi, acc[j][i], 0, 0, 0);
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(up, lo, acc[j][i], 0, 0, 0);
        }
      }
    }
  }
}

// Low-rank branch for the 256 x 64 wave tiles of the scale-group path.  The
// accumulators live in the accumulation registers, which vector
// instructions cannot scale in place, so instead of g_a g_w acc + L_up T^T
// the tile computes g_a g_w (L_up (T / (g_a g_w))^T + acc): this function
// runs first, on the zeroed accumulators, before the product's main loop
// (the decoded-A buffers are still free), and the store multiplies by
// g_a g_w (tscale = 1 / (g_a g_w)).  With g_a g_w = 0 the caller skips the
// product and passes tscale = 1 (store multiplier 1).  With g_a g_w outside
// [2^-64, 2^64] the branch divided by it could leave the fp32 range: the
// caller then skips this, stores the product alone and adds the branch to
// the stored tile (add_branch_frag).  T is staged as bf16
// hi + lo parts as in lora_epilogue, one thread per row of the tile (256 T
// rows and 256 L_up rows per 32-rank chunk).
__device__ __forceinline__ void lora_branch_n64(float16v (&acc)[2][8], float tscale,
                                                const float* __restrict__ lora_t,
                                                const uint16_t* __restrict__ lora_up, int r, int M, int N, int m0,
                                                int n0, int wave, int h, int r32) {
  const auto tr = buffer_of(lora_t, (uint32_t)M * (uint32_t)r * 4u);
  const auto ur = buffer_of(lora_up, (uint32_t)N * (uint32_t)r * 2u);
  uint4* st = (uint4*)g_af0;      // [256 rows][8 pieces]
  uint4* su = (uint4*)g_af1;      // [256 rows][4 pieces]
  const int srow = threadIdx.x;
  for (int c0 = 0; c0 < r; c0 += 32) {
    __syncthreads();              // previous users of the buffers are done
    {
      const uint32_t m = (uint32_t)(m0 + srow), n = (uint32_t)(n0 + srow);
      uint4 tv[8], uv[4];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t k = (uint32_t)(c0 + 4 * e);
        tv[e] = buffer_load16(tr, m < (uint32_t)M && k < (uint32_t)r ? 4u * (m * r + k) : kBufferOob);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t k = (uint32_t)(c0 + 8 * e);
        uv[e] = buffer_load16(ur, n < (uint32_t)N && k < (uint32_t)r ? 2u * (n * r + k) : kBufferOob);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 t0 = tv[2 * q], t1 = tv[2 * q + 1];
        const float f[8] = {__uint_as_float(t0.x) * tscale, __uint_as_float(t0.y) * tscale,
                            __uint_as_float(t0.z) * tscale, __uint_as_float(t0.w) * tscale,
                            __uint_as_float(t1.x) * tscale, __uint_as_float(t1.y) * tscale,
                            __uint_as_float(t1.z) * tscale, __uint_as_float(t1.w) * tscale};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const uint32_t h0 = f32_to_bf16_rne(f[2 * x]), h1 = f32_to_bf16_rne(f[2 * x + 1]);
          const uint32_t l0 = f32_to_bf16_rne(f[2 * x] - bf16_bits_to_f32(h0));
          const uint32_t l1 = f32_to_bf16_rne(f[2 * x + 1] - bf16_bits_to_f32(h1));
          hi[x] = h0 | (h1 << 16);
          lo[x] = l0 | (l1 << 16);
        }
        st[srow * 8 + ((2 * q) ^ (srow & 7))] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        st[srow * 8 + ((2 * q + 1) ^ (srow & 7))] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        su[srow * 4 + (q ^ (srow & 3))] = uv[q];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if (c0 + 16 * kk >= r) break;
      const int q = 2 * kk + h;
      short8v up[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = 64 * wave + 32 * j + r32;
        up[j] = __builtin_bit_cast(short8v, su[col * 4 + (q ^ (col & 3))]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 32 * i + r32;
        const short8v hi = __builtin_bit_cast(short8v, st[row * 8 + ((2 * q) ^ (row & 7))]);
        const short8v lo = __builtin_bit_cast(short8v, st[row * 8 + ((2 * q + 1) ^ (row & 7))]);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(up[j], hi, acc[j][i], 0, 0, 0);
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(up[j], lo, acc[j][i], 0, 0, 0);
        }
      }
    }
  }
}

// Grid: full_tiles whole tiles and (tiles - full_tiles) x splits K parts
// (half of the parts dispatched before the whole tiles, half after).
// Whole tiles are visited in an XCD-aware order when full_tiles % 8 == 0.
// Part p of leftover tile t takes stages [p nst / S, (p + 1) nst / S) and
// stores its unscaled fp32 accumulators to part[(t S + p)] in lane order
// (kW == 4 only).  kLora: add the low-rank branch T L_up^T (T fp32 [M, r],
// L_up bf16 [N, r]) to each output before the bf16 rounding (launched
// with kW == 8 and without splits).  kAmax (kW == 4, no low-rank branch):
// amax[tile] receives the largest |bf16| pattern of the tile's outputs;
// for a split tile it is set to 0 here and raised by the reduce kernel.
// kGroups (kW == 4, K a multiple of 256, scale arrays 16-byte aligned):
// scales move in groups of four stages, and part boundaries are multiples
// of four stages (part p of S: groups [p G / S, (p + 1) G / S) of the
// G = K / 256).
template <int kW, bool kLora, bool kAmax = false, bool kGroups = false>
__global__ __launch_bounds__(64 * kW, 1) void nvfp4_gemm_tiled_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const float* __restrict__ w_g,
    uint16_t* __restrict__ out, int M, int N, int K, int tiles_m, int tiles_n, int full_tiles, int splits,
    float* __restrict__ part, const float* __restrict__ lora_t, const uint16_t* __restrict__ lora_up, int r,
    uint32_t* __restrict__ amax) {
  static_assert(!kAmax || (kW == 4 && !kLora), "amax slots: 4-wave kernel without the low-rank branch");
  static_assert(!kGroups || kW == 4, "scale groups: 4-wave kernel");
  static_assert(!kLora || kW == 8 || kGroups, "low-rank branch: 8-wave kernel or the scale-group path");
  using Ctx = TiledCtx<kW>;
  constexpr int kFr = Ctx::kFr, kJ = Ctx::kJ;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Dispatch order when the last round is split: half of the K parts first,
  // then the whole tiles, then the other half of the parts.  On every XCD
  // the CUs that start with a part run a fraction of a tile ahead of the
  // others from then on, so the tiles of one XCD do not all request the
  // same lines at the same moment (measured faster than every tile in step,
  // though the XCD's L2 then re-fetches more of their shared panels).
  int bid = blockIdx.x;
  {
    const int nunits = (int)gridDim.x - full_tiles, first = (nunits / 2) & ~7;
    if (full_tiles > 0 && first > 0) bid = bid < first ? full_tiles + bid : (bid < first + full_tiles ? bid - first : bid);
  }
  const int nst_all = K / TK;
  int tile_id, st0 = 0, st1 = nst_all, unit = -1;
  if (bid < full_tiles) {
    tile_id = (full_tiles & 7) == 0 ? (bid & 7) * (full_tiles >> 3) + (bid >> 3) : bid;
  } else {
    // K part p of leftover tile t is dispatched as u = p * left + t, and
    // each XCD takes a contiguous range of u (when the counts divide by 8):
    // the parts that run together on an XCD then read the same K range of
    // neighbouring tiles and share their operand panels in its L2.  `unit`
    // = t * splits + p is where the part's sums go (the reduce kernel's
    // order), so the results do not depend on this order.
    const int nunits = (int)gridDim.x - full_tiles, left = nunits / splits;
    const int uo = bid - full_tiles;
    const int u = ((full_tiles | nunits) & 7) == 0 ? (uo & 7) * (nunits >> 3) + (uo >> 3) : uo;
    const int p = u / left, t = u % left;
    unit = t * splits + p;
    tile_id = full_tiles + t;
    if (kGroups) {
      const int ng = nst_all / kGroupStages;
      st0 = kGroupStages * (p * ng / splits);
      st1 = kGroupStages * ((p + 1) * ng / splits);
    } else {
      st0 = p * nst_all / splits;
      st1 = (p + 1) * nst_all / splits;
    }
  }
  int tile_m, tile_n;
  tile_of(tile_id, tiles_m, tiles_n, tile_m, tile_n);
  const int m0 = tile_m * TM, n0 = tile_n * TN;
  const int64_t row_bytes = K / 2, row_scales = K / 16;

  Ctx c;
  c.wave = wave;
  c.lane = lane;
  c.wm = wave / (kW / 2);           // wave's A rows 128 wm ..
  c.wn = wave % (kW / 2);           // wave's W rows 32 kJ wn ..
  c.h = lane >> 5;
  c.r32 = lane & 31;
  c.st0 = st0;
  c.nst = st1 - st0;
  // Buffer resources over the tile's rows (at most 256 x K/2 < 2^31 bytes:
  // the tiled kernel takes K < 2^24).  Rows past M or N re-read the last
  // row: those results are never stored.
  const int rows_a = min(TM, M - m0), rows_w = min(TN, N - n0);
  c.rca = buffer_of(a_codes + (int64_t)m0 * row_bytes, (uint32_t)(rows_a * row_bytes));
  c.rcw = buffer_of(w_codes + (int64_t)n0 * row_bytes, (uint32_t)(rows_w * row_bytes));
  const auto rsa = buffer_of(a_scales + (int64_t)m0 * row_scales, (uint32_t)(rows_a * row_scales));
  const auto rsw = buffer_of(w_scales + (int64_t)n0 * row_scales, (uint32_t)(rows_w * row_scales));
  if constexpr (kGroups) {
    // Pair copy k (0-3) of this wave: rows 16 (4 wave + k) + lane / 4, slot
    // lane % 4 of the row's 64 bytes, which holds piece (lane % 4) ^
    // pair_swz(row).  Scale groups: copy slot vw = 2 wave + q moves rows
    // 64 (vw % 4) + lane of operand vw / 4.
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rr = 16 * (4 * wave + k) + (lane >> 2);
      const int piece = (lane & 3) ^ pair_swz(rr);
      c.opa[k] = (uint32_t)(min(rr, rows_a - 1) * row_bytes + 16 * piece);
      c.opw[k] = (uint32_t)(min(rr, rows_w - 1) * row_bytes + 16 * piece);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int vw = 2 * wave + q, sr = 64 * (vw & 3) + lane;
      c.rsq[q] = vw < 4 ? rsa : rsw;
      c.os[q] = (uint32_t)(min(sr, (vw < 4 ? rows_a : rows_w) - 1) * row_scales);
    }
  } else {
#pragma unroll
    for (int q = 0; q < kFr; ++q) {
      // Code copies of copy slot vw: lane l holds row 32 vw + l/2 and piece
      // (l%2) ^ piece_swz(row), so it lands at piece_slot(row, piece).
      // Scale copies: slots 0-3 copy A's rows 64 (vw%4) + lane, 4-7 W's;
      // laid out [operand][row][4 bytes].
      const int vw = kFr * wave + q;
      const int rr = 32 * vw + (lane >> 1);
      const int piece = (lane & 1) ^ piece_swz(rr);
      c.oa[q] = (uint32_t)(min(rr, rows_a - 1) * row_bytes + 16 * piece);
      c.ow[q] = (uint32_t)(min(rr, rows_w - 1) * row_bytes + 16 * piece);
      const int sr = 64 * (vw & 3) + lane;
      c.rsq[q] = vw < 4 ? rsa : rsw;
      c.os[q] = (uint32_t)(min(sr, (vw < 4 ? rows_a : rows_w) - 1) * row_scales);
    }
  }

  float16v acc[kJ][4];
#pragma unroll
  for (int j = 0; j < kJ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = float16v{};

  if constexpr (kGroups) {
    float16v acc2[2][8];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc2[j][i] = float16v{};
    // With the low-rank branch and g_a g_w = 0 the product adds nothing: it
    // is skipped, and the branch alone is stored (store multiplier 1).  With
    // g_a g_w far from 1 the branch is added after the store instead.
    const float gg = (*a_g) * (*w_g);
    const float gmul = kLora && gg == 0.f ? 1.f : gg;
    const bool late = kLora && gg != 0.f && !(gg >= 0x1p-64f && gg <= 0x1p64f);
    if constexpr (kLora) {
      if (!late) lora_branch_n64(acc2, 1.f / gmul, lora_t, lora_up, r, M, N, m0, n0, wave, c.h, c.r32);
      __syncthreads();            // the decoded-A buffers are free again
    }
    // Prologue: scale group 0 and code pairs 0 and 1 in flight, then stage
    // 0's A decoded and its W read.
    group_copy<0>(c, 0);
#pragma unroll
    for (int part = 0; part < 4; ++part) pair_copy_part<0>(c, 0, part);
#pragma unroll
    for (int part = 0; part < 4; ++part) pair_copy_part<1>(c, 1, part);
    NVFP4_WAIT_VMCNT(8);
    stage_barrier();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const ADecodeRaw d = decode_a_load_p<0, 0, 0, 0>(2 * wave + q, lane);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) decode_a_step_raw<0>(d, jj);
    }
    WPre2 pw[2];
    w_prefetch_p<0, 0, 0, 0>(c, pw[0]);
    int ls = kLora && gg == 0.f ? c.nst : 0;
    for (; ls + 8 <= c.nst; ls += 8) {
      tiled_stage_n64<0>(c, ls, acc2, pw);
      tiled_stage_n64<1>(c, ls + 1, acc2, pw);
      tiled_stage_n64<2>(c, ls + 2, acc2, pw);
      tiled_stage_n64<3>(c, ls + 3, acc2, pw);
      tiled_stage_n64<4>(c, ls + 4, acc2, pw);
      tiled_stage_n64<5>(c, ls + 5, acc2, pw);
      tiled_stage_n64<6>(c, ls + 6, acc2, pw);
      tiled_stage_n64<7>(c, ls + 7, acc2, pw);
    }
    if (ls < c.nst) {      // nst is a multiple of 4: one group left
      tiled_stage_n64<0>(c, ls, acc2, pw);
      tiled_stage_n64<1>(c, ls + 1, acc2, pw);
      tiled_stage_n64<2>(c, ls + 2, acc2, pw);
      tiled_stage_n64<3>(c, ls + 3, acc2, pw);
    }
    NVFP4_WAIT_VMCNT(0);
    const int h = c.h, r32 = c.r32;
    if (unit >= 0) {
      if (kAmax && tid == 0 && unit % splits == 0) amax[tile_id] = 0u;
      // fragment (j, i) of wave w at part[unit][(w * 16 + j * 8 + i) * 64 + lane][16]
      float* dst = part + (int64_t)unit * kPartFloats + (int64_t)wave * 16 * 64 * 16 + lane * 16;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float4* d4 = (float4*)(dst + (j * 8 + i) * 64 * 16);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            d4[e] = make_float4(acc2[j][i][4 * e], acc2[j][i][4 * e + 1], acc2[j][i][4 * e + 2], acc2[j][i][4 * e + 3]);
        }
      return;
    }
    uint32_t mx = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        mx = max(mx, store_frag(acc2[j][i], gmul, out, M, N, m0 + 32 * i + r32, n0 + 64 * wave + 32 * j, h));
    if constexpr (kLora) {
      if (late) {
#pragma unroll 1
        for (int f = 0; f < 16; ++f)
          add_branch_frag(lora_t, lora_up, r, out, M, N, m0 + 32 * (f & 7) + r32, n0 + 64 * wave + 32 * (f >> 3), h);
      }
    }
    if (kAmax) {
      static_assert(!(kAmax && kLora), "the low-rank variant reports no amax");
      __shared__ uint32_t red2[4];
      const uint32_t m = block_max_u32<4>(mx, red2);
      if (tid == 0) amax[tile_id] = m;
    }
    return;
  } else if constexpr (kW == 4) {
    tiled_prologue<kW>(c);
    WPre pw[2];
    w_prefetch<0>(c, pw[0]);
    int ls = 0;
    for (; ls + 4 <= c.nst; ls += 4) {
      tiled_stage4<0, false>(c, ls, acc, pw);
      tiled_stage4<1, false>(c, ls + 1, acc, pw);
      tiled_stage4<2, false>(c, ls + 2, acc, pw);
      tiled_stage4<3, false>(c, ls + 3, acc, pw);
    }
    if (ls < c.nst) {
      tiled_stage4<0, true>(c, ls, acc, pw);
      tiled_stage4<1, true>(c, ls + 1, acc, pw);
      tiled_stage4<2, true>(c, ls + 2, acc, pw);
      tiled_stage4<3, true>(c, ls + 3, acc, pw);
    }
  } else {
    tiled_prologue<kW>(c);
    for (int ls = 0; ls < c.nst; ls += 4) {
      tiled_stage<0>(c, ls, acc);
      tiled_stage<1>(c, ls + 1, acc);
      tiled_stage<2>(c, ls + 2, acc);
      tiled_stage<3>(c, ls + 3, acc);
    }
  }
  NVFP4_WAIT_VMCNT(0);      // no copy may land in LDS after the workgroup ends

  const int h = c.h, r32 = c.r32, wm = c.wm, wn = c.wn;
  if (kW == 4 && unit >= 0) {
    if (kAmax && tid == 0 && unit % splits == 0) amax[tile_id] = 0u;
    // K part of a split tile: fragment (j, i) of wave w at
    // part[unit][(w * 16 + j * 4 + i) * 64 + lane][16].
    float* dst = part + (int64_t)unit * kPartFloats + (int64_t)wave * 16 * 64 * 16 + lane * 16;
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4* d4 = (float4*)(dst + (j * 4 + i) * 64 * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          d4[e] = make_float4(acc[j][i][4 * e], acc[j][i][4 * e + 1], acc[j][i][4 * e + 2], acc[j][i][4 * e + 3]);
      }
    return;
  }
  const float gg = (*a_g) * (*w_g);
  if (kLora) lora_epilogue<kW>(acc, gg, lora_t, lora_up, r, M, N, m0, n0, wm, wn, h, r32);
  const uint32_t mx = store_tile<kJ>(acc, kLora ? 1.0f : gg, out, M, N, m0, n0, wm, wn, h, r32);
  if (kAmax) {
    __shared__ uint32_t red[kW];
    const uint32_t m = block_max_u32<kW>(mx, red);
    if (tid == 0) amax[tile_id] = m;
  }
}

// Leftover tile t: workgroup (t, g) sums, for fragments 4g .. 4g + 3 of
// the tile (one per wave), the `splits` K parts in order, scales by
// g_a g_w, rounds to bf16 and stores.  Fragment f of the GEMM's wave w is
// f = 16 w + 4 j + i with 128 x 128 wave tiles (rows 128 (w / 2) + 32 i,
// columns 128 (w % 2) + 32 j) and f = 16 w + 8 j + i with 256 x 64 wave
// tiles (kN64: rows 32 i, columns 64 w + 32 j).  With amax, it raises
// amax[full_tiles + t] (zeroed by the tile kernel) to the largest |bf16|
// pattern it stored.
template <bool kN64>
__global__ __launch_bounds__(256) void nvfp4_gemm_tiled_reduce_kernel(const float* __restrict__ part,
                                                                      const float* __restrict__ a_g,
                                                                      const float* __restrict__ w_g,
                                                                      uint16_t* __restrict__ out, int M, int N,
                                                                      int tiles_m, int tiles_n, int full_tiles,
                                                                      int splits, uint32_t* __restrict__ amax) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x >> 4;
  const int f = 4 * (blockIdx.x & 15) + (threadIdx.x >> 6);
  const int w = f >> 4;
  const int fm = kN64 ? 32 * (f & 7) : 128 * (w >> 1) + 32 * (f & 3);
  const int fn = kN64 ? 64 * w + 32 * ((f >> 3) & 1) : 128 * (w & 1) + 32 * ((f >> 2) & 3);
  int tile_m, tile_n;
  tile_of(full_tiles + t, tiles_m, tiles_n, tile_m, tile_n);
  const float* src = part + (int64_t)t * splits * kPartFloats + ((int64_t)f * 64 + lane) * 16;
  float16v s = *(const float16v*)src;
  for (int p = 1; p < splits; ++p) s += *(const float16v*)(src + p * kPartFloats);
  const uint32_t mx = store_frag(s, (*a_g) * (*w_g), out, M, N, tile_m * TM + fm + (lane & 31), tile_n * TN + fn,
                                 lane >> 5);
  if (amax != nullptr) {
    __shared__ uint32_t red[4];
    const uint32_t m = block_max_u32<4>(mx, red);
    if (threadIdx.x == 0) atomicMax(amax + full_tiles + t, m);
  }
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

namespace {

struct TiledPlan {
  int tiles_m, tiles_n, full_tiles, splits;
  bool groups;          // scales in groups of four stages (K a multiple of 256)
  int64_t part_bytes;
};

// Whole tiles for every full round; the leftover tiles of a partial round
// are split along K so that they fill the CUs (no split without leftovers
// or when the parts would be shorter than kMinPartStages stages).  Only a
// last round at most half full is split (S = CUs / leftover >= 2): the chip
// is power bound, so when fewer CUs run they clock higher, and a round 3/4
// full (192 of 256 tiles, the DiT down GEMM) measured as fast unsplit as
// split into 4 parts was slow (0.27 vs 0.34 ms, the parts' traffic
// included).
TiledPlan plan_tiled(int64_t M, int64_t N, int64_t K, bool allow_split) {
  TiledPlan p;
  p.tiles_m = (int)((M + TM - 1) / TM);
  p.tiles_n = (int)((N + TN - 1) / TN);
  const int tiles = p.tiles_m * p.tiles_n;
  p.full_tiles = tiles;
  p.splits = 1;
  // Scale groups need K % 256 == 0; their buffer offsets cover a tile's
  // rows, 256 x K/2 bytes, which must stay below 2^31.
  p.groups = K % (kGroupStages * TK) == 0 && K < ((int64_t)1 << 24);
  p.part_bytes = 0;
  if (!allow_split) return p;
  const int cus = device_cus();
  const int left = tiles % cus;
  if (left == 0) return p;
  int s = cus / left;
  const int nst = (int)(K / TK);
  if (s > kMaxSplit) s = kMaxSplit;
  if (s > nst / kMinPartStages) s = nst / kMinPartStages;
  if (s < 2) return p;
  p.full_tiles = tiles - left;
  p.splits = s;
  p.part_bytes = (int64_t)left * s * kPartFloats * 4;
  if (p.groups) {
    // With scale groups a stage runs about 4% faster, but a split part is
    // whole groups, so the longest part can have up to 3 more stages (84
    // stages in 4 parts: 24 instead of 21).  Keep groups when the estimated
    // time of the full rounds plus the split round is lower.
    const int64_t rounds = p.full_tiles / cus;
    const int64_t ng = nst / kGroupStages;
    const int64_t t_groups = 24 * (rounds * nst + kGroupStages * ((ng + s - 1) / s));
    const int64_t t_stages = 25 * (rounds * nst + (nst + s - 1) / s);
    p.groups = t_groups < t_stages;
  }
  return p;
}
}  // namespace

int64_t nvfp4_gemm_tiled_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0) return 0;
  return plan_tiled(M, N, K, true).part_bytes;
}

int64_t nvfp4_gemm_tiled_amax_slots(int64_t M, int64_t N) {
  return ((M + TM - 1) / TM) * ((N + TN - 1) / TN);
}

hipError_t launch_nvfp4_gemm_tiled_ws(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                      const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                      int64_t K, void* workspace, int64_t workspace_bytes, hipStream_t stream,
                                      uint32_t* amax) {
  TiledPlan p = plan_tiled(M, N, K, workspace != nullptr);
  if (p.part_bytes > workspace_bytes) p = plan_tiled(M, N, K, false);
  const int tiles = p.tiles_m * p.tiles_n;
  const int grid = p.full_tiles + (tiles - p.full_tiles) * p.splits;
  // Scale groups copy 16 bytes per row: the scale arrays must be 16-byte
  // aligned (rows are, as K is a multiple of 256).  The C entry points
  // require that alignment; other callers get the per-stage copies.
  const bool groups = p.groups && ((reinterpret_cast<uintptr_t>(as) | reinterpret_cast<uintptr_t>(ws)) & 15) == 0;
  auto kernel = amax != nullptr ? (groups ? nvfp4_gemm_tiled_kernel<4, false, true, true>
                                          : nvfp4_gemm_tiled_kernel<4, false, true, false>)
                                : (groups ? nvfp4_gemm_tiled_kernel<4, false, false, true>
                                          : nvfp4_gemm_tiled_kernel<4, false, false, false>);
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(256), 0, stream, ac, as, ag, wc, ws, wg, (uint16_t*)out,
                     (int)M, (int)N, (int)K, p.tiles_m, p.tiles_n, p.full_tiles, p.splits, (float*)workspace,
                     nullptr, nullptr, 0, amax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.full_tiles == tiles) return e;
  hipLaunchKernelGGL(groups ? nvfp4_gemm_tiled_reduce_kernel<true> : nvfp4_gemm_tiled_reduce_kernel<false>,
                     dim3((unsigned)(16 * (tiles - p.full_tiles))), dim3(256), 0, stream,
                     (const float*)workspace, ag, wg, (uint16_t*)out, (int)M, (int)N, p.tiles_m, p.tiles_n,
                     p.full_tiles, p.splits, amax);
  return hipGetLastError();
}

hipError_t launch_nvfp4_gemm_tiled(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                   const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N, int64_t K,
                                   hipStream_t stream) {
  return launch_nvfp4_gemm_tiled_ws(ac, as, ag, wc, ws, wg, out, M, N, K, nullptr, 0, stream);
}

hipError_t launch_nvfp4_gemm_tiled_lora(const uint8_t* ac, const uint8_t* as, const float* ag, const uint8_t* wc,
                                        const uint8_t* ws, const float* wg, void* out, int64_t M, int64_t N,
                                        int64_t K, const float* lora_t, const void* lora_up, int64_t r,
                                        hipStream_t stream) {
  // The 4-wave scale-group kernel for grids of at least half a round of
  // tiles; a lone tile runs faster on the 8-wave kernel (two waves per SIMD
  // hide more latency: 28 vs 34 us for 6 tiles, 300 x 700 x 1024).
  const TiledPlan p = plan_tiled(M, N, K, false);
  const int tiles = p.tiles_m * p.tiles_n;
  if (p.groups && 2 * tiles >= device_cus() &&
      ((reinterpret_cast<uintptr_t>(as) | reinterpret_cast<uintptr_t>(ws)) & 15) == 0)
    hipLaunchKernelGGL((nvfp4_gemm_tiled_kernel<4, true, false, true>), dim3((unsigned)tiles), dim3(256), 0, stream,
                       ac, as, ag, wc, ws, wg, (uint16_t*)out, (int)M, (int)N, (int)K, p.tiles_m, p.tiles_n, tiles, 1,
                       nullptr, lora_t, (const uint16_t*)lora_up, (int)r, nullptr);
  else
    hipLaunchKernelGGL((nvfp4_gemm_tiled_kernel<8, true>), dim3((unsigned)tiles), dim3(512), 0, stream, ac, as, ag,
                       wc, ws, wg, (uint16_t*)out, (int)M, (int)N, (int)K, p.tiles_m, p.tiles_n, tiles, 1, nullptr,
                       lora_t, (const uint16_t*)lora_up, (int)r, nullptr);
  return hipGetLastError();
}

}  // namespace nvfp4k
