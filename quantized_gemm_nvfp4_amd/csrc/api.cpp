// C ABI of libnvfp4.so (declared in include/nvfp4.h): argument validation,
// kernel choice and error reporting.  Every check runs on the host before
// any HIP call, so a rejected call enqueues nothing and touches no device.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "../../include/nvfp4.h"
#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

nvfp4_status fail(nvfp4_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

nvfp4_status ok() {
  g_last_error[0] = '\0';
  return NVFP4_OK;
}

nvfp4_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
  const void* p;
  int64_t bytes;
  const char* name;
};

bool overlap(const Range& a, const Range& b) {
  if (a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

// Checks that no output range overlaps any other listed range.
nvfp4_status check_disjoint(const Range* outs, int nout, const Range* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j]))
        return fail(NVFP4_ERR_INVALID_ARG, "output %s overlaps input %s", outs[i].name, ins[j].name);
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j]))
        return fail(NVFP4_ERR_INVALID_ARG, "output %s overlaps output %s", outs[i].name, outs[j].name);
  }
  return NVFP4_OK;
}

constexpr int64_t kMaxDim = 0x7FFFFFFF;
// The INT4 and weight-only NVFP4 tiled kernels address a tile's rows of x
// (128 x 2K bytes) with 32-bit buffer offsets.
constexpr int64_t kInt4TiledKLimit = (int64_t)1 << 22;
// The weight-streaming kernels address at most kDecodeMaxRows packed weight
// rows (the 112-row workgroup of the INT4 decode kernel is the largest) and
// the whole bf16 activation of M <= 16 rows through buffer resources with
// 32-bit byte ranges.  Offsets at or past 2^31 mark loads that must read
// zero, so every range must stay below 2^31; K <= 2^24 guarantees it.
constexpr int64_t kDecodeMaxK = int64_t(1) << 24;
constexpr int64_t kDecodeMaxRows = 112;
constexpr int64_t kBufferOobOffset = int64_t(1) << 31;
static_assert(kDecodeMaxRows * (kDecodeMaxK / 2) < kBufferOobOffset, "weight rows of a decode workgroup");
static_assert(16 * kDecodeMaxK * 2 < kBufferOobOffset, "bf16 activation of a decode call");
// The NVFP4 tiled kernel addresses a tile's rows (256 x K/2 bytes) with
// 32-bit buffer offsets.
constexpr int64_t kTiledKLimit = int64_t(1) << 24;

#define REQUIRE_PTR(p)                                                               \
  do {                                                                               \
    if ((p) == nullptr) return fail(NVFP4_ERR_INVALID_ARG, "%s is a null pointer", #p); \
  } while (0)
#define REQUIRE_ALIGN(p, a)                                                                  \
  do {                                                                                       \
    if (!aligned((p), (a))) return fail(NVFP4_ERR_ALIGNMENT, "%s is not %d-byte aligned", #p, (int)(a)); \
  } while (0)

nvfp4_status check_dims(int64_t a, const char* an, int64_t b, const char* bn, int64_t c, const char* cn) {
  if (a < 0 || b < 0 || c < 0)
    return fail(NVFP4_ERR_INVALID_ARG, "negative size (%s=%lld, %s=%lld, %s=%lld)", an, (long long)a, bn,
                (long long)b, cn, (long long)c);
  if (a > kMaxDim || b > kMaxDim || c > kMaxDim)
    return fail(NVFP4_ERR_UNSUPPORTED, "a dimension exceeds 2^31-1 (%s=%lld, %s=%lld, %s=%lld)", an,
                (long long)a, bn, (long long)b, cn, (long long)c);
  return NVFP4_OK;
}

// Matrix sizes whose element counts stay below 2^40 (far past any device
// memory), so byte counts and ranges never overflow int64.
constexpr int64_t kMaxElems = int64_t(1) << 40;
nvfp4_status check_products(int64_t M, int64_t N, int64_t K) {
  if ((N > 0 && M > kMaxElems / N) || (K > 0 && M > kMaxElems / K) || (K > 0 && N > kMaxElems / K))
    return fail(NVFP4_ERR_UNSUPPORTED, "a matrix exceeds 2^40 elements (M=%lld, N=%lld, K=%lld)", (long long)M,
                (long long)N, (long long)K);
  return NVFP4_OK;
}

// Which kernel AUTO picks for the NVFP4 GEMM.
int auto_algo(int64_t M, int64_t K) {
  const bool k128 = (K % 128) == 0 && K > 0;
  return !k128 ? NVFP4_ALGO_SIMPLE
               : (M <= 16 ? (K <= kDecodeMaxK ? NVFP4_ALGO_DECODE : NVFP4_ALGO_SIMPLE)
                          : (K < kTiledKLimit ? NVFP4_ALGO_TILED : NVFP4_ALGO_SIMPLE));
}

// Slots nvfp4_gemm_amax writes for AUTO's kernel choice: one per output tile
// of the tiled kernel, else the partial maxima of a separate pass over out.
int64_t amax_slots(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0) return 0;
  if (auto_algo(M, K) == NVFP4_ALGO_TILED) return nvfp4k::nvfp4_gemm_tiled_amax_slots(M, N);
  return nvfp4k::amax_partial_count(M * N);
}

// Shared by nvfp4_gemm_ex, nvfp4_gemm_lora_ex and nvfp4_gemm_amax; lora_t ==
// nullptr means no low-rank branch (its arguments were validated by the
// caller); amax != nullptr (AUTO, no branch, N % 16 == 0) also writes the
// output's amax slots.
nvfp4_status gemm_impl(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                       const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale, void* out_bf16,
                       int64_t M, int64_t N, int64_t K, int algo, const float* lora_t, const void* lora_up,
                       int64_t r, void* workspace, size_t workspace_bytes, void* stream, uint32_t* amax = nullptr) {
  if (nvfp4_status s = check_dims(M, "M", N, "N", K, "K")) return s;
  if (nvfp4_status s = check_products(M, N, K)) return s;
  if (K > 0) {  // with K == 0 the packed operands are empty and never read
    REQUIRE_PTR(a_codes);
    REQUIRE_PTR(a_scales);
    REQUIRE_PTR(w_codes);
    REQUIRE_PTR(w_scales);
  }
  REQUIRE_PTR(a_gscale);
  REQUIRE_PTR(w_gscale);
  REQUIRE_PTR(out_bf16);
  if (K % 16 != 0) return fail(NVFP4_ERR_SHAPE, "K=%lld is not a multiple of 16", (long long)K);
  if (algo < NVFP4_ALGO_AUTO || algo > NVFP4_ALGO_SIMPLE) return fail(NVFP4_ERR_INVALID_ARG, "unknown algo %d", algo);
  REQUIRE_ALIGN(a_codes, 16);
  REQUIRE_ALIGN(a_scales, 16);
  REQUIRE_ALIGN(w_codes, 16);
  REQUIRE_ALIGN(w_scales, 16);
  REQUIRE_ALIGN(out_bf16, 16);
  REQUIRE_ALIGN(a_gscale, 4);
  REQUIRE_ALIGN(w_gscale, 4);
  if (workspace != nullptr) {
    REQUIRE_ALIGN(workspace, 256);
    if (workspace_bytes > (size_t)INT64_MAX) return fail(NVFP4_ERR_INVALID_ARG, "workspace_bytes is too large");
  }
  const Range outs[3] = {{out_bf16, M * N * 2, "out"},
                         {workspace, workspace ? (int64_t)workspace_bytes : 0, "workspace"},
                         {amax, amax ? 4 * amax_slots(M, N, K) : 0, "amax_slots"}};
  const Range ins[8] = {{a_codes, M * K / 2, "a_codes"}, {a_scales, M * K / 16, "a_scales"},
                        {a_gscale, 4, "a_gscale"},       {w_codes, N * K / 2, "w_codes"},
                        {w_scales, N * K / 16, "w_scales"}, {w_gscale, 4, "w_gscale"},
                        {lora_t, lora_t ? M * r * 4 : 0, "lora_t"}, {lora_up, lora_t ? N * r * 2 : 0, "lora_up"}};
  if (M == 0 || N == 0) return ok();
  if (nvfp4_status s = check_disjoint(outs, 3, ins, 8)) return s;
  const bool k128 = (K % 128) == 0 && K > 0;
  if (algo == NVFP4_ALGO_AUTO) algo = auto_algo(M, K);
  hipStream_t st = (hipStream_t)stream;
  if (amax && algo != NVFP4_ALGO_TILED) {    // the output's maxima from a separate pass
    nvfp4_status s = gemm_impl(a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, out_bf16, M, N, K, algo,
                               nullptr, nullptr, 0, workspace, workspace_bytes, stream);
    if (s != NVFP4_OK) return s;
    return hip_status(nvfp4k::launch_amax_partials(out_bf16, M * N, amax, st), "nvfp4_gemm_amax amax pass");
  }
  switch (algo) {
    case NVFP4_ALGO_TILED:
      if (!k128 || K >= kTiledKLimit)
        return fail(NVFP4_ERR_UNSUPPORTED, "tiled kernel needs K %% 128 == 0 and 0 < K < 2^24 (K=%lld)", (long long)K);
      if (lora_t)
        return hip_status(nvfp4k::launch_nvfp4_gemm_tiled_lora(a_codes, a_scales, a_gscale, w_codes, w_scales,
                                                               w_gscale, out_bf16, M, N, K, lora_t, lora_up, r, st),
                          "nvfp4_gemm_lora tiled launch");
      return hip_status(nvfp4k::launch_nvfp4_gemm_tiled_ws(a_codes, a_scales, a_gscale, w_codes, w_scales,
                                                           w_gscale, out_bf16, M, N, K, workspace,
                                                           (int64_t)workspace_bytes, st, amax),
                        "nvfp4_gemm tiled launch");
    case NVFP4_ALGO_DECODE:
      if (!k128 || M > 16 || K > kDecodeMaxK)
        return fail(NVFP4_ERR_UNSUPPORTED, "decode kernel needs M <= 16, K %% 128 == 0 and K <= 2^24 (M=%lld, K=%lld)",
                    (long long)M, (long long)K);
      return hip_status(nvfp4k::launch_nvfp4_gemm_decode_lora(a_codes, a_scales, a_gscale, w_codes, w_scales,
                                                              w_gscale, out_bf16, M, N, K, lora_t, lora_up, r, st),
                        "nvfp4_gemm decode launch");
    default:
      return hip_status(nvfp4k::launch_nvfp4_gemm_simple_lora(a_codes, a_scales, a_gscale, w_codes, w_scales,
                                                              w_gscale, out_bf16, M, N, K, lora_t, lora_up, r, st),
                        "nvfp4_gemm simple launch");
  }
}

// Rank limits shared by the two low-rank entry points.
nvfp4_status check_rank(int64_t r) {
  if (r < 8 || r > nvfp4k::kLoraMaxRank || r % 8 != 0)
    return fail(NVFP4_ERR_UNSUPPORTED, "rank r=%lld; supported ranks are multiples of 8 in [8, %d]", (long long)r,
                nvfp4k::kLoraMaxRank);
  return NVFP4_OK;
}

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return 1; }

size_t nvfp4_quantize_workspace_bytes(void) { return sizeof(uint32_t) * nvfp4k::kAmaxPartials; }

size_t nvfp4_quantize_lora_workspace_bytes(int64_t rows, int64_t cols, int64_t r) {
  if (rows < 0 || cols < 0 || r < 0 || rows > kMaxDim || cols > kMaxDim || r > nvfp4k::kLoraMaxRank) return 0;
  return (size_t)nvfp4k::lora_workspace_bytes(rows, cols, r);
}

const char* nvfp4_status_string(nvfp4_status s) {
  switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_INVALID_ARG: return "invalid argument";
    case NVFP4_ERR_SHAPE: return "shape violates the format";
    case NVFP4_ERR_ALIGNMENT: return "misaligned pointer";
    case NVFP4_ERR_UNSUPPORTED: return "unsupported request";
    case NVFP4_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* nvfp4_last_error(void) { return g_last_error; }

nvfp4_status nvfp4_quantize_ex(const void* x_bf16, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                               float* global_scale, int use_given_global_scale, int scale_rule, void* workspace,
                               void* stream) {
  REQUIRE_PTR(x_bf16);
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scales);
  REQUIRE_PTR(global_scale);
  if (!use_given_global_scale) REQUIRE_PTR(workspace);
  if (scale_rule < NVFP4_SCALE_ABSMAX || scale_rule > NVFP4_SCALE_MSE)
    return fail(NVFP4_ERR_INVALID_ARG, "unknown scale rule %d", scale_rule);
  if (nvfp4_status s = check_dims(rows, "rows", cols, "cols", 0, "-")) return s;
  if (cols % 16 != 0) return fail(NVFP4_ERR_SHAPE, "cols=%lld is not a multiple of 16", (long long)cols);
  if (rows > 0 && cols > INT64_MAX / 2 / rows) return fail(NVFP4_ERR_UNSUPPORTED, "rows*cols overflows");
  REQUIRE_ALIGN(x_bf16, 16);
  REQUIRE_ALIGN(codes, 16);
  REQUIRE_ALIGN(scales, 16);
  REQUIRE_ALIGN(global_scale, 4);
  if (!use_given_global_scale) REQUIRE_ALIGN(workspace, 4);
  const int64_t n = rows * cols;
  const Range outs[3] = {{codes, n / 2, "codes"}, {scales, n / 16, "scales"}, {global_scale, 4, "global_scale"}};
  const Range ins[2] = {{x_bf16, n * 2, "x"},
                        {workspace, use_given_global_scale ? 0 : (int64_t)nvfp4_quantize_workspace_bytes(),
                         "workspace"}};
  if (n == 0) return ok();
  if (nvfp4_status s = check_disjoint(outs, 3, ins, 2)) return s;
  return hip_status(nvfp4k::launch_nvfp4_quantize(x_bf16, rows, cols, codes, scales, global_scale,
                                                  use_given_global_scale, scale_rule, (uint32_t*)workspace,
                                                  (hipStream_t)stream),
                    "nvfp4_quantize launch");
}

nvfp4_status nvfp4_quantize(const void* x_bf16, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                            float* global_scale, int use_given_global_scale, void* workspace, void* stream) {
  return nvfp4_quantize_ex(x_bf16, rows, cols, codes, scales, global_scale, use_given_global_scale,
                           NVFP4_SCALE_ABSMAX, workspace, stream);
}

nvfp4_status nvfp4_quantize_noalloc(const void* x_bf16, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                    float* global_scale, int use_given_global_scale, void* stream) {
  REQUIRE_PTR(x_bf16);
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scales);
  REQUIRE_PTR(global_scale);
  if (nvfp4_status s = check_dims(rows, "rows", cols, "cols", 0, "-")) return s;
  if (cols % 16 != 0) return fail(NVFP4_ERR_SHAPE, "cols=%lld is not a multiple of 16", (long long)cols);
  if (rows > 0 && cols > kMaxElems / rows) return fail(NVFP4_ERR_UNSUPPORTED, "rows*cols exceeds 2^40");
  REQUIRE_ALIGN(x_bf16, 16);
  REQUIRE_ALIGN(codes, 16);
  REQUIRE_ALIGN(scales, 16);
  REQUIRE_ALIGN(global_scale, 4);
  const int64_t n = rows * cols;
  const Range outs[3] = {{codes, n / 2, "codes"}, {scales, n / 16, "scales"}, {global_scale, 4, "global_scale"}};
  const Range ins[1] = {{x_bf16, n * 2, "x"}};
  if (n == 0) return ok();
  if (nvfp4_status s = check_disjoint(outs, 3, ins, 1)) return s;
  // the first pass writes at most kAmaxPartials partial maxima, which is
  // exactly the scratch's size, for every input size accepted above
  uint32_t* partials = nullptr;
  if (!use_given_global_scale) {
    const hipError_t e = nvfp4k::quantize_scratch((hipStream_t)stream, &partials);
    if (e != hipSuccess) return hip_status(e, "nvfp4_quantize_noalloc scratch lookup");
  }
  return hip_status(nvfp4k::launch_nvfp4_quantize(x_bf16, rows, cols, codes, scales, global_scale,
                                                  use_given_global_scale, NVFP4_SCALE_ABSMAX, partials,
                                                  (hipStream_t)stream),
                    "nvfp4_quantize_noalloc launch");
}

nvfp4_status nvfp4_gemm_ex(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                           const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale, void* out_bf16,
                           int64_t M, int64_t N, int64_t K, int algo, void* stream) {
  return gemm_impl(a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, out_bf16, M, N, K, algo, nullptr,
                   nullptr, 0, nullptr, 0, stream);
}

size_t nvfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 16 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K >= kTiledKLimit) return 0;
  return (size_t)nvfp4k::nvfp4_gemm_tiled_workspace_bytes(M, N, K);
}

nvfp4_status nvfp4_gemm_ws(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                           const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale, void* out_bf16,
                           int64_t M, int64_t N, int64_t K, int algo, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return gemm_impl(a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, out_bf16, M, N, K, algo, nullptr,
                   nullptr, 0, workspace, workspace_bytes, stream);
}

size_t nvfp4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N < 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
  if (nvfp4k::nvfp4_linear_fused_supported(M, K)) return 0;
  // the quantizer's partial maxima, then (stream-ordered, after the
  // quantizer is done with them) the GEMM's split-K partial sums
  const size_t g = nvfp4_gemm_workspace_bytes(M, N, K), q = nvfp4_quantize_workspace_bytes();
  return g > q ? g : q;
}

nvfp4_status nvfp4_linear(const void* x_bf16, const uint8_t* w_codes, const uint8_t* w_scales,
                          const float* w_gscale, void* out_bf16, int64_t M, int64_t N, int64_t K, uint8_t* x_codes,
                          uint8_t* x_scales, float* x_gscale, void* workspace, size_t workspace_bytes, void* stream) {
  REQUIRE_PTR(x_bf16);
  REQUIRE_PTR(w_codes);
  REQUIRE_PTR(w_scales);
  REQUIRE_PTR(w_gscale);
  REQUIRE_PTR(out_bf16);
  REQUIRE_PTR(x_codes);
  REQUIRE_PTR(x_scales);
  REQUIRE_PTR(x_gscale);
  if (nvfp4_status s = check_dims(M, "M", N, "N", K, "K")) return s;
  if (nvfp4_status s = check_products(M, N, K)) return s;
  if (K <= 0 || K % 16 != 0)
    return fail(NVFP4_ERR_SHAPE, "K=%lld is not a positive multiple of 16", (long long)K);
  REQUIRE_ALIGN(x_bf16, 16);
  REQUIRE_ALIGN(w_codes, 16);
  REQUIRE_ALIGN(w_scales, 16);
  REQUIRE_ALIGN(w_gscale, 4);
  REQUIRE_ALIGN(out_bf16, 16);
  REQUIRE_ALIGN(x_codes, 16);
  REQUIRE_ALIGN(x_scales, 16);
  REQUIRE_ALIGN(x_gscale, 4);
  const size_t need = nvfp4_linear_workspace_bytes(M, N, K);
  if (need > 0) {
    REQUIRE_PTR(workspace);
    REQUIRE_ALIGN(workspace, 256);
    if (workspace_bytes < need)
      return fail(NVFP4_ERR_INVALID_ARG, "workspace_bytes=%zu is below nvfp4_linear_workspace_bytes=%zu",
                  workspace_bytes, need);
  }
  const Range outs[5] = {{out_bf16, M * N * 2, "out"},
                         {x_codes, M * K / 2, "x_codes"},
                         {x_scales, M * K / 16, "x_scales"},
                         {x_gscale, 4, "x_gscale"},
                         {workspace, need > 0 ? (int64_t)need : 0, "workspace"}};
  const Range ins[4] = {{x_bf16, M * K * 2, "x"},
                        {w_codes, N * K / 2, "w_codes"},
                        {w_scales, N * K / 16, "w_scales"},
                        {w_gscale, 4, "w_gscale"}};
  if (M == 0) return ok();
  if (nvfp4_status s = check_disjoint(outs, 5, ins, 4)) return s;
  hipStream_t st = (hipStream_t)stream;
  if (N > 0 && nvfp4k::nvfp4_linear_fused_supported(M, K))
    return hip_status(nvfp4k::launch_nvfp4_linear_fused(x_bf16, w_codes, w_scales, w_gscale, out_bf16, M, N, K,
                                                        x_codes, x_scales, x_gscale, st),
                      "nvfp4_linear fused launch");
  nvfp4_status s = hip_status(nvfp4k::launch_nvfp4_quantize(x_bf16, M, K, x_codes, x_scales, x_gscale, 0,
                                                             NVFP4_SCALE_ABSMAX, (uint32_t*)workspace, st),
                              "nvfp4_linear quantize launch");
  if (s != NVFP4_OK || N == 0) return s;
  return gemm_impl(x_codes, x_scales, x_gscale, w_codes, w_scales, w_gscale, out_bf16, M, N, K, NVFP4_ALGO_AUTO,
                   nullptr, nullptr, 0, workspace, workspace_bytes, stream);
}

size_t nvfp4_gemm_amax_slots(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
  if (check_products(M, N, K) != NVFP4_OK) return 0;
  return (size_t)amax_slots(M, N, K);
}

nvfp4_status nvfp4_gemm_amax(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                             const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale, void* out_bf16,
                             int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                             uint32_t* amax_slots, void* stream) {
  REQUIRE_PTR(amax_slots);
  REQUIRE_ALIGN(amax_slots, 4);
  if (N % 16 != 0)
    return fail(NVFP4_ERR_SHAPE, "N=%lld is not a multiple of 16 (the output is quantized along N)", (long long)N);
  return gemm_impl(a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, out_bf16, M, N, K, NVFP4_ALGO_AUTO,
                   nullptr, nullptr, 0, workspace, workspace_bytes, stream, amax_slots);
}

nvfp4_status nvfp4_quantize_amax(const void* x_bf16, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                 float* global_scale, const uint32_t* amax_slots, int64_t nslots, void* stream) {
  REQUIRE_PTR(x_bf16);
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scales);
  REQUIRE_PTR(global_scale);
  REQUIRE_PTR(amax_slots);
  if (nvfp4_status s = check_dims(rows, "rows", cols, "cols", nslots, "nslots")) return s;
  if (nslots < 1 || nslots > (int64_t(1) << 28))
    return fail(NVFP4_ERR_INVALID_ARG, "nslots=%lld is outside [1, 2^28]", (long long)nslots);
  if (cols % 16 != 0) return fail(NVFP4_ERR_SHAPE, "cols=%lld is not a multiple of 16", (long long)cols);
  if (rows > 0 && cols > kMaxElems / rows) return fail(NVFP4_ERR_UNSUPPORTED, "rows*cols exceeds 2^40");
  REQUIRE_ALIGN(x_bf16, 16);
  REQUIRE_ALIGN(codes, 16);
  REQUIRE_ALIGN(scales, 16);
  REQUIRE_ALIGN(global_scale, 4);
  REQUIRE_ALIGN(amax_slots, 4);
  const int64_t n = rows * cols;
  const Range outs[3] = {{codes, n / 2, "codes"}, {scales, n / 16, "scales"}, {global_scale, 4, "global_scale"}};
  const Range ins[2] = {{x_bf16, n * 2, "x"}, {amax_slots, 4 * nslots, "amax_slots"}};
  if (n == 0) return ok();
  if (nvfp4_status s = check_disjoint(outs, 3, ins, 2)) return s;
  return hip_status(nvfp4k::launch_nvfp4_quantize_pass2(x_bf16, rows, cols, codes, scales, global_scale, 0,
                                                        nvfp4k::kRuleAbsmax, (int)nslots,
                                                        const_cast<uint32_t*>(amax_slots), (hipStream_t)stream),
                    "nvfp4_quantize_amax launch");
}

nvfp4_status nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                        const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale, void* out_bf16,
                        int64_t M, int64_t N, int64_t K, void* stream) {
  return nvfp4_gemm_ex(a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, out_bf16, M, N, K,
                       NVFP4_ALGO_AUTO, stream);
}

nvfp4_status nvfp4_gemm_w4a16_ex(const void* x_bf16, const uint8_t* w_codes, const uint8_t* w_scales,
                                 const float* w_gscale, void* out_bf16, int64_t M, int64_t N, int64_t K, int algo,
                                 void* stream) {
  if (nvfp4_status s = check_dims(M, "M", N, "N", K, "K")) return s;
  if (nvfp4_status s = check_products(M, N, K)) return s;
  if (K > 0) {
    REQUIRE_PTR(x_bf16);
    REQUIRE_PTR(w_codes);
    REQUIRE_PTR(w_scales);
  }
  REQUIRE_PTR(w_gscale);
  REQUIRE_PTR(out_bf16);
  if (K % 16 != 0) return fail(NVFP4_ERR_SHAPE, "K=%lld is not a multiple of 16", (long long)K);
  if (algo < NVFP4_ALGO_AUTO || algo > NVFP4_ALGO_SIMPLE) return fail(NVFP4_ERR_INVALID_ARG, "unknown algo %d", algo);
  REQUIRE_ALIGN(x_bf16, 16);
  REQUIRE_ALIGN(w_codes, 16);
  REQUIRE_ALIGN(w_scales, 16);
  REQUIRE_ALIGN(out_bf16, 16);
  REQUIRE_ALIGN(w_gscale, 4);
  const Range outs[1] = {{out_bf16, M * N * 2, "out"}};
  const Range ins[4] = {{x_bf16, M * K * 2, "x"}, {w_codes, N * K / 2, "w_codes"},
                        {w_scales, N * K / 16, "w_scales"}, {w_gscale, 4, "w_gscale"}};
  if (M == 0 || N == 0) return ok();
  if (nvfp4_status s = check_disjoint(outs, 1, ins, 4)) return s;
  const bool decode_ok = nvfp4k::nvfp4_w4a16_decode_supported(M, K);
  // the tiled kernel stages 128 values per step and addresses a tile's rows
  // of x (128 x 2K bytes) with 32-bit buffer offsets
  const bool tiled_ok = K > 0 && K % 128 == 0 && K < kInt4TiledKLimit;
  if (algo == NVFP4_ALGO_AUTO)
    algo = decode_ok ? NVFP4_ALGO_DECODE : (tiled_ok ? NVFP4_ALGO_TILED : NVFP4_ALGO_SIMPLE);
  hipStream_t st = (hipStream_t)stream;
  if (algo == NVFP4_ALGO_TILED) {
    if (!tiled_ok)
      return fail(NVFP4_ERR_UNSUPPORTED, "weight-only tiled kernel needs K %% 128 == 0 and 0 < K < 2^22 (K=%lld)",
                  (long long)K);
    return hip_status(nvfp4k::launch_nvfp4_w4a16_tiled(x_bf16, w_codes, w_scales, w_gscale, out_bf16, M, N, K, st),
                      "nvfp4_gemm_w4a16 tiled launch");
  }
  if (algo == NVFP4_ALGO_DECODE) {
    if (!decode_ok)
      return fail(NVFP4_ERR_UNSUPPORTED, "weight-only decode kernel needs M <= 16, K %% 128 == 0 and K <= 32768 "
                  "(M=%lld, K=%lld)", (long long)M, (long long)K);
    return hip_status(nvfp4k::launch_nvfp4_w4a16_decode(x_bf16, w_codes, w_scales, w_gscale, out_bf16, M, N, K, st),
                      "nvfp4_gemm_w4a16 decode launch");
  }
  return hip_status(nvfp4k::launch_nvfp4_w4a16_simple(x_bf16, w_codes, w_scales, w_gscale, out_bf16, M, N, K, st),
                    "nvfp4_gemm_w4a16 simple launch");
}

nvfp4_status nvfp4_gemm_w4a16(const void* x_bf16, const uint8_t* w_codes, const uint8_t* w_scales,
                              const float* w_gscale, void* out_bf16, int64_t M, int64_t N, int64_t K, void* stream) {
  return nvfp4_gemm_w4a16_ex(x_bf16, w_codes, w_scales, w_gscale, out_bf16, M, N, K, NVFP4_ALGO_AUTO, stream);
}

nvfp4_status int4g_quantize(const void* w_bf16, int64_t N, int64_t K, int64_t group, uint8_t* q, void* scales_fp16,
                            void* stream) {
  REQUIRE_PTR(w_bf16);
  REQUIRE_PTR(q);
  REQUIRE_PTR(scales_fp16);
  if (nvfp4_status s = check_dims(N, "N", K, "K", group, "group")) return s;
  if (group != 128) return fail(NVFP4_ERR_UNSUPPORTED, "group=%lld; only 128 is supported", (long long)group);
  if (K % 128 != 0) return fail(NVFP4_ERR_SHAPE, "K=%lld is not a multiple of the group (128)", (long long)K);
  REQUIRE_ALIGN(w_bf16, 16);
  REQUIRE_ALIGN(q, 16);
  REQUIRE_ALIGN(scales_fp16, 16);
  const Range outs[2] = {{q, N * K / 2, "q"}, {scales_fp16, N * (K / 128) * 2, "scales"}};
  const Range ins[1] = {{w_bf16, N * K * 2, "w"}};
  if (N == 0 || K == 0) return ok();
  if (nvfp4_status s = check_disjoint(outs, 2, ins, 1)) return s;
  return hip_status(nvfp4k::launch_int4g_quantize(w_bf16, N, K, q, scales_fp16, (hipStream_t)stream),
                    "int4g_quantize launch");
}

nvfp4_status int4g_gemv_ex(const void* x_bf16, const uint8_t* q, const void* scales_fp16, void* out_bf16, int64_t M,
                           int64_t N, int64_t K, int64_t group, int algo, void* stream) {
  REQUIRE_PTR(x_bf16);
  REQUIRE_PTR(q);
  REQUIRE_PTR(scales_fp16);
  REQUIRE_PTR(out_bf16);
  if (nvfp4_status s = check_dims(M, "M", N, "N", K, "K")) return s;
  if (nvfp4_status s = check_products(M, N, K)) return s;
  if (group != 128) return fail(NVFP4_ERR_UNSUPPORTED, "group=%lld; only 128 is supported", (long long)group);
  if (K % 128 != 0) return fail(NVFP4_ERR_SHAPE, "K=%lld is not a multiple of the group (128)", (long long)K);
  if (algo < NVFP4_ALGO_AUTO || algo > NVFP4_ALGO_SIMPLE) return fail(NVFP4_ERR_INVALID_ARG, "unknown algo %d", algo);
  REQUIRE_ALIGN(x_bf16, 16);
  REQUIRE_ALIGN(q, 16);
  REQUIRE_ALIGN(scales_fp16, 16);
  REQUIRE_ALIGN(out_bf16, 16);
  const Range outs[1] = {{out_bf16, M * N * 2, "out"}};
  const Range ins[3] = {{x_bf16, M * K * 2, "x"}, {q, N * K / 2, "q"}, {scales_fp16, N * (K / 128) * 2, "scales"}};
  if (M == 0 || N == 0) return ok();
  if (nvfp4_status s = check_disjoint(outs, 1, ins, 3)) return s;
  if (algo == NVFP4_ALGO_AUTO)
    algo = (K == 0) ? NVFP4_ALGO_SIMPLE
                    : (M <= 16 ? (K <= kDecodeMaxK ? NVFP4_ALGO_DECODE : NVFP4_ALGO_SIMPLE)
                               : (K < kInt4TiledKLimit ? NVFP4_ALGO_TILED : NVFP4_ALGO_SIMPLE));
  hipStream_t st = (hipStream_t)stream;
  switch (algo) {
    case NVFP4_ALGO_TILED:
      if (K == 0 || K >= kInt4TiledKLimit)
        return fail(NVFP4_ERR_UNSUPPORTED, "tiled kernel needs 0 < K < 2^22 (K=%lld)", (long long)K);
      return hip_status(nvfp4k::launch_int4g_gemm_tiled(x_bf16, q, scales_fp16, out_bf16, M, N, K, st),
                        "int4g_gemv tiled launch");
    case NVFP4_ALGO_DECODE:
      if (M > 16 || K == 0 || K > kDecodeMaxK)
        return fail(NVFP4_ERR_UNSUPPORTED, "decode kernel needs M <= 16 and 0 < K <= 2^24 (M=%lld, K=%lld)",
                    (long long)M, (long long)K);
      return hip_status(nvfp4k::launch_int4g_gemm_decode(x_bf16, q, scales_fp16, out_bf16, M, N, K, st),
                        "int4g_gemv decode launch");
    default:
      return hip_status(nvfp4k::launch_int4g_gemm_simple(x_bf16, q, scales_fp16, out_bf16, M, N, K, st),
                        "int4g_gemv simple launch");
  }
}

nvfp4_status int4g_gemv(const void* x_bf16, const uint8_t* q, const void* scales_fp16, void* out_bf16, int64_t M,
                        int64_t N, int64_t K, int64_t group, void* stream) {
  return int4g_gemv_ex(x_bf16, q, scales_fp16, out_bf16, M, N, K, group, NVFP4_ALGO_AUTO, stream);
}

nvfp4_status int4g_asym_quantize(const void* w_bf16, int64_t N, int64_t K, int64_t group, uint8_t* q,
                                 void* scales_fp16, uint8_t* zeros, void* stream) {
  REQUIRE_PTR(w_bf16);
  REQUIRE_PTR(q);
  REQUIRE_PTR(scales_fp16);
  REQUIRE_PTR(zeros);
  if (nvfp4_status s = check_dims(N, "N", K, "K", group, "group")) return s;
  if (group != 128) return fail(NVFP4_ERR_UNSUPPORTED, "group=%lld; only 128 is supported", (long long)group);
  if (K % 128 != 0) return fail(NVFP4_ERR_SHAPE, "K=%lld is not a multiple of the group (128)", (long long)K);
  REQUIRE_ALIGN(w_bf16, 16);
  REQUIRE_ALIGN(q, 16);
  REQUIRE_ALIGN(scales_fp16, 16);
  const Range outs[3] = {{q, N * K / 2, "q"}, {scales_fp16, N * (K / 128) * 2, "scales"},
                         {zeros, N * (K / 128), "zeros"}};
  const Range ins[1] = {{w_bf16, N * K * 2, "w"}};
  if (N == 0 || K == 0) return ok();
  if (nvfp4_status s = check_disjoint(outs, 3, ins, 1)) return s;
  return hip_status(nvfp4k::launch_int4g_asym_quantize(w_bf16, N, K, q, scales_fp16, zeros, (hipStream_t)stream),
                    "int4g_asym_quantize launch");
}

nvfp4_status int4g_asym_gemv_ex(const void* x_bf16, const uint8_t* q, const void* scales_fp16, const uint8_t* zeros,
                                void* out_bf16, int64_t M, int64_t N, int64_t K, int64_t group, int algo,
                                void* stream) {
  REQUIRE_PTR(x_bf16);
  REQUIRE_PTR(q);
  REQUIRE_PTR(scales_fp16);
  REQUIRE_PTR(zeros);
  REQUIRE_PTR(out_bf16);
  if (nvfp4_status s = check_dims(M, "M", N, "N", K, "K")) return s;
  if (nvfp4_status s = check_products(M, N, K)) return s;
  if (group != 128) return fail(NVFP4_ERR_UNSUPPORTED, "group=%lld; only 128 is supported", (long long)group);
  if (K % 128 != 0) return fail(NVFP4_ERR_SHAPE, "K=%lld is not a multiple of the group (128)", (long long)K);
  if (algo < NVFP4_ALGO_AUTO || algo > NVFP4_ALGO_SIMPLE) return fail(NVFP4_ERR_INVALID_ARG, "unknown algo %d", algo);
  REQUIRE_ALIGN(x_bf16, 16);
  REQUIRE_ALIGN(q, 16);
  REQUIRE_ALIGN(scales_fp16, 16);
  REQUIRE_ALIGN(out_bf16, 16);
  const Range outs[1] = {{out_bf16, M * N * 2, "out"}};
  const Range ins[4] = {{x_bf16, M * K * 2, "x"}, {q, N * K / 2, "q"}, {scales_fp16, N * (K / 128) * 2, "scales"},
                        {zeros, N * (K / 128), "zeros"}};
  if (M == 0 || N == 0) return ok();
  if (nvfp4_status s = check_disjoint(outs, 1, ins, 4)) return s;
  const bool decode_ok = nvfp4k::int4g_asym_decode_supported(M, K);
  if (algo == NVFP4_ALGO_AUTO)
    algo = decode_ok ? NVFP4_ALGO_DECODE : (K < kInt4TiledKLimit ? NVFP4_ALGO_TILED : NVFP4_ALGO_SIMPLE);
  hipStream_t st = (hipStream_t)stream;
  if (algo == NVFP4_ALGO_TILED) {
    if (K >= kInt4TiledKLimit)
      return fail(NVFP4_ERR_UNSUPPORTED, "tiled kernel needs 0 < K < 2^22 (K=%lld)", (long long)K);
    return hip_status(nvfp4k::launch_int4g_asym_tiled(x_bf16, q, scales_fp16, zeros, out_bf16, M, N, K, st),
                      "int4g_asym_gemv tiled launch");
  }
  if (algo == NVFP4_ALGO_DECODE) {
    if (!decode_ok)
      return fail(NVFP4_ERR_UNSUPPORTED, "asymmetric decode kernel needs M <= 2 and 0 < K <= 32768 (M=%lld, K=%lld)",
                  (long long)M, (long long)K);
    return hip_status(nvfp4k::launch_int4g_asym_decode(x_bf16, q, scales_fp16, zeros, out_bf16, M, N, K, st),
                      "int4g_asym_gemv decode launch");
  }
  return hip_status(nvfp4k::launch_int4g_asym_simple(x_bf16, q, scales_fp16, zeros, out_bf16, M, N, K, st),
                    "int4g_asym_gemv simple launch");
}

nvfp4_status int4g_asym_gemv(const void* x_bf16, const uint8_t* q, const void* scales_fp16, const uint8_t* zeros,
                             void* out_bf16, int64_t M, int64_t N, int64_t K, int64_t group, void* stream) {
  return int4g_asym_gemv_ex(x_bf16, q, scales_fp16, zeros, out_bf16, M, N, K, group, NVFP4_ALGO_AUTO, stream);
}

nvfp4_status nvfp4_quantize_lora(const void* x_bf16, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                 float* global_scale, int use_given_global_scale, const void* lora_down_bf16,
                                 int64_t r, float* lora_t, void* workspace, void* stream) {
  REQUIRE_PTR(x_bf16);
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scales);
  REQUIRE_PTR(global_scale);
  REQUIRE_PTR(lora_down_bf16);
  REQUIRE_PTR(lora_t);
  REQUIRE_PTR(workspace);
  if (nvfp4_status s = check_dims(rows, "rows", cols, "cols", r, "r")) return s;
  if (nvfp4_status s = check_rank(r)) return s;
  if (cols % 16 != 0) return fail(NVFP4_ERR_SHAPE, "cols=%lld is not a multiple of 16", (long long)cols);
  if (rows > 0 && cols > INT64_MAX / 2 / rows) return fail(NVFP4_ERR_UNSUPPORTED, "rows*cols overflows");
  if (r * cols * 2 > (int64_t)INT32_MAX || 16 * cols * 2 > (int64_t)INT32_MAX)
    return fail(NVFP4_ERR_UNSUPPORTED, "r*cols or 16*cols exceeds 2^30 values (r=%lld, cols=%lld)", (long long)r,
                (long long)cols);
  REQUIRE_ALIGN(x_bf16, 16);
  REQUIRE_ALIGN(codes, 16);
  REQUIRE_ALIGN(scales, 16);
  REQUIRE_ALIGN(global_scale, 4);
  REQUIRE_ALIGN(lora_down_bf16, 16);
  REQUIRE_ALIGN(lora_t, 16);
  REQUIRE_ALIGN(workspace, 4);
  const int64_t n = rows * cols;
  const Range outs[4] = {{codes, n / 2, "codes"}, {scales, n / 16, "scales"}, {global_scale, 4, "global_scale"},
                         {lora_t, rows * r * 4, "lora_t"}};
  const Range ins[3] = {{x_bf16, n * 2, "x"}, {lora_down_bf16, r * cols * 2, "lora_down"},
                        {workspace, nvfp4k::lora_workspace_bytes(rows, cols, r), "workspace"}};
  if (rows == 0) return ok();
  if (nvfp4_status s = check_disjoint(outs, 4, ins, 3)) return s;
  return hip_status(nvfp4k::launch_nvfp4_quantize_lora(x_bf16, rows, cols, codes, scales, global_scale,
                                                       use_given_global_scale, lora_down_bf16, r, lora_t,
                                                       (uint32_t*)workspace, (hipStream_t)stream),
                    "nvfp4_quantize_lora launch");
}

nvfp4_status nvfp4_gemm_lora_ex(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                                const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale,
                                const float* lora_t, const void* lora_up_bf16, int64_t r, void* out_bf16, int64_t M,
                                int64_t N, int64_t K, int algo, void* stream) {
  REQUIRE_PTR(lora_t);
  REQUIRE_PTR(lora_up_bf16);
  if (nvfp4_status s = check_dims(M, "M", N, "N", r, "r")) return s;
  if (nvfp4_status s = check_rank(r)) return s;
  if (M * r * 4 > (int64_t)INT32_MAX || N * r * 2 > (int64_t)INT32_MAX)
    return fail(NVFP4_ERR_UNSUPPORTED, "lora_t or lora_up exceeds 2 GiB (M=%lld, N=%lld, r=%lld)", (long long)M,
                (long long)N, (long long)r);
  REQUIRE_ALIGN(lora_t, 16);
  REQUIRE_ALIGN(lora_up_bf16, 16);
  return gemm_impl(a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, out_bf16, M, N, K, algo, lora_t,
                   lora_up_bf16, r, nullptr, 0, stream);
}

nvfp4_status nvfp4_gemm_lora(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                             const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale,
                             const float* lora_t, const void* lora_up_bf16, int64_t r, void* out_bf16, int64_t M,
                             int64_t N, int64_t K, void* stream) {
  return nvfp4_gemm_lora_ex(a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, lora_t, lora_up_bf16, r,
                            out_bf16, M, N, K, NVFP4_ALGO_AUTO, stream);
}

}  // extern "C"
