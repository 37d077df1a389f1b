// C ABI of the library: argument validation (host only, before any HIP call),
// status codes and text, and dispatch to the kernel launchers.
#include <algorithm>
#include <cmath>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "launchers.h"
#include "w4a16.h"

namespace {

thread_local char g_last_error[512];

w4a16_status fail(w4a16_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_last_error[0] = '\0'; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr int64_t kMaxM = int64_t(1) << 16;
constexpr int64_t kMaxT = int64_t(1) << 20;
constexpr int64_t kMaxTiles = (int64_t(1) << 31) - 1;  // one workgroup per loss tile, 1-D grid
// automatic dispatch, from sweeps on MI355X over the LLaMA projection shapes: the GEMV
// kernel at M = 1, and at M = 2 on rows of up to 24576 inputs or where the GEMV takes narrow
// tiles (its batched cross-lane sums keep the doubled dot work under the weight stream:
// 9.3 against 9.8 us at 8192 -> 8192, 20.9 against 29.6 at 22016 -> 8192, 19.3 against 23.1
// at 8192 -> 22016, 7.6 against 8.1 at 4096 -> 11008, 8.4 against 8.8 at 11008 -> 4096, 4.4
// against 4.8 at 4096 -> 4096; on 28672 -> 8192 the small-batch kernel is ahead, 28.9
// against 29.2); the small-batch MFMA kernel up to skinny_max_m(); the tiled MFMA kernel
// beyond
bool auto_gemv(int64_t M, int64_t N, int64_t K) {
  return M == 1 || (M == 2 && (K <= 24576 || w4a16::gemv_narrow(M, N, K)));
}

// NF4 codes and 3-bit codes at M = 1 take the GEMV on every shape. At M = 2 NF4 goes to the
// small-batch kernel: its 16-entry lookups cost the GEMV more than the shared x saves (blocks
// of 64: 8192 -> 8192 14.7 against 12.9 us, 8192 -> 22016 32.6 against 29.4, 8192 -> 28672
// 40.8 against 37.0, 22016 -> 8192 58.0 against 39.6); 3-bit codes have their own M = 2 rule
// below
bool auto_gemv_variant(int64_t M) { return M == 1; }

// 33 <= M <= 64 on layers with N <= 8192 and K <= 16384: the small-batch kernel twice (rows
// 0..31, then the rest) beats the tiled kernel there, for every code format (group 128:
// 14.9-20.9 against 26.0-26.7 us at 4096 -> 4096, 33.1-46.9 against 47.2-49.2 at 8192 -> 8192,
// 34.0-51.2 against 61.8-63.8 at 11008 -> 4096); on wider or longer layers (4096 -> 11008,
// 8192 -> 22016, 22016 -> 8192) the tiled kernel is ahead
bool two_small_batch_passes(int64_t M, int64_t N, int64_t K) {
  return M > w4a16::skinny_max_m() && M <= 2 * w4a16::skinny_max_m() && N <= 8192 && K <= 16384;
}

// From M = 256, 4-bit codes with groups of 128: the one-range split-K kernel (64 x 128 tiles,
// fp16 written directly, no workspace) where its tiles fill the chip's 256 CUs a whole number
// of times or come to at least 1280. Its time follows the rounds of tiles per CU, so a
// partial last round costs it a whole one. From a sweep of M = 128..1024 over nine layer
// shapes (MI355X, graph-timed), one-range / the kernel the rules below pick: 8192 -> 8192 at
// M = 256 64.7 / 68.4 us, M = 512 115.9 / 132.3, M = 1024 228.3 / 259.1; 22016 -> 8192 at
// M = 512 286.3 / 356.4, M = 1024 566.4 / 714.7; 8192 -> 22016 at M = 512 328.6 / 337.6;
// 8192 -> 28672 at M = 768 608.8 / 664.0; 4096 -> 4096 at M = 512 29.6 / 35.2;
// 11008 -> 4096 at M = 512 84.8 / 91.5. With a partial round it loses: 8192 -> 8192 at
// M = 384 (384 tiles) 113.0 / 97.3, 8192 -> 22016 at M = 384 (1032) 268.6 / 263.9,
// 4096 -> 11008 at M = 256 (344) 56.6 / 46.8.
bool auto_one_range(int64_t M, int64_t N) {
  if (M < 256) return false;
  const int64_t tiles = w4a16::splitk_tiles(M, N);
  return tiles % 256 == 0 || tiles >= 1280;
}

// Above the small-batch kernel, 4-bit codes with groups of 128: the K-lane kernel where the
// tiled kernel has at most one workgroup per CU, or where the K-lane grid fills the chip at
// most once (two workgroups per CU, K >= 8192) or 1.5 times (K > 8192); the tiled kernel
// otherwise. From a sweep of M = 33..512 over nine layer shapes (MI355X, graph-timed), K-lane /
// tiled: 4096 -> 4096 at M = 128 16.2 / 24.1 us, 8192 -> 8192 at M = 128 49.3 / 51.2,
// 11008 -> 4096 at M = 256 55.4 / 66.1 and at M = 384 79.8 / 80.7, 22016 -> 8192 at M = 128
// 111.5 / 130.1, 8192 -> 1024 at M = 512 24.7 / 39.4; the tiled kernel keeps 4096 -> 4096
// from M = 192 (25.9 / 26.6), every 4096 -> 11008, 4096 -> 12288 and 8192 -> 22016 shape,
// 8192 -> 8192 from M = 192 (61.6 / 69.2), 11008 -> 4096 at M = 512 (89.4 / 107.6) and
// 22016 -> 8192 at M = 256 (175.6 / 208.1). This also replaces the two small-batch passes
// at M = 33..64 where the tiled grid is short (11008 -> 4096, M = 64: 34.6 against 51.0 us).
bool auto_klane(int64_t M, int64_t N, int64_t K) {
  const int64_t tiled = w4a16::mfma_workgroups(M, N), klane = w4a16::klane_workgroups(M, N);
  return M > w4a16::skinny_max_m() && (tiled <= 256 || (K >= 8192 && klane <= 512) || (K > 8192 && klane <= 768));
}

// 17 <= M <= 32 with K > 16384: the small-batch kernel's two-m-tile variants fall off on
// such long rows (22016 -> 8192: 91 us at M = 24 and 106 at M = 32, against 44.5 at
// M = 16), where the K-lane kernel takes 60-69 us; on 8192 -> 22016 it stays ahead
// (57 / 65 against 73 / 75 us)
bool auto_klane_small(int64_t M, int64_t K) { return M > 16 && M <= w4a16::skinny_max_m() && K > 16384; }

// The automatic path's split-K choice when the caller lends a workspace (4-bit codes, groups
// of 128): the number of K ranges, or 0 for the kernels of w4a16_linear. No split up to
// M = 16. Over K >= 8192: up to M = 32, none on rows of at most 16384 inputs where the
// small-batch kernel's grid fills the chip in whole rounds (below); else the largest S of 8,
// 4, 2 with S * tiles < 1024 (at most 256 on up to 64 tiles) and at least 8 groups per range
// (a single range is left to the automatic path without a workspace, which runs the one-range
// kernel itself where it is ahead). Over 4096 <= K < 8192, from M = 21: two ranges on
// 65..128 tiles, four on at most 48 tiles at M > 32. Tiles are the partial kernel's (32 x 128
// up to M = 32, else 64 x 128). From sweeps of M = 12..512 over nine layer shapes (MI355X,
// graph-timed us, split-K / the automatic path without a workspace): 22016 -> 8192 at M = 17
// 42.1 (S = 4) / 56.8, at M = 32 43.5 / 60.3, at M = 128 90.0 / 109.3; 28672 -> 8192 at
// M = 17 58.5 / 79.1; 11008 -> 4096 at M = 17 15.2 (S = 8) / 16.8, at M = 64 20.2 / 34.1
// and at M = 256 47.9 (S = 4) / 54.0; 8192 -> 22016 at M = 20 49.9 / 53.0; 8192 -> 8192 at
// M = 128 42.3 / 48.0; 8192 -> 1024 at M = 32 11.0 / 14.7; 4096 -> 4096 at M = 256 23.4
// (S = 2) / 26.0; 4096 -> 11008 at M = 32 19.0 / 20.8. On 64 tiles four ranges beat eight
// (8192 -> 8192 at M = 64 25.8 / 28.8). Up to M = 16 the small-batch kernel stays ahead on
// most shapes (8192 -> 8192 at M = 16: 20.8 / 14.5). The rule costs up to 5 % where it
// misjudges (8192 -> 22016 at M = 128: 102.4 / 98.2; 8192 -> 28672 at M = 32: 68.1 with
// four ranges against 65.4 with two).
int auto_splits(int64_t M, int64_t N, int64_t K) {
  if (M <= 16) return 0;
  const int64_t tiles = w4a16::splitk_tiles(M, N), G = K / 128;
  if (K >= 8192) {
    // up to M = 32 on rows of at most 16384 inputs, the small-batch kernel wherever its
    // 32-column workgroups fill the 256 CUs in whole rounds (8192 -> 8192 at M = 21 / 32:
    // 19.4 / 21.1 against 20.8 / 21.4 us with four ranges)
    if (M <= 32 && K <= 16384 && ((N + 31) / 32) % 256 == 0) return 0;
    int s = 8;
    while (s > 1 && (tiles * s >= (tiles <= 64 ? 257 : 1024) || G / s < 8)) s >>= 1;
    return s == 1 ? 0 : s;  // one range: the automatic choice without a workspace covers it
  }
  if (K >= 4096 && M > 20) {
    if (tiles > 64 && tiles <= 128) return 2;
    if (M > 32 && tiles <= 48) return 4;
  }
  return 0;
}

// The x-resident kernel on the automatic path with a workspace (4-bit, groups of 128, scales
// and zeros 4-byte aligned, an even number of groups per row, K > 2048). Up to M = 16 (its
// 64-column workgroups): from M = 4 on layers of at least 2^27 weights, from M = 8 on layers
// of at least 2^25 weights wider than they are long, or where the small-batch kernel's grid is
// at most 64 workgroups on rows of 8192 inputs or more, and from M = 12 on layers of at least
// 2^25 weights. From M = 17 (128-column workgroups) where W = ceil(N / 128) * ceil(K / 2048)
// >= 160. From sweeps of M = 4..32 over nine layer shapes (MI355X, graph-timed us, x-resident /
// the automatic choice before it): 22016 -> 8192 at M = 4 / 16 / 32 23.9 / 27.4 / 36.0 against
// 31.5 / 42.5 / 44.2; 8192 -> 28672 at M = 4 / 16 / 32 27.5 / 33.4 / 41.6 against 30.4 / 50.0 /
// 68.2; 8192 -> 1024 at M = 8 / 16 6.5 / 6.6 against 7.1 / 9.4; 4096 -> 11008 at M = 8 / 32
// 10.3 / 14.4 against 11.6 / 19.1; 11008 -> 4096 at M = 12 / 32 12.3 / 15.4 against 13.5 /
// 17.2; 8192 -> 8192 at M = 12 / 16 / 32 12.6 / 12.9 / 15.5 against 14.0 / 14.6 / 21.1. It
// loses on 4096 -> 4096 at every M (7.1 against 6.0 at M = 16), below the thresholds above
// (8192 -> 8192 at M = 8: 12.3 against 12.1; 4096 -> 11008 at M = 4: 9.8 against 8.6) and from
// M = 20 on 8192 -> 1024 (13.3 against 12.6).
bool auto_xres(int64_t M, int64_t N, int64_t K) {
  // K > 2048: the kernel then takes its workspace (one range needs none and is not measured here)
  if (M < 4 || K <= 2048 || !w4a16::xres_supports(M, K)) return false;
  if (M <= 16) {
    const int64_t w = N * K;
    if (w >= (int64_t(1) << 27)) return true;
    if (M >= 8 && ((N > K && w >= (int64_t(1) << 25)) || ((N + 31) / 32 <= 64 && K >= 8192))) return true;
    return M >= 12 && w >= (int64_t(1) << 25);
  }
  const int64_t W = ((N + 127) / 128) * ((K / 128 + 15) / 16);  // eight-wave 128-column workgroups
  return W >= 160;
}

// float32 workspace the automatic path may use (groups of 128): the larger of the two
// kernels' needs where both may run (the x-resident kernel falls back to the split-K choice
// when scales or zeros are not 4-byte aligned)
int64_t ws_floats(int64_t M, int64_t N, int64_t K) {
  int64_t f = 0;
  const int s = auto_splits(M, N, K);
  if (s > 0) f = w4a16::splitk_workspace_floats(M, N, s);
  if (auto_xres(M, N, K)) f = std::max(f, w4a16::xres_workspace_floats(M, N, K));
  return f;
}

w4a16_status hip_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(W4A16_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return W4A16_OK;
}

w4a16_status check_linear(const void* x, const void* qweight, const void* scales, const void* zeros, int64_t M,
                          int64_t N, int64_t K, int32_t group, const void* y) {
  if (!x || !qweight || !scales || !zeros || !y) return fail(W4A16_ERR_NULL, "x, qweight, scales, zeros and y are required");
  if (group != 128 && group != 64 && group != 32)
    return fail(W4A16_ERR_UNSUPPORTED, "group must be 32, 64 or 128 (got %d)", (int)group);
  if (M <= 0 || N <= 0 || K <= 0) return fail(W4A16_ERR_SHAPE, "M, N, K must be positive (got %lld, %lld, %lld)",
                                              (long long)M, (long long)N, (long long)K);
  if (K % 128 != 0) return fail(W4A16_ERR_SHAPE, "K must be a multiple of 128 (got %lld)", (long long)K);
  if (K > W4A16_MAX_K || N > kMaxN || M > kMaxM)
    return fail(W4A16_ERR_SHAPE, "size beyond the limits (M <= 65536, N <= 2^24, K <= %d)", W4A16_MAX_K);
  if (!aligned(x, 16) || !aligned(qweight, 16)) return fail(W4A16_ERR_ALIGN, "x and qweight must be 16-byte aligned");
  if (!aligned(scales, 2) || !aligned(zeros, 2) || !aligned(y, 2))
    return fail(W4A16_ERR_ALIGN, "scales, zeros and y must be 2-byte aligned");
  return W4A16_OK;
}

// The NF4 codebook ("Quantization for LLMs", chapter 11, section 11.5): 8 positive
// levels at the standard normal quantiles of OFFSET - i (OFFSET - 1/2) / 8 (i = 0..7),
// 7 negative levels mirrored from OFFSET - i (OFFSET - 1/2) / 7 (i = 0..6), and 0, all
// divided by the largest; OFFSET = 0.9677083. The quantiles come from bisection on
// the normal CDF 1/2 erfc(-x / sqrt 2) to double precision; each level is then
// rounded once to fp16. Built once per process (thread-safe static init).
double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double normal_quantile_upper(double p) {  // p in (1/2, 1)
  double lo = 0.0, hi = 40.0;
  for (int i = 0; i < 400 && lo < hi; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (normal_cdf(mid) < p)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

const w4a16::Nf4Table& nf4_table() {
  static const w4a16::Nf4Table table = [] {
    constexpr double kOffset = 0.9677083;
    const double span = kOffset - 0.5;
    const double top = normal_quantile_upper(kOffset);
    double levels[16];
    for (int i = 0; i < 7; ++i) levels[i] = -normal_quantile_upper(kOffset - i * span / 7.0) / top;
    levels[7] = 0.0;
    for (int i = 0; i < 8; ++i) levels[15 - i] = normal_quantile_upper(kOffset - i * span / 8.0) / top;
    w4a16::Nf4Table t;
    for (int i = 0; i < 8; ++i)
      t.pairs[i] = (uint32_t)w4a16::f64_to_f16_rne(levels[2 * i]) |
                   ((uint32_t)w4a16::f64_to_f16_rne(levels[2 * i + 1]) << 16);
    return t;
  }();
  return table;
}

w4a16_status check_nf4_linear(const void* x, const void* qweight, const void* absmax, int64_t M, int64_t N, int64_t K,
                              int32_t block, const void* y) {
  if (!x || !qweight || !absmax || !y) return fail(W4A16_ERR_NULL, "x, qweight, absmax and y are required");
  if (block != 64 && block != 32 && block != 128)
    return fail(W4A16_ERR_UNSUPPORTED, "block must be 32, 64 or 128 (got %d)", (int)block);
  if (M <= 0 || N <= 0 || K <= 0) return fail(W4A16_ERR_SHAPE, "M, N, K must be positive (got %lld, %lld, %lld)",
                                              (long long)M, (long long)N, (long long)K);
  if (K % 128 != 0) return fail(W4A16_ERR_SHAPE, "K must be a multiple of 128 (got %lld)", (long long)K);
  if (K > W4A16_MAX_K || N > kMaxN || M > kMaxM)
    return fail(W4A16_ERR_SHAPE, "size beyond the limits (M <= 65536, N <= 2^24, K <= %d)", W4A16_MAX_K);
  if (!aligned(x, 16) || !aligned(qweight, 16)) return fail(W4A16_ERR_ALIGN, "x and qweight must be 16-byte aligned");
  if (!aligned(absmax, 4) || !aligned(y, 2)) return fail(W4A16_ERR_ALIGN, "absmax must be 4-byte and y 2-byte aligned");
  return W4A16_OK;
}

// bits 4 with group 128 runs the tuned kernels; every other format the variant kernels
w4a16_status run_linear(int32_t bits, int32_t path, const void* x, const void* qweight, const void* scales,
                        const void* zeros, int64_t M, int64_t N, int64_t K, int32_t group, void* y,
                        hipStream_t stream) {
  const uint16_t* xh = static_cast<const uint16_t*>(x);
  const uint32_t* qw = static_cast<const uint32_t*>(qweight);
  const uint16_t* sc = static_cast<const uint16_t*>(scales);
  const uint16_t* zr = static_cast<const uint16_t*>(zeros);
  uint16_t* yh = static_cast<uint16_t*>(y);
  if (bits != 4 || group != 128) {
    const bool gemv_ok = w4a16::gemv_format_supports(bits, group, M, N, K);
    // the small-batch kernel loads a row's scales (zeros) of 128 inputs in one 2-, 4- or 8-byte load
    const uintptr_t sz_align = group == 128 ? 2 : 4;
    const bool sz_aligned = aligned(scales, sz_align) && aligned(zeros, sz_align);
    const bool skinny_ok = M <= w4a16::skinny_max_m() && sz_aligned;
    bool two_passes = false;
    int32_t kernel = path;
    if (path == 0) {
      // 4-bit groups of 64 and 32 run the tuned GEMV, which at M = 2 is ahead on every LLaMA
      // shape measured, rows of up to 28672 inputs (8192 -> 8192: 9.5 against 11.0 us for 64,
      // 10.0 against 12.4 for 32; 28672 -> 8192: 30.0 against 31.9, 31.1 against 33.8;
      // 4096 -> 4096: 4.5 against 4.9, 4.8 against 5.2). 3-bit codes keep the GEMV variant at
      // M = 2 where rows are no longer than the layer is wide (its dequant VALU is shared by
      // both rows: 8192 -> 8192 11.2 against 12.5 us, 8192 -> 22016 24.6 against 28.0,
      // 4096 -> 11008 10.8 against 11.0) except on square layers below 2^26 weights
      // (4096 -> 4096: 6.9 against 5.9), and leave longer rows to the small-batch kernel
      // (11008 -> 4096: 11.3 against 10.5, 22016 -> 8192: 38.6 against 32.6)
      const bool gemv_first =
          bits == 4 ? M == 1 || (M == 2 && K <= 32768)
                    : auto_gemv_variant(M) ||
                          (bits == 3 && M == 2 && (K < N || (K == N && N * K >= (int64_t(1) << 26))));
      two_passes = sz_aligned && two_small_batch_passes(M, N, K);
      kernel = gemv_first && gemv_ok ? 1 : skinny_ok || two_passes ? 3 : gemv_ok ? 1 : 2;
    } else if (path == 1 && !gemv_ok) {
      return fail(W4A16_ERR_UNSUPPORTED, "the GEMV kernels for this format take M <= %d and K <= 32768 "
                  "(M <= 4 above K = 16384), or for 4-bit codes M * ceil(K / 16384) <= 8; got M=%lld K=%lld",
                  w4a16::gemv_max_m(), (long long)M, (long long)K);
    } else if (path == 3) {
      if (M > w4a16::skinny_max_m())
        return fail(W4A16_ERR_UNSUPPORTED, "the small-batch MFMA kernel takes M <= %d; got M=%lld",
                    w4a16::skinny_max_m(), (long long)M);
      if (!skinny_ok)
        return fail(W4A16_ERR_ALIGN, "the small-batch MFMA kernel needs scales and zeros 4-byte aligned "
                    "for groups of 32 and 64");
    }
    if (kernel == 1)
      return hip_result(w4a16::launch_gemv_variant(bits, group, xh, qw, sc, zr, M, N, K, yh, stream), "GEMV launch");
    if (kernel == 3 && two_passes) {
      const int64_t m1 = w4a16::skinny_max_m();
      hipError_t e = w4a16::launch_skinny_variant(bits, group, xh, qw, sc, zr, m1, N, K, yh, stream);
      if (e == hipSuccess)
        e = w4a16::launch_skinny_variant(bits, group, xh + m1 * K, qw, sc, zr, M - m1, N, K, yh + m1 * N, stream);
      return hip_result(e, "small-batch MFMA launch");
    }
    if (kernel == 3)
      return hip_result(w4a16::launch_skinny_variant(bits, group, xh, qw, sc, zr, M, N, K, yh, stream),
                        "small-batch MFMA launch");
    return hip_result(w4a16::launch_mfma_variant(bits, group, xh, qw, sc, zr, M, N, K, yh, stream), "MFMA launch");
  }
  int32_t kernel = path;
  bool two_passes = false;
  if (path == 0) {
    if (auto_gemv(M, N, K) && w4a16::gemv_supports(M, K)) {
      kernel = 1;
    } else if (auto_one_range(M, N)) {
      kernel = 5;
    } else if (auto_klane_small(M, K)) {
      kernel = 4;
    } else if (M <= w4a16::skinny_max_m()) {
      kernel = 3;
    } else if (auto_klane(M, N, K)) {
      kernel = 4;
    } else if (two_small_batch_passes(M, N, K)) {
      kernel = 3;
      two_passes = true;
    } else {
      kernel = 2;
    }
  } else if (path == 1 && !w4a16::gemv_supports(M, K)) {
    return fail(W4A16_ERR_UNSUPPORTED, "the GEMV kernel takes M <= %d (M * ceil(K / 16384) <= 8); got M=%lld K=%lld",
                w4a16::gemv_max_m(), (long long)M, (long long)K);
  } else if (path == 3 && M > w4a16::skinny_max_m()) {
    return fail(W4A16_ERR_UNSUPPORTED, "the small-batch MFMA kernel takes M <= %d; got M=%lld",
                w4a16::skinny_max_m(), (long long)M);
  }
  if (kernel == 1) return hip_result(w4a16::launch_gemv(xh, qw, sc, zr, M, N, K, yh, stream), "GEMV launch");
  if (kernel == 3 && two_passes) {
    const int64_t m1 = w4a16::skinny_max_m();
    hipError_t e = w4a16::launch_skinny(xh, qw, sc, zr, m1, N, K, yh, stream);
    if (e == hipSuccess) e = w4a16::launch_skinny(xh + m1 * K, qw, sc, zr, M - m1, N, K, yh + m1 * N, stream);
    return hip_result(e, "small-batch MFMA launch");
  }
  if (kernel == 3)
    return hip_result(w4a16::launch_skinny(xh, qw, sc, zr, M, N, K, yh, stream), "small-batch MFMA launch");
  if (kernel == 4) return hip_result(w4a16::launch_klane(xh, qw, sc, zr, M, N, K, yh, stream), "K-lane MFMA launch");
  if (kernel == 5)
    return hip_result(w4a16::launch_splitk(xh, qw, sc, zr, M, N, K, 1, nullptr, yh, stream), "one-range MFMA launch");
  return hip_result(w4a16::launch_mfma(xh, qw, sc, zr, M, N, K, yh, stream), "MFMA launch");
}

}  // namespace

namespace {

// awq_search_alpha's workspace, each region 256-byte aligned: y_ref float32 [T][N], the 21
// candidate scales float32 [21][K], x_s fp16 [T][K], qweight u32 [N][K/8], scales and zeros
// fp16 [N][K/128], and the loss partials float64 [awq_alpha_loss_workspace(T, N)]
struct SearchSpace {
  int64_t y_ref, s_all, x_s, qweight, scales, zeros, partials, total;
};

int64_t round256(int64_t b) { return (b + 255) & ~int64_t(255); }

bool search_space(int64_t T, int64_t N, int64_t K, SearchSpace* sp) {
  if (T <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || T > kMaxM || N > kMaxN || K > W4A16_MAX_K) return false;
  const int64_t parts = awq_alpha_loss_workspace(T, N);
  if (parts < 0) return false;
  int64_t at = 0;
  auto take = [&](int64_t bytes) {
    const int64_t here = at;
    at += round256(bytes);
    return here;
  };
  sp->y_ref = take(T * N * 4);
  sp->s_all = take(int64_t(W4A16_ALPHA_GRID_POINTS) * K * 4);
  sp->x_s = take(T * K * 2);
  sp->qweight = take(N * K / 2);
  sp->scales = take(N * (K / 128) * 2);
  sp->zeros = take(N * (K / 128) * 2);
  sp->partials = take(parts * 8);
  sp->total = at;
  return true;
}

}  // namespace

extern "C" {

int32_t w4a16_layout_version(void) { return 1; }

const char* w4a16_status_str(int32_t status) {
  switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_NULL: return "null pointer";
    case W4A16_ERR_SHAPE: return "bad shape";
    case W4A16_ERR_UNSUPPORTED: return "unsupported configuration";
    case W4A16_ERR_ALIGN: return "misaligned pointer";
    case W4A16_ERR_HIP: return "HIP runtime error";
    case W4A16_ERR_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

const char* w4a16_last_error(void) { return g_last_error; }

int32_t w4a16_gemv_max_m(void) { return w4a16::gemv_max_m(); }

int64_t w4a16_stream_read_sink_bytes(int64_t bytes) {
  if (bytes <= 0 || bytes % 16 != 0) return -1;
  return w4a16::stream_read_blocks(bytes) * 4;
}

w4a16_status w4a16_stream_read(const void* buf, int64_t bytes, void* sink, void* stream) {
  if (!buf || !sink) return fail(W4A16_ERR_NULL, "buf and sink are required");
  if (bytes <= 0 || bytes % 16 != 0) return fail(W4A16_ERR_SHAPE, "bytes must be positive and a multiple of 16");
  if (w4a16::stream_read_blocks(bytes) > (int64_t(1) << 31) - 1) return fail(W4A16_ERR_SHAPE, "bytes beyond the limit");
  if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(W4A16_ERR_ALIGN, "buf must be 16-byte and sink 4-byte aligned");
  return hip_result(w4a16::launch_stream_read(buf, bytes, static_cast<uint32_t*>(sink),
                                              static_cast<hipStream_t>(stream)),
                    "stream read launch");
}

w4a16_status w4a16_stream_read_grid(const void* buf, int64_t bytes, int32_t threads, int32_t blocks, int32_t unroll,
                                    void* sink, void* stream) {
  clear_error();
  if (!buf || !sink) return fail(W4A16_ERR_NULL, "buf and sink are required");
  if (bytes <= 0 || bytes % 16 != 0) return fail(W4A16_ERR_SHAPE, "bytes must be positive and a multiple of 16");
  if (bytes / 16 > (int64_t(1) << 40)) return fail(W4A16_ERR_SHAPE, "bytes beyond the limit");
  if (threads != 64 && threads != 128 && threads != 256 && threads != 512 && threads != 1024)
    return fail(W4A16_ERR_ARG, "threads must be 64, 128, 256, 512 or 1024 (got %d)", (int)threads);
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8 && unroll != 16)
    return fail(W4A16_ERR_ARG, "unroll must be 1, 2, 4, 8 or 16 (got %d)", (int)unroll);
  if (blocks <= 0 || blocks > (1 << 20)) return fail(W4A16_ERR_ARG, "blocks must lie in [1, 2^20] (got %d)", (int)blocks);
  if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(W4A16_ERR_ALIGN, "buf must be 16-byte and sink 4-byte aligned");
  return hip_result(w4a16::launch_stream_read_grid(buf, bytes, threads, blocks, unroll, static_cast<uint32_t*>(sink),
                                                   static_cast<hipStream_t>(stream)),
                    "grid-stride read launch");
}

w4a16_status awq_channel_scale(const void* x_cal, int64_t T, int64_t K, double alpha, float* s, void* stream) {
  clear_error();
  if (!x_cal || !s) return fail(W4A16_ERR_NULL, "x_cal and s are required");
  if (T <= 0 || K <= 0) return fail(W4A16_ERR_SHAPE, "T and K must be positive");
  if (T > kMaxT || K > W4A16_MAX_K) return fail(W4A16_ERR_SHAPE, "size beyond the limits (T <= 2^20, K <= %d)", W4A16_MAX_K);
  if (!(alpha >= 0.0 && alpha <= 1.0)) return fail(W4A16_ERR_ARG, "alpha must lie in [0, 1]");
  if (!aligned(x_cal, 2) || !aligned(s, 4)) return fail(W4A16_ERR_ALIGN, "x_cal must be 2-byte and s 4-byte aligned");
  return hip_result(w4a16::launch_channel_scale(static_cast<const uint16_t*>(x_cal), T, K, alpha, s,
                                                static_cast<hipStream_t>(stream)),
                    "channel-scale launch");
}

w4a16_status awq_scale_input(const void* x, const float* s, int64_t M, int64_t K, void* x_s, void* stream) {
  clear_error();
  if (!x || !s || !x_s) return fail(W4A16_ERR_NULL, "x, s and x_s are required");
  if (M <= 0 || K <= 0) return fail(W4A16_ERR_SHAPE, "M and K must be positive");
  if (M > kMaxM || K > W4A16_MAX_K) return fail(W4A16_ERR_SHAPE, "size beyond the limits (M <= 65536, K <= %d)", W4A16_MAX_K);
  if (!aligned(x, 2) || !aligned(x_s, 2) || !aligned(s, 4))
    return fail(W4A16_ERR_ALIGN, "x and x_s must be 2-byte and s 4-byte aligned");
  return hip_result(w4a16::launch_scale_input(static_cast<const uint16_t*>(x), s, M, K, static_cast<uint16_t*>(x_s),
                                              static_cast<hipStream_t>(stream)),
                    "scale-input launch");
}

w4a16_status awq_rmsnorm_fold(const void* h, const void* gamma, const float* s, int64_t M, int64_t K, double eps,
                              void* x_s, void* stream) {
  clear_error();
  if (!h || !gamma || !x_s) return fail(W4A16_ERR_NULL, "h, gamma and x_s are required");
  if (M <= 0 || K <= 0 || K % 8 != 0) return fail(W4A16_ERR_SHAPE, "M, K must be positive and K a multiple of 8");
  if (M > kMaxT || K > W4A16_MAX_K) return fail(W4A16_ERR_SHAPE, "size beyond the limits (M <= 2^20, K <= %d)", W4A16_MAX_K);
  if (!(eps > 0.0) || !std::isfinite(eps)) return fail(W4A16_ERR_ARG, "eps must be finite and positive");
  if (!aligned(h, 16) || !aligned(x_s, 16) || !aligned(gamma, 2) || (s && !aligned(s, 4)))
    return fail(W4A16_ERR_ALIGN, "h and x_s must be 16-byte, gamma 2-byte and s 4-byte aligned");
  return hip_result(w4a16::launch_rmsnorm_fold(static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(gamma), s,
                                               M, K, eps, static_cast<uint16_t*>(x_s), static_cast<hipStream_t>(stream)),
                    "RMSNorm-fold launch");
}

w4a16_status awq_quantize_pack(const void* w, const float* s, int64_t N, int64_t K, int32_t bits, int32_t group,
                               void* qweight, void* scales, void* zeros, void* stream) {
  clear_error();
  if (!w || !qweight || !scales || !zeros) return fail(W4A16_ERR_NULL, "w, qweight, scales and zeros are required");
  if ((bits != 4 && bits != 3) || (group != 128 && group != 64 && group != 32))
    return fail(W4A16_ERR_UNSUPPORTED, "bits must be 3 or 4 and group 32, 64 or 128 (got bits=%d, group=%d)",
                (int)bits, (int)group);
  if (N <= 0 || K <= 0) return fail(W4A16_ERR_SHAPE, "N and K must be positive");
  if (K % group != 0) return fail(W4A16_ERR_SHAPE, "K must be a multiple of the group (got K=%lld, group=%d)",
                                  (long long)K, (int)group);
  if (K > W4A16_MAX_K || N > kMaxN) return fail(W4A16_ERR_SHAPE, "size beyond the limits (N <= 2^24, K <= %d)", W4A16_MAX_K);
  if (!aligned(w, 16) || !aligned(qweight, 16) || (s && !aligned(s, 16)))
    return fail(W4A16_ERR_ALIGN, "w, qweight and s must be 16-byte aligned");
  if (!aligned(scales, 2) || !aligned(zeros, 2)) return fail(W4A16_ERR_ALIGN, "scales and zeros must be 2-byte aligned");
  return hip_result(w4a16::launch_quantize_pack(static_cast<const uint16_t*>(w), s, N, K, bits, group,
                                                static_cast<uint32_t*>(qweight), static_cast<uint16_t*>(scales),
                                                static_cast<uint16_t*>(zeros), static_cast<hipStream_t>(stream)),
                    "quantize-pack launch");
}

w4a16_status w4a16_linear(const void* x, const void* qweight, const void* scales, const void* zeros, int64_t M,
                          int64_t N, int64_t K, int32_t group, void* y, void* stream) {
  clear_error();
  const w4a16_status st = check_linear(x, qweight, scales, zeros, M, N, K, group, y);
  if (st != W4A16_OK) return st;
  return run_linear(4, 0, x, qweight, scales, zeros, M, N, K, group, y, static_cast<hipStream_t>(stream));
}

int64_t w4a16_linear_workspace(int64_t M, int64_t N, int64_t K, int32_t group) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || M > kMaxM || N > kMaxN || K > W4A16_MAX_K) return -1;
  if (group != 128 && group != 64 && group != 32) return -1;
  if (group == 64) return auto_xres(M, N, K) ? w4a16::xres_workspace_floats(M, N, K) * 4 : 0;
  return group == 128 ? ws_floats(M, N, K) * 4 : 0;
}

w4a16_status w4a16_linear_ws(const void* x, const void* qweight, const void* scales, const void* zeros, int64_t M,
                             int64_t N, int64_t K, int32_t group, void* workspace, int64_t workspace_bytes, void* y,
                             void* stream) {
  clear_error();
  const w4a16_status st = check_linear(x, qweight, scales, zeros, M, N, K, group, y);
  if (st != W4A16_OK) return st;
  // groups of 64 take the x-resident kernel on the same shapes (measured ahead of the small-batch
  // kernel on each of them: 22016 -> 8192 at M = 16 44.4 -> 28.2 us, 8192 -> 28672 at M = 32
  // 79.8 -> 46.1, 8192 x 8192 at M = 32 21.9 -> 17.0) and behind it on the others tried
  if ((group == 128 || group == 64) && workspace && auto_xres(M, N, K) && aligned(scales, 4) && aligned(zeros, 4)) {
    const int64_t need = w4a16::xres_workspace_floats(M, N, K) * 4;
    if (workspace_bytes < need)
      return fail(W4A16_ERR_ARG, "workspace holds %lld bytes, %lld needed", (long long)workspace_bytes, (long long)need);
    if (!aligned(workspace, 16)) return fail(W4A16_ERR_ALIGN, "workspace must be 16-byte aligned");
    return hip_result(w4a16::launch_xres(group, static_cast<const uint16_t*>(x), static_cast<const uint32_t*>(qweight),
                                         static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), M,
                                         N, K, static_cast<float*>(workspace), static_cast<uint16_t*>(y),
                                         static_cast<hipStream_t>(stream)),
                      "x-resident MFMA launch");
  }
  const int s = (group == 128 && workspace) ? auto_splits(M, N, K) : 0;
  if (s > 0) {
    const int64_t need = w4a16::splitk_workspace_floats(M, N, s) * 4;
    if (workspace_bytes < need)
      return fail(W4A16_ERR_ARG, "workspace holds %lld bytes, %lld needed", (long long)workspace_bytes, (long long)need);
    if (!aligned(workspace, 16)) return fail(W4A16_ERR_ALIGN, "workspace must be 16-byte aligned");
    return hip_result(w4a16::launch_splitk(static_cast<const uint16_t*>(x), static_cast<const uint32_t*>(qweight),
                                           static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros),
                                           M, N, K, s, static_cast<float*>(workspace), static_cast<uint16_t*>(y),
                                           static_cast<hipStream_t>(stream)),
                      "split-K launch");
  }
  return run_linear(4, 0, x, qweight, scales, zeros, M, N, K, group, y, static_cast<hipStream_t>(stream));
}

int32_t w4a16_linear_ws_splits(int64_t M, int64_t N, int64_t K, int32_t group) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || M > kMaxM || N > kMaxN || K > W4A16_MAX_K) return -1;
  if (group != 128 && group != 64 && group != 32) return -1;
  return group == 128 ? auto_splits(M, N, K) : 0;
}

int32_t w4a16_linear_ws_kernel(int64_t M, int64_t N, int64_t K, int32_t group) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || M > kMaxM || N > kMaxN || K > W4A16_MAX_K) return -1;
  if (group != 128 && group != 64 && group != 32) return -1;
  if (group != 128) return group == 64 && auto_xres(M, N, K) ? 2 : 0;
  if (auto_xres(M, N, K)) return 2;
  return auto_splits(M, N, K) > 0 ? 1 : 0;
}

w4a16_status w4a16_linear_path(int32_t path, const void* x, const void* qweight, const void* scales,
                               const void* zeros, int64_t M, int64_t N, int64_t K, int32_t group, void* y,
                               void* stream) {
  clear_error();
  if (path < 0 || path > 5)
    return fail(W4A16_ERR_UNSUPPORTED, "path must be 0 (auto), 1 (GEMV), 2 (tiled MFMA), 3 (small-batch MFMA), "
                "4 (K-lane MFMA) or 5 (one-range split-K MFMA)");
  if ((path == 4 || path == 5) && group != 128)
    return fail(W4A16_ERR_UNSUPPORTED, "the K-lane and one-range MFMA kernels take groups of 128 (got %d)", (int)group);
  const w4a16_status st = check_linear(x, qweight, scales, zeros, M, N, K, group, y);
  if (st != W4A16_OK) return st;
  return run_linear(4, path, x, qweight, scales, zeros, M, N, K, group, y, static_cast<hipStream_t>(stream));
}

w4a16_status w3a16_linear(const void* x, const void* qweight, const void* scales, const void* zeros, int64_t M,
                          int64_t N, int64_t K, int32_t group, void* y, void* stream) {
  clear_error();
  const w4a16_status st = check_linear(x, qweight, scales, zeros, M, N, K, group, y);
  if (st != W4A16_OK) return st;
  return run_linear(3, 0, x, qweight, scales, zeros, M, N, K, group, y, static_cast<hipStream_t>(stream));
}

w4a16_status w3a16_linear_path(int32_t path, const void* x, const void* qweight, const void* scales,
                               const void* zeros, int64_t M, int64_t N, int64_t K, int32_t group, void* y,
                               void* stream) {
  clear_error();
  if (path < 0 || path > 3)
    return fail(W4A16_ERR_UNSUPPORTED, "path must be 0 (auto), 1 (GEMV), 2 (tiled MFMA) or 3 (small-batch MFMA)");
  const w4a16_status st = check_linear(x, qweight, scales, zeros, M, N, K, group, y);
  if (st != W4A16_OK) return st;
  return run_linear(3, path, x, qweight, scales, zeros, M, N, K, group, y, static_cast<hipStream_t>(stream));
}

int64_t w4a16_linear_splitk_workspace(int64_t M, int64_t N, int64_t K, int32_t splits) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || M > kMaxM || N > kMaxN || K > W4A16_MAX_K) return -1;
  if (splits < 0 || splits > w4a16::splitk_max_splits()) return -1;
  int s = splits == 0 ? w4a16::splitk_default_splits(M, N, K) : splits;
  if (s > K / 128) return -1;
  return w4a16::splitk_workspace_floats(M, N, s) * 4;
}

w4a16_status w4a16_linear_splitk(const void* x, const void* qweight, const void* scales, const void* zeros, int64_t M,
                                 int64_t N, int64_t K, int32_t group, int32_t splits, void* workspace,
                                 int64_t workspace_bytes, void* y, void* stream) {
  clear_error();
  const w4a16_status st = check_linear(x, qweight, scales, zeros, M, N, K, group, y);
  if (st != W4A16_OK) return st;
  if (group != 128) return fail(W4A16_ERR_UNSUPPORTED, "the split-K kernel takes groups of 128 (got %d)", (int)group);
  if (!workspace) return fail(W4A16_ERR_NULL, "workspace is required");
  if (splits < 0 || splits > w4a16::splitk_max_splits() || splits > K / 128)
    return fail(W4A16_ERR_ARG, "splits must lie in [0, min(%d, K/128)] (got %d)", w4a16::splitk_max_splits(), (int)splits);
  const int s = splits == 0 ? w4a16::splitk_default_splits(M, N, K) : splits;
  const int64_t need = w4a16::splitk_workspace_floats(M, N, s) * 4;
  if (workspace_bytes < need)
    return fail(W4A16_ERR_ARG, "workspace holds %lld bytes, %lld needed", (long long)workspace_bytes, (long long)need);
  if (!aligned(workspace, 16)) return fail(W4A16_ERR_ALIGN, "workspace must be 16-byte aligned");
  return hip_result(w4a16::launch_splitk(static_cast<const uint16_t*>(x), static_cast<const uint32_t*>(qweight),
                                         static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), M,
                                         N, K, s, static_cast<float*>(workspace), static_cast<uint16_t*>(y),
                                         static_cast<hipStream_t>(stream)),
                    "split-K launch");
}

int64_t w4a16_linear_xres_workspace(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || M > kMaxM || N > kMaxN || K > W4A16_MAX_K) return -1;
  if (!w4a16::xres_supports(M, K)) return -1;
  return w4a16::xres_workspace_floats(M, N, K) * 4;
}

w4a16_status w4a16_linear_xres(const void* x, const void* qweight, const void* scales, const void* zeros, int64_t M,
                               int64_t N, int64_t K, int32_t group, void* workspace, int64_t workspace_bytes, void* y,
                               void* stream) {
  clear_error();
  const w4a16_status st = check_linear(x, qweight, scales, zeros, M, N, K, group, y);
  if (st != W4A16_OK) return st;
  if (group != 128 && group != 64)
    return fail(W4A16_ERR_UNSUPPORTED, "the x-resident kernel takes groups of 128 or 64 (got %d)", (int)group);
  if (!w4a16::xres_supports(M, K))
    return fail(W4A16_ERR_UNSUPPORTED, "the x-resident kernel takes M <= %d and an even number of groups per row "
                "(got M=%lld K=%lld)", w4a16::xres_max_m(), (long long)M, (long long)K);
  if (!aligned(scales, 4) || !aligned(zeros, 4))
    return fail(W4A16_ERR_ALIGN, "the x-resident kernel needs scales and zeros 4-byte aligned");
  const int64_t need = w4a16::xres_workspace_floats(M, N, K) * 4;
  if (need > 0) {
    if (!workspace) return fail(W4A16_ERR_NULL, "a workspace of %lld bytes is required", (long long)need);
    if (workspace_bytes < need)
      return fail(W4A16_ERR_ARG, "workspace holds %lld bytes, %lld needed", (long long)workspace_bytes, (long long)need);
    if (!aligned(workspace, 16)) return fail(W4A16_ERR_ALIGN, "workspace must be 16-byte aligned");
  }
  return hip_result(w4a16::launch_xres(group, static_cast<const uint16_t*>(x), static_cast<const uint32_t*>(qweight),
                                       static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), M, N,
                                       K, static_cast<float*>(workspace), static_cast<uint16_t*>(y),
                                       static_cast<hipStream_t>(stream)),
                    "x-resident MFMA launch");
}

w4a16_status w4a16_linear_splitk_noalloc(const void* x, const void* qweight, const void* scales, const void* zeros,
                                         int64_t M, int64_t N, int64_t K, int32_t group, int32_t splits, void* y,
                                         void* stream) {
  clear_error();
  const w4a16_status st = check_linear(x, qweight, scales, zeros, M, N, K, group, y);
  if (st != W4A16_OK) return st;
  if (group != 128) return fail(W4A16_ERR_UNSUPPORTED, "the split-K kernel takes groups of 128 (got %d)", (int)group);
  if (splits < 0 || splits > w4a16::splitk_max_splits() || splits > K / 128)
    return fail(W4A16_ERR_ARG, "splits must lie in [0, min(%d, K/128)] (got %d)", w4a16::splitk_max_splits(), (int)splits);
  const int s = splits == 0 ? w4a16::splitk_default_splits(M, N, K) : splits;
  const int64_t need = w4a16::splitk_workspace_floats(M, N, s);
  if (need > w4a16::kSplitkScratchFloats)
    return fail(W4A16_ERR_SHAPE, "splits * M * N = %lld float partials exceed the library's scratch of %lld",
                (long long)need, (long long)w4a16::kSplitkScratchFloats);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  float* scratch = nullptr;
  const w4a16_status rs = hip_result(w4a16::splitk_scratch(hs, &scratch), "scratch address");
  if (rs != W4A16_OK) return rs;
  return hip_result(w4a16::launch_splitk(static_cast<const uint16_t*>(x), static_cast<const uint32_t*>(qweight),
                                         static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), M,
                                         N, K, s, scratch, static_cast<uint16_t*>(y), hs),
                    "split-K launch");
}

int64_t awq_alpha_loss_workspace(int64_t T, int64_t N) {
  if (T <= 0 || N <= 0 || T > kMaxT || N > kMaxN) return -1;
  const int64_t tiles = w4a16::alpha_loss_partials(T, N);
  return tiles > kMaxTiles ? -1 : tiles;
}

int64_t awq_search_alpha_workspace(int64_t T, int64_t N, int64_t K) {
  SearchSpace sp;
  return search_space(T, N, K, &sp) ? sp.total : -1;
}

w4a16_status awq_search_alpha(const void* x_cal, const void* w, int64_t T, int64_t N, int64_t K, void* workspace,
                              int64_t workspace_bytes, double* losses, int32_t* best, double* alpha, float* s,
                              void* stream) {
  clear_error();
  if (!x_cal || !w || !workspace || !losses || !best || !alpha)
    return fail(W4A16_ERR_NULL, "x_cal, w, workspace, losses, best and alpha are required");
  if (T <= 0 || N <= 0 || K <= 0) return fail(W4A16_ERR_SHAPE, "T, N, K must be positive (got %lld, %lld, %lld)",
                                              (long long)T, (long long)N, (long long)K);
  if (K % 128 != 0) return fail(W4A16_ERR_SHAPE, "K must be a multiple of 128 (got %lld)", (long long)K);
  SearchSpace sp;
  if (!search_space(T, N, K, &sp))
    return fail(W4A16_ERR_SHAPE, "size beyond the limits (T <= 65536, N <= 2^24, K <= %d)", W4A16_MAX_K);
  if (workspace_bytes < sp.total)
    return fail(W4A16_ERR_ARG, "workspace holds %lld bytes, %lld needed", (long long)workspace_bytes,
                (long long)sp.total);
  if (!aligned(x_cal, 16) || !aligned(w, 16) || !aligned(workspace, 256))
    return fail(W4A16_ERR_ALIGN, "x_cal and w must be 16-byte, workspace 256-byte aligned");
  if (!aligned(losses, 8) || !aligned(alpha, 8) || !aligned(best, 4) || (s && !aligned(s, 4)))
    return fail(W4A16_ERR_ALIGN, "losses and alpha must be 8-byte, best and s 4-byte aligned");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  const uint16_t* xc = static_cast<const uint16_t*>(x_cal);
  const uint16_t* wh = static_cast<const uint16_t*>(w);
  float* y_ref = reinterpret_cast<float*>(base + sp.y_ref);
  float* s_all = reinterpret_cast<float*>(base + sp.s_all);
  uint16_t* x_s = reinterpret_cast<uint16_t*>(base + sp.x_s);
  uint32_t* qw = reinterpret_cast<uint32_t*>(base + sp.qweight);
  uint16_t* sc = reinterpret_cast<uint16_t*>(base + sp.scales);
  uint16_t* zr = reinterpret_cast<uint16_t*>(base + sp.zeros);
  double* parts = reinterpret_cast<double*>(base + sp.partials);
  // the original output once, then per grid point: s = s_X^alpha, x_s = f16(x / s),
  // quantize-pack of W * s, and the output-error loss (L13 guide, AWQ section, slide 28)
  hipError_t e = w4a16::launch_output_reference(xc, wh, T, N, K, y_ref, hs);
  for (int i = 0; i < W4A16_ALPHA_GRID_POINTS && e == hipSuccess; ++i) {
    const double a = (double)i / (double)(W4A16_ALPHA_GRID_POINTS - 1);
    float* si = s_all + (int64_t)i * K;
    e = w4a16::launch_channel_scale(xc, T, K, a, si, hs);
    if (e == hipSuccess) e = w4a16::launch_scale_input(xc, si, T, K, x_s, hs);
    if (e == hipSuccess) e = w4a16::launch_quantize_pack(wh, si, N, K, 4, 128, qw, sc, zr, hs);
    if (e == hipSuccess) e = w4a16::launch_alpha_loss(x_s, qw, sc, zr, y_ref, T, N, K, parts, losses + i, hs);
  }
  if (e == hipSuccess) e = w4a16::launch_search_select(losses, W4A16_ALPHA_GRID_POINTS, s_all, K, best, alpha, s, hs);
  return hip_result(e, "alpha-search launch");
}

void nf4_codebook(uint16_t* levels) {
  if (!levels) return;
  const w4a16::Nf4Table& t = nf4_table();
  for (int i = 0; i < 8; ++i) {
    levels[2 * i] = (uint16_t)(t.pairs[i] & 0xFFFFu);
    levels[2 * i + 1] = (uint16_t)(t.pairs[i] >> 16);
  }
}

w4a16_status nf4_quantize_pack(const void* w, const float* s, int64_t N, int64_t K, int32_t block, void* qweight,
                               float* absmax, void* stream) {
  clear_error();
  if (!w || !qweight || !absmax) return fail(W4A16_ERR_NULL, "w, qweight and absmax are required");
  if (block != 64 && block != 32 && block != 128)
    return fail(W4A16_ERR_UNSUPPORTED, "block must be 32, 64 or 128 (got %d)", (int)block);
  if (N <= 0 || K <= 0) return fail(W4A16_ERR_SHAPE, "N and K must be positive");
  if (K % block != 0) return fail(W4A16_ERR_SHAPE, "K must be a multiple of the block (got K=%lld)", (long long)K);
  if (K > W4A16_MAX_K || N > kMaxN) return fail(W4A16_ERR_SHAPE, "size beyond the limits (N <= 2^24, K <= %d)", W4A16_MAX_K);
  if (!aligned(w, 16) || !aligned(qweight, 16) || (s && !aligned(s, 16)))
    return fail(W4A16_ERR_ALIGN, "w, qweight and s must be 16-byte aligned");
  if (!aligned(absmax, 4)) return fail(W4A16_ERR_ALIGN, "absmax must be 4-byte aligned");
  return hip_result(w4a16::launch_nf4_quantize_pack(static_cast<const uint16_t*>(w), s, N, K, block,
                                                    nf4_table().pairs, static_cast<uint32_t*>(qweight), absmax,
                                                    static_cast<hipStream_t>(stream)),
                    "NF4 quantize-pack launch");
}

w4a16_status nf4_linear_path(int32_t path, const void* x, const void* qweight, const float* absmax, int64_t M,
                             int64_t N, int64_t K, int32_t block, void* y, void* stream) {
  clear_error();
  if (path < 0 || path > 3)
    return fail(W4A16_ERR_UNSUPPORTED, "path must be 0 (auto), 1 (GEMV), 2 (tiled MFMA) or 3 (small-batch MFMA)");
  const w4a16_status st = check_nf4_linear(x, qweight, absmax, M, N, K, block, y);
  if (st != W4A16_OK) return st;
  const bool gemv_ok = w4a16::gemv_format_supports(0, block, M, N, K);
  if (path == 1 && !gemv_ok)
    return fail(W4A16_ERR_UNSUPPORTED, "the NF4 GEMV kernels take M <= %d and K <= 32768 (M <= 4 above K = 16384), "
                "or M = 1 with N * K < 2^26 and K <= 131072; got M=%lld K=%lld", w4a16::gemv_max_m(), (long long)M,
                (long long)K);
  if (path == 3 && M > w4a16::skinny_max_m())
    return fail(W4A16_ERR_UNSUPPORTED, "the small-batch MFMA kernel takes M <= %d; got M=%lld", w4a16::skinny_max_m(),
                (long long)M);
  const uint16_t* xh = static_cast<const uint16_t*>(x);
  const uint32_t* qw = static_cast<const uint32_t*>(qweight);
  uint16_t* yh = static_cast<uint16_t*>(y);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int32_t kernel = path;
  const bool two_passes = path == 0 && two_small_batch_passes(M, N, K);
  if (path == 0)
    kernel = auto_gemv_variant(M) && gemv_ok ? 1 : M <= w4a16::skinny_max_m() || two_passes ? 3 : gemv_ok ? 1 : 2;
  if (kernel == 1)
    return hip_result(w4a16::launch_gemv_nf4(nf4_table(), block, xh, qw, absmax, M, N, K, yh, hs), "NF4 GEMV launch");
  if (kernel == 3 && two_passes) {
    const int64_t m1 = w4a16::skinny_max_m();
    hipError_t e = w4a16::launch_skinny_nf4(nf4_table(), block, xh, qw, absmax, m1, N, K, yh, hs);
    if (e == hipSuccess) e = w4a16::launch_skinny_nf4(nf4_table(), block, xh + m1 * K, qw, absmax, M - m1, N, K, yh + m1 * N, hs);
    return hip_result(e, "NF4 small-batch MFMA launch");
  }
  if (kernel == 3)
    return hip_result(w4a16::launch_skinny_nf4(nf4_table(), block, xh, qw, absmax, M, N, K, yh, hs),
                      "NF4 small-batch MFMA launch");
  return hip_result(w4a16::launch_mfma_nf4(nf4_table(), block, xh, qw, absmax, M, N, K, yh, hs), "NF4 MFMA launch");
}

w4a16_status nf4_linear(const void* x, const void* qweight, const float* absmax, int64_t M, int64_t N, int64_t K,
                        int32_t block, void* y, void* stream) {
  return nf4_linear_path(0, x, qweight, absmax, M, N, K, block, y, stream);
}

w4a16_status awq_quantize_pack_sym(const void* w, const float* s, int64_t N, int64_t K, int32_t bits, int32_t group,
                                   void* qweight, void* scales, void* zeros, void* stream) {
  clear_error();
  if (!w || !qweight || !scales || !zeros) return fail(W4A16_ERR_NULL, "w, qweight, scales and zeros are required");
  if ((bits != 4 && bits != 3) || (group != 128 && group != 64 && group != 32))
    return fail(W4A16_ERR_UNSUPPORTED, "bits must be 3 or 4 and group 32, 64 or 128 (got bits=%d, group=%d)",
                (int)bits, (int)group);
  if (N <= 0 || K <= 0) return fail(W4A16_ERR_SHAPE, "N and K must be positive");
  if (K % group != 0) return fail(W4A16_ERR_SHAPE, "K must be a multiple of the group (got K=%lld, group=%d)",
                                  (long long)K, (int)group);
  if (K > W4A16_MAX_K || N > kMaxN) return fail(W4A16_ERR_SHAPE, "size beyond the limits (N <= 2^24, K <= %d)", W4A16_MAX_K);
  if (!aligned(w, 16) || !aligned(qweight, 16) || (s && !aligned(s, 16)))
    return fail(W4A16_ERR_ALIGN, "w, qweight and s must be 16-byte aligned");
  if (!aligned(scales, 2) || !aligned(zeros, 2)) return fail(W4A16_ERR_ALIGN, "scales and zeros must be 2-byte aligned");
  return hip_result(w4a16::launch_quantize_pack_sym(static_cast<const uint16_t*>(w), s, N, K, bits, group,
                                                    static_cast<uint32_t*>(qweight), static_cast<uint16_t*>(scales),
                                                    static_cast<uint16_t*>(zeros), static_cast<hipStream_t>(stream)),
                    "symmetric quantize-pack launch");
}

w4a16_status awq_output_reference(const void* x, const void* w, int64_t T, int64_t N, int64_t K, float* y_ref,
                                  void* stream) {
  clear_error();
  if (!x || !w || !y_ref) return fail(W4A16_ERR_NULL, "x, w and y_ref are required");
  if (T <= 0 || N <= 0 || K <= 0) return fail(W4A16_ERR_SHAPE, "T, N, K must be positive (got %lld, %lld, %lld)",
                                              (long long)T, (long long)N, (long long)K);
  if (K % 128 != 0) return fail(W4A16_ERR_SHAPE, "K must be a multiple of 128 (got %lld)", (long long)K);
  if (K > W4A16_MAX_K || awq_alpha_loss_workspace(T, N) < 0)
    return fail(W4A16_ERR_SHAPE, "size beyond the limits (T <= 2^20, N <= 2^24, K <= %d)", W4A16_MAX_K);
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y_ref, 4))
    return fail(W4A16_ERR_ALIGN, "x and w must be 16-byte, y_ref 4-byte aligned");
  return hip_result(w4a16::launch_output_reference(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                                                   T, N, K, y_ref, static_cast<hipStream_t>(stream)),
                    "output-reference launch");
}

w4a16_status awq_alpha_loss(const void* x_s, const void* qweight, const void* scales, const void* zeros,
                            const float* y_ref, int64_t T, int64_t N, int64_t K, int32_t group, double* workspace,
                            int64_t workspace_len, double* loss, void* stream) {
  clear_error();
  if (!x_s || !qweight || !scales || !zeros || !y_ref || !workspace || !loss)
    return fail(W4A16_ERR_NULL, "x_s, qweight, scales, zeros, y_ref, workspace and loss are required");
  if (group != 128) return fail(W4A16_ERR_UNSUPPORTED, "group must be 128 (got %d)", (int)group);
  if (T <= 0 || N <= 0 || K <= 0) return fail(W4A16_ERR_SHAPE, "T, N, K must be positive (got %lld, %lld, %lld)",
                                              (long long)T, (long long)N, (long long)K);
  if (K % 128 != 0) return fail(W4A16_ERR_SHAPE, "K must be a multiple of 128 (got %lld)", (long long)K);
  const int64_t need = awq_alpha_loss_workspace(T, N);
  if (K > W4A16_MAX_K || need < 0)
    return fail(W4A16_ERR_SHAPE, "size beyond the limits (T <= 2^20, N <= 2^24, K <= %d)", W4A16_MAX_K);
  if (workspace_len < need)
    return fail(W4A16_ERR_ARG, "workspace holds %lld float64 values, %lld needed", (long long)workspace_len,
                (long long)need);
  if (!aligned(x_s, 16) || !aligned(qweight, 16))
    return fail(W4A16_ERR_ALIGN, "x_s and qweight must be 16-byte aligned");
  if (!aligned(scales, 2) || !aligned(zeros, 2) || !aligned(y_ref, 4) || !aligned(workspace, 8) || !aligned(loss, 8))
    return fail(W4A16_ERR_ALIGN, "scales and zeros must be 2-byte, y_ref 4-byte, workspace and loss 8-byte aligned");
  return hip_result(w4a16::launch_alpha_loss(static_cast<const uint16_t*>(x_s), static_cast<const uint32_t*>(qweight),
                                             static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros),
                                             y_ref, T, N, K, workspace, loss, static_cast<hipStream_t>(stream)),
                    "alpha-loss launch");
}

}  // extern "C"
