// C ABI of the library: argument validation (host only, before any HIP call),
// status codes and text, and dispatch to the kernel launchers.
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
// kernel at M = 1, and at M = 2 on layers of at least 2^27 weights with K <= 24576 (there
// the GEMV's doubled dot work still hides under the weight stream: 21.8 against 24.0 us at
// 8192 -> 22016, 28.7 against 29.9 at 22016 -> 8192, 26.9 against 28.9 at 8192 -> 28672; on
// 8192 -> 8192 and on 28672 -> 8192 the small-batch kernel is ahead: 9.9 against 10.3 us at
// 8192 -> 8192, 29.5 against 33.8 at 28672 -> 8192), and at M = 2 on the small layers where
// the GEMV takes narrow tiles (8.1 against 8.3 us at 4096 -> 11008, 8.7 against 9.0 at
// 11008 -> 4096, 8.4 against 8.6 at 4096 -> 12288, 4.8 both at 4096 -> 4096); the
// small-batch MFMA kernel up to skinny_max_m(); the tiled MFMA kernel beyond
bool auto_gemv(int64_t M, int64_t N, int64_t K) {
  return M == 1 || (M == 2 && K <= 24576 && N * K >= (int64_t(1) << 27)) ||
         (M == 2 && w4a16::gemv_narrow(M, N, K));
}

// the same hand-off for groups of 32 and 64 and for NF4, whose GEMV variant has no long-row
// plan: at M = 2 it keeps the large layers with K <= 16384 (8192 -> 22016, groups of 64:
// 23.2 against 25.1 us; NF4: 26.7 against 29.3) and loses the long rows (22016 -> 8192:
// 47.7 against 29.5 us)
bool auto_gemv_variant(int64_t M, int64_t N, int64_t K) {
  return M == 1 || (M == 2 && K <= 16384 && N * K >= (int64_t(1) << 27));
}

// 33 <= M <= 64 on layers with N <= 8192 and K <= 16384: the small-batch kernel twice (rows
// 0..31, then the rest) beats the tiled kernel there, for every code format (group 128:
// 14.9-20.9 against 26.0-26.7 us at 4096 -> 4096, 33.1-46.9 against 47.2-49.2 at 8192 -> 8192,
// 34.0-51.2 against 61.8-63.8 at 11008 -> 4096); on wider or longer layers (4096 -> 11008,
// 8192 -> 22016, 22016 -> 8192) the tiled kernel is ahead
bool two_small_batch_passes(int64_t M, int64_t N, int64_t K) {
  return M > w4a16::skinny_max_m() && M <= 2 * w4a16::skinny_max_m() && N <= 8192 && K <= 16384;
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
    const bool gemv_ok = w4a16::gemv_variant_supports(M, K, group);
    // the small-batch kernel loads a row's scales (zeros) of 128 inputs in one 2-, 4- or 8-byte load
    const uintptr_t sz_align = group == 128 ? 2 : 4;
    const bool sz_aligned = aligned(scales, sz_align) && aligned(zeros, sz_align);
    const bool skinny_ok = M <= w4a16::skinny_max_m() && sz_aligned;
    bool two_passes = false;
    int32_t kernel = path;
    if (path == 0) {
      // 3-bit codes keep the GEMV variant at M = 2 on every shape: its dequant VALU is shared
      // by both rows there (8192 -> 8192: 12.5 against 12.8 us for groups of 128, 12.6 against
      // 13.3 for 64, 12.8 against 15.2 for 32). 4-bit groups of 64 and 32 run the tuned GEMV,
      // which at M = 2 stays ahead from 2^26 weights (8192 -> 8192: 10.5 against 11.1 us for
      // 64, 10.7 against 12.4 for 32; 8192 -> 22016: 21.1 against 25.1) and on the small layers
      // where it takes 4-row tiles (4096 -> 11008: 8.3 against 8.6 us for 64, 8.5 against 9.4
      // for 32; 11008 -> 4096: 8.9 against 9.4, 9.1 against 11.4; 4096 -> 4096: 4.8 against 4.9)
      const bool gemv_first =
          bits == 4 ? M == 1 || (M == 2 && ((K <= 24576 && N * K >= (int64_t(1) << 26)) || w4a16::gemv_narrow(M, N, K)))
                    : auto_gemv_variant(M, N, K) || (bits == 3 && M == 2);
      two_passes = sz_aligned && two_small_batch_passes(M, N, K);
      kernel = gemv_first && gemv_ok ? 1 : skinny_ok || two_passes ? 3 : gemv_ok ? 1 : 2;
    } else if (path == 1 && !gemv_ok) {
      return fail(W4A16_ERR_UNSUPPORTED, "the GEMV kernel for this format takes M <= %d and K <= 32768 "
                  "(M <= 4 above K = 16384); got M=%lld K=%lld", w4a16::gemv_max_m(), (long long)M, (long long)K);
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
    } else if (M <= w4a16::skinny_max_m()) {
      kernel = 3;
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
  return hip_result(w4a16::launch_mfma(xh, qw, sc, zr, M, N, K, yh, stream), "MFMA launch");
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

w4a16_status w4a16_linear_path(int32_t path, const void* x, const void* qweight, const void* scales,
                               const void* zeros, int64_t M, int64_t N, int64_t K, int32_t group, void* y,
                               void* stream) {
  clear_error();
  if (path < 0 || path > 3)
    return fail(W4A16_ERR_UNSUPPORTED, "path must be 0 (auto), 1 (GEMV), 2 (tiled MFMA) or 3 (small-batch MFMA)");
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

int64_t awq_alpha_loss_workspace(int64_t T, int64_t N) {
  if (T <= 0 || N <= 0 || T > kMaxT || N > kMaxN) return -1;
  const int64_t tiles = w4a16::alpha_loss_partials(T, N);
  return tiles > kMaxTiles ? -1 : tiles;
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
  const bool gemv_ok = w4a16::gemv_variant_supports(M, K, block);
  if (path == 1 && !gemv_ok)
    return fail(W4A16_ERR_UNSUPPORTED, "the NF4 GEMV kernel takes M <= %d and K <= 32768 (M <= 4 above K = 16384); "
                "got M=%lld K=%lld", w4a16::gemv_max_m(), (long long)M, (long long)K);
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
    kernel = auto_gemv_variant(M, N, K) && gemv_ok ? 1 : M <= w4a16::skinny_max_m() || two_passes ? 3 : gemv_ok ? 1 : 2;
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
