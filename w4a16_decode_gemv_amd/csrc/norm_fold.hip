// RMSNorm with the AWQ 1/s folded in: the operator that produces x_s in front of
// the scaled projections of a decoder block.
//
// The pages merge the division by s into the operator in front of the scaled
// layer, so that inference needs no extra kernel ("MIT 6.5940 Lab 4 + Lab 5"
// guide, AWQ skeleton part 2.3: the scales are merged into the preceding
// LayerNorm or linear layer; "Quantization for LLMs" chapter 11, AWQ section:
// the division by s is merged into the LayerNorm in front). The LLaMA-shaped
// blocks put an RMSNorm there:
//
//   x_s[m][k] = f16( ((h[m][k] * r[m]) * gamma[k]) / s[k] ),
//   r[m]      = 1 / sqrt( sum_k h[m][k]^2 / K + eps ),
//
// every step in float64 in that order (correctly rounded square root and
// division), one float64 -> float16 rounding at the end. The sum of squares is
// accumulated in a fixed order (per thread in k order, then a fixed tree), so
// results are reproducible run to run.
//
// Work split: a row is cut into S slices of its 16-byte chunks, one workgroup per
// (row, slice). Every workgroup of a row forms the whole sum of squares in the same
// fixed order (so r is bit-identical across them) and writes its own slice. Small
// batches (M < 64) take S = ceil(chunks / 256), one chunk per thread: the float64
// division and rounding work of a row then spreads over several CUs instead of
// queueing on one. Larger batches take S = 1 and loop. A thread's first chunk of
// the second pass, with its gamma and s, is loaded before the reduction, so the
// latency of those loads overlaps the first pass; that chunk of h is kept from the
// first pass. The first pass issues up to four of a thread's chunk loads before it
// adds any (in k order), and gamma and s arrive in 16-byte loads when aligned:
// measured on MI355X, one 4096-wide row took 4.0 us against 5.5 us with one chunk
// load in flight and element-wise gamma and s loads.
#include "device_utils.h"
#include "launchers.h"

namespace w4a16 {

namespace {

constexpr int kThreads = 256;
constexpr int64_t kSplitBelowM = 64;
constexpr int kInFlight = 4;  // chunks of h each thread has in flight in the first pass

// VEC: gamma and s are 16-byte aligned, so a chunk's eight gamma and eight s values arrive in
// one and two 16-byte loads instead of eight 2-byte and eight 4-byte ones
template <bool VEC>
__global__ __launch_bounds__(kThreads) void rmsnorm_fold_kernel(const u32x4_t* __restrict__ h,
                                                                const uint16_t* __restrict__ gamma,
                                                                const float* __restrict__ s, int K, int S,
                                                                double eps, u32x4_t* __restrict__ out) {
  __shared__ double wsum[kThreads / 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int row = blockIdx.x / S, slice = blockIdx.x - row * S;
  const int chunks = K >> 3;  // 8 fp16 per 16-byte chunk
  // slices are whole multiples of kThreads chunks, so thread t's first chunk c0 + t is one
  // the first pass below visits (c = t, t + kThreads, ...)
  const int per = ((chunks + S - 1) / S + kThreads - 1) / kThreads * kThreads;
  const int c0 = slice * per, c1 = min(chunks, c0 + per);
  const int64_t base = (int64_t)row * chunks;

  // this thread's first chunk of the second pass: gamma and s now, h from the first pass
  const int cp = c0 + t;
  const bool has = cp < c1;
  uint16_t gp[8];
  float sp[8];
  auto load_gs = [&](int c, bool in, uint16_t (&g)[8], float (&sv)[8]) {
    if constexpr (VEC) {
      const u32x4_t gz = {0u, 0u, 0u, 0u};
      const u32x4_t sone = {0x3F800000u, 0x3F800000u, 0x3F800000u, 0x3F800000u};
      const u32x4_t gw = in ? reinterpret_cast<const u32x4_t*>(gamma)[c] : gz;
      const bool sin = in && s != nullptr;
      const u32x4_t s0 = sin ? reinterpret_cast<const u32x4_t*>(s)[2 * c] : sone;
      const u32x4_t s1 = sin ? reinterpret_cast<const u32x4_t*>(s)[2 * c + 1] : sone;
      const uint32_t gwv[4] = {gw.x, gw.y, gw.z, gw.w};
      const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        g[e] = (uint16_t)(gwv[e >> 1] >> (16 * (e & 1)));
        sv[e] = __builtin_bit_cast(float, sw[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        g[e] = in ? gamma[8 * c + e] : (uint16_t)0;
        sv[e] = (in && s != nullptr) ? s[8 * c + e] : 1.0f;
      }
    }
  };
  load_gs(cp, has, gp, sp);
  u32x4_t hp = {0u, 0u, 0u, 0u};

  // first pass: kInFlight chunks issued before any is added, added in k order
  double acc = 0.0;
  for (int cb = t; cb < chunks; cb += kInFlight * kThreads) {
    u32x4_t v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int c = cb + u * kThreads;
      v[u] = c < chunks ? h[base + c] : (u32x4_t){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int c = cb + u * kThreads;
      if (c >= chunks) break;
      if (c == cp) hp = v[u];
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double a = (double)half_bits_to_float((uint16_t)(w[i] & 0xFFFFu));
        const double b = (double)half_bits_to_float((uint16_t)(w[i] >> 16));
        acc += a * a;
        acc += b * b;
      }
    }
  }
  // fixed-order tree: xor butterfly inside the wave, then the waves in index order
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) wsum[wave] = acc;
  __syncthreads();
  // every thread forms r from the same four sums in the same order (no second barrier)
  double ms = 0.0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) ms += wsum[w];
  ms = ms / (double)K;
  const double r = 1.0 / sqrt(ms + eps);

  for (int c = cp; c < c1; c += kThreads) {
    u32x4_t v = hp;
    uint16_t g[8];
    float sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      g[e] = gp[e];
      sv[e] = sp[e];
    }
    if (c != cp) {
      v = h[base + c];
      load_gs(c, true, g, sv);
    }
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t res[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int e = 2 * i + hh;
        const double hv = (double)half_bits_to_float((uint16_t)(hh ? (w[i] >> 16) : (w[i] & 0xFFFFu)));
        double val = (hv * r) * (double)half_bits_to_float(g[e]);
        if (s != nullptr) val = val / (double)sv[e];
        res[hh] = f64_to_f16_rne(val);
      }
      o[i] = (uint32_t)res[0] | ((uint32_t)res[1] << 16);
    }
    out[base + c] = (u32x4_t){o[0], o[1], o[2], o[3]};
  }
}

}  // namespace

hipError_t launch_rmsnorm_fold(const uint16_t* h, const uint16_t* gamma, const float* s, int64_t M, int64_t K,
                               double eps, uint16_t* x_s, hipStream_t stream) {
  const int64_t chunks = K / 8;
  const int S = M < kSplitBelowM ? (int)((chunks + kThreads - 1) / kThreads) : 1;
  const bool vec = (reinterpret_cast<uintptr_t>(gamma) & 15) == 0 && (reinterpret_cast<uintptr_t>(s) & 15) == 0;
  if (vec)
    hipLaunchKernelGGL(rmsnorm_fold_kernel<true>, dim3((unsigned)(M * S)), dim3(kThreads), 0, stream,
                       reinterpret_cast<const u32x4_t*>(h), gamma, s, (int)K, S, eps, reinterpret_cast<u32x4_t*>(x_s));
  else
    hipLaunchKernelGGL(rmsnorm_fold_kernel<false>, dim3((unsigned)(M * S)), dim3(kThreads), 0, stream,
                       reinterpret_cast<const u32x4_t*>(h), gamma, s, (int)K, S, eps, reinterpret_cast<u32x4_t*>(x_s));
  return hipGetLastError();
}

}  // namespace w4a16
