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
// One workgroup per row; the row is read twice (the second read is an L2 hit),
// so registers do not bound K.
#include "device_utils.h"
#include "launchers.h"

namespace w4a16 {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void rmsnorm_fold_kernel(const u32x4_t* __restrict__ h,
                                                                const uint16_t* __restrict__ gamma,
                                                                const float* __restrict__ s, int K, double eps,
                                                                u32x4_t* __restrict__ out) {
  __shared__ double wsum[kThreads / 64];
  __shared__ double rrow;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int chunks = K >> 3;  // 8 fp16 per 16-byte chunk
  const int64_t base = (int64_t)blockIdx.x * chunks;

  double acc = 0.0;
  for (int c = t; c < chunks; c += kThreads) {
    const u32x4_t v = h[base + c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double a = (double)half_bits_to_float((uint16_t)(w[i] & 0xFFFFu));
      const double b = (double)half_bits_to_float((uint16_t)(w[i] >> 16));
      acc += a * a;
      acc += b * b;
    }
  }
  // fixed-order tree: xor butterfly inside the wave, then the waves in index order
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) wsum[wave] = acc;
  __syncthreads();
  if (t == 0) {
    double ms = 0.0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) ms += wsum[w];
    ms = ms / (double)K;
    rrow = 1.0 / sqrt(ms + eps);
  }
  __syncthreads();
  const double r = rrow;

  for (int c = t; c < chunks; c += kThreads) {
    const u32x4_t v = h[base + c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t res[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int k = 8 * c + 2 * i + hh;
        const double hv = (double)half_bits_to_float((uint16_t)(hh ? (w[i] >> 16) : (w[i] & 0xFFFFu)));
        double val = (hv * r) * (double)half_bits_to_float(gamma[k]);
        if (s != nullptr) val = val / (double)s[k];
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
  hipLaunchKernelGGL(rmsnorm_fold_kernel, dim3((unsigned)M), dim3(kThreads), 0, stream,
                     reinterpret_cast<const u32x4_t*>(h), gamma, s, (int)K, eps, reinterpret_cast<u32x4_t*>(x_s));
  return hipGetLastError();
}

}  // namespace w4a16
