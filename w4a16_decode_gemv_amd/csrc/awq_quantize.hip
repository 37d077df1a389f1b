// AWQ calibration statistic, the 1/s input fold, and RTN group quantize-pack
// for gfx950.
//
// What is computed follows the "MIT 6.5940 L13 LLM Deployment" guide (AWQ
// section: s = s_X^alpha, Q(w) = Delta * Round(w / Delta), 1/s folded into the
// input), the Lab 4 setup of the "MIT 6.5940 Lab 4 + Lab 5" guide (mean |input|
// per channel), and the "CMU 11-868 Model Quantization" guide, L19 zero-point
// quantizer (range max - min, zero range counts as 1, integer zero offset,
// clipped codes). Every quantity that decides a stored bit is computed in
// float64 with IEEE division and round-half-even, so results are bit-identical
// to the plain definition.
#include "device_utils.h"
#include "launchers.h"

#pragma clang fp contract(off)

namespace w4a16 {

// ---------------------------------------------------------------------------
// s[k] = (sum_t |x_cal[t][k]| / T)^alpha. The float64 sum of fp16 magnitudes is
// exact while T * max|x| < 2^29 (every fp16 value is a multiple of 2^-24), so it
// does not depend on the order of the additions: the tokens can be split freely.

__device__ __forceinline__ float channel_power(double sum, int T, double alpha) {
  const double mean = sum / (double)T;
  double r;
  if (mean == 0.0)
    r = 1.0;
  else if (alpha == 0.5)
    r = sqrt(mean);
  else if (alpha == 1.0)
    r = mean;
  else if (alpha == 0.0)
    r = 1.0;
  else
    r = pow(mean, alpha);
  return (float)r;
}

// Any K and alignment: one thread per channel, the loop over tokens coalesced
// across channels.
__global__ __launch_bounds__(256) void channel_scale_kernel(const uint16_t* __restrict__ x_cal, int T, int K,
                                                            double alpha, float* __restrict__ s) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  double acc0 = 0.0, acc1 = 0.0, acc2 = 0.0, acc3 = 0.0;
  const uint16_t* p = x_cal + k;
  int t = 0;
  for (; t + 4 <= T; t += 4) {
    acc0 += fabs((double)half_bits_to_float(p[(int64_t)(t + 0) * K]));
    acc1 += fabs((double)half_bits_to_float(p[(int64_t)(t + 1) * K]));
    acc2 += fabs((double)half_bits_to_float(p[(int64_t)(t + 2) * K]));
    acc3 += fabs((double)half_bits_to_float(p[(int64_t)(t + 3) * K]));
  }
  for (; t < T; ++t) acc0 += fabs((double)half_bits_to_float(p[(int64_t)t * K]));
  s[k] = channel_power((acc0 + acc1) + (acc2 + acc3), T, alpha);
}

// K % 8 == 0 and x_cal 16-byte aligned: a workgroup owns 128 channels; its 16
// rows of 16 threads split the tokens (thread (ty, tx) reads the 16 bytes of
// channels 8tx .. 8tx+7 of tokens ty, ty + 16, ...), and the 16 partial sums of
// each channel meet in LDS.
constexpr int kScaleRows = 16;

__global__ __launch_bounds__(256) void channel_scale_wide_kernel(const uint4* __restrict__ x_cal, int T, int K,
                                                                 double alpha, float* __restrict__ s) {
  __shared__ double part[kScaleRows][129];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int k0 = blockIdx.x * 128 + 8 * tx;  // first of this thread's 8 channels
  const bool active = k0 < K;                // K % 8 == 0: all 8 channels exist
  const int KC = K >> 3;
  double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  if (active) {
    const uint4* p = x_cal + (k0 >> 3);
    int t = ty;
    for (; t + 3 * kScaleRows < T; t += 4 * kScaleRows) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = p[(int64_t)(t + u * kScaleRows) * KC];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += fabs((double)half_bits_to_float((uint16_t)(w[i] & 0xFFFFu)));
          acc[2 * i + 1] += fabs((double)half_bits_to_float((uint16_t)(w[i] >> 16)));
        }
      }
    }
    for (; t < T; t += kScaleRows) {
      const uint4 v = p[(int64_t)t * KC];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += fabs((double)half_bits_to_float((uint16_t)(w[i] & 0xFFFFu)));
        acc[2 * i + 1] += fabs((double)half_bits_to_float((uint16_t)(w[i] >> 16)));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[ty][8 * tx + i] = acc[i];
  __syncthreads();
  if (threadIdx.x < 128) {
    const int k = blockIdx.x * 128 + threadIdx.x;
    if (k < K) {
      double sum = 0.0;
#pragma unroll
      for (int r = 0; r < kScaleRows; ++r) sum += part[r][threadIdx.x];
      s[k] = channel_power(sum, T, alpha);
    }
  }
}

hipError_t launch_channel_scale(const uint16_t* x_cal, int64_t T, int64_t K, double alpha, float* s,
                                hipStream_t stream) {
  if (K % 8 == 0 && (reinterpret_cast<uintptr_t>(x_cal) & 15) == 0) {
    const int grid = (int)((K + 127) / 128);
    hipLaunchKernelGGL(channel_scale_wide_kernel, dim3(grid), dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(x_cal), (int)T, (int)K, alpha, s);
  } else {
    const int block = 256;
    const int grid = (int)((K + block - 1) / block);
    hipLaunchKernelGGL(channel_scale_kernel, dim3(grid), dim3(block), 0, stream, x_cal, (int)T, (int)K, alpha, s);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// x_s = f16(float64(x) / float64(s)), one correctly rounded division and one
// round-to-nearest-even to binary16.
__global__ __launch_bounds__(256) void scale_input_kernel(const uint16_t* __restrict__ x, const float* __restrict__ s,
                                                          int64_t total, int K, uint16_t* __restrict__ x_s) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int k = (int)(i % K);
    const double v = (double)half_bits_to_float(x[i]) / (double)s[k];
    x_s[i] = f64_to_f16_rne(v);
  }
}

hipError_t launch_scale_input(const uint16_t* x, const float* s, int64_t M, int64_t K, uint16_t* x_s,
                              hipStream_t stream) {
  const int64_t total = M * K;
  const int block = 256;
  int64_t grid = (total + block - 1) / block;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(scale_input_kernel, dim3((unsigned)grid), dim3(block), 0, stream, x, s, total, (int)K, x_s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Quantize-pack. A group of GROUP inputs of one output row belongs to GROUP / 8
// consecutive lanes: lane j of the group loads the 8 fp16 weights
// k = GROUP g + 8j .. +7 (16 bytes, so a wave reads 1 KB contiguous per load),
// multiplies by s in float64 (exact), takes part in the group's min/max
// reduction, and computes its 8 codes. 4-bit codes: the lane writes exactly one
// layout-v1 word (the codes of 8 consecutive inputs). 3-bit codes: the four
// lanes of a 32-input block OR their bits into the block's three bit-plane words
// (two low-bit words, one high-bit word) and three of them write one word each.
// Lane 0 of the group writes the fp16 scale and zero.
template <int BITS, int GROUP, bool SYM>
__global__ __launch_bounds__(256) void quantize_pack_kernel(const uint4* __restrict__ w, const float4* __restrict__ s,
                                                            int64_t n_groups, int G, uint32_t* __restrict__ qweight,
                                                            uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros) {
  constexpr int LPG = GROUP / 8;  // lanes per group
  constexpr double kQmax = (double)((1 << BITS) - 1);
  const int64_t gid_raw = (int64_t)blockIdx.x * (blockDim.x / LPG) + (threadIdx.x / LPG);
  const int j = threadIdx.x % LPG;
  const bool valid = gid_raw < n_groups;  // uniform over the lanes of a group
  const int64_t gid = valid ? gid_raw : 0;
  const int64_t n = gid / G;
  const int g = (int)(gid - n * G);
  const int64_t chunk = n * ((int64_t)G * LPG) + (int64_t)LPG * g + j;  // the lane's 16-byte weight chunk

  const uint4 wv = w[chunk];
  const uint32_t wu[4] = {wv.x, wv.y, wv.z, wv.w};
  double v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = (double)half_bits_to_float((uint16_t)(wu[i] & 0xFFFFu));
    v[2 * i + 1] = (double)half_bits_to_float((uint16_t)(wu[i] >> 16));
  }
  if (s != nullptr) {
    const int64_t kc = (int64_t)GROUP * g + 8 * j;  // first input of the chunk
    const float4 s0 = s[kc / 4];
    const float4 s1 = s[kc / 4 + 1];
    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = v[i] * (double)sv[i];  // exact: 11 x 24 significant bits
  }
  double delta, z;
  uint32_t c[8];
  if constexpr (!SYM) {
    double mn = v[0], mx = v[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      mn = fmin(mn, v[i]);
      mx = fmax(mx, v[i]);
    }
#pragma unroll
    for (int off = 1; off < LPG; off <<= 1) {
      mn = fmin(mn, __shfl_xor(mn, off, LPG));
      mx = fmax(mx, __shfl_xor(mx, off, LPG));
    }
    double range = mx - mn;
    if (range == 0.0) range = 1.0;
    delta = range / kQmax;
    z = rint(-mn / delta) + 0.0;  // + 0.0 makes a zero offset +0
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      double q = rint(v[i] / delta) + z;
      q = fmin(fmax(q, 0.0), kQmax);
      c[i] = (uint32_t)q;
    }
  } else {
    // symmetric absmax: Delta = max|w| / (2^(b-1) - 1), codes rint(w / Delta) clipped to
    // the symmetric range, stored with the fixed zero 2^(b-1)
    constexpr double kHalf = (double)((1 << (BITS - 1)) - 1);
    double m = fabs(v[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) m = fmax(m, fabs(v[i]));
#pragma unroll
    for (int off = 1; off < LPG; off <<= 1) m = fmax(m, __shfl_xor(m, off, LPG));
    if (m == 0.0) m = 1.0;
    delta = m / kHalf;
    z = (double)(1 << (BITS - 1));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double q = fmin(fmax(rint(v[i] / delta), -kHalf), kHalf);
      c[i] = (uint32_t)(q + z);
    }
  }
  if constexpr (BITS == 4) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= c[i] << ((i & 1) ? (16 + 4 * (i >> 1)) : (4 * (i >> 1)));
    if (valid) qweight[chunk] = word;
  } else {
    // position of this lane's 8 inputs in its 32-input block: quarter jb = j & 3
    const int jb = j & 3;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int pl = 4 * (jb & 1) + (i >> 1);  // pair index within the 16-input half
      const int ph = 4 * jb + (i >> 1);        // pair index within the block
      lo |= (c[i] & 3u) << ((i & 1) ? (16 + 2 * pl) : (2 * pl));
      hi |= (c[i] >> 2) << ((i & 1) ? (16 + ph) : ph);
    }
    lo |= __shfl_xor(lo, 1, LPG);  // quarters 0|1 and 2|3 share a low-bit word
    hi |= __shfl_xor(hi, 1, LPG);
    hi |= __shfl_xor(hi, 2, LPG);
    // block index within the row, and its three words
    const int64_t block = (int64_t)(GROUP / 32) * g + (j >> 2);
    const int64_t base = n * ((int64_t)G * (GROUP / 32) * 3) + 3 * block;
    if (valid) {
      if (jb == 0) qweight[base] = lo;      // quarters 0, 1
      if (jb == 2) qweight[base + 1] = lo;  // quarters 2, 3
      if (jb == 1) qweight[base + 2] = hi;
    }
  }
  if (valid && j == 0) {
    scales[gid] = f64_to_f16_rne(delta);
    zeros[gid] = f64_to_f16_rne(z);
  }
}

template <int BITS, int GROUP, bool SYM>
hipError_t launch_qp(const uint16_t* w, const float* s, int64_t N, int64_t K, uint32_t* qweight, uint16_t* scales,
                     uint16_t* zeros, hipStream_t stream) {
  const int G = (int)(K / GROUP);
  const int64_t n_groups = N * G;
  const int block = 256;
  const int per_block = block / (GROUP / 8);
  const int64_t grid = (n_groups + per_block - 1) / per_block;
  hipLaunchKernelGGL((quantize_pack_kernel<BITS, GROUP, SYM>), dim3((unsigned)grid), dim3(block), 0, stream,
                     reinterpret_cast<const uint4*>(w), reinterpret_cast<const float4*>(s), n_groups, G, qweight,
                     scales, zeros);
  return hipGetLastError();
}

template <bool SYM>
hipError_t launch_qp_any(const uint16_t* w, const float* s, int64_t N, int64_t K, int bits, int group,
                         uint32_t* qweight, uint16_t* scales, uint16_t* zeros, hipStream_t stream) {
  if (bits == 4) {
    if (group == 128) return launch_qp<4, 128, SYM>(w, s, N, K, qweight, scales, zeros, stream);
    if (group == 64) return launch_qp<4, 64, SYM>(w, s, N, K, qweight, scales, zeros, stream);
    if (group == 32) return launch_qp<4, 32, SYM>(w, s, N, K, qweight, scales, zeros, stream);
  } else if (bits == 3) {
    if (group == 128) return launch_qp<3, 128, SYM>(w, s, N, K, qweight, scales, zeros, stream);
    if (group == 64) return launch_qp<3, 64, SYM>(w, s, N, K, qweight, scales, zeros, stream);
    if (group == 32) return launch_qp<3, 32, SYM>(w, s, N, K, qweight, scales, zeros, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_quantize_pack(const uint16_t* w, const float* s, int64_t N, int64_t K, int bits, int group,
                                uint32_t* qweight, uint16_t* scales, uint16_t* zeros, hipStream_t stream) {
  return launch_qp_any<false>(w, s, N, K, bits, group, qweight, scales, zeros, stream);
}

hipError_t launch_quantize_pack_sym(const uint16_t* w, const float* s, int64_t N, int64_t K, int bits, int group,
                                    uint32_t* qweight, uint16_t* scales, uint16_t* zeros, hipStream_t stream) {
  return launch_qp_any<true>(w, s, N, K, bits, group, qweight, scales, zeros, stream);
}

// ---------------------------------------------------------------------------
// NF4 quantize-pack. A block of BLOCK inputs of one row belongs to BLOCK / 8
// lanes (8 weights each, as above); a = f32(max |w|) of the block, and each
// weight's code is the index of the nearest fp16 codebook level to w / a
// (float64 division): the number of level midpoints at or below it, so an
// exact midpoint goes to the larger level. A block with a = 0 stores a = 0 and
// the code of level 0. Codes are packed in layout v1.
template <int BLOCK>
__global__ __launch_bounds__(256) void nf4_quantize_kernel(const uint4* __restrict__ w, const float4* __restrict__ s,
                                                           int64_t n_blocks, int G, Nf4Table table,
                                                           uint32_t* __restrict__ qweight, float* __restrict__ absmax) {
  constexpr int LPB = BLOCK / 8;
  const int64_t bid_raw = (int64_t)blockIdx.x * (blockDim.x / LPB) + (threadIdx.x / LPB);
  const int j = threadIdx.x % LPB;
  const bool valid = bid_raw < n_blocks;
  const int64_t bid = valid ? bid_raw : 0;
  const int64_t n = bid / G;
  const int g = (int)(bid - n * G);
  const int64_t chunk = n * ((int64_t)G * LPB) + (int64_t)LPB * g + j;

  const uint4 wv = w[chunk];
  const uint32_t wu[4] = {wv.x, wv.y, wv.z, wv.w};
  double v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = (double)half_bits_to_float((uint16_t)(wu[i] & 0xFFFFu));
    v[2 * i + 1] = (double)half_bits_to_float((uint16_t)(wu[i] >> 16));
  }
  if (s != nullptr) {
    const int64_t kc = (int64_t)BLOCK * g + 8 * j;
    const float4 s0 = s[kc / 4];
    const float4 s1 = s[kc / 4 + 1];
    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = v[i] * (double)sv[i];
  }
  double m = fabs(v[0]);
#pragma unroll
  for (int i = 1; i < 8; ++i) m = fmax(m, fabs(v[i]));
#pragma unroll
  for (int off = 1; off < LPB; off <<= 1) m = fmax(m, __shfl_xor(m, off, LPB));
  const float a = (float)m;  // round to nearest even
  // midpoints of consecutive fp16 levels (exact in float64); the level-0 code
  double mid[15];
  int zero_code = 0;
#pragma unroll
  for (int i = 0; i < 15; ++i) {
    const uint32_t w0 = table.pairs[i >> 1], w1 = table.pairs[(i + 1) >> 1];
    const double l0 = (double)half_bits_to_float((uint16_t)((i & 1) ? (w0 >> 16) : (w0 & 0xFFFFu)));
    const double l1 = (double)half_bits_to_float((uint16_t)(((i + 1) & 1) ? (w1 >> 16) : (w1 & 0xFFFFu)));
    mid[i] = (l0 + l1) * 0.5;
    if (l1 == 0.0) zero_code = i + 1;
  }
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t c = (uint32_t)zero_code;
    if (a != 0.0f) {
      const double x = v[i] / (double)a;
      c = 0;
#pragma unroll
      for (int t = 0; t < 15; ++t) c += (mid[t] <= x) ? 1u : 0u;
    }
    word |= c << ((i & 1) ? (16 + 4 * (i >> 1)) : (4 * (i >> 1)));
  }
  if (valid) {
    qweight[chunk] = word;
    if (j == 0) absmax[bid] = a;
  }
}

template <int BLOCK>
hipError_t launch_nf4q(const uint16_t* w, const float* s, int64_t N, int64_t K, const uint32_t* lut,
                       uint32_t* qweight, float* absmax, hipStream_t stream) {
  const int G = (int)(K / BLOCK);
  const int64_t n_blocks = N * G;
  const int per_block = 256 / (BLOCK / 8);
  const int64_t grid = (n_blocks + per_block - 1) / per_block;
  Nf4Table t;
  for (int i = 0; i < 8; ++i) t.pairs[i] = lut[i];
  hipLaunchKernelGGL((nf4_quantize_kernel<BLOCK>), dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(w), reinterpret_cast<const float4*>(s), n_blocks, G, t, qweight,
                     absmax);
  return hipGetLastError();
}

hipError_t launch_nf4_quantize_pack(const uint16_t* w, const float* s, int64_t N, int64_t K, int block,
                                    const uint32_t* lut, uint32_t* qweight, float* absmax, hipStream_t stream) {
  if (block == 64) return launch_nf4q<64>(w, s, N, K, lut, qweight, absmax, stream);
  if (block == 32) return launch_nf4q<32>(w, s, N, K, lut, qweight, absmax, stream);
  if (block == 128) return launch_nf4q<128>(w, s, N, K, lut, qweight, absmax, stream);
  return hipErrorInvalidValue;
}

}  // namespace w4a16
