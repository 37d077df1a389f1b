// The output-error loss of the AWQ scale search, for one candidate scale.
//
//   L(s) = sum_{t,n} ( sum_k x_s[t][k] * w_hat[n][k]  -  sum_k x[t][k] * w[n][k] )^2
//
// "MIT 6.5940 L13 LLM Deployment" guide, AWQ section (slide 28): the scale is
// chosen by a grid search over alpha on L(s) = ||Q(W s)(s^-1 X) - W X|| with
// s = s_X^alpha, the error measured on the layer's output; chapter 11, AWQ
// section, the same. Here x_s = f16(x / s) is the input the deployed kernel
// consumes and w_hat = (q - z) * d is rebuilt from the packed codes and the stored
// fp16 scale and zero of W * s (both produced by this library's own kernels), so
// the loss is the one of the layer as it would run.
//
// One fused tiled MFMA pass computes both products for a 64 x 64 (t, n) tile,
// one quantization group (128 inputs) per step:
//   * the quantized product takes exact fp16 q in the B operand and applies each
//     group as d * (sum_k x_s q - z * sum_k x_s): exact q - z for every storable
//     zero; sum_k x_s per (row, group) is formed once while the tile is staged;
//   * the reference product takes the fp16 weights directly;
// both accumulate in float32. x and x_s are shared by the four waves and staged
// through LDS (double-buffered, the next group's global loads in flight while the
// current one is computed); the weights, codes and (scale, zero) of a wave's 16
// output rows are its own and go straight to registers. The tile's squared
// differences are summed in float64 in a fixed order into one partial; a second
// one-workgroup kernel adds the partials in index order into the loss, so the
// result is reproducible run to run.
//
// Fragments as in the tiled linear kernel (v_mfma_f32_16x16x32_f16): at step st
// of a group, slot group j holds the 8 inputs of chunk 4j + st, so lane (j, c)
// reads 64 contiguous bytes of its weight row and one 16-byte code chunk per
// group.
#include "device_utils.h"
#include "launchers.h"

namespace w4a16 {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 64;   // calibration rows t per tile (4 MFMA tiles of 16)
constexpr int BN = 64;   // output rows n per tile (4 waves x 16)
constexpr int kThreads = 256;
constexpr int XP = 17;   // x tiles: 16 chunks of 16 bytes per row, padded to 17

__device__ __forceinline__ half8_t as_half8(u32x4_t v) { return __builtin_bit_cast(half8_t, v); }

// the eight codes q of one code word as exact fp16, in k order
__device__ __forceinline__ half8_t codes_word(uint32_t w) {
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t c_lo = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  const half2_t c_hi = {(_Float16)-64.0f, (_Float16)-64.0f};
  const uint32_t w8 = w >> 8;
  const half2_t p0 = as_half2(and_or(w, 0x000F000Fu, 0x64006400u)) + c_lo;
  const half2_t p1 = __builtin_elementwise_fma(as_half2(and_or(w, 0x00F000F0u, 0x64006400u)), sixteenth, c_hi);
  const half2_t p2 = as_half2(and_or(w8, 0x000F000Fu, 0x64006400u)) + c_lo;
  const half2_t p3 = __builtin_elementwise_fma(as_half2(and_or(w8, 0x00F000F0u, 0x64006400u)), sixteenth, c_hi);
  const u32x4_t v = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                     __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
  return __builtin_bit_cast(half8_t, v);
}

// sum of the eight fp16 values of one 16-byte chunk, float32, in k order
__device__ __forceinline__ float chunk_sum(u32x4_t v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s += half_bits_to_float((uint16_t)(w[i] & 0xFFFFu));
    s += half_bits_to_float((uint16_t)(w[i] >> 16));
  }
  return s;
}

struct Smem {
  u32x4_t xs[2][BM][XP];  // x_s tile of the group
  u32x4_t x[2][BM][XP];   // x tile of the group
  float sxs[2][BM];       // sum over the group's 128 inputs of x_s, per row
};

// Tiles are numbered so that the eight XCDs (workgroups go to them round-robin)
// each take a contiguous run of output-row tiles, all calibration tiles of one
// output-row tile back to back: a weight tile is fetched by one XCD's L2.
__device__ __forceinline__ int tile_of_block(int id, int nb) {
  const int xcd = id & 7, slot = id >> 3;
  const int per = nb >> 3, rem = nb & 7;
  return xcd * per + min(xcd, rem) + slot;
}

__global__ __launch_bounds__(kThreads) void alpha_loss_kernel(const u32x4_t* __restrict__ x, const u32x4_t* __restrict__ xs,
                                                             const u32x4_t* __restrict__ w, const u32x4_t* __restrict__ qw,
                                                             const uint16_t* __restrict__ scales,
                                                             const uint16_t* __restrict__ zeros, int T, int N, int K,
                                                             int GT, double* __restrict__ partials) {
  __shared__ Smem sm;
  __shared__ double wsum[kThreads / 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int j = lane >> 4, c = lane & 15;
  const int tile = tile_of_block(blockIdx.x, gridDim.x);
  const int m0 = (tile % GT) * BM, n0 = (tile / GT) * BN;
  const int G = K >> 7, KX = K >> 3, KQ = K >> 5;

  // staging of x and x_s: chunk i = t + 256 u -> row (t >> 4) + 16 u, chunk t & 15; the
  // 16 lanes of a row form one DPP row
  const int ch = t & 15;
  int64_t xoff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) xoff[u] = (int64_t)min(m0 + (t >> 4) + 16 * u, T - 1) * KX + ch;
  // this lane's output row
  const int nl = wave * 16 + c;
  const int nrow = min(n0 + nl, N - 1);
  const u32x4_t* wrow = w + (int64_t)nrow * KX + 4 * j;
  const u32x4_t* qrow = qw + (int64_t)nrow * KQ + j;
  const int64_t szrow = (int64_t)nrow * G;

  u32x4_t rxs[4], rx[4];
  u32x4_t wn[4], qn;
  uint16_t sn, zn;
  auto load_stage = [&](int g) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      rxs[u] = xs[xoff[u] + 16 * g];
      rx[u] = x[xoff[u] + 16 * g];
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) wn[st] = wrow[16 * g + st];
    qn = qrow[4 * g];
    sn = scales[szrow + g];
    zn = zeros[szrow + g];
  };
  auto store_stage = [&](int b) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = (t >> 4) + 16 * u;
      sm.xs[b][r][ch] = rxs[u];
      sm.x[b][r][ch] = rx[u];
      const float sr = dpp_row_sum16(chunk_sum(rxs[u]));
      if (ch == 0) sm.sxs[b][r] = sr;
    }
  };

  float4_t dq[4], dr[4];  // quantized and reference products, per MFMA tile of rows
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    dq[mt] = (float4_t){0.f, 0.f, 0.f, 0.f};
    dr[mt] = (float4_t){0.f, 0.f, 0.f, 0.f};
  }

  load_stage(0);
  store_stage(0);
  u32x4_t wc[4] = {wn[0], wn[1], wn[2], wn[3]};
  u32x4_t qc = qn;
  uint16_t sc = sn, zc = zn;
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const int b = g & 1;
    if (g + 1 < G) load_stage(g + 1);
    const half8_t bq[4] = {codes_word(qc.x), codes_word(qc.y), codes_word(qc.z), codes_word(qc.w)};
    const float d = half_bits_to_float(sc);
    const float zf = half_bits_to_float(zc);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int row = 16 * mt + c;
      float4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        a = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(sm.xs[b][row][4 * j + st]), bq[st], a, 0, 0, 0);
        dr[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(sm.x[b][row][4 * j + st]), as_half8(wc[st]), dr[mt],
                                                        0, 0, 0);
      }
      const float4_t sx = *reinterpret_cast<const float4_t*>(&sm.sxs[b][16 * mt + 4 * j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) dq[mt][i] = __builtin_fmaf(d, __builtin_fmaf(-zf, sx[i], a[i]), dq[mt][i]);
    }
    if (g + 1 < G) {
      store_stage(b ^ 1);  // the buffer every wave finished reading before the last barrier
#pragma unroll
      for (int st = 0; st < 4; ++st) wc[st] = wn[st];
      qc = qn;
      sc = sn;
      zc = zn;
    }
    __syncthreads();
  }

  // squared differences of this tile's valid outputs, float64, fixed order
  double acc = 0.0;
  const int n = n0 + nl;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 16 * mt + 4 * j + i;
      const double e = (double)dq[mt][i] - (double)dr[mt][i];
      if (m < T && n < N) acc += e * e;
    }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) wsum[wave] = acc;
  __syncthreads();
  if (t == 0) {
    double s = 0.0;
#pragma unroll
    for (int ww = 0; ww < kThreads / 64; ++ww) s += wsum[ww];
    partials[tile] = s;
  }
}

__global__ __launch_bounds__(kThreads) void sum_partials_kernel(const double* __restrict__ partials, int64_t count,
                                                               double* __restrict__ loss) {
  __shared__ double wsum[kThreads / 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  double acc = 0.0;
  for (int64_t i = t; i < count; i += kThreads) acc += partials[i];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) wsum[wave] = acc;
  __syncthreads();
  if (t == 0) {
    double s = 0.0;
#pragma unroll
    for (int ww = 0; ww < kThreads / 64; ++ww) s += wsum[ww];
    *loss = s;
  }
}

}  // namespace

int64_t alpha_loss_partials(int64_t T, int64_t N) { return ((T + BM - 1) / BM) * ((N + BN - 1) / BN); }

hipError_t launch_alpha_loss(const uint16_t* x, const uint16_t* x_s, const uint16_t* w, const uint32_t* qweight,
                             const uint16_t* scales, const uint16_t* zeros, int64_t T, int64_t N, int64_t K,
                             double* partials, double* loss, hipStream_t stream) {
  const int64_t tiles = alpha_loss_partials(T, N);
  hipLaunchKernelGGL(alpha_loss_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, stream,
                     reinterpret_cast<const u32x4_t*>(x), reinterpret_cast<const u32x4_t*>(x_s),
                     reinterpret_cast<const u32x4_t*>(w), reinterpret_cast<const u32x4_t*>(qweight), scales, zeros,
                     (int)T, (int)N, (int)K, (int)((T + BM - 1) / BM), partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sum_partials_kernel, dim3(1), dim3(kThreads), 0, stream, partials, tiles, loss);
  return hipGetLastError();
}

}  // namespace w4a16
