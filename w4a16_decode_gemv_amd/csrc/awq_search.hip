// The output-error loss of the AWQ scale search.
//
//   loss(s) = sum_{t,n} ( sum_k x_s[t][k] * w_hat[n][k]  -  y_ref[t][n] )^2,
//   y_ref[t][n] = sum_k x[t][k] * w[n][k]
//
// "MIT 6.5940 L13 LLM Deployment" guide, AWQ section (slide 28): the scale is
// picked by a grid search over alpha that minimises the distance between the
// quantized layer's output on (s^-1 X) and the original layer's output W X,
// with s = s_X^alpha; "Quantization for LLMs" chapter 11, AWQ section, the same.
// x_s = f16(x / s) is the input the deployed kernel consumes and w_hat =
// (q - z) * d is rebuilt from the packed codes and the stored fp16 scale and zero
// of W * s, so the loss is that of the layer as it would run.
//
// The original layer's output does not depend on the candidate scale, so it is
// computed once per search (output_reference_kernel) and every grid point runs
// only the quantized product (alpha_loss_kernel), whose epilogue subtracts the
// stored reference, squares and sums.
//
// Both kernels tile the (t, n) plane in BM x BN = 64 x 128 tiles, one workgroup of
// eight waves per tile, each wave owning 16 output rows n and all 64 rows t, one
// quantization group (128 inputs) per stage:
//   * the 64 x 128 input tile (x or x_s) is shared by the eight waves and passes
//     through LDS; the weights of a wave's 16 rows (codes with (scale, zero), or
//     the fp16 weights) are its own and stay in registers;
//   * loads run R = 2 stages ahead of the compute in register sets that are
//     written to LDS one stage ahead; every load is a buffer load, so rows past T
//     or N and stages past the last group read as zero with no memory traffic and
//     the pipeline has no data-dependent branch; the workgroup barrier orders LDS
//     only, so loads stay in flight across it;
//   * the quantized product takes exact fp16 (q - z) in the B operand while the
//     zero lies in [-2032, 1024] (OR-ing a nibble pair into 0x6400 gives 1024 + q;
//     a packed add, or a packed FMA by 1/16 for the high nibbles, with -(1024 + z)
//     or -(64 + z) gives q - z without rounding), and acc += d * sum; a wave that
//     meets a zero outside that range (only one-signed groups have one) takes the
//     general route for that stage: exact q, and the zero applied as
//     z * sum_k x_s with sum_k x_s from an MFMA of the same fragment against ones;
//   * products accumulate in float32; the loss epilogue forms each residual, its
//     square and the tile's sum in float64 in a fixed order and writes one partial;
//     a one-workgroup kernel adds the partials in index order, so the loss is
//     reproducible run to run.
//
// Fragments (v_mfma_f32_16x16x32_f16): lane (j, c) = (l / 16, l % 16) holds
// A[m = c][8 k-slots of slot group j] and B[the same slots][n = c]; D[m = 4 j + i]
// [n = c]. At step st of a stage, slot group j takes the 8 inputs of chunk
// 4 j + st, so a lane reads 64 contiguous weight bytes, or one 16-byte chunk of
// codes, per stage of its row.
#include <algorithm>

#include "device_utils.h"
#include "launchers.h"

namespace w4a16 {

namespace {


constexpr int MT = 4;                 // 16-row MFMA tiles of t per workgroup
constexpr int WAVES = 8;
constexpr int BM = 16 * MT;           // 64 rows t
constexpr int BN = 16 * WAVES;        // 128 rows n
constexpr int kThreads = 64 * WAVES;
constexpr int XU = BM * 16 / kThreads;  // 16-byte input chunks per thread per stage
constexpr int R = 2;                  // stages of loads in flight ahead of the compute

static_assert(R % 2 == 0, "the LDS buffer of each unrolled stage must be fixed");




// Loads of one stage's input tile into registers, and their store into LDS (rows
// XOR-free: the row pitch of 17 chunks keeps the 16 lanes of a read on distinct banks).
struct InputTile {
  int off[XU];
  __device__ InputTile(int t, int K) {
#pragma unroll
    for (int u = 0; u < XU; ++u) off[u] = ((t >> 4) + (kThreads / 16) * u) * K * 2 + (t & 15) * 16;
  }
};

struct Lds {
  u32x4_t x[2][BM][17];
};

__device__ __forceinline__ void store_tile(Lds& lds, int b, const u32x4_t (&v)[XU], int t) {
#pragma unroll
  for (int u = 0; u < XU; ++u) lds.x[b][(t >> 4) + (kThreads / 16) * u][t & 15] = v[u];
}

// ---------------------------------------------------------------- the quantized product

struct QuantStage {
  u32x4_t x[XU];
  u32x4_t q;
  uint16_t s, z;
};

__global__ __launch_bounds__(kThreads) void alpha_loss_kernel(const uint16_t* __restrict__ xs,
                                                             const uint32_t* __restrict__ qw,
                                                             const uint16_t* __restrict__ scales,
                                                             const uint16_t* __restrict__ zeros,
                                                             const float* __restrict__ yref, int T, int N, int K,
                                                             int GT, double* __restrict__ partials) {
  __shared__ Lds lds;
  __shared__ double wsum[WAVES];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int j = lane >> 4, c = lane & 15;
  // the calibration tiles of one weight tile share an XCD
  const int tile = xcd_contiguous_item(blockIdx.x, gridDim.x);
  const int m0 = (tile % GT) * BM, n0 = (tile / GT) * BN;
  const int G = K >> 7;
  const int nl = wave * 16 + c;  // this lane's output row within the tile

  // each resource spans only this tile's rows (at most 32 MiB), so an offset plus
  // kOutOfRange always lies past it
  const int64_t rows_t = min(T - m0, BM), rows_n = min(N - n0, BN);
  const __amdgpu_buffer_rsrc_t rx = rsrc(xs + (int64_t)m0 * K, rows_t * K * 2);
  const __amdgpu_buffer_rsrc_t rq = rsrc(qw + (int64_t)n0 * (K >> 3), rows_n * (K >> 1));
  const __amdgpu_buffer_rsrc_t rs = rsrc(scales + (int64_t)n0 * G, rows_n * G * 2);
  const __amdgpu_buffer_rsrc_t rz = rsrc(zeros + (int64_t)n0 * G, rows_n * G * 2);
  const InputTile xin(t, K);
  const int qo = nl * (K >> 1) + j * 16;
  const int so = nl * G * 2;

  QuantStage set[R];
  auto issue = [&](int g, QuantStage& r) {
    const int past = (int)(g >= G) * kOutOfRange;
#pragma unroll
    for (int u = 0; u < XU; ++u) r.x[u] = load16(rx, xin.off[u] + g * 256 + past);
    r.q = load16(rq, qo + g * 64 + past);
    r.s = __builtin_amdgcn_raw_buffer_load_b16(rs, so + g * 2 + past, 0, 0);
    r.z = __builtin_amdgcn_raw_buffer_load_b16(rz, so + g * 2 + past, 0, 0);
  };

  float4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = (float4_t){0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const QuantStage& r, int b) {
    // x fragments one m-tile ahead: the next tile's LDS reads overlap this tile's MFMAs
    half8_t xa[2][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) xa[0][st] = as_half8(lds.x[b][c][4 * j + st]);
    const float d = half_bits_to_float(r.s);
    const _Float16 zh = __builtin_bit_cast(_Float16, r.z);
    const float zf = (float)zh;
    const bool exact = zf >= -2032.0f && zf <= 1024.0f;
    const bool fast = __builtin_amdgcn_ballot_w64(!exact) == 0;
    const _Float16 clo = fast ? -((_Float16)1024.0f + zh) : (_Float16)-1024.0f;
    const _Float16 chi = fast ? -((_Float16)64.0f + zh) : (_Float16)-64.0f;
    const half2_t c_lo = {clo, clo}, c_hi = {chi, chi};
    const half8_t bq[4] = {dequant_word(r.q.x, c_lo, c_hi), dequant_word(r.q.y, c_lo, c_hi),
                           dequant_word(r.q.z, c_lo, c_hi), dequant_word(r.q.w, c_lo, c_hi)};
    const u32x4_t ones_bits = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
    const half8_t ones = as_half8(ones_bits);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt + 1 < MT) {
#pragma unroll
        for (int st = 0; st < 4; ++st) xa[(mt + 1) & 1][st] = as_half8(lds.x[b][16 * (mt + 1) + c][4 * j + st]);
      }
      float4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) a = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[mt & 1][st], bq[st], a, 0, 0, 0);
      if (fast) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][i] = __builtin_fmaf(d, a[i], acc[mt][i]);
      } else {
        float4_t sx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[mt & 1][st], ones, sx, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][i] = __builtin_fmaf(d, __builtin_fmaf(-zf, sx[i], a[i]), acc[mt][i]);
      }
    }
  };

#pragma unroll
  for (int r = 0; r < R; ++r) {
    issue(r, set[r]);
    __builtin_amdgcn_sched_barrier(0);  // stages stay in issue order: the waits count on it
  }
  store_tile(lds, 0, set[0].x, t);
  lds_barrier();
  for (int g0 = 0; g0 < G; g0 += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int g = g0 + r;
      if (g < G) compute(set[r], r & 1);
      __builtin_amdgcn_sched_barrier(0);
      issue(g + R, set[r]);  // this set's stage is computed: refill it
      __builtin_amdgcn_sched_barrier(0);
      store_tile(lds, (r + 1) & 1, set[(r + 1) % R].x, t);  // the buffer every wave left at the last barrier
      lds_barrier();
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load in flight at exit

  // the reference entries of this lane's 16 outputs, loaded together (indices clamped
  // into the matrix, invalid outputs masked afterwards)
  const int n = n0 + nl;
  const int64_t ncol = min(n, N - 1);
  float yr[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) yr[mt][i] = yref[(int64_t)min(m0 + 16 * mt + 4 * j + i, T - 1) * N + ncol];
  double e2 = 0.0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = m0 + 16 * mt + 4 * j + i < T && n < N;
      const double e = valid ? (double)acc[mt][i] - (double)yr[mt][i] : 0.0;
      e2 += e * e;
    }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) e2 += __shfl_xor(e2, off, 64);
  if (lane == 0) wsum[wave] = e2;
  __syncthreads();
  if (t == 0) {
    double sum = 0.0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += wsum[w];
    partials[tile] = sum;
  }
}

__global__ __launch_bounds__(256) void sum_partials_kernel(const double* __restrict__ partials, int64_t count,
                                                          double* __restrict__ loss) {
  __shared__ double wsum[4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  double acc = 0.0;
  for (int64_t i = t; i < count; i += 256) acc += partials[i];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) wsum[wave] = acc;
  __syncthreads();
  if (t == 0) *loss = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
}

// ---------------------------------------------------------------- the original layer's output

struct DenseStage {
  u32x4_t x[XU];
  u32x4_t w[4];
};

__global__ __launch_bounds__(kThreads) void output_reference_kernel(const uint16_t* __restrict__ x,
                                                                   const uint16_t* __restrict__ w, int T, int N,
                                                                   int K, int GT, float* __restrict__ y) {
  __shared__ Lds lds;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int j = lane >> 4, c = lane & 15;
  // the calibration tiles of one weight tile share an XCD
  const int tile = xcd_contiguous_item(blockIdx.x, gridDim.x);
  const int m0 = (tile % GT) * BM, n0 = (tile / GT) * BN;
  const int G = K >> 7;
  const int nl = wave * 16 + c;

  const int64_t rows_t = min(T - m0, BM), rows_n = min(N - n0, BN);
  const __amdgpu_buffer_rsrc_t rx = rsrc(x + (int64_t)m0 * K, rows_t * K * 2);
  const __amdgpu_buffer_rsrc_t rw = rsrc(w + (int64_t)n0 * K, rows_n * K * 2);
  const InputTile xin(t, K);
  const int wo = nl * K * 2 + j * 64;

  DenseStage set[R];
  auto issue = [&](int g, DenseStage& r) {
    const int past = (int)(g >= G) * kOutOfRange;
#pragma unroll
    for (int u = 0; u < XU; ++u) r.x[u] = load16(rx, xin.off[u] + g * 256 + past);
#pragma unroll
    for (int st = 0; st < 4; ++st) r.w[st] = load16(rw, wo + g * 256 + st * 16 + past);
  };

  float4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = (float4_t){0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const DenseStage& r, int b) {
    // x fragments one m-tile ahead, as in the loss kernel
    half8_t xa[2][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) xa[0][st] = as_half8(lds.x[b][c][4 * j + st]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt + 1 < MT) {
#pragma unroll
        for (int st = 0; st < 4; ++st) xa[(mt + 1) & 1][st] = as_half8(lds.x[b][16 * (mt + 1) + c][4 * j + st]);
      }
#pragma unroll
      for (int st = 0; st < 4; ++st)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[mt & 1][st], as_half8(r.w[st]), acc[mt], 0, 0, 0);
    }
  };

#pragma unroll
  for (int r = 0; r < R; ++r) {
    issue(r, set[r]);
    __builtin_amdgcn_sched_barrier(0);
  }
  store_tile(lds, 0, set[0].x, t);
  lds_barrier();
  for (int g0 = 0; g0 < G; g0 += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int g = g0 + r;
      if (g < G) compute(set[r], r & 1);
      __builtin_amdgcn_sched_barrier(0);
      issue(g + R, set[r]);
      __builtin_amdgcn_sched_barrier(0);
      store_tile(lds, (r + 1) & 1, set[(r + 1) % R].x, t);
      lds_barrier();
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);

  const int n = n0 + nl;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 16 * mt + 4 * j + i;
      if (m < T && n < N) y[(int64_t)m * N + n] = acc[mt][i];
    }
}

int64_t tiles(int64_t T, int64_t N) { return ((T + BM - 1) / BM) * ((N + BN - 1) / BN); }

}  // namespace

int64_t alpha_loss_partials(int64_t T, int64_t N) { return tiles(T, N); }

namespace {

// The grid search's choice: the first index of the smallest loss (strictly smaller losses
// replace the best so far, so equal losses keep the smaller alpha), its alpha = index / 20,
// and the candidate scale of that index copied out. Every workgroup takes the (tiny) argmin
// itself and copies its slice of the scale.
__global__ __launch_bounds__(256) void search_select_kernel(const double* __restrict__ losses, int count,
                                                            const float* __restrict__ s_all, int64_t K,
                                                            int32_t* __restrict__ best, double* __restrict__ alpha,
                                                            float* __restrict__ s) {
  int b = 0;
  double v = losses[0];
  for (int i = 1; i < count; ++i) {
    const double l = losses[i];
    if (l < v) {
      v = l;
      b = i;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *best = b;
    *alpha = (double)b / (double)(count - 1);
  }
  if (s) {
    const float* src = s_all + (int64_t)b * K;
    for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < K; k += (int64_t)gridDim.x * 256) s[k] = src[k];
  }
}

}  // namespace

hipError_t launch_search_select(const double* losses, int count, const float* s_all, int64_t K, int32_t* best,
                                double* alpha, float* s, hipStream_t stream) {
  const int64_t blocks = s ? std::min<int64_t>((K + 255) / 256, 1024) : 1;
  hipLaunchKernelGGL(search_select_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, losses, count, s_all, K, best,
                     alpha, s);
  return hipGetLastError();
}

hipError_t launch_output_reference(const uint16_t* x, const uint16_t* w, int64_t T, int64_t N, int64_t K, float* y,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(output_reference_kernel, dim3((unsigned)tiles(T, N)), dim3(kThreads), 0, stream, x, w, (int)T,
                     (int)N, (int)K, (int)((T + BM - 1) / BM), y);
  return hipGetLastError();
}

hipError_t launch_alpha_loss(const uint16_t* x_s, const uint32_t* qweight, const uint16_t* scales,
                             const uint16_t* zeros, const float* y_ref, int64_t T, int64_t N, int64_t K,
                             double* partials, double* loss, hipStream_t stream) {
  const int64_t nt = tiles(T, N);
  hipLaunchKernelGGL(alpha_loss_kernel, dim3((unsigned)nt), dim3(kThreads), 0, stream, x_s, qweight, scales, zeros,
                     y_ref, (int)T, (int)N, (int)K, (int)((T + BM - 1) / BM), partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sum_partials_kernel, dim3(1), dim3(256), 0, stream, partials, nt, loss);
  return hipGetLastError();
}

}  // namespace w4a16
