// W4A16 GEMM on fp16 MFMA for batches large enough to be a dense contraction.
//
// y[m][n] = sum_g d[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g])
//
// Same fused dequantize + multiply as the GEMV ("MIT 6.5940 L13 LLM Deployment"
// guide, TinyChat kernel fusion), but once many rows of x share each weight
// the work is compute-bound and belongs on the matrix cores ("CMU 11-868 Model
// Quantization" guide: large-batch speedups do not carry over; L13 QServe:
// dequantization inside a GEMM main loop costs ALU time, so it is kept to a
// few VALU operations per 8 weights, once per weight per workgroup).
//
// Tile: 64 output columns n (4 waves x 16) by BM = 16 * MB rows of x, stepping
// one quantization group (128 inputs) per stage, double-buffered in LDS:
//   * x[m0:m0+BM][128g : 128g+128] and the 64 rows' codes of group g are
//     copied to LDS (global loads for group g+1 are in flight while group g
//     is computed), with the 64 (scale, zero) pairs;
//   * each wave rebuilds its 16 rows' weights as exact fp16 (q - z): OR-ing a
//     nibble pair into 0x6400 gives 1024 + q, and one packed add (or a packed
//     FMA by 1/16 for the high nibbles) with -(1024 + z) (or -(64 + z)) gives
//     q - z with no rounding while z lies in [-2032, 1024];
//   * v_mfma_f32_16x16x32_f16 over the group's 128 inputs gives
//     sum x (q - z) in float32, and acc += d * that.
// A wave meeting a group whose zero lies outside that range (possible only
// for one-signed groups) takes the general route for that group: exact q in
// the MFMA, and the zero applied as z * sum_k x, with sum_k x from an MFMA
// against ones.
//
// MFMA fragments (16x16x32 f16): lane l holds A[m = l%16][8 k-slots of slot
// group l/16] and B[the same 8 k-slots][n = l%16]; D[m = 4(l/16) + i][n = l%16].
// Step s of the 4 steps of a group gives slot group j the 8 inputs of code
// word 4j + s of the row (any assignment of inputs to slots works as long as
// A and B agree), so lane (j, n) needs words 4j..4j+3 of row n: one 16-byte
// read per group, and x[m][32j .. 32j+31]: four 16-byte reads per group.
// LDS rows are padded (17 chunks of x, 20 words of codes) so that the eight
// lanes served together by a 16-byte LDS read hit distinct banks.
#include "device_utils.h"
#include "launchers.h"

namespace w4a16 {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int BN = 64;          // output columns per workgroup (4 waves x 16)
constexpr int kThreads = 256;

__device__ __forceinline__ half8_t as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4_t v = {a, b, c, d};
  return __builtin_bit_cast(half8_t, v);
}

// the four exact fp16 pairs (q - z) of one code word; c_lo = -(1024 + z), c_hi = -(64 + z)
__device__ __forceinline__ half8_t dequant_word(uint32_t w, half2_t c_lo, half2_t c_hi) {
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w8 = w >> 8;
  const half2_t p0 = as_half2(and_or(w, 0x000F000Fu, 0x64006400u)) + c_lo;
  const half2_t p1 = __builtin_elementwise_fma(as_half2(and_or(w, 0x00F000F0u, 0x64006400u)), sixteenth, c_hi);
  const half2_t p2 = as_half2(and_or(w8, 0x000F000Fu, 0x64006400u)) + c_lo;
  const half2_t p3 = __builtin_elementwise_fma(as_half2(and_or(w8, 0x00F000F0u, 0x64006400u)), sixteenth, c_hi);
  return as_half8(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1), __builtin_bit_cast(uint32_t, p2),
                  __builtin_bit_cast(uint32_t, p3));
}

template <int MB>
struct Smem {
  uint4 a[2][16 * MB][17];  // x tile: BM rows x 128 fp16 (16 chunks of 16 B, padded to 17)
  uint32_t b[2][BN][20];    // codes: 64 rows x 16 words (padded to 20)
  uint32_t sz[2][BN];       // (scale | zero << 16)
};

template <int MB>
__global__ __launch_bounds__(kThreads) void mfma_kernel(const uint4* __restrict__ x, const uint4* __restrict__ qw,
                                                        const uint16_t* __restrict__ scales,
                                                        const uint16_t* __restrict__ zeros, int M, int N, int K,
                                                        uint16_t* __restrict__ y) {
  constexpr int BM = 16 * MB;
  constexpr int AU = (BM * 16 + kThreads - 1) / kThreads;  // x chunks per thread per stage
  __shared__ Smem<MB> sm;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int j = lane >> 4, c = lane & 15;  // slot group, row within the wave's 16
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int G = K >> 7;
  const int KX = K >> 3;    // 16-byte x chunks per row
  const int KQ = K >> 5;    // 16-byte code chunks per row

  // staging assignment: codes chunk (row t/4, quarter t%4 = words 4q..4q+3);
  // x chunk index i = t + u * 256 -> (row i / 16, chunk i % 16)
  const int b_row = t >> 2, b_q = t & 3;
  const int64_t b_src = (int64_t)min(n0 + b_row, N - 1) * KQ + b_q;
  const int s_row = min(n0 + (t & 63), N - 1);

  uint4 areg[AU];
  uint4 breg;
  uint16_t sreg = 0, zreg = 0;

  auto load_stage = [&](int g) {
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const int i = t + u * kThreads;
      const int r = i >> 4, ch = i & 15;
      uint4 v = {0u, 0u, 0u, 0u};
      if (i < BM * 16 && m0 + r < M) v = x[(int64_t)(m0 + r) * KX + g * 16 + ch];
      areg[u] = v;
    }
    breg = qw[b_src + 4 * g];
    if (t < BN) {
      sreg = scales[(int64_t)s_row * G + g];
      zreg = zeros[(int64_t)s_row * G + g];
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const int i = t + u * kThreads;
      if (i < BM * 16) sm.a[buf][i >> 4][i & 15] = areg[u];
    }
    *reinterpret_cast<uint4*>(&sm.b[buf][b_row][4 * b_q]) = breg;  // words 4q .. 4q+3, natural order
    if (t < BN) sm.sz[buf][t] = (uint32_t)sreg | ((uint32_t)zreg << 16);
  };

  float4_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = (float4_t){0.f, 0.f, 0.f, 0.f};

  load_stage(0);
  store_stage(0);
  __syncthreads();

  const int n_loc = wave * 16 + c;  // this lane's output column within the tile
  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    if (g + 1 < G) load_stage(g + 1);

    // ---- this lane's (scale, zero) and the 4 code words (one per MFMA step)
    const uint32_t szv = sm.sz[buf][n_loc];
    const float d = half_bits_to_float((uint16_t)(szv & 0xFFFFu));
    const _Float16 zh = __builtin_bit_cast(_Float16, (uint16_t)(szv >> 16));
    const uint4 wq = *reinterpret_cast<const uint4*>(&sm.b[buf][n_loc][4 * j]);
    const uint32_t words[4] = {wq.x, wq.y, wq.z, wq.w};
    const float zf = (float)zh;
    const bool z_ok = (zf >= -2032.0f) && (zf <= 1024.0f);
    const bool wave_ok = __builtin_amdgcn_ballot_w64(!z_ok) == 0;

    if (wave_ok) {
      const _Float16 clo = -((_Float16)1024.0f + zh);
      const _Float16 chi = -((_Float16)64.0f + zh);
      const half2_t c_lo = {clo, clo}, c_hi = {chi, chi};
      half8_t bfrag[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) bfrag[s] = dequant_word(words[s], c_lo, c_hi);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint4* arow = &sm.a[buf][16 * mb + c][4 * j];
        float4_t accg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint4 av = arow[s];
          accg = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(av.x, av.y, av.z, av.w), bfrag[s], accg, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mb][i] = __builtin_fmaf(d, accg[i], acc[mb][i]);
      }
    } else {
      // general route: exact q, zero applied through sum_k x
      const half2_t c_lo = {(_Float16)-1024.0f, (_Float16)-1024.0f};
      const half2_t c_hi = {(_Float16)-64.0f, (_Float16)-64.0f};
      const half8_t ones = as_half8(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
      half8_t bfrag[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) bfrag[s] = dequant_word(words[s], c_lo, c_hi);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint4* arow = &sm.a[buf][16 * mb + c][4 * j];
        float4_t accg = {0.f, 0.f, 0.f, 0.f}, sx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint4 av = arow[s];
          const half8_t a = as_half8(av.x, av.y, av.z, av.w);
          accg = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bfrag[s], accg, 0, 0, 0);
          sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ones, sx, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mb][i] = __builtin_fmaf(d, __builtin_fmaf(-zf, sx[i], accg[i]), acc[mb][i]);
      }
    }

    if (g + 1 < G) {
      __syncthreads();  // every wave is done with the buffer about to be refilled
      store_stage(buf ^ 1);
      __syncthreads();
    }
  }

  const int n = n0 + n_loc;
  if (n < N) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 16 * mb + 4 * j + i;
        if (m < M) y[(int64_t)m * N + n] = float_to_half_bits(acc[mb][i]);
      }
  }
}

template <int MB>
hipError_t launch_mb(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                     int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + 16 * MB - 1) / (16 * MB)));
  hipLaunchKernelGGL(mfma_kernel<MB>, grid, dim3(kThreads), 0, stream, reinterpret_cast<const uint4*>(x),
                     reinterpret_cast<const uint4*>(qweight), scales, zeros, (int)M, (int)N, (int)K, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                       int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  if (M <= 16) return launch_mb<1>(x, qweight, scales, zeros, M, N, K, y, stream);
  if (M <= 32) return launch_mb<2>(x, qweight, scales, zeros, M, N, K, y, stream);
  return launch_mb<4>(x, qweight, scales, zeros, M, N, K, y, stream);
}

}  // namespace w4a16
