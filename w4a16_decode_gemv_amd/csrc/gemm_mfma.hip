// W4A16 GEMM on fp16 MFMA for batches large enough to be a dense contraction.
//
// y[m][n] = sum_g d[n][g] * ( sum_{k in g} x[m][k] * q[n][k]  -  z[n][g] * sum_{k in g} x[m][k] )
//
// Same fused dequantize + multiply as the GEMV ("MIT 6.5940 L13 LLM Deployment"
// guide, TinyChat kernel fusion), but once many rows of x share each weight
// the work is compute-bound and belongs on the matrix cores ("CMU 11-868 Model
// Quantization" guide: large-batch speedups do not carry over; L13 QServe:
// dequantization inside a GEMM main loop costs ALU time, so it is done once per
// tile into LDS and the MFMA main loop reads fp16 only).
//
// Tile: 64 (m) x 64 (n), stepping one quantization group (128 inputs) at a
// time; 4 waves, each owning a 32 x 32 block computed with
// v_mfma_f32_32x32x16_f16. Per group:
//   * x[m0:m0+64][128g : 128g+128] is copied to LDS;
//   * the matching codes are unpacked to exact fp16 q in LDS (one AND-OR and
//     one packed add per input pair, as in the GEMV);
//   * sum_k x over the group is formed per row m (zero-point term);
//   * the MFMA chain over the group's 128 inputs gives sum q x in float32, and
//     the group is folded in as acc += d * (sum q x - z * sum x).
// Applying d per group keeps q exact in fp16 for every z, so the only
// roundings are the float32 accumulation and the final fp16 store.
#include "device_utils.h"
#include "launchers.h"

namespace w4a16 {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 64;
constexpr int BN = 64;
constexpr int GK = 128;        // inputs per group = K-step
constexpr int LDA = GK + 8;    // padded LDS row (halves)

__device__ __forceinline__ uint32_t q_pair_lo_bits(uint32_t w) {
  const half2_t b = as_half2(and_or(w, 0x000F000Fu, 0x64006400u));
  return __builtin_bit_cast(uint32_t, b - (half2_t){(_Float16)1024.0f, (_Float16)1024.0f});
}

__device__ __forceinline__ uint32_t q_pair_hi_bits(uint32_t w) {
  const half2_t b = as_half2(and_or(w, 0x00F000F0u, 0x64006400u));
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(b, (half2_t){(_Float16)0.0625f, (_Float16)0.0625f},
                                                                (half2_t){(_Float16)-64.0f, (_Float16)-64.0f}));
}

__global__ __launch_bounds__(256) void mfma_kernel(const uint4* __restrict__ x, const uint32_t* __restrict__ qw,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint16_t* __restrict__ zeros, int M, int N, int K,
                                                   uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) _Float16 As[BM * LDA];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[BN * LDA];
  __shared__ float Sx[BM];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int G = K >> 7;
  const int KX = K >> 3;  // uint4 per x row
  const int KW = K >> 3;  // words per code row

  // this lane's output column and its group constants
  const int n_lane = n0 + wn * 32 + (lane & 31);
  const bool n_ok = n_lane < N;

  float16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;

  for (int g = 0; g < G; ++g) {
    // ---- stage A (x) : 64 rows x 16 uint4
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = t + u * 256;
      const int r = i >> 4, c = i & 15;
      uint4 v = {0u, 0u, 0u, 0u};
      if (m0 + r < M) v = x[(int64_t)(m0 + r) * KX + g * 16 + c];
      *reinterpret_cast<uint4*>(&As[r * LDA + c * 8]) = v;
    }
    // ---- stage B (exact q) : 64 rows x 16 words -> 8 halves each
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = t + u * 256;
      const int r = i >> 4, c = i & 15;
      uint32_t w = 0x88888888u;  // any codes: rows past N are never stored
      if (n0 + r < N) w = __builtin_nontemporal_load(&qw[(int64_t)(n0 + r) * KW + g * 16 + c]);
      const uint32_t w8 = w >> 8;
      uint4 h;
      h.x = q_pair_lo_bits(w);   // k = 8c + 0, 1
      h.y = q_pair_hi_bits(w);   // k = 8c + 2, 3
      h.z = q_pair_lo_bits(w8);  // k = 8c + 4, 5
      h.w = q_pair_hi_bits(w8);  // k = 8c + 6, 7
      *reinterpret_cast<uint4*>(&Bs[r * LDA + c * 8]) = h;
    }
    __syncthreads();
    // ---- sum of x over the group, per row (4 threads per row, 32 inputs each)
    {
      const int r = t >> 2, part = t & 3;
      float s = 0.f;
      const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 v = *reinterpret_cast<const uint4*>(&As[r * LDA + part * 32 + c * 8]);
        s = __builtin_amdgcn_fdot2(as_half2(v.x), ones, s, false);
        s = __builtin_amdgcn_fdot2(as_half2(v.y), ones, s, false);
        s = __builtin_amdgcn_fdot2(as_half2(v.z), ones, s, false);
        s = __builtin_amdgcn_fdot2(as_half2(v.w), ones, s, false);
      }
      s += __shfl_xor(s, 1, 4);
      s += __shfl_xor(s, 2, 4);
      if (part == 0) Sx[r] = s;
    }
    // ---- MFMA chain over the group: lane holds A[m = l%32][k = 8(l/32) + i], B[k][n = l%32]
    float16_t accg;
#pragma unroll
    for (int i = 0; i < 16; ++i) accg[i] = 0.f;
    const int arow = wm * 32 + (lane & 31);
    const int brow = wn * 32 + (lane & 31);
    const int kofs = 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < GK; ks += 16) {
      const half8_t a = *reinterpret_cast<const half8_t*>(&As[arow * LDA + ks + kofs]);
      const half8_t b = *reinterpret_cast<const half8_t*>(&Bs[brow * LDA + ks + kofs]);
      accg = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, accg, 0, 0, 0);
    }
    __syncthreads();  // Sx written; also every wave is done reading As/Bs
    float d = 0.f, z = 0.f;
    if (n_ok) {
      d = half_bits_to_float(scales[(int64_t)n_lane * G + g]);
      z = half_bits_to_float(zeros[(int64_t)n_lane * G + g]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int mloc = wm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      acc[i] = __builtin_fmaf(d, __builtin_fmaf(-z, Sx[mloc], accg[i]), acc[i]);
    }
    __syncthreads();  // Sx is rewritten next group
  }

  if (n_ok) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = m0 + wm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (m < M) y[(int64_t)m * N + n_lane] = float_to_half_bits(acc[i]);
    }
  }
}

}  // namespace

hipError_t launch_mfma(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                       int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  hipLaunchKernelGGL(mfma_kernel, grid, dim3(256), 0, stream, reinterpret_cast<const uint4*>(x), qweight, scales,
                     zeros, (int)M, (int)N, (int)K, y);
  return hipGetLastError();
}

}  // namespace w4a16
