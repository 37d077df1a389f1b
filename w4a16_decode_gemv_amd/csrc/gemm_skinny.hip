// W4A16 product for small batches (2 <= M <= 32) on fp16 MFMA.
//
// y[m][n] = sum_g d[n][g] * (sum_{k in g} x[m][k] * q[n][k] - z[n][g] * sum_{k in g} x[m][k])
//
// Small-batch decode is still bound by the weight stream ("MIT 6.5940 L13 LLM
// Deployment" guide: decode reads every weight once per step; the W4A16
// benefit fades only once the batch makes the layer compute-bound), but with
// M > 1 the per-weight multiply work grows M-fold, which a matrix-core tile
// absorbs without extra VALU time.
//
// Shape of the kernel, chosen for a weight stream that must stay at HBM rate:
//   * a workgroup owns ROWS = 16 * NTW output columns n and the whole of K, so
//     no partial sums leave the chip; its 8 waves split the K groups evenly and
//     their 16 x 16 fp32 tiles are summed in a fixed order at the end;
//   * each wave streams its groups in stages of two (16 rows x 128 bytes of
//     codes per 8 lanes: whole 128-byte lines), two stages in flight; a stage's
//     codes pass through a one-stage LDS area private to the wave (no
//     workgroup barrier) to reach the MFMA B-fragment layout;
//   * x reaches the A fragments straight from L2 (it is small and shared by all
//     workgroups); the k-slot assignment makes each x load 64 contiguous bytes
//     per row. For M <= 8 a stage's x rows instead arrive in M/2 full-width loads
//     (512 contiguous bytes per row) and pass through a wave-private LDS area: a
//     16-row fragment load spends its lanes on rows past M, and this cuts the
//     x load instructions per stage from 8 to 1-4 (measured 6-20 % faster at
//     M = 2..8 on the LLaMA shapes);
//   * every load is a buffer load: rows past M or N and groups past a wave's
//     share read as zero through the range check, which costs no memory
//     traffic and adds exactly zero, so the stage sequence is a fixed,
//     branch-free pipeline whose waits the compiler can count statically.
//
// The weights enter the MFMA as exact fp16 integers q (OR-ing a nibble pair into
// 0x6400 gives 1024 + q; one packed add, or a packed FMA by 1/16 for the high
// nibbles, removes the 1024), and the zero is applied per group as
// z * sum_k x, with sum_k x from an MFMA of the same x fragment against ones;
// this is exact for every zero the quantizer can store, so there is no
// data-dependent branch (a branch on the zeros would let the compiler delay the
// whole weight stream behind the zero loads).
//
// MFMA 16x16x32 f16 fragments: lane l holds A[m = l%16][8 k-slots of slot group
// l/16] and B[the same k-slots][n = l%16]; D[m = 4(l/16) + i][n = l%16]. At step
// q (0..3) of a group, slot group j takes the 8 inputs of code word 4q + j, so
// lane (j, n) needs words j, 4+j, 8+j, 12+j of row n's group: the LDS area is
// written in that order, one 16-byte slot per (row, group, j), XOR-swizzled by
// row so that neither the writes nor the reads collide in LDS banks.
#include "device_utils.h"
#include "launchers.h"

namespace w4a16 {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int KS = 8;               // waves per workgroup, splitting K
constexpr int kThreads = KS * 64;
constexpr int D = 2;                // stages in flight per wave
constexpr int kMaxStages = 8;       // stages per chunk of the largest kernel variant
constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3: 32-bit raw data, range-checked
constexpr int kOutOfRange = 1 << 30;      // added to an offset: past every buffer range used here
constexpr int kNonTemporal = 2;           // streaming hint for the code loads (read once)

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

// NS stages (2 * NS groups) per wave and chunk; K beyond one chunk per wave loops over chunks
// XI > 0 (M <= 2 XI <= 8, MT = 1): a stage's x rows arrive in XI full-width loads (lane l of
// load i takes row 2i + l/32, 16-byte piece l%32 of the stage's 512 bytes) and reach the A
// fragments through a wave-private LDS area; XI = 0: A fragments loaded straight from L2
template <int NTW, int MT, int NS, int XI>
__global__ __launch_bounds__(kThreads) void skinny_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint16_t* __restrict__ zeros, int M, int N, int K,
                                                         uint16_t* __restrict__ y) {
  constexpr int ROWS = 16 * NTW;
  constexpr int CG = 2 * NS;                       // groups per wave and chunk
  constexpr int SZL = (ROWS * CG + 63) / 64;       // (scale, zero) pairs per lane and chunk
  static_assert(ROWS * 8 >= NTW * MT * 64, "the final combine reuses the code staging area");
  __shared__ u32x4_t lds_b[KS][ROWS * 8];          // one stage of codes: ROWS x (2 groups x 4 slots)
  __shared__ uint32_t lds_sz[KS][ROWS][CG + 1];    // one chunk of (scale | zero << 16)
  __shared__ u32x4_t lds_x[XI > 0 ? KS : 1][XI > 0 ? D : 1][XI > 0 ? 2 * XI : 1][33];  // x rows, padded

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int j = lane >> 4, c = lane & 15;   // fragment slot group, fragment row
  const int lr = lane & 7, lq = lane >> 3;  // code load: row within 8, 16-byte piece within the stage
  const int n0 = blockIdx.x * ROWS;
  const int rows = min(ROWS, N - n0);
  const int G = K >> 7;
  const int gb = (w * G) / KS;
  const int ng = ((w + 1) * G) / KS - gb;   // this wave's groups [gb, gb + ng); may be 0 when G < 8
  const int nchunks = (((G + KS - 1) / KS) + CG - 1) / CG;

  // buffer views: this workgroup's code, scale and zero rows, and all of x
  const __amdgpu_buffer_rsrc_t q_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(qw + (int64_t)n0 * (K >> 3)), (short)0, rows * (K >> 1), kBufferFlags);
  const __amdgpu_buffer_rsrc_t s_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(scales + (int64_t)n0 * G), (short)0, rows * G * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t z_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(zeros + (int64_t)n0 * G), (short)0, rows * G * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t x_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, M * K * 2, kBufferFlags);

  const u32x4_t ones_bits = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
  const half8_t ones = as_half8(ones_bits);
  uint32_t* lds_words = reinterpret_cast<uint32_t*>(&lds_b[w][0]);

  float4_t acc[NTW][MT];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = (float4_t){0.f, 0.f, 0.f, 0.f};

  for (int ch = 0; ch < nchunks; ++ch) {
    const int g0 = gb + ch * CG;            // first group of the chunk
    const int nv = ng - ch * CG;            // groups of the chunk inside the wave's share (may be <= 0)
    // plain arithmetic, not a select: a select would let the compiler split each load in two
    auto bias = [&](int gi) { return (int)(gi >= nv) * kOutOfRange; };

    // (scale, zero) of the chunk: lane -> (row, SZL consecutive groups)
    uint16_t sv[SZL], zv[SZL];
    const int sz_row = (lane * SZL) / CG, sz_g = (lane * SZL) % CG;
#pragma unroll
    for (int e = 0; e < SZL; ++e) {
      const int gi = sz_g + e;
      const int o = min(sz_row, ROWS - 1) * G * 2 + (g0 + gi) * 2 + bias(gi) + (int)(sz_row >= ROWS) * kOutOfRange;
      sv[e] = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, o, 0, 0);
      zv[e] = __builtin_amdgcn_raw_buffer_load_b16(z_rsrc, o, 0, 0);
    }

    u32x4_t cr[D][NTW][2];
    u32x4_t xr[D][2][MT][4];
    u32x4_t xl[D][XI > 0 ? XI : 1];
    auto load_codes = [&](int s, int slot) {
      const int gi = 2 * s + (lq >> 2);
      const int off = (g0 + gi) * 64 + 16 * (lq & 3) + bias(gi);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          cr[slot][nt][h] = __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, off + (16 * nt + 8 * h + lr) * (K >> 1), 0,
                                                                  kNonTemporal);
    };
    auto load_x = [&](int s, int slot) {
      if constexpr (XI > 0) {
        const int gi = 2 * s + ((lane & 31) >> 4);
        const int off = (g0 + 2 * s) * 256 + 16 * (lane & 31) + bias(gi);
#pragma unroll
        for (int i = 0; i < XI; ++i)
          xl[slot][i] = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, off + (2 * i + (lane >> 5)) * K * 2, 0, 0);
        return;
      }
#pragma unroll
      for (int gs = 0; gs < 2; ++gs) {
        const int gi = 2 * s + gs;
        const int off = (g0 + gi) * 256 + 16 * j + bias(gi);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int o = (16 * mt + c) * K * 2 + off;  // rows past M: out of range (buffer size M * K * 2)
#pragma unroll
          for (int q = 0; q < 4; ++q) xr[slot][gs][mt][q] = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, o + 64 * q, 0, 0);
        }
      }
    };
#pragma unroll
    for (int s = 0; s < D && s < NS; ++s) {
      load_codes(s, s);
      load_x(s, s);
    }
    // the scheduler would otherwise sink prefetches down to their first use
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int e = 0; e < SZL; ++e)
      if (sz_row < ROWS) lds_sz[w][sz_row][sz_g + e] = (uint32_t)sv[e] | ((uint32_t)zv[e] << 16);

#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int u = s % D;
      // stage codes -> LDS: piece lq holds words 4(lq%4) .. +3 of group lq/4; word 4p + e goes to
      // slot (row, group, j = e) at dword p
      {
        const int gs = lq >> 2, p = lq & 3;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int row = 16 * nt + 8 * h + lr;
            const int swz = (row >> 1) & 7;
            const u32x4_t v = cr[u][nt][h];
            lds_words[(row * 8 + ((gs * 4 + 0) ^ swz)) * 4 + p] = v.x;
            lds_words[(row * 8 + ((gs * 4 + 1) ^ swz)) * 4 + p] = v.y;
            lds_words[(row * 8 + ((gs * 4 + 2) ^ swz)) * 4 + p] = v.z;
            lds_words[(row * 8 + ((gs * 4 + 3) ^ swz)) * 4 + p] = v.w;
          }
      }
      if constexpr (XI > 0) {
#pragma unroll
        for (int i = 0; i < XI; ++i) lds_x[w][u][2 * i + (lane >> 5)][lane & 31] = xl[u][i];
      }
      if (s + D < NS) load_codes(s + D, u);
      if constexpr (XI > 0) {
        if (s + D < NS) load_x(s + D, u);
      }
      __builtin_amdgcn_sched_barrier(0);

#pragma unroll
      for (int gs = 0; gs < 2; ++gs) {
        const int gi = 2 * s + gs;
        if constexpr (XI > 0) {
          // A fragments from the LDS copy; rows past M read row 0 (their results are never stored)
          const int xrow = c < M ? c : 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) xr[u][gs][0][q] = lds_x[w][u][xrow][16 * gs + 4 * q + j];
        }
        float4_t sx[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          sx[mt] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            sx[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(xr[u][gs][mt][q]), ones, sx[mt], 0, 0, 0);
        }
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const int row = 16 * nt + c;
          const u32x4_t wq = lds_b[w][row * 8 + ((gs * 4 + j) ^ ((row >> 1) & 7))];
          const uint32_t szv = lds_sz[w][row][gi];
          const float d = half_bits_to_float((uint16_t)(szv & 0xFFFFu));
          const float zf = half_bits_to_float((uint16_t)(szv >> 16));
          const half8_t b0 = codes_word(wq.x), b1 = codes_word(wq.y), b2 = codes_word(wq.z), b3 = codes_word(wq.w);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            float4_t a4 = {0.f, 0.f, 0.f, 0.f};
            a4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(xr[u][gs][mt][0]), b0, a4, 0, 0, 0);
            a4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(xr[u][gs][mt][1]), b1, a4, 0, 0, 0);
            a4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(xr[u][gs][mt][2]), b2, a4, 0, 0, 0);
            a4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(xr[u][gs][mt][3]), b3, a4, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[nt][mt][i] = __builtin_fmaf(d, __builtin_fmaf(-zf, sx[mt][i], a4[i]), acc[nt][mt][i]);
          }
        }
      }
      if constexpr (XI == 0) {
        if (s + D < NS) load_x(s + D, u);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // combine the 8 waves' tiles in a fixed order; each wave's partials go to its own staging area
  float4_t* red = reinterpret_cast<float4_t*>(&lds_b[w][0]);
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[(nt * MT + mt) * 64 + lane] = acc[nt][mt];
  __syncthreads();
  for (int o = t; o < 16 * MT * ROWS; o += kThreads) {
    const int m = o / ROWS, nl = o - m * ROWS;
    if (m < M && nl < rows) {
      const int nt = nl >> 4, mt = m >> 4, mm = m & 15;
      const int ln = (mm >> 2) * 16 + (nl & 15), i = mm & 3;
      float sum = 0.f;
#pragma unroll
      for (int ww = 0; ww < KS; ++ww) sum += reinterpret_cast<const float4_t*>(&lds_b[ww][0])[(nt * MT + mt) * 64 + ln][i];
      y[(int64_t)m * N + n0 + nl] = float_to_half_bits(sum);
    }
  }
}

template <int NTW, int MT, int NS, int XI>
hipError_t launch_tile_x(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                         int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const dim3 grid((unsigned)((N + 16 * NTW - 1) / (16 * NTW)));
  hipLaunchKernelGGL((skinny_kernel<NTW, MT, NS, XI>), grid, dim3(kThreads), 0, stream, x, qweight, scales, zeros,
                     (int)M, (int)N, (int)K, y);
  return hipGetLastError();
}

template <int NTW, int MT, int NS>
hipError_t launch_tile(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                       int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  if constexpr (MT == 1) {
    if (M <= 2) return launch_tile_x<NTW, MT, NS, 1>(x, qweight, scales, zeros, M, N, K, y, stream);
    if (M <= 4) return launch_tile_x<NTW, MT, NS, 2>(x, qweight, scales, zeros, M, N, K, y, stream);
    if (M <= 8) return launch_tile_x<NTW, MT, NS, 4>(x, qweight, scales, zeros, M, N, K, y, stream);
  }
  return launch_tile_x<NTW, MT, NS, 0>(x, qweight, scales, zeros, M, N, K, y, stream);
}

template <int NTW, int MT>
hipError_t launch_stages(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                         int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const int64_t stages = ((K / 128 + KS - 1) / KS + 1) / 2;  // per wave
  if (stages <= 2) return launch_tile<NTW, MT, 2>(x, qweight, scales, zeros, M, N, K, y, stream);
  if (stages <= 4) return launch_tile<NTW, MT, 4>(x, qweight, scales, zeros, M, N, K, y, stream);
  if (stages <= 6) return launch_tile<NTW, MT, 6>(x, qweight, scales, zeros, M, N, K, y, stream);
  return launch_tile<NTW, MT, kMaxStages>(x, qweight, scales, zeros, M, N, K, y, stream);
}

}  // namespace

int skinny_max_m() { return 32; }

hipError_t launch_skinny(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                         int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  // two column tiles per wave halve the x traffic per code byte, as long as that still leaves
  // one workgroup for each of the 256 compute units
  // (with two m-tiles, only up to 4 stages per wave: beyond that the two-tile variant runs out
  // of registers)
  const bool wide = (N + 31) / 32 >= 256;
  if (M <= 16) return wide ? launch_stages<2, 1>(x, qweight, scales, zeros, M, N, K, y, stream)
                           : launch_stages<1, 1>(x, qweight, scales, zeros, M, N, K, y, stream);
  const bool short_k = ((K / 128 + KS - 1) / KS + 1) / 2 <= 4;
  return wide && short_k ? launch_stages<2, 2>(x, qweight, scales, zeros, M, N, K, y, stream)
                         : launch_stages<1, 2>(x, qweight, scales, zeros, M, N, K, y, stream);
}

}  // namespace w4a16
