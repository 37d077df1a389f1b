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
// one quantization group (128 inputs) per stage, double-buffered in LDS, with the
// global loads of two groups in flight in a register ring for 32- and 64-row tiles
// (group g + 2 is loaded while group g is computed and group g + 1 waits in registers
// for its LDS store; 3-7 % faster than one group ahead on the LLaMA serving shapes):
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


constexpr int BN = 64;          // output columns per workgroup (4 waves x 16)
constexpr int kThreads = 256;
constexpr int kRing = 2;        // stages whose global loads are in flight


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
  constexpr int RING = MB == 1 ? 1 : kRing;  // 16-row tiles (explicit path only, M <= 16) keep one group ahead
  __shared__ Smem<MB> sm;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int j = lane >> 4, c = lane & 15;  // slot group, row within the wave's 16
  // item = n-tile * TM + m-tile: the m-tiles of one weight tile run on one XCD
  const int TM = (M + BM - 1) / BM;
  const int item = xcd_contiguous_item(blockIdx.x, gridDim.x);
  const int m0 = (item % TM) * BM;
  const int n0 = (item / TM) * BN;
  const int G = K >> 7;
  const int KX = K >> 3;    // 16-byte x chunks per row
  const int KQ = K >> 5;    // 16-byte code chunks per row

  // staging assignment: codes chunk (row t/4, quarter t%4 = words 4q..4q+3);
  // x chunk index i = t + u * 256 -> (row i / 16, chunk i % 16)
  const int b_row = t >> 2, b_q = t & 3;
  const int64_t b_src = (int64_t)min(n0 + b_row, N - 1) * KQ + b_q;
  const int s_row = min(n0 + (t & 63), N - 1);

  // register ring of RING groups; native vectors, so that the ring stays in registers
  u32x4_t areg[RING][AU];
  u32x4_t breg[RING];
  uint16_t sreg[RING] = {}, zreg[RING] = {};

  auto load_stage = [&](int g, int sl) {
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const int i = t + u * kThreads;
      const int r = i >> 4, ch = i & 15;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (i < BM * 16 && m0 + r < M) v = *reinterpret_cast<const u32x4_t*>(&x[(int64_t)(m0 + r) * KX + g * 16 + ch]);
      areg[sl][u] = v;
    }
    breg[sl] = *reinterpret_cast<const u32x4_t*>(&qw[b_src + 4 * g]);
    if (t < BN) {
      sreg[sl] = scales[(int64_t)s_row * G + g];
      zreg[sl] = zeros[(int64_t)s_row * G + g];
    }
  };
  auto store_stage = [&](int buf, int sl) {
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const int i = t + u * kThreads;
      if (i < BM * 16) *reinterpret_cast<u32x4_t*>(&sm.a[buf][i >> 4][i & 15]) = areg[sl][u];
    }
    *reinterpret_cast<u32x4_t*>(&sm.b[buf][b_row][4 * b_q]) = breg[sl];  // words 4q .. 4q+3, natural order
    if (t < BN) sm.sz[buf][t] = (uint32_t)sreg[sl] | ((uint32_t)zreg[sl] << 16);
  };

  float4_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = (float4_t){0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int p = 0; p < RING; ++p)
    if (p < G) load_stage(p, p);
  store_stage(0, 0);
  __syncthreads();

  const int n_loc = wave * 16 + c;  // this lane's output column within the tile
  // unrolled by the ring size so that every ring slot is a compile-time index
  for (int g0 = 0; g0 < G; g0 += RING)
#pragma unroll
  for (int kk = 0; kk < RING; ++kk) {
    const int g = g0 + kk;
    if (g >= G) continue;
    const int buf = g & 1;
    // slot kk held group g, stored to LDS one iteration ago: refill it with group g + RING
    if (g + RING < G) load_stage(g + RING, kk);

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
      store_stage(buf ^ 1, (kk + 1) % RING);
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

// ---------------------------------------------------------------------------
// Variants: 3-bit codes and groups of 32 or 64 (and 3-bit with groups of 128), and
// NF4 codes (layout v1 codes into the 16-level codebook, a float32 absmax per block).
// A stage is still 128 inputs, but MFMA step st covers exactly the 32 inputs
// 32 st .. 32 st + 31 (lane (j, c) takes inputs 32 st + 8 j .. + 7), so every
// step lies inside one group and gets its own (scale, zero): acc += d_st * step.
// The LDS code rows are laid out so that a lane reads the words of its four
// steps with one 16-byte read: 4-bit, position 4 j + st holds word 4 st + j (the
// lane's 8 inputs of step st); 3-bit, positions 0..3 / 4..7 / 8..11 hold the
// low-bit word of inputs 0..15, of inputs 16..31, and the high-bit word, of
// pieces 0..3.

constexpr int kNF4 = 16;

template <int MB, int BITS>
struct VarSmem {
  uint4 a[2][16 * MB][17];
  uint32_t b[2][BN][20];
  uint32_t sz[2][BN][4];  // (scale | zero << 16) per row and step
};

// exact fp16 pairs (q - z) of lane j's 8 inputs of a 3-bit piece
__device__ __forceinline__ half8_t dequant3(uint32_t lo, uint32_t hi, int j, half2_t c) {
  const int i0 = 4 * (j & 1), p0 = 4 * j;
  uint32_t v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // bits p and 16 + p of hi (p = p0 + e) rotated to bits 2 and 18
    const uint32_t hp = __builtin_amdgcn_alignbit(hi, hi, (uint32_t)(p0 + e + 30) & 31u);
    const uint32_t t = and_or(hp, 0x00040004u, 0x64006400u);
    v[e] = __builtin_bit_cast(uint32_t, as_half2(and_or(lo >> (2 * (i0 + e)), 0x00030003u, t)) + c);
  }
  return as_half8(v[0], v[1], v[2], v[3]);
}

// fast route of one stage: SPG consecutive steps share a group (SPG = group / 32) and
// chain into one MFMA accumulator, which is scaled once by that group's scale
template <int MB, int SPG>
__device__ __forceinline__ void fast_steps(const uint4 (&a_tile)[16 * MB][17], const half8_t (&bfrag)[4],
                                           const float (&d)[4], int c, int j, float4_t (&acc)[MB]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int g0 = 0; g0 < 4; g0 += SPG) {
      float4_t p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = g0; st < g0 + SPG; ++st) {
        const uint4 av = a_tile[16 * mb + c][4 * st + j];
        p = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(av.x, av.y, av.z, av.w), bfrag[st], p, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[mb][i] = __builtin_fmaf(d[g0], p[i], acc[mb][i]);
    }
  }
}

template <int MB, int BITS>
__global__ __launch_bounds__(kThreads) void mfma_var_kernel(const uint4* __restrict__ x, const uint32_t* __restrict__ qw,
                                                            const void* __restrict__ scales,
                                                            const uint16_t* __restrict__ zeros, int M, int N, int K,
                                                            int gsh, Nf4Table table, uint16_t* __restrict__ y) {
  constexpr int BM = 16 * MB;
  constexpr int AU = (BM * 16 + kThreads - 1) / kThreads;
  constexpr bool NF4 = BITS == kNF4;
  constexpr int RING = MB == 4 ? kRing : 1;
  constexpr int WPS = BITS == 3 ? 12 : 16;  // code words per row per stage
  __shared__ VarSmem<MB, BITS> sm;
  __shared__ __align__(16) _Float16 lut[16];
  if constexpr (NF4) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (threadIdx.x == i) reinterpret_cast<uint32_t*>(lut)[i] = table.pairs[i];
  }

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int j = lane >> 4, c = lane & 15;
  // item = n-tile * TM + m-tile: the m-tiles of one weight tile run on one XCD
  const int TM = (M + BM - 1) / BM;
  const int item = xcd_contiguous_item(blockIdx.x, gridDim.x);
  const int m0 = (item % TM) * BM;
  const int n0 = (item / TM) * BN;
  const int S = K >> 7;            // stages
  const int G = K >> (5 + gsh);    // groups per row
  const int KX = K >> 3;
  const int64_t row_words = (int64_t)(K >> 7) * WPS;

  // codes staging: 4-bit, thread t < 256 copies words 4q..4q+3 of row t / 4; 3-bit, thread t < 192
  // copies words 4q..4q+3 (q = t % 3) of row t / 3
  const int b_row = BITS != 3 ? (t >> 2) : (t / 3);
  const int b_q = BITS != 3 ? (t & 3) : (t % 3);
  const bool b_act = BITS != 3 || t < 192;
  const int64_t b_src = (int64_t)min(n0 + b_row, N - 1) * row_words + 4 * b_q;
  // (scale, zero) staging: thread t -> row t / 4, step t % 4
  const int s_row = min(n0 + (t >> 2), N - 1), s_st = t & 3;

  // register ring of RING stages, as in the 4-bit kernel, with 64-row tiles only (same-box
  // medians, outputs bit-identical: 1-5.5 % faster at M = 256 on 8192 -> 8192 and
  // 4096 -> 11008; with 32-row tiles neutral to 12 % slower, NF4 worst); scale and zero stay in separate
  // registers until the LDS store: combining them at load time would make the wave wait for
  // those loads at once
  u32x4_t areg[RING][AU];
  u32x4_t breg[RING] = {};
  uint32_t sreg[RING] = {};
  uint16_t zreg[RING] = {};
  auto load_stage = [&](int g, int sl) {
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const int i = t + u * kThreads;
      const int r = i >> 4, ch = i & 15;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (i < BM * 16 && m0 + r < M) v = *reinterpret_cast<const u32x4_t*>(&x[(int64_t)(m0 + r) * KX + g * 16 + ch]);
      areg[sl][u] = v;
    }
    if (b_act) breg[sl] = *reinterpret_cast<const u32x4_t*>(qw + b_src + (int64_t)g * WPS);
    const int64_t off = (int64_t)s_row * G + (((g << 2) + s_st) >> gsh);
    if constexpr (NF4) {
      sreg[sl] = __builtin_bit_cast(uint32_t, static_cast<const float*>(scales)[off]);
    } else {
      sreg[sl] = static_cast<const uint16_t*>(scales)[off];
      zreg[sl] = zeros[off];
    }
  };
  auto store_stage = [&](int buf, int sl) {
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const int i = t + u * kThreads;
      if (i < BM * 16) *reinterpret_cast<u32x4_t*>(&sm.a[buf][i >> 4][i & 15]) = areg[sl][u];
    }
    if (b_act) {
      const uint32_t wv[4] = {breg[sl].x, breg[sl].y, breg[sl].z, breg[sl].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int w = 4 * b_q + e;  // word of the stage
        const int pos = BITS != 3 ? (4 * (w & 3) + (w >> 2))    // word 4 st + j -> 4 j + st
                                  : (4 * (w % 3) + w / 3);      // piece w / 3, kind w % 3 -> 4 kind + piece
        sm.b[buf][b_row][pos] = wv[e];
      }
    }
    sm.sz[buf][t >> 2][s_st] = NF4 ? sreg[sl] : (sreg[sl] | ((uint32_t)zreg[sl] << 16));
  };

  float4_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = (float4_t){0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int p = 0; p < RING; ++p)
    if (p < S) load_stage(p, p);
  store_stage(0, 0);
  __syncthreads();  // also publishes the codebook

  const int n_loc = wave * 16 + c;
  const half8_t ones = as_half8(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
  // unrolled by the ring size so that every ring slot is a compile-time index
  for (int g0 = 0; g0 < S; g0 += RING)
#pragma unroll
  for (int kk = 0; kk < RING; ++kk) {
    const int g = g0 + kk;
    if (g >= S) continue;
    const int buf = g & 1;
    // slot kk held stage g, stored to LDS one iteration ago: refill it with stage g + RING
    if (g + RING < S) load_stage(g + RING, kk);

    const uint4 szq = *reinterpret_cast<const uint4*>(&sm.sz[buf][n_loc][0]);
    const uint32_t szs[4] = {szq.x, szq.y, szq.z, szq.w};
    float d[4], zf[4];
    _Float16 zh[4];
    bool ok = true;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if constexpr (NF4) {
        d[st] = __builtin_bit_cast(float, szs[st]);
        zh[st] = (_Float16)0.0f;
      } else {
        d[st] = half_bits_to_float((uint16_t)(szs[st] & 0xFFFFu));
        zh[st] = __builtin_bit_cast(_Float16, (uint16_t)(szs[st] >> 16));
      }
      zf[st] = (float)zh[st];
      ok = ok && zf[st] >= -2032.0f && zf[st] <= 1024.0f;
    }
    const bool fast = NF4 || __builtin_amdgcn_ballot_w64(!ok) == 0;
    // B fragments of the four steps: exact (q - z) on the fast route, exact q otherwise;
    // NF4: the codebook levels
    half8_t bfrag[4];
    if constexpr (NF4) {
      const uint4 wq = *reinterpret_cast<const uint4*>(&sm.b[buf][n_loc][4 * j]);
      const uint32_t words[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        uint32_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t n = words[st] >> (4 * i);
          v[i] = __builtin_bit_cast(uint32_t, (half2_t){lut[n & 15u], lut[(n >> 16) & 15u]});
        }
        bfrag[st] = as_half8(v[0], v[1], v[2], v[3]);
      }
    } else if constexpr (BITS == 4) {
      const uint4 wq = *reinterpret_cast<const uint4*>(&sm.b[buf][n_loc][4 * j]);
      const uint32_t words[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const _Float16 zz = fast ? zh[st] : (_Float16)0.0f;
        const _Float16 clo = -((_Float16)1024.0f + zz), chi = -((_Float16)64.0f + zz);
        bfrag[st] = dequant_word(words[st], (half2_t){clo, clo}, (half2_t){chi, chi});
      }
    } else {
      const uint4 lo = *reinterpret_cast<const uint4*>(&sm.b[buf][n_loc][4 * (j >> 1)]);
      const uint4 hi = *reinterpret_cast<const uint4*>(&sm.b[buf][n_loc][8]);
      const uint32_t los[4] = {lo.x, lo.y, lo.z, lo.w}, his[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const _Float16 zz = fast ? zh[st] : (_Float16)0.0f;
        const _Float16 cc = -((_Float16)1024.0f + zz);
        bfrag[st] = dequant3(los[st], his[st], j, (half2_t){cc, cc});
      }
    }
    if (fast) {
      // the steps of one group chain into one accumulator, scaled once
      if (gsh == 2)
        fast_steps<MB, 4>(sm.a[buf], bfrag, d, c, j, acc);
      else if (gsh == 1)
        fast_steps<MB, 2>(sm.a[buf], bfrag, d, c, j, acc);
      else
        fast_steps<MB, 1>(sm.a[buf], bfrag, d, c, j, acc);
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const uint4 av = sm.a[buf][16 * mb + c][4 * st + j];
          const half8_t a = as_half8(av.x, av.y, av.z, av.w);
          const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};
          const float4_t p = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bfrag[st], zero4, 0, 0, 0);
          const float4_t sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ones, zero4, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mb][i] = __builtin_fmaf(d[st], __builtin_fmaf(-zf[st], sx[i], p[i]), acc[mb][i]);
        }
      }
    }

    if (g + 1 < S) {
      __syncthreads();
      store_stage(buf ^ 1, (kk + 1) % RING);
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

template <int MB, int BITS>
hipError_t launch_var(const uint16_t* x, const uint32_t* qweight, const void* scales, const uint16_t* zeros,
                      int64_t M, int64_t N, int64_t K, int gsh, const Nf4Table& table, uint16_t* y,
                      hipStream_t stream) {
  const dim3 grid((unsigned)(((N + BN - 1) / BN) * ((M + 16 * MB - 1) / (16 * MB))));
  hipLaunchKernelGGL((mfma_var_kernel<MB, BITS>), grid, dim3(kThreads), 0, stream, reinterpret_cast<const uint4*>(x),
                     qweight, scales, zeros, (int)M, (int)N, (int)K, gsh, table, y);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_var_m(const uint16_t* x, const uint32_t* qweight, const void* scales, const uint16_t* zeros,
                        int64_t M, int64_t N, int64_t K, int gsh, const Nf4Table& table, uint16_t* y,
                        hipStream_t stream) {
  if (M <= 16) return launch_var<1, BITS>(x, qweight, scales, zeros, M, N, K, gsh, table, y, stream);
  if (M <= 32) return launch_var<2, BITS>(x, qweight, scales, zeros, M, N, K, gsh, table, y, stream);
  // 32-row tiles while 64-row ones would give fewer than two workgroups per CU (as launch_mfma)
  const int64_t tiles64 = ((M + 63) / 64) * ((N + BN - 1) / BN);
  if (tiles64 < 512) return launch_var<2, BITS>(x, qweight, scales, zeros, M, N, K, gsh, table, y, stream);
  return launch_var<4, BITS>(x, qweight, scales, zeros, M, N, K, gsh, table, y, stream);
}

template <int MB>
hipError_t launch_mb(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                     int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const dim3 grid((unsigned)(((N + BN - 1) / BN) * ((M + 16 * MB - 1) / (16 * MB))));
  hipLaunchKernelGGL(mfma_kernel<MB>, grid, dim3(kThreads), 0, stream, reinterpret_cast<const uint4*>(x),
                     reinterpret_cast<const uint4*>(qweight), scales, zeros, (int)M, (int)N, (int)K, y);
  return hipGetLastError();
}

}  // namespace

int64_t mfma_workgroups(int64_t M, int64_t N) {
  const int64_t tn = (N + BN - 1) / BN;
  if (M <= 16) return tn * M;
  if (M <= 32) return tn * ((M + 31) / 32);
  const int64_t tiles64 = ((M + 63) / 64) * tn;
  return tiles64 < 512 ? ((M + 31) / 32) * tn : tiles64;
}

hipError_t launch_mfma(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                       int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  if (M <= 16) return launch_mb<1>(x, qweight, scales, zeros, M, N, K, y, stream);
  if (M <= 32) return launch_mb<2>(x, qweight, scales, zeros, M, N, K, y, stream);
  // 32-row tiles while 64-row ones would give fewer than two workgroups per CU: measured on
  // MI355X at M = 128, 27.7 against 32.9 us (4096 x 4096), 33.9 against 38.2 (4096 -> 11008),
  // 67.7 against 82.4 (11008 -> 4096); at 688 tiles (4096 -> 11008, M = 256) 64-row tiles
  // stay ahead, 50.2 against 61.7 us
  const int64_t tiles64 = ((M + 63) / 64) * ((N + BN - 1) / BN);
  if (tiles64 < 512) return launch_mb<2>(x, qweight, scales, zeros, M, N, K, y, stream);
  return launch_mb<4>(x, qweight, scales, zeros, M, N, K, y, stream);
}

hipError_t launch_mfma_variant(int bits, int group, const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                               const uint16_t* zeros, int64_t M, int64_t N, int64_t K, uint16_t* y,
                               hipStream_t stream) {
  const int gsh = group == 32 ? 0 : group == 64 ? 1 : 2;
  const Nf4Table none = {};
  if (bits == 4) return launch_var_m<4>(x, qweight, scales, zeros, M, N, K, gsh, none, y, stream);
  return launch_var_m<3>(x, qweight, scales, zeros, M, N, K, gsh, none, y, stream);
}

hipError_t launch_mfma_nf4(const Nf4Table& table, int block, const uint16_t* x, const uint32_t* qweight,
                           const float* absmax, int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const int gsh = block == 32 ? 0 : block == 64 ? 1 : 2;
  return launch_var_m<kNF4>(x, qweight, absmax, nullptr, M, N, K, gsh, table, y, stream);
}

}  // namespace w4a16
