// W4A16 GEMV for small batches (M = 1..8) on gfx950.
//
// y[m][n] = sum_k x[m][k] * (q[n][k] - z[n][g]) * d[n][g], float32 accumulation.
// This is TinyChat's fused dequantize + GEMV ("MIT 6.5940 L13 LLM Deployment"
// guide, TinyChat kernel fusion, slide 37): weights are rebuilt in registers
// and never written back. Batch-1 decode reads every weight once, so the kernel
// is bound by HBM bandwidth ("CMU 11-868 Model Quantization" guide, where the
// speed comes from; "MIT 6.5940 Lab 4 + Lab 5" guide, Lab 4 starting point).
//
// Work split
//   * A workgroup owns R consecutive output rows and spans all of K: thread t
//     owns the 16-byte code pieces p = t, t + T, ... of every row (a piece is
//     32 inputs, i.e. 16 bytes of codes). A wave's code load is therefore
//     1 KB of contiguous HBM per row (eight 128-byte lines).
//   * Each thread keeps its x pieces in VGPRs for the whole tile (reused by
//     all R rows) and issues the loads of all R rows before computing, so a
//     wave has R KB in flight. Code loads are non-temporal: the weights are
//     streamed once and should not displace x or the scales in the caches.
//   * Each piece lies inside one group of 128, so each (row, piece) needs one
//     (scale, zero) pair; each wave stages the pairs of its own 16 groups in
//     its own LDS area (no workgroup barrier before compute).
//   * The lane partials of all the tile's (row, input) outputs are added
//     across the wave in one batched pass after the last row (permlane swaps
//     halve each set of eight values, DPP finishes them), in one fixed order
//     for every output; one barrier at the end adds the waves' sums in a fixed
//     order (deterministic). Measured on MI355X at K = N = 8192 against one
//     DPP reduction per output as its row finished: 7.95 against 8.26 us at
//     M = 1, 9.32 against 10.23 us at M = 2.
//   * Issue order: the (scale, zero) pairs, the codes of the first row, the x
//     pieces, then the codes of the other rows, pinned with sched_barrier. The
//     tile's rows are visited in a rotated order (slot r holds row
//     (r + blockIdx) mod R of the tile), so neighbouring workgroups do not all
//     open their streams on rows 32 KB apart. Measured on MI355X at
//     K = N = 8192, M = 1: 8.27 us against 8.40 us for the compiler's own order
//     without rotation.
//
// Dequantization (layout v1: nibble i of a word is input 2i, nibble i + 4 is
// input 2i + 1):
//   * gemv_kernel: w & 0x0F0F0F0F and (w >> 4) & 0x0F0F0F0F put one code in
//     each byte. Read as OCP E4M3 (fp8) values, the bytes 0..15 are the
//     subnormals and the first normal binade, whose value is exactly
//     byte * 2^-9, so v_cvt_scalef32_pk_f16_fp8 with scale 2^9 turns two
//     bytes into the fp16 pair (q_a, q_b) exactly, one instruction per pair.
//     The pairs come out as inputs (0, 4), (1, 5), (2, 6), (3, 7) of the word,
//     so the thread regroups its x pairs the same way once (v_perm_b32) and
//     reuses them for every row. This is 7 VALU operations per word against 9
//     for the OR-into-0x6400 route below.
//   * gemv_var_kernel: OR-ing a nibble pair into 0x6400 gives the fp16 pair
//     1024 + q exactly (0x00F0 nibbles give 1024 + 16q); one v_pk_add_f16
//     (resp. v_pk_fma_f16 by 1/16) turns that into q exactly.
//   v_dot2_f32_f16 multiplies q pairs by x pairs into float32 (single rounding
//   per instruction on normal operands). The zero point is applied once per
//   piece: sum (q - z) x = sum q x - z sum x, exact in the integer part for any
//   z, so no zero range is special.
#include "device_utils.h"
#include "launchers.h"

namespace w4a16 {

namespace {

constexpr int kMaxThreads = 512;
// At M <= 2 a workgroup may have up to 1024 threads when that gives every thread a
// single piece (K <= 32768). Measured on MI355X against two pieces per thread in 512
// threads, N = 8192: at M = 1, 19.5 against 21.5 us at K = 22016 and 24.5 against 27.2
// us at K = 32768 (25.9 against 25.5 us at K = 28672); at M = 2, 28.8 against 39.8 us at
// K = 22016 and 34.0 against 41.9 us at K = 28672.
constexpr int kMaxThreadsOnePiece = 1024;
constexpr int kMaxM = 8;

// Rows per workgroup. Measured on MI355X at K = N = 8192: for M = 1, 8 rows
// per 4-wave workgroup (1024 workgroups, four per CU) streams better than 16
// rows (512 workgroups) or 4 rows (2048 workgroups, where the per-workgroup x
// reads double): 8.31 against 8.53 us. On smaller layers 8 rows leave fewer
// than 16 waves per CU (a workgroup has one wave per 2048 inputs of K), and
// there 4 rows win: 4.08 against 4.75 us at 4096 x 4096, 6.47 against 7.17 at
// 4096 -> 11008, 6.90 against 7.51 at 11008 -> 4096 ("Narrow" tiles). For
// M >= 2 the x reads grow with M, and R * M * PPT <= 16 keeps more rows
// sharing them. M = 2 takes narrow tiles (4 rows) on the same small layers:
// 4.8 against 6.0 us at 4096 x 4096, 8.1 against 8.9 at 4096 -> 11008, 8.7
// against 9.6 at 11008 -> 4096; at 8192 x 8192 8 rows stay ahead (10.3
// against 10.7).
template <int M, int PPT, bool Narrow = false>
struct Tile {
  static constexpr int kBudget = (M == 1) ? (Narrow ? 4 : 8) : (M == 2 && Narrow) ? 8 : 16;
  static constexpr int R = (kBudget / (M * PPT)) > 0 ? (kBudget / (M * PPT)) : 1;
  static constexpr int V = R * M;
};

__device__ __forceinline__ half2_t q_pair_lo(uint32_t w) {  // nibbles at bits 0-3 / 16-19
  const half2_t b = as_half2(and_or(w, 0x000F000Fu, 0x64006400u));
  return b - (half2_t){(_Float16)1024.0f, (_Float16)1024.0f};
}

__device__ __forceinline__ half2_t q_pair_hi(uint32_t w) {  // nibbles at bits 4-7 / 20-23
  const half2_t b = as_half2(and_or(w, 0x00F000F0u, 0x64006400u));
  return __builtin_elementwise_fma(b, (half2_t){(_Float16)0.0625f, (_Float16)0.0625f},
                                   (half2_t){(_Float16)-64.0f, (_Float16)-64.0f});
}

// PSH: 2^PSH 32-input pieces per quantization group (2: groups of 128, 1: 64, 0: 32).
// NF4: the codes index the 16-level codebook (a copy per wave in LDS; the lookups give the
// same (0,4), (1,5), (2,6), (3,7) input pairs as the fp8 route) and `scales` holds the
// float32 absmax per block; there is no zero.
template <int M, int PPT, bool Narrow, int PSH, bool NF4>
__global__ __launch_bounds__(M <= 2 && PPT == 1 ? kMaxThreadsOnePiece : kMaxThreads) void gemv_kernel(const uint4* __restrict__ x, const u32x4_t* __restrict__ qw,
                                                           const void* __restrict__ scales,
                                                           const uint16_t* __restrict__ zeros, int N, int K,
                                                           uint16_t* __restrict__ y, Nf4Table table) {
  constexpr int R = Tile<M, PPT, Narrow>::R;
  constexpr int V = Tile<M, PPT, Narrow>::V;
  constexpr int GPW = 64 >> PSH;         // groups one wave's 64 pieces of a slot span
  constexpr int E = R * PPT * GPW;       // (scale, zero) pairs one wave needs: R rows x PPT slots x GPW groups
  constexpr int NE = (E + 63) / 64;      // ... per lane
  constexpr int WS = E + V + (NF4 ? 8 : 0);  // LDS words per wave
  extern __shared__ uint32_t lds[];      // per wave: E staged pairs, V partial sums (NF4: then the codebook)

  const int T = blockDim.x;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int G = K >> (5 + PSH);  // groups per row
  const int P = K >> 5;   // 16-byte code pieces per row
  const int KX = K >> 3;  // 16-byte x chunks per input row
  const int row0 = blockIdx.x * R;
  const int rot = (int)(blockIdx.x % R);
  // the row held in slot r (rows past N are loaded as row N - 1 and never stored)
  auto row_of = [&](int r) {
    const int rr = r + rot;
    return row0 + (rr >= R ? rr - R : rr);
  };
  uint32_t* wsz = lds + wave * WS;  // this wave's staging area
  float* wred = reinterpret_cast<float*>(wsz + E);
  _Float16* lut = reinterpret_cast<_Float16*>(wsz + E + V);
  if constexpr (NF4) {
    // stored and read as fp16 by this wave only; the wave-scope fences and wave barrier
    // order the other lanes' reads after lanes 0..15's stores for the compiler (they cost
    // nothing at run time: one wave's LDS accesses complete in order)
    if (lane < 16)
      lut[lane] = __builtin_bit_cast(_Float16, (uint16_t)(table.pairs[lane >> 1] >> (16 * (lane & 1))));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  }

  // Every load below is unconditional, with indices clamped into the tensors,
  // so the compiler can count outstanding loads exactly and let each row's
  // compute start as soon as that row's codes have landed. Lanes past K (the
  // last wave of a ragged K) compute with a zero scale; rows past N are never
  // stored.

  // (1) the (scale, zero) pairs this wave needs: lanes of piece slot pp cover
  //     GPW consecutive groups starting at GPW * wave + pp * T / 2^PSH
  uint32_t sreg[NE];
  uint16_t zreg[NF4 ? 1 : NE];
#pragma unroll
  for (int u = 0; u < NE; ++u) {
    const int e = min(lane + 64 * u, E - 1);
    const int r = e / (GPW * PPT), pp = (e / GPW) % PPT, gl = e % GPW;
    const int g = min(GPW * wave + pp * (T >> PSH) + gl, G - 1);
    const int64_t off = (int64_t)min(row_of(r), N - 1) * G + g;
    if constexpr (NF4) {
      sreg[u] = static_cast<const uint32_t*>(scales)[off];
    } else {
      sreg[u] = static_cast<const uint16_t*>(scales)[off];
      zreg[u] = zeros[off];
    }
  }

  // (2) code pieces of the first slot, (3) x pieces: 32 inputs = four 16-byte
  //     chunks per row of x, (4) code pieces of the other slots. Code loads are
  //     non-temporal (read once).
  u32x4_t cw[R][PPT];
  auto load_codes = [&](int r) {
    const int64_t row = min(row_of(r), N - 1);
#pragma unroll
    for (int pp = 0; pp < PPT; ++pp) {
      const int p = min(t + pp * T, P - 1);
      cw[r][pp] = __builtin_nontemporal_load(&qw[row * P + p]);
    }
  };
  load_codes(0);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t xr[PPT][M][16];
#pragma unroll
  for (int pp = 0; pp < PPT; ++pp) {
    const int p = min(t + pp * T, P - 1);
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 v = x[(int64_t)m * KX + 4 * p + c];
        xr[pp][m][4 * c + 0] = v.x;
        xr[pp][m][4 * c + 1] = v.y;
        xr[pp][m][4 * c + 2] = v.z;
        xr[pp][m][4 * c + 3] = v.w;
      }
    }
  }

  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 1; r < R; ++r) load_codes(r);
  __builtin_amdgcn_sched_barrier(0);

  // (5) stage this wave's (scale, zero) pairs; only this wave reads them, and
  //     a wave sees its own LDS writes in order, so no workgroup barrier
#pragma unroll
  for (int u = 0; u < NE; ++u) {
    const int e = lane + 64 * u;
    if constexpr (NF4) {
      if (e < E) wsz[e] = sreg[u];
    } else {
      if (e < E) wsz[e] = sreg[u] | ((uint32_t)zreg[u] << 16);
    }
  }

  // sum of x over each piece (for the zero-point term)
  const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
  float sx[PPT][M];
#pragma unroll
  for (int pp = 0; pp < PPT; ++pp)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) a = __builtin_amdgcn_fdot2(as_half2(xr[pp][m][j]), ones, a, false);
      sx[pp][m] = a;
    }

  // x pairs regrouped to match the converted code pairs: inputs (0, 4), (1, 5),
  // (2, 6), (3, 7) of each 8-input word
  uint32_t xp[PPT][M][16];
#pragma unroll
  for (int pp = 0; pp < PPT; ++pp)
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int wi = 0; wi < 4; ++wi) {
        const uint32_t x01 = xr[pp][m][4 * wi + 0], x23 = xr[pp][m][4 * wi + 1];
        const uint32_t x45 = xr[pp][m][4 * wi + 2], x67 = xr[pp][m][4 * wi + 3];
        xp[pp][m][4 * wi + 0] = __builtin_amdgcn_perm(x45, x01, 0x05040100u);
        xp[pp][m][4 * wi + 1] = __builtin_amdgcn_perm(x45, x01, 0x07060302u);
        xp[pp][m][4 * wi + 2] = __builtin_amdgcn_perm(x67, x23, 0x05040100u);
        xp[pp][m][4 * wi + 3] = __builtin_amdgcn_perm(x67, x23, 0x07060302u);
      }

  // (6) slot by slot as the loads land: dequantize and multiply; then (7) the partials are
  //     summed across the wave in batches (swaps and DPP): all V of them in one pass at the
  //     end, or, with 8 inputs, each row's 8 as soon as the row is done (measured on MI355X
  //     at 8192 x 8192, M = 8: 37.25 against 37.43 us, groups of 64: 35.61 against 36.10)
  float vsum[V];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float* acc = vsum + r * M;
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;
#pragma unroll
    for (int pp = 0; pp < PPT; ++pp) {
      const int p_raw = t + pp * T;
      const uint32_t szv = wsz[(r * PPT + pp) * GPW + (lane >> PSH)];
      const float dv = NF4 ? __builtin_bit_cast(float, szv) : half_bits_to_float((uint16_t)(szv & 0xFFFFu));
      const float d = (p_raw < P) ? dv : 0.f;
      const float z = NF4 ? 0.f : half_bits_to_float((uint16_t)(szv >> 16));
      const uint32_t wd[4] = {cw[r][pp].x, cw[r][pp].y, cw[r][pp].z, cw[r][pp].w};
      float part[M];
#pragma unroll
      for (int m = 0; m < M; ++m) part[m] = 0.f;
#pragma unroll
      for (int wi = 0; wi < 4; ++wi) {
        half2_t q04, q15, q26, q37;
        if constexpr (NF4) {
          const uint32_t w = wd[wi];  // nibble i holds input 2i (i < 4) or 2(i - 4) + 1
          q04 = (half2_t){lut[w & 15u], lut[(w >> 8) & 15u]};
          q15 = (half2_t){lut[(w >> 16) & 15u], lut[(w >> 24) & 15u]};
          q26 = (half2_t){lut[(w >> 4) & 15u], lut[(w >> 12) & 15u]};
          q37 = (half2_t){lut[(w >> 20) & 15u], lut[w >> 28]};
        } else {
          const uint32_t lo = wd[wi] & 0x0F0F0F0Fu, hi = (wd[wi] >> 4) & 0x0F0F0F0Fu;
          q04 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false);
          q15 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true);
          q26 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, false);
          q37 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, true);
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
          float a = part[m];
          a = __builtin_amdgcn_fdot2(q04, as_half2(xp[pp][m][4 * wi + 0]), a, false);
          a = __builtin_amdgcn_fdot2(q15, as_half2(xp[pp][m][4 * wi + 1]), a, false);
          a = __builtin_amdgcn_fdot2(q26, as_half2(xp[pp][m][4 * wi + 2]), a, false);
          a = __builtin_amdgcn_fdot2(q37, as_half2(xp[pp][m][4 * wi + 3]), a, false);
          part[m] = a;
        }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if constexpr (NF4)
          acc[m] = __builtin_fmaf(d, part[m], acc[m]);
        else
          acc[m] = __builtin_fmaf(d, __builtin_fmaf(-z, sx[pp][m], part[m]), acc[m]);
      }
    }
    if constexpr (M >= 8) wave_sums<M>(acc, wred + r * M, lane);
  }
  if constexpr (M < 8) wave_sums<V>(vsum, wred, lane);

  // (8) add the waves' sums in a fixed order and store
  __syncthreads();
  const int nw = T >> 6;
  for (int v = t; v < R * M; v += T) {
    float s = 0.f;
    for (int w = 0; w < nw; ++w) s += reinterpret_cast<const float*>(lds + w * WS + E)[v];
    const int r = v / M;
    const int m = v - r * M;
    const int row = row_of(r);
    if (row < N) y[(int64_t)m * N + row] = float_to_half_bits(s);
  }
}

// ---------------------------------------------------------------------------
// Variants: 3-bit codes, and groups of 32 or 64 (the same work split; the batch
// size M is a runtime value up to the template's MT, rows past M are loaded as
// copies of row M - 1 and never stored; the group size is a runtime shift).
//
// 3-bit pieces are the 12 bytes of one 32-input block of the bit-plane layout:
// low-bit words lo0 (inputs 0..15), lo1 (16..31) and the high-bit word hi. The
// pair of inputs (2j, 2j+1) is rebuilt as the fp16 pair 1024 + q by OR-ing
// ((lo >> 2i) & 0x00030003) and the high bits moved to bits 2 and 18 into 0x6400.

// code formats of the variant kernels: 4-bit and 3-bit integer codes with a
// (scale, zero) per group, and NF4 (4-bit codes into the 16-level codebook, layout
// v1) with a float32 absmax per block
constexpr int kNF4 = 16;

template <int FMT>
struct Piece {
  u32x4_t w;  // layout v1: 4-bit integer codes and NF4 codes
};
template <>
struct Piece<3> {
  uint32_t lo0, lo1, hi;
};

template <int FMT>
__device__ __forceinline__ Piece<FMT> load_piece(const uint32_t* qw, int64_t row, int P, int p, Piece<FMT>*) {
  Piece<FMT> r;
  r.w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(qw) + row * P + p);
  return r;
}

__device__ __forceinline__ Piece<3> load_piece(const uint32_t* qw, int64_t row, int P, int p, Piece<3>*) {
  const uint32_t* b = qw + (row * P + p) * 3;
  Piece<3> r;
  r.lo0 = __builtin_nontemporal_load(b);
  r.lo1 = __builtin_nontemporal_load(b + 1);
  r.hi = __builtin_nontemporal_load(b + 2);
  return r;
}

// the 16 exact fp16 code pairs of a piece, pair j = inputs (2j, 2j+1)
// NF4: pair i of word wi is (codebook[(w >> 4i) & 15], codebook[(w >> 16 + 4i) & 15])
__device__ __forceinline__ void piece_pairs(const Piece<kNF4>& pc, half2_t (&q)[16], const _Float16* lut) {
  const uint32_t wd[4] = {pc.w.x, pc.w.y, pc.w.z, pc.w.w};
#pragma unroll
  for (int wi = 0; wi < 4; ++wi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t n = wd[wi] >> (4 * i);
      q[4 * wi + i] = (half2_t){lut[n & 15u], lut[(n >> 16) & 15u]};
    }
}

__device__ __forceinline__ void piece_pairs(const Piece<4>& pc, half2_t (&q)[16], const _Float16*) {
  const uint32_t wd[4] = {pc.w.x, pc.w.y, pc.w.z, pc.w.w};
#pragma unroll
  for (int wi = 0; wi < 4; ++wi) {
    const uint32_t w8 = wd[wi] >> 8;
    q[4 * wi + 0] = q_pair_lo(wd[wi]);
    q[4 * wi + 1] = q_pair_hi(wd[wi]);
    q[4 * wi + 2] = q_pair_lo(w8);
    q[4 * wi + 3] = q_pair_hi(w8);
  }
}

__device__ __forceinline__ void piece_pairs(const Piece<3>& pc, half2_t (&q)[16], const _Float16*) {
  const half2_t m1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t lo = (j < 8) ? pc.lo0 : pc.lo1;
    // bits j and 16 + j of hi moved to bits 2 and 18
    const uint32_t hj = j >= 2 ? (pc.hi >> (j - 2)) : (pc.hi << (2 - j));
    const uint32_t t = and_or(hj, 0x00040004u, 0x64006400u);
    q[j] = as_half2(and_or(lo >> (2 * (j & 7)), 0x00030003u, t)) + m1024;
  }
}

template <int MT, int PPT, int FMT>
__global__ __launch_bounds__(kMaxThreads) void gemv_var_kernel(const uint4* __restrict__ x, const uint32_t* __restrict__ qw,
                                                               const void* __restrict__ scales,
                                                               const uint16_t* __restrict__ zeros, int M, int N, int K,
                                                               int gsh, Nf4Table table, uint16_t* __restrict__ y) {
  constexpr int R = Tile<MT, PPT>::R;
  constexpr int V = Tile<MT, PPT>::V;
  constexpr int E = R * PPT * 64;        // staged (scale, zero) pairs per wave, enough for groups of 32
  constexpr int NE = E / 64;
  extern __shared__ uint32_t lds[];

  const int T = blockDim.x;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int G = K >> (5 + gsh);  // groups per row
  const int P = K >> 5;          // 32-input pieces per row
  const int KX = K >> 3;
  const int row0 = blockIdx.x * R;
  const int rows = min(R, N - row0);
  uint32_t* wsz = lds + wave * (E + V);
  float* wred = reinterpret_cast<float*>(wsz + E);

  __shared__ __align__(16) _Float16 lut[16];
  if constexpr (FMT == kNF4) {
    // constant indices keep the codebook words in scalar registers (no memory round trip)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (t == i) reinterpret_cast<uint32_t*>(lut)[i] = table.pairs[i];
  }

  // (1) (scale, zero) pairs, or NF4 absmax: slot pp of this wave covers 64 >> gsh groups from
  //     (64 wave + pp T) >> gsh. Scale and zero stay in separate registers until they are
  //     staged, so no wait on these loads comes before the weight loads are issued.
  uint32_t sreg[NE];
  uint16_t zreg[NE];
#pragma unroll
  for (int u = 0; u < NE; ++u) {
    const int e = lane + 64 * u;
    const int r = e / (64 * PPT), pp = (e >> 6) % PPT, gl = e & 63;
    const int g = min(((64 * wave + pp * T) >> gsh) + gl, G - 1);
    const int64_t off = (int64_t)min(row0 + r, N - 1) * G + g;
    if constexpr (FMT == kNF4) {
      sreg[u] = __builtin_bit_cast(uint32_t, static_cast<const float*>(scales)[off]);
      zreg[u] = 0;
    } else {
      sreg[u] = static_cast<const uint16_t*>(scales)[off];
      zreg[u] = zeros[off];
    }
  }

  // (2) x pieces (rows past M repeat row M - 1)
  uint32_t xr[PPT][MT][16];
#pragma unroll
  for (int pp = 0; pp < PPT; ++pp) {
    const int p = min(t + pp * T, P - 1);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int mr = min(m, M - 1);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 v = x[(int64_t)mr * KX + 4 * p + c];
        xr[pp][m][4 * c + 0] = v.x;
        xr[pp][m][4 * c + 1] = v.y;
        xr[pp][m][4 * c + 2] = v.z;
        xr[pp][m][4 * c + 3] = v.w;
      }
    }
  }

  // (3) code pieces of all rows of the tile
  Piece<FMT> cw[R][PPT];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = min(row0 + r, N - 1);
#pragma unroll
    for (int pp = 0; pp < PPT; ++pp)
      cw[r][pp] = load_piece(qw, row, P, min(t + pp * T, P - 1), (Piece<FMT>*)nullptr);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load is issued before anything waits on one

  // (4) stage this wave's pairs (read by this wave only)
#pragma unroll
  for (int u = 0; u < NE; ++u) wsz[lane + 64 * u] = sreg[u] | ((uint32_t)zreg[u] << 16);
  if constexpr (FMT == kNF4) {
    // the codebook written by wave 0 becomes visible to every wave; the barrier orders LDS
    // only, so the weight loads stay in flight across it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }

  const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
  float sx[PPT][MT];
#pragma unroll
  for (int pp = 0; pp < PPT; ++pp)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) a = __builtin_amdgcn_fdot2(as_half2(xr[pp][m][j]), ones, a, false);
      sx[pp][m] = a;
    }

  // (5) per row: dequantize, multiply; then the wave sums in batches as in gemv_kernel
  //     (measured on MI355X at 8192 x 8192 against one wave sum per value: 3-bit groups of
  //     128, M = 2: 11.15 against 12.35 us, M = 4: 15.37 against 16.79; M = 8 within 1 %)
  float vsum[V];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float* acc = vsum + r * MT;
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.f;
#pragma unroll
    for (int pp = 0; pp < PPT; ++pp) {
      const int p_raw = t + pp * T;
      const uint32_t szv = wsz[(r * PPT + pp) * 64 + (lane >> gsh)];
      float d, z;
      if constexpr (FMT == kNF4) {
        d = (p_raw < P) ? __builtin_bit_cast(float, szv) : 0.f;
        z = 0.f;
      } else {
        d = (p_raw < P) ? half_bits_to_float((uint16_t)(szv & 0xFFFFu)) : 0.f;
        z = half_bits_to_float((uint16_t)(szv >> 16));
      }
      half2_t q[16];
      piece_pairs(cw[r][pp], q, lut);
      float part[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) a = __builtin_amdgcn_fdot2(q[j], as_half2(xr[pp][m][j]), a, false);
        part[m] = a;
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if constexpr (FMT == kNF4)
          acc[m] = __builtin_fmaf(d, part[m], acc[m]);
        else
          acc[m] = __builtin_fmaf(d, __builtin_fmaf(-z, sx[pp][m], part[m]), acc[m]);
      }
    }
    if constexpr (MT >= 8) wave_sums<MT>(acc, wred + r * MT, lane);
  }
  if constexpr (MT < 8) wave_sums<V>(vsum, wred, lane);

  // (6) the waves' sums in a fixed order
  __syncthreads();
  const int nw = T >> 6;
  for (int v = t; v < rows * MT; v += T) {
    const int r = v / MT;
    const int m = v - r * MT;
    if (m >= M) continue;
    float sum = 0.f;
    for (int w = 0; w < nw; ++w) sum += reinterpret_cast<const float*>(lds + w * (E + V) + E)[v];
    y[(int64_t)m * N + row0 + r] = float_to_half_bits(sum);
  }
}

struct Launch {
  int ppt;
  int threads;
};

// pieces per thread and threads per workgroup; one_piece_max: the largest workgroup
// allowed when that gives every thread a single piece
Launch plan(int64_t K, int one_piece_max = kMaxThreads) {
  const int P = (int)(K >> 5);
  if (P <= one_piece_max) return {1, (P + 63) & ~63};
  int ppt = 1;
  while ((P + ppt - 1) / ppt > kMaxThreads) ppt <<= 1;
  int t = (P + ppt - 1) / ppt;
  t = (t + 63) & ~63;
  return {ppt, t};
}

// narrow tiles (M <= 2, one piece per thread) when the default ones would give fewer than
// 16 waves per CU
bool narrow_tiles(int64_t M, int64_t N, int threads) {
  const int R = M == 1 ? Tile<1, 1>::R : Tile<2, 1>::R;
  return M <= 2 && (N + R - 1) / R * (threads / 64) < 16 * 256;
}

template <int M, int PPT, bool Narrow, int PSH, bool NF4>
hipError_t launch_mp(const uint16_t* x, const uint32_t* qweight, const void* scales, const uint16_t* zeros,
                     int64_t N, int64_t K, uint16_t* y, int threads, const Nf4Table& table, hipStream_t stream) {
  constexpr int R = Tile<M, PPT, Narrow>::R;
  constexpr int V = Tile<M, PPT, Narrow>::V;
  constexpr int E = R * PPT * (64 >> PSH);
  const size_t lds = (size_t)(threads / 64) * (E + V + (NF4 ? 8 : 0)) * 4;
  const int grid = (int)((N + R - 1) / R);
  hipLaunchKernelGGL((gemv_kernel<M, PPT, Narrow, PSH, NF4>), dim3(grid), dim3(threads), lds, stream,
                     reinterpret_cast<const uint4*>(x), reinterpret_cast<const u32x4_t*>(qweight), scales, zeros,
                     (int)N, (int)K, y, table);
  return hipGetLastError();
}

template <int M, int PSH = 2, bool NF4 = false>
hipError_t launch_m(const uint16_t* x, const uint32_t* qweight, const void* scales, const uint16_t* zeros,
                    int64_t N, int64_t K, uint16_t* y, hipStream_t stream, const Nf4Table& table = {}) {
  const Launch l = plan(K, M <= 2 ? kMaxThreadsOnePiece : kMaxThreads);
  switch (l.ppt) {
    case 1:
      if constexpr (M <= 2) {
        if (narrow_tiles(M, N, l.threads))
          return launch_mp<M, 1, true, PSH, NF4>(x, qweight, scales, zeros, N, K, y, l.threads, table, stream);
      }
      return launch_mp<M, 1, false, PSH, NF4>(x, qweight, scales, zeros, N, K, y, l.threads, table, stream);
    case 2:
      if constexpr (M <= 4) return launch_mp<M, 2, false, PSH, NF4>(x, qweight, scales, zeros, N, K, y, l.threads, table, stream);
      break;
    case 4:
      if constexpr (M <= 2) return launch_mp<M, 4, false, PSH, NF4>(x, qweight, scales, zeros, N, K, y, l.threads, table, stream);
      break;
    case 8:
      if constexpr (M <= 1) return launch_mp<M, 8, false, PSH, NF4>(x, qweight, scales, zeros, N, K, y, l.threads, table, stream);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <int MT, int PPT, int FMT>
hipError_t launch_var(const uint16_t* x, const uint32_t* qweight, const void* scales, const uint16_t* zeros,
                      int64_t M, int64_t N, int64_t K, int gsh, const Nf4Table& table, uint16_t* y, int threads,
                      hipStream_t stream) {
  constexpr int R = Tile<MT, PPT>::R;
  constexpr int V = Tile<MT, PPT>::V;
  constexpr int E = R * PPT * 64;
  const size_t lds = (size_t)(threads / 64) * (E + V) * 4;
  const int grid = (int)((N + R - 1) / R);
  hipLaunchKernelGGL((gemv_var_kernel<MT, PPT, FMT>), dim3(grid), dim3(threads), lds, stream,
                     reinterpret_cast<const uint4*>(x), qweight, scales, zeros, (int)M, (int)N, (int)K, gsh, table, y);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_var_fmt(const uint16_t* x, const uint32_t* qweight, const void* scales, const uint16_t* zeros,
                          int64_t M, int64_t N, int64_t K, int gsh, const Nf4Table& table, uint16_t* y,
                          hipStream_t stream) {
  const Launch l = plan(K);
  const int mt = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
  if (l.ppt == 1) {
    switch (mt) {
      case 1: return launch_var<1, 1, FMT>(x, qweight, scales, zeros, M, N, K, gsh, table, y, l.threads, stream);
      case 2: return launch_var<2, 1, FMT>(x, qweight, scales, zeros, M, N, K, gsh, table, y, l.threads, stream);
      case 4: return launch_var<4, 1, FMT>(x, qweight, scales, zeros, M, N, K, gsh, table, y, l.threads, stream);
      default: return launch_var<8, 1, FMT>(x, qweight, scales, zeros, M, N, K, gsh, table, y, l.threads, stream);
    }
  }
  if (l.ppt == 2) {
    switch (mt) {
      case 1: return launch_var<1, 2, FMT>(x, qweight, scales, zeros, M, N, K, gsh, table, y, l.threads, stream);
      case 2: return launch_var<2, 2, FMT>(x, qweight, scales, zeros, M, N, K, gsh, table, y, l.threads, stream);
      case 4: return launch_var<4, 2, FMT>(x, qweight, scales, zeros, M, N, K, gsh, table, y, l.threads, stream);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

int gemv_max_m() { return kMaxM; }

bool gemv_variant_supports(int64_t M, int64_t K, int group) {
  if (M < 1 || M > kMaxM || K <= 0 || K % group != 0) return false;
  const int ppt = plan(K).ppt;
  const int mt = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
  return ppt == 1 || (ppt == 2 && mt <= 4);
}

template <int PSH>
hipError_t launch_gemv_groups(const uint16_t* x, const uint32_t* qweight, const void* scales, const uint16_t* zeros,
                              int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  switch (M) {
    case 1: return launch_m<1, PSH>(x, qweight, scales, zeros, N, K, y, stream);
    case 2: return launch_m<2, PSH>(x, qweight, scales, zeros, N, K, y, stream);
    case 3: return launch_m<3, PSH>(x, qweight, scales, zeros, N, K, y, stream);
    case 4: return launch_m<4, PSH>(x, qweight, scales, zeros, N, K, y, stream);
    case 5: return launch_m<5, PSH>(x, qweight, scales, zeros, N, K, y, stream);
    case 6: return launch_m<6, PSH>(x, qweight, scales, zeros, N, K, y, stream);
    case 7: return launch_m<7, PSH>(x, qweight, scales, zeros, N, K, y, stream);
    case 8: return launch_m<8, PSH>(x, qweight, scales, zeros, N, K, y, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv_variant(int bits, int group, const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                               const uint16_t* zeros, int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const int gsh = group == 32 ? 0 : group == 64 ? 1 : 2;
  const Nf4Table none = {};
  // 4-bit codes with groups of 64 or 32: the tuned kernel with two or one pieces per group
  if (bits == 4 && gemv_supports(M, K)) {
    if (gsh == 1) return launch_gemv_groups<1>(x, qweight, scales, zeros, M, N, K, y, stream);
    if (gsh == 0) return launch_gemv_groups<0>(x, qweight, scales, zeros, M, N, K, y, stream);
  }
  if (bits == 4) return launch_var_fmt<4>(x, qweight, scales, zeros, M, N, K, gsh, none, y, stream);
  return launch_var_fmt<3>(x, qweight, scales, zeros, M, N, K, gsh, none, y, stream);
}

hipError_t launch_gemv_nf4(const Nf4Table& table, int block, const uint16_t* x, const uint32_t* qweight,
                           const float* absmax, int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const int gsh = block == 32 ? 0 : block == 64 ? 1 : 2;
  // One row on layers below 2^26 weights: the tuned kernel with the block's pieces per group
  // (measured 14-15 % faster at 4096 x 11008 and 11008 x 4096). On larger layers and at
  // M = 2 the per-piece kernel measured 5-10 % faster; there both run near 2.9 TB/s, well
  // under the 4-bit integer codes' rate on the same bytes, so the 16-entry lookups (eight
  // LDS reads per 32-bit code word) rather than HBM set the pace.
  if (M == 1 && N * K < (int64_t{1} << 26) && gemv_supports(M, K)) {
    if (gsh == 2) return launch_m<1, 2, true>(x, qweight, absmax, nullptr, N, K, y, stream, table);
    if (gsh == 1) return launch_m<1, 1, true>(x, qweight, absmax, nullptr, N, K, y, stream, table);
    return launch_m<1, 0, true>(x, qweight, absmax, nullptr, N, K, y, stream, table);
  }
  return launch_var_fmt<kNF4>(x, qweight, absmax, nullptr, M, N, K, gsh, table, y, stream);
}

bool gemv_format_supports(int bits, int group, int64_t M, int64_t N, int64_t K) {
  // the routes launch_gemv_variant and launch_gemv_nf4 take: the tuned kernel for 4-bit
  // groups of 64/32 (and NF4 rows on small layers) wherever it fits, the variant kernel otherwise
  if (bits == 4 && gemv_supports(M, K)) return true;
  if (bits == 0 && M == 1 && N * K < (int64_t{1} << 26) && gemv_supports(M, K)) return true;
  return gemv_variant_supports(M, K, group);
}

bool gemv_narrow(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > 2 || K <= 0) return false;
  const Launch l = plan(K, kMaxThreadsOnePiece);
  return l.ppt == 1 && narrow_tiles(M, N, l.threads);
}

bool gemv_supports(int64_t M, int64_t K) {
  if (M < 1 || M > kMaxM || K <= 0 || K % 128 != 0) return false;
  return plan(K).ppt * M <= 8;
}

hipError_t launch_gemv(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                       int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  switch (M) {
    case 1: return launch_m<1>(x, qweight, scales, zeros, N, K, y, stream);
    case 2: return launch_m<2>(x, qweight, scales, zeros, N, K, y, stream);
    case 3: return launch_m<3>(x, qweight, scales, zeros, N, K, y, stream);
    case 4: return launch_m<4>(x, qweight, scales, zeros, N, K, y, stream);
    case 5: return launch_m<5>(x, qweight, scales, zeros, N, K, y, stream);
    case 6: return launch_m<6>(x, qweight, scales, zeros, N, K, y, stream);
    case 7: return launch_m<7>(x, qweight, scales, zeros, N, K, y, stream);
    case 8: return launch_m<8>(x, qweight, scales, zeros, N, K, y, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w4a16
