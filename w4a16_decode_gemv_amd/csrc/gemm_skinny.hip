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
//
// Groups of 64 or 32 (and NF4 blocks of 128, 64 or 32) use the same code stream:
// the code layout does not depend on the group. Step q covers inputs 32q..32q+31
// of a 128-input group, which lie inside one group of 32 or 64, so the steps of
// one group chain into one MFMA accumulator that is scaled once (and its zero
// applied once, through the sum of x over the same steps). The SUB = 128 / group
// (scale, zero) pairs of a row's 128 inputs are contiguous in memory and arrive
// in one load. NF4 codes become fp16 levels through a 16-entry codebook in LDS
// (16 fp16 values: 8 banks, so every lookup is conflict-free or a broadcast) and
// are scaled by the float32 absmax of the block; there is no zero.
//
// 3-bit codes (the packed 3-bit layout: per 32-input block, the low two bits of
// inputs 0..15 and of 16..31 in two words, the high bits of all 32 in a third)
// keep the k-slot assignment: step q is block q of the group, and slot group j
// needs the low-bit word j / 2 of that block and its high-bit word. A stage is
// 96 bytes per row (six 16-byte pieces, spread over the lanes); the LDS area holds
// each row's two groups transposed, as [group][low word 0 | low word 1 | high
// word][block], so that a lane reads its four steps' low words and high words in
// two 16-byte reads.
#include "device_utils.h"
#include "launchers.h"

namespace w4a16 {

namespace {


constexpr int KS = 8;               // waves per workgroup, splitting K
constexpr int kThreads = KS * 64;
constexpr int D = 2;                // stages in flight per wave
constexpr int kMaxStages = 8;       // stages per chunk of the largest kernel variant


// code formats of the kernel
constexpr int kFmt4 = 0;    // 4-bit codes in layout v1, fp16 scales and zeros
constexpr int kFmtNf4 = 1;  // 4-bit NF4 codes in layout v1, float32 absmax
constexpr int kFmt3 = 2;    // 3-bit codes in the packed 3-bit layout, fp16 scales and zeros
constexpr int kRowStride3 = 28;  // dwords per row of the 3-bit LDS area (24 used; 28 keeps 16 rows apart in banks)

// the eight 3-bit codes q (exact fp16) that slot group j takes from one block: the low bits
// of pairs 4(j % 2) .. 4(j % 2) + 3 of `lo`, the high bits at bits 4j + e and 16 + 4j + e of
// `hi` (rotated to bits 2 and 18); OR-ed into 0x6400 and rebased by 1024 like the 4-bit codes
__device__ __forceinline__ half8_t codes3_word(uint32_t lo, uint32_t hi, int j) {
  const half2_t c_lo = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  const uint32_t l = lo >> (8 * (j & 1));
  const uint32_t h = __builtin_amdgcn_alignbit(hi, hi, (uint32_t)(4 * j + 30) & 31u);
  uint32_t v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t t = and_or(h >> e, 0x00040004u, 0x64006400u);
    v[e] = __builtin_bit_cast(uint32_t, as_half2(and_or(l >> (2 * e), 0x00030003u, t)) + c_lo);
  }
  return as_half8((u32x4_t){v[0], v[1], v[2], v[3]});
}

// the eight NF4 codes of one code word as their fp16 levels, in k order
__device__ __forceinline__ half8_t nf4_word(uint32_t w, const _Float16* lut) {
  uint32_t v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t n = w >> (4 * i);
    v[i] = __builtin_bit_cast(uint32_t, (half2_t){lut[n & 15u], lut[(n >> 16) & 15u]});
  }
  return as_half8((u32x4_t){v[0], v[1], v[2], v[3]});
}

// the scale-side bytes of one (row, 128-input group) item: SUB fp16 scales (or zeros), or
// SUB float32 absmax values, contiguous in memory; one load, little-endian words
template <int BYTES>
__device__ __forceinline__ void load_item(__amdgpu_buffer_rsrc_t r, int off, uint32_t (&v)[BYTES >= 4 ? BYTES / 4 : 1]) {
  if constexpr (BYTES == 2) {
    v[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  } else if constexpr (BYTES == 4) {
    v[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else if constexpr (BYTES == 8) {
    const auto t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    v[0] = t[0];
    v[1] = t[1];
  } else {
    static_assert(BYTES == 16, "items of 2, 4, 8 or 16 bytes");
    const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    v[0] = t.x;
    v[1] = t.y;
    v[2] = t.z;
    v[3] = t.w;
  }
}

// NS stages (2 * NS groups) per wave and chunk; K beyond one chunk per wave loops over chunks
// XI > 0 (M <= 2 XI <= 16, MT = 1): a stage's x rows arrive in XI full-width loads (lane l of
// load i takes row 2i + l/32, 16-byte piece l%32 of the stage's 512 bytes) and reach the A
// fragments through a wave-private LDS area; XI = 0: A fragments loaded straight from L2.
// "Group" below is a 128-input group of the code stream; SUB = 128 / (quantization group)
// scales per row and group (NF4: float32 absmax values passed through `scales`, no zeros).
template <int NTW, int MT, int NS, int XI, int SUB, int FMT>
__global__ __launch_bounds__(kThreads) void skinny_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw,
                                                         const void* __restrict__ scales,
                                                         const uint16_t* __restrict__ zeros, int M, int N, int K,
                                                         Nf4Table table, uint16_t* __restrict__ y) {
  constexpr bool NF4 = FMT == kFmtNf4, B3 = FMT == kFmt3;
  constexpr int ROWS = 16 * NTW;
  constexpr int CG = 2 * NS;                       // groups per wave and chunk
  constexpr int CL = B3 ? (6 * ROWS + 63) / 64 : 2 * NTW;  // 16-byte code loads per lane and stage
  constexpr int SZL = (ROWS * CG + 63) / 64;       // (row, group) scale items per lane and chunk
  constexpr int QS = 4 / SUB;                      // MFMA steps per quantization group
  constexpr int IB = (NF4 ? 4 : 2) * SUB;          // bytes of one scale item (per tensor)
  constexpr int IW = IB >= 4 ? IB / 4 : 1;         // 32-bit words holding it
  static_assert(SUB == 1 || SUB == 2 || SUB == 4, "groups of 128, 64 or 32");
  static_assert(ROWS * 8 >= NTW * MT * 64, "the final combine reuses the code staging area");
  static_assert(kRowStride3 <= 32, "the 3-bit staging area fits the 4-bit one");
  __shared__ u32x4_t lds_b[KS][ROWS * 8];            // one stage of codes: ROWS x (2 groups x 4 slots)
  __shared__ uint32_t lds_sz[KS][ROWS][CG * SUB + 1];  // one chunk of (scale | zero << 16), or absmax
  // x rows, padded; 16 rows keep one LDS stage per wave (a wave reads its stage before it
  // stores the next, in program order), which fits the chip's LDS next to two column tiles
  constexpr int XS = XI > 4 ? 1 : D;
  __shared__ u32x4_t lds_x[XI > 0 ? KS : 1][XI > 0 ? XS : 1][XI > 0 ? 2 * XI : 1][33];
  __shared__ __align__(16) _Float16 lut[NF4 ? 16 : 2];
  if constexpr (NF4) {
    if (threadIdx.x < 8) reinterpret_cast<uint32_t*>(lut)[threadIdx.x] = table.pairs[threadIdx.x];
    __syncthreads();
  }

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
  const int row_bytes = B3 ? 3 * (K >> 3) : K >> 1;  // code bytes per row
  const __amdgpu_buffer_rsrc_t q_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const uint8_t*>(qw) + (int64_t)n0 * row_bytes), (short)0, rows * row_bytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const uint8_t*>(scales) + (int64_t)n0 * G * IB), (short)0, rows * G * IB, kBufferFlags);
  const __amdgpu_buffer_rsrc_t z_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(NF4 ? nullptr : zeros + (int64_t)n0 * G * SUB), (short)0, NF4 ? 0 : rows * G * IB, kBufferFlags);
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

    // scales (and zeros) of the chunk: lane -> (row, SZL consecutive groups)
    uint32_t sv[SZL][IW], zv[NF4 ? 1 : SZL][IW];
    const int sz_row = (lane * SZL) / CG, sz_g = (lane * SZL) % CG;
#pragma unroll
    for (int e = 0; e < SZL; ++e) {
      const int gi = sz_g + e;
      const int o = min(sz_row, ROWS - 1) * G * IB + (g0 + gi) * IB + bias(gi) + (int)(sz_row >= ROWS) * kOutOfRange;
      load_item<IB>(s_rsrc, o, sv[e]);
      if constexpr (!NF4) load_item<IB>(z_rsrc, o, zv[e]);
    }

    u32x4_t cr[D][CL];
    u32x4_t xr[D][2][MT][4];
    u32x4_t xl[D][XI > 0 ? XI : 1];
    auto load_codes = [&](int s, int slot) {
      if constexpr (B3) {
        // piece p = lane + 64 i: row p / 6, 16-byte piece p % 6 of the row's 96 bytes (pieces
        // 0..2 group 2s, 3..5 group 2s + 1); rows from ROWS on are past the buffer range
#pragma unroll
        for (int i = 0; i < CL; ++i) {
          const int p = lane + 64 * i, row = p / 6, piece = p - 6 * row;
          const int gi = 2 * s + (int)(piece >= 3);
          cr[slot][i] = __builtin_amdgcn_raw_buffer_load_b128(
              q_rsrc, row * row_bytes + (g0 + 2 * s) * 48 + 16 * piece + bias(gi), 0, kNonTemporal);
        }
        return;
      }
      const int gi = 2 * s + (lq >> 2);
      const int off = (g0 + gi) * 64 + 16 * (lq & 3) + bias(gi);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          cr[slot][2 * nt + h] = __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, off + (16 * nt + 8 * h + lr) * (K >> 1), 0,
                                                                       kNonTemporal);
    };
    // x rows 0 .. 2 XI - 1 in full-width loads (to LDS, stored before the compute), and the
    // 16-row fragment loads of the m-tiles not taken through LDS: all of them when XI = 0, the
    // second when XI > 0 and MT = 2 (those land in the registers the compute reads, so the next
    // stage's are issued after it)
    constexpr int MT0 = XI > 0 ? 1 : 0;
    auto load_x_rows = [&](int s, int slot) {
      if constexpr (XI > 0) {
        const int gi = 2 * s + ((lane & 31) >> 4);
        const int off = (g0 + 2 * s) * 256 + 16 * (lane & 31) + bias(gi);
#pragma unroll
        for (int i = 0; i < XI; ++i)
          xl[slot][i] = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, off + (2 * i + (lane >> 5)) * K * 2, 0, 0);
      }
    };
    auto load_x_frag = [&](int s, int slot) {
#pragma unroll
      for (int gs = 0; gs < 2; ++gs) {
        const int gi = 2 * s + gs;
        const int off = (g0 + gi) * 256 + 16 * j + bias(gi);
#pragma unroll
        for (int mt = MT0; mt < MT; ++mt) {
          const int o = (16 * mt + c) * K * 2 + off;  // rows past M: out of range (buffer size M * K * 2)
#pragma unroll
          for (int q = 0; q < 4; ++q) xr[slot][gs][mt][q] = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, o + 64 * q, 0, 0);
        }
      }
    };
    auto load_x = [&](int s, int slot) {
      load_x_rows(s, slot);
      load_x_frag(s, slot);
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
#pragma unroll
      for (int sub = 0; sub < SUB; ++sub) {
        uint32_t v;
        if constexpr (NF4) {
          v = sv[e][sub];
        } else {
          const int sh = 16 * (sub & 1);
          v = ((sv[e][sub >> 1] >> sh) & 0xFFFFu) | (((zv[e][sub >> 1] >> sh) & 0xFFFFu) << 16);
        }
        if (sz_row < ROWS) lds_sz[w][sz_row][(sz_g + e) * SUB + sub] = v;
      }

#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int u = s % D;
      if constexpr (B3) {
        // stage codes -> LDS: word 4 piece + e of the row's 24 is word wi = that % 12 of group
        // that / 12, i.e. kind wi % 3 (low 0, low 1, high) of block wi / 3
#pragma unroll
        for (int i = 0; i < CL; ++i) {
          const int p = lane + 64 * i, row = p / 6, piece = p - 6 * row;
          const u32x4_t v = cr[u][i];
          const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
          if (p < 6 * ROWS) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int wd = 4 * piece + e, gsw = wd / 12, wi = wd - 12 * gsw;
              lds_words[row * kRowStride3 + gsw * 12 + (wi % 3) * 4 + wi / 3] = vw[e];
            }
          }
        }
      } else {
        // stage codes -> LDS: piece lq holds words 4(lq%4) .. +3 of group lq/4; word 4p + e goes
        // to slot (row, group, j = e) at dword p
        const int gs = lq >> 2, p = lq & 3;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int row = 16 * nt + 8 * h + lr;
            const int swz = (row >> 1) & 7;
            const u32x4_t v = cr[u][2 * nt + h];
            lds_words[(row * 8 + ((gs * 4 + 0) ^ swz)) * 4 + p] = v.x;
            lds_words[(row * 8 + ((gs * 4 + 1) ^ swz)) * 4 + p] = v.y;
            lds_words[(row * 8 + ((gs * 4 + 2) ^ swz)) * 4 + p] = v.z;
            lds_words[(row * 8 + ((gs * 4 + 3) ^ swz)) * 4 + p] = v.w;
          }
      }
      if constexpr (XI > 0) {
#pragma unroll
        for (int i = 0; i < XI; ++i) lds_x[w][u % XS][2 * i + (lane >> 5)][lane & 31] = xl[u][i];
      }
      if (s + D < NS) load_codes(s + D, u);
      if constexpr (XI > 0) {
        if (s + D < NS) load_x_rows(s + D, u);
      }
      __builtin_amdgcn_sched_barrier(0);

#pragma unroll
      for (int gs = 0; gs < 2; ++gs) {
        const int gi = 2 * s + gs;
        if constexpr (XI > 0) {
          // A fragments from the LDS copy; rows past M read row 0 (their results are never stored)
          const int xrow = c < M ? c : 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) xr[u][gs][0][q] = lds_x[w][u % XS][xrow][16 * gs + 4 * q + j];
        }
        // sum of x over each quantization group's steps (for the zero)
        float4_t sx[NF4 ? 1 : MT][SUB];
        if constexpr (!NF4) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int sub = 0; sub < SUB; ++sub) {
              sx[mt][sub] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int q = sub * QS; q < (sub + 1) * QS; ++q)
                sx[mt][sub] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(xr[u][gs][mt][q]), ones, sx[mt][sub], 0, 0, 0);
            }
        }
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const int row = 16 * nt + c;
          float d[SUB], zf[SUB];
#pragma unroll
          for (int sub = 0; sub < SUB; ++sub) {
            const uint32_t szv = lds_sz[w][row][gi * SUB + sub];
            if constexpr (NF4) {
              d[sub] = __builtin_bit_cast(float, szv);
              zf[sub] = 0.f;
            } else {
              d[sub] = half_bits_to_float((uint16_t)(szv & 0xFFFFu));
              zf[sub] = half_bits_to_float((uint16_t)(szv >> 16));
            }
          }
          half8_t b[4];
          if constexpr (B3) {
            const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(&lds_words[row * kRowStride3 + gs * 12 + (j >> 1) * 4]);
            const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(&lds_words[row * kRowStride3 + gs * 12 + 8]);
            b[0] = codes3_word(lo.x, hi.x, j);
            b[1] = codes3_word(lo.y, hi.y, j);
            b[2] = codes3_word(lo.z, hi.z, j);
            b[3] = codes3_word(lo.w, hi.w, j);
          } else if constexpr (NF4) {
            const u32x4_t wq = lds_b[w][row * 8 + ((gs * 4 + j) ^ ((row >> 1) & 7))];
            b[0] = nf4_word(wq.x, lut);
            b[1] = nf4_word(wq.y, lut);
            b[2] = nf4_word(wq.z, lut);
            b[3] = nf4_word(wq.w, lut);
          } else {
            const u32x4_t wq = lds_b[w][row * 8 + ((gs * 4 + j) ^ ((row >> 1) & 7))];
            b[0] = codes_word(wq.x);
            b[1] = codes_word(wq.y);
            b[2] = codes_word(wq.z);
            b[3] = codes_word(wq.w);
          }
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int sub = 0; sub < SUB; ++sub) {
              float4_t a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int q = sub * QS; q < (sub + 1) * QS; ++q)
                a4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(xr[u][gs][mt][q]), b[q], a4, 0, 0, 0);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                if constexpr (NF4)
                  acc[nt][mt][i] = __builtin_fmaf(d[sub], a4[i], acc[nt][mt][i]);
                else
                  acc[nt][mt][i] = __builtin_fmaf(d[sub], __builtin_fmaf(-zf[sub], sx[mt][sub][i], a4[i]), acc[nt][mt][i]);
              }
            }
        }
        // with several scales per group, keep the two groups' work apart: interleaved, their
        // per-group sums and scales no longer fit in registers
        if constexpr (SUB > 1) __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (MT0 < MT) {
        if (s + D < NS) load_x_frag(s + D, u);
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

}  // namespace

struct SkinnyArgs {
  const uint16_t* x;
  const uint32_t* qweight;
  const void* scales;  // fp16 scales, or float32 absmax (NF4)
  const uint16_t* zeros;
  int64_t M, N, K;
  Nf4Table table;
  uint16_t* y;
  hipStream_t stream;
};

namespace {

using Args = SkinnyArgs;

template <int NTW, int MT, int NS, int XI, int SUB, int FMT>
hipError_t launch_tile_x(const Args& a) {
  const dim3 grid((unsigned)((a.N + 16 * NTW - 1) / (16 * NTW)));
  hipLaunchKernelGGL((skinny_kernel<NTW, MT, NS, XI, SUB, FMT>), grid, dim3(kThreads), 0, a.stream, a.x, a.qweight,
                     a.scales, a.zeros, (int)a.M, (int)a.N, (int)a.K, a.table, a.y);
  return hipGetLastError();
}

// M <= 8 (MT = 1): x rows through LDS in M/2 full-width loads; otherwise 16-row fragment loads
// (two column tiles with groups of 32 meet M <= 8 in two-stage chunks only). 4-bit integer
// codes take the LDS route for 12 <= M <= 16 too (eight loads for 16 rows), and 3-bit codes at
// M = 16; measured on MI355X against the fragment loads (same-process interleaved replays,
// outputs bit-identical), 4-bit groups of 128 at M = 16: 14.5 against 16.1 us at 8192 x 8192,
// 14.4 against 16.4 at 4096 -> 11008, 13.7 against 15.7 at 11008 -> 4096, 5.9 against 7.1 at
// 4096 x 4096, 37.9 against 43.7 at 8192 -> 22016, 42.7 against 44.4 at 22016 -> 8192;
// at M = 12 4-6 % faster on most shapes; at M = 9 up to 5 % slower (eight loads for nine rows);
// 3-bit codes at M = 16 1-18 % faster, at M = 12 mixed; NF4 at M = 16 from 8 % faster to 4 %
// slower, so NF4 keeps the fragment loads.
template <int NTW, int MT, int NS, int SUB, int FMT>
hipError_t launch_tile(const Args& a) {
  if constexpr (MT == 1 && !(NTW == 2 && SUB == 4 && NS > 2)) {
    if (a.M <= 2) return launch_tile_x<NTW, MT, NS, 1, SUB, FMT>(a);
    if (a.M <= 4) return launch_tile_x<NTW, MT, NS, 2, SUB, FMT>(a);
    if (a.M <= 8) return launch_tile_x<NTW, MT, NS, 4, SUB, FMT>(a);
    if constexpr (FMT != kFmtNf4 && !(FMT == kFmt3 && NS > 6)) {  // 3-bit eight-stage chunks would spill
      if (a.M >= (FMT == kFmt3 ? 16 : 12) && a.M <= 16) return launch_tile_x<NTW, MT, NS, 8, SUB, FMT>(a);
    }
  }
  // two m-tiles, 4- and 3-bit integer codes: the first m-tile's x rows through LDS, the
  // second's as fragment loads, wherever the variant fits the registers (one column tile, or
  // two with two-stage chunks; two tiles with longer chunks spill 200-400 bytes per lane).
  // 3-bit codes measured 3-25 % faster at M = 17..32 on the shapes it reaches (4096 x 4096
  // groups of 128: 9.5 against 11.7 us at M = 32; 8192 -> 22016 groups of 32: 60.6 against
  // 81.1); NF4 keeps the fragment loads (its codebook lookups share the LDS).
  if constexpr (MT == 2 && FMT != kFmtNf4 && (NTW == 1 || NS == 2)) return launch_tile_x<NTW, MT, NS, 8, SUB, FMT>(a);
  return launch_tile_x<NTW, MT, NS, 0, SUB, FMT>(a);
}

// stages per chunk: enough for the wave's whole share, up to CAP (2, 4 or 8; 4 at most with
// groups of 32, whose chunk of scales is four times as large)
template <int NTW, int MT, int SUB, int FMT, int CAP>
hipError_t launch_stages(const Args& a) {
  const int64_t stages = ((a.K / 128 + KS - 1) / KS + 1) / 2;  // per wave
  if constexpr (CAP == 2) {
    return launch_tile<NTW, MT, 2, SUB, FMT>(a);
  } else if constexpr (SUB == 4 || CAP == 4) {
    return stages <= 2 ? launch_tile<NTW, MT, 2, SUB, FMT>(a) : launch_tile<NTW, MT, 4, SUB, FMT>(a);
  } else {
    if (stages <= 2) return launch_tile<NTW, MT, 2, SUB, FMT>(a);
    if (stages <= 4) return launch_tile<NTW, MT, 4, SUB, FMT>(a);
    if (stages <= 6) return launch_tile<NTW, MT, 6, SUB, FMT>(a);
    return launch_tile<NTW, MT, kMaxStages, SUB, FMT>(a);
  }
}

// Column tiles per wave (NTW) and the stage cap, measured on MI355X at K = N = 8192,
// K = 4096 -> N = 11008 and K = 11008 -> N = 4096 for every format and M = 2..32:
//   * one column tile while M <= 4, on layers too narrow for 256 two-tile workgroups, and on
//     K <= 4096 up to M = 8: twice the workgroups and waves in flight (K = N = 8192, M = 2:
//     10.2 against 10.9 us; 4096 -> 11008, M = 2: 8.3 against 9.5 us); beyond, two column
//     tiles halve the x reads from L2, which then dominate (M = 8: 11.8 against 13.5 us);
//   * a two-stage cap where the longer chunk costs too many registers: groups of 32 always
//     (their four scales, zeros and x sums per group), groups of 64 with one column tile when
//     the grid needs two workgroups per CU (10.9 against 12.5 us at M = 4), groups of 64
//     at two m-tiles (M = 32: 25.2 against 27.0 us), NF4 at M = 5..8 (15.2 against
//     16.6 us) and NF4 blocks of 32 with one column tile at M <= 4;
//   * groups of 128 at two m-tiles keep two column tiles only up to 4 stages per wave (beyond
//     that the two-tile variant runs out of registers);
//   * 3-bit codes have rules of their own (below).
template <int SUB, int FMT>
hipError_t launch_format(const Args& a) {
  constexpr bool NF4 = FMT == kFmtNf4, B3 = FMT == kFmt3, zp = !NF4;
  const int64_t M = a.M;
  const bool wide = (a.N + 31) / 32 >= 256;
  if constexpr (B3) {
    // 3-bit codes, measured the same way (their dequant holds more registers and VALU time):
    // one column tile on narrow layers (full chunks for groups of 128 up to M = 16) and for
    // groups of 128 on K <= 4096 up to M = 4; otherwise two column tiles, with the two-stage
    // cap up to M = 8 (groups of 64, M = 4: 13.2 against 17.0 us with one tile) and for
    // groups of 32 at two m-tiles (groups of 64 there: four stages, as eight spill)
    if (!wide) {
      if (M > 16) return launch_stages<1, 2, SUB, FMT, 2>(a);
      if constexpr (SUB == 1) return launch_stages<1, 1, SUB, FMT, 8>(a);
      else return launch_stages<1, 1, SUB, FMT, 2>(a);
    }
    if (SUB == 1 && a.K <= 4096 && M <= 4) return launch_stages<1, 1, SUB, FMT, 2>(a);
    if (M <= 8) return launch_stages<2, 1, SUB, FMT, 2>(a);
    if (M <= 16) return launch_stages<2, 1, SUB, FMT, 8>(a);
    return launch_stages<2, 2, SUB, FMT, SUB == 4 ? 2 : SUB == 2 ? 4 : 8>(a);
  } else {
    if (M <= 4 || !wide || (a.K <= 4096 && M <= 8)) {
      const bool many = (a.N + 15) / 16 > 256;  // more than one one-tile workgroup per CU
      if (M > 16) return launch_stages<1, 2, SUB, FMT, zp && SUB == 4 ? 2 : 8>(a);
      if ((zp && SUB == 4) || (zp && SUB == 2 && M <= 4 && many) || (NF4 && SUB == 4 && M <= 4))
        return launch_stages<1, 1, SUB, FMT, 2>(a);
      return launch_stages<1, 1, SUB, FMT, 8>(a);
    }
    if (M <= 8) return launch_stages<2, 1, SUB, FMT, SUB == 4 || NF4 ? 2 : 8>(a);
    if (M <= 16) return launch_stages<2, 1, SUB, FMT, 8>(a);
    if constexpr (SUB == 1 && FMT == kFmt4) {
      const bool short_k = ((a.K / 128 + KS - 1) / KS + 1) / 2 <= 4;
      // from M = 24 two-stage chunks, which take the x route above (8192 x 8192 at M = 32:
      // 20.9 against 23.6 us; at M = 17 the longer chunks stay ahead, 18.1 against 19.2)
      if (short_k && M >= 24) return launch_stages<2, 2, SUB, FMT, 2>(a);
      return short_k ? launch_stages<2, 2, SUB, FMT, 8>(a) : launch_stages<1, 2, SUB, FMT, 8>(a);
    } else {
      return launch_stages<2, 2, SUB, FMT, zp ? 2 : 8>(a);
    }
  }
}

}  // namespace

// One launcher per (SUB, FMT) pair. The build compiles this file once per part
// (W4A16_SKINNY_PART = 0..4), each part holding some of the formats, so that the
// kernel instances compile in parallel; without the macro one object holds them all.
template <int SUB, int FMT>
hipError_t skinny_format(const SkinnyArgs& a);
template <> hipError_t skinny_format<1, kFmt4>(const SkinnyArgs& a);
template <> hipError_t skinny_format<2, kFmt4>(const SkinnyArgs& a);
template <> hipError_t skinny_format<4, kFmt4>(const SkinnyArgs& a);
template <> hipError_t skinny_format<1, kFmt3>(const SkinnyArgs& a);
template <> hipError_t skinny_format<2, kFmt3>(const SkinnyArgs& a);
template <> hipError_t skinny_format<4, kFmt3>(const SkinnyArgs& a);
template <> hipError_t skinny_format<1, kFmtNf4>(const SkinnyArgs& a);
template <> hipError_t skinny_format<2, kFmtNf4>(const SkinnyArgs& a);
template <> hipError_t skinny_format<4, kFmtNf4>(const SkinnyArgs& a);

#ifdef W4A16_SKINNY_PART
#define W4A16_SKINNY_IN_PART(p) (W4A16_SKINNY_PART == (p))
#else
#define W4A16_SKINNY_IN_PART(p) 1
#endif

#if W4A16_SKINNY_IN_PART(0)
template <>
hipError_t skinny_format<1, kFmt4>(const SkinnyArgs& a) { return launch_format<1, kFmt4>(a); }
#endif
#if W4A16_SKINNY_IN_PART(1)
template <>
hipError_t skinny_format<2, kFmt4>(const SkinnyArgs& a) { return launch_format<2, kFmt4>(a); }
template <>
hipError_t skinny_format<4, kFmt4>(const SkinnyArgs& a) { return launch_format<4, kFmt4>(a); }
#endif
#if W4A16_SKINNY_IN_PART(2)
template <>
hipError_t skinny_format<1, kFmt3>(const SkinnyArgs& a) { return launch_format<1, kFmt3>(a); }
template <>
hipError_t skinny_format<2, kFmt3>(const SkinnyArgs& a) { return launch_format<2, kFmt3>(a); }
#endif
#if W4A16_SKINNY_IN_PART(3)
template <>
hipError_t skinny_format<4, kFmt3>(const SkinnyArgs& a) { return launch_format<4, kFmt3>(a); }
template <>
hipError_t skinny_format<1, kFmtNf4>(const SkinnyArgs& a) { return launch_format<1, kFmtNf4>(a); }
#endif
#if W4A16_SKINNY_IN_PART(4)
template <>
hipError_t skinny_format<2, kFmtNf4>(const SkinnyArgs& a) { return launch_format<2, kFmtNf4>(a); }
template <>
hipError_t skinny_format<4, kFmtNf4>(const SkinnyArgs& a) { return launch_format<4, kFmtNf4>(a); }
#endif

#if W4A16_SKINNY_IN_PART(0)
int skinny_max_m() { return 32; }

hipError_t launch_skinny(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                         int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  return skinny_format<1, kFmt4>({x, qweight, scales, zeros, M, N, K, {}, y, stream});
}

hipError_t launch_skinny_variant(int bits, int group, const uint16_t* x, const uint32_t* qweight,
                                 const uint16_t* scales, const uint16_t* zeros, int64_t M, int64_t N, int64_t K,
                                 uint16_t* y, hipStream_t stream) {
  const SkinnyArgs a = {x, qweight, scales, zeros, M, N, K, {}, y, stream};
  if (bits == 4) {
    if (group == 128) return skinny_format<1, kFmt4>(a);
    if (group == 64) return skinny_format<2, kFmt4>(a);
    if (group == 32) return skinny_format<4, kFmt4>(a);
  } else if (bits == 3) {
    if (group == 128) return skinny_format<1, kFmt3>(a);
    if (group == 64) return skinny_format<2, kFmt3>(a);
    if (group == 32) return skinny_format<4, kFmt3>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_skinny_nf4(const Nf4Table& table, int block, const uint16_t* x, const uint32_t* qweight,
                             const float* absmax, int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const SkinnyArgs a = {x, qweight, absmax, nullptr, M, N, K, table, y, stream};
  if (block == 128) return skinny_format<1, kFmtNf4>(a);
  if (block == 64) return skinny_format<2, kFmtNf4>(a);
  if (block == 32) return skinny_format<4, kFmtNf4>(a);
  return hipErrorInvalidValue;
}
#endif

}  // namespace w4a16
