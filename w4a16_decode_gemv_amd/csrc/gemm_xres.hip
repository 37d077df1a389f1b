// Small-batch W4A16 GEMM (M <= 32, 4-bit codes, groups of 128 or 64) with each wave's block of
// x held in registers for the whole launch and K split across workgroups.
//
// y[m][n] = f16( sum_s P_s[m][n] ),
// P_s[m][n] = sum_{g in range s} d[n][g] * sum_{k in g} x[m][k] (q[n][k] - z[n][g])
//
// The fused dequantize + multiply of the other kernels ("MIT 6.5940 L13 LLM Deployment"
// guide, TinyChat kernel fusion), on the matrix cores because every weight serves up to 32
// rows of x ("CMU 11-868 Model Quantization" guide, where the speed comes from).
//
// Why another small-batch kernel. The small-batch kernel's workgroups own 32 output columns
// and all of K, so each of them reads all of x: at M = 32 on an 8192 x 8192 layer that is
// 128 MB of L2-to-L1 traffic beside 34 MB of codes, and that path sets its time. Here a
// workgroup owns 64 or 128 columns and one range of 256 inputs per wave (eight or four waves,
// see xres_config). Each of its waves loads the x fragments of its 256 inputs (two groups, 16
// or 32 rows) once, keeps them in registers, and streams the codes of all the workgroup's
// columns past them: x crosses L2 -> L1 once per 64 or 128 columns (8 MB at M = 32 on
// 8192 x 8192). Every x, scale, zero and code load of a wave is issued before its first MFMA
// (8 or 16 KB of codes per wave in flight), so the weight stream keeps the GEMV's depth.
//
// Per 16-column n-tile and group the group's MFMA steps (four for groups of 128; two for
// groups of 64, where each step takes 32 contiguous inputs) accumulate sum x (q - z) exactly (fp16
// (q - z) B fragments while every zero of the wave lies in [-2032, 1024]; otherwise the wave
// takes exact q and z * sum x for all its groups, sum x from an MFMA against ones), then
// acc += d * that. The waves' float32 tiles are added through LDS in wave order. With one K range the sums are
// rounded to fp16 and written to y; otherwise range s writes its tile to the
// caller's workspace P[s][m][n] and the split-K reduction kernel adds the ranges in index
// order and rounds once. Results are reproducible.
#include <type_traits>

#include "device_utils.h"
#include "launchers.h"

namespace w4a16 {

namespace {

constexpr int kXrGroups = 2;                           // groups of 128 inputs per wave

// grid: ceil(N / (16 NT)) * S items, item = n-tile * S + range (ranges of one n-tile
// adjacent); WV waves, each with NT 16-column n-tiles and MT 16-row m-tiles (M <= 16 * MT)
//
// Loads are whole 128-byte lines: a code row's two groups (128 bytes) come from 8 lanes, an x
// row's 512 bytes from 32 lanes. The MFMA fragments need lane (c, j) to hold row c, so codes
// and x pass through LDS (XOR-swizzled, conflict-free both ways), inside the wave's slice of
// the reduction area: x once, before that slice holds any partial tile, and each n-tile's codes
// through two slots that hold no partial tile yet (with one m-tile and eight n-tiles the last
// n-tile uses the wave's (scale, zero) table for its second half, read before). Each wave keeps
// its own (scale, zero) table: no workgroup barrier before the final sums. With one m-tile and
// four n-tiles a workgroup needs 35 or 70 KB of LDS and at most 128 VGPRs, so 16 waves share a
// CU. Measured (timing-only copies, 8192 x 8192 at M = 4): half-line code loads cost 2.5 us;
// on 22016 -> 8192 at M = 16 (three rounds of workgroups) one workgroup per CU cost 6-8 us
// against two.
template <int MT, int WV, int NT, int GS, bool DIRECT>
__global__ __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(MT == 1 ? 4 : 2)))
void xres_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw,
                 const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int M, int N, int K, int S,
                 float* __restrict__ part, uint16_t* __restrict__ y) {
  // red[wave]: first the wave's x rows [16 MT][32 pieces], then the code stage, then its
  // partial tiles
  constexpr int kXrThreads = 64 * WV;
  constexpr int kXrRangeGroups = WV * kXrGroups;  // groups per K range
  constexpr int kXrTiles = NT;                     // 16-column n-tiles per wave
  constexpr int kXrCols = 16 * NT;                 // output columns per workgroup
  constexpr int kSlotTiles = NT < 8 ? 8 : NT;      // slots per m-tile: x needs 8 KB per m-tile
  constexpr bool kSpare = NT * MT <= kSlotTiles * MT - 2;  // two slots past the partial tiles
  constexpr int kGB = 128 / GS;                     // groups per 128 inputs
  constexpr int kSPG = 4 / kGB;                     // MFMA steps per group
  constexpr int kGSh = GS == 128 ? 7 : (GS == 64 ? 6 : 5);
  __shared__ float4_t red[WV][kSlotTiles * MT][64];
  __shared__ u32x4_t wsz[WV][12 * NT * kGB];  // the wave's (scale, zero) table: 3 kGB x 16 NT words
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int j = lane >> 4, c = lane & 15;
  const int item = xcd_contiguous_item(blockIdx.x, gridDim.x);
  const int range = item % S, tn = item / S;
  const int n0 = tn * kXrCols;
  const int G = K >> kGSh;
  const int g0 = range * kXrRangeGroups + wave * kXrGroups;  // this wave's first 128 inputs, in 128s
  // G is even and so is g0: a wave holds both of its groups or neither; a wave past the last
  // group reads zeros everywhere (no traffic) and adds exact zeros
  const int past = (int)(g0 >= (K >> 7)) * kOutOfRange;
  const int rows_n = min(N - n0, kXrCols);
  const __amdgpu_buffer_rsrc_t rx = rsrc(x, (int64_t)M * K * 2);  // rows past M read zero
  const __amdgpu_buffer_rsrc_t rq = rsrc(qw + (int64_t)n0 * (K >> 3), (int64_t)rows_n * (K >> 1));
  const __amdgpu_buffer_rsrc_t rs = rsrc(scales + (int64_t)n0 * G, (int64_t)rows_n * G * 2);
  const __amdgpu_buffer_rsrc_t rz = rsrc(zeros + (int64_t)n0 * G, (int64_t)rows_n * G * 2);

  // (1) the wave's (scale, zero) pairs (its 2 kGB groups, two per word) of rows lane and lane + 64
  uint32_t sv[NT / 4][kGB], zv[NT / 4][kGB];
#pragma unroll
  for (int u = 0; u < NT / 4; ++u)
#pragma unroll
    for (int w = 0; w < kGB; ++w) {
      const int off = (lane + 64 * u) * G * 2 + g0 * kGB * 2 + 4 * w + past;
      sv[u][w] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
      zv[u][w] = __builtin_amdgcn_raw_buffer_load_b32(rz, off, 0, 0);
    }
  __builtin_amdgcn_sched_barrier(0);
  // (2) x rows of the wave's 256 inputs: load i takes row 2i + lane / 32, piece lane % 32 (16
  //     bytes; piece p is input chunk p % 16 of group g0 + p / 16)
  u32x4_t xl[8 * MT];
#pragma unroll
  for (int i = 0; i < 8 * MT; ++i) xl[i] = load16(rx, (2 * i + (lane >> 5)) * K * 2 + g0 * 256 + (lane & 31) * 16 + past);
  __builtin_amdgcn_sched_barrier(0);
  // (3) codes: n-tile tt, load i takes row 16 tt + 8i + lane / 8, piece lane % 8 (piece p holds
  //     words 4 (p % 4) .. + 3 of group g0 + p / 4); non-temporal (read once)
  //     With one m-tile the last n-tile's codes are issued after the first n-tile's compute (its
  //     registers then free), which keeps the wave within 128 VGPRs (two workgroups per CU).
  u32x4_t q[kXrTiles][2];
  constexpr int kLate = MT == 1 && NT == 8 ? kXrTiles - 1 : kXrTiles;  // n-tiles issued up front
  auto issue_codes = [&](int tt) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      q[tt][i] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                       rq, (16 * tt + 8 * i + (lane >> 3)) * (K >> 1) + g0 * 64 + (lane & 7) * 16 + past, 0,
                       kNonTemporal));
  };
#pragma unroll
  for (int tt = 0; tt < kLate; ++tt) {
    issue_codes(tt);
    __builtin_amdgcn_sched_barrier(0);  // loads stay in compute order: each n-tile waits only for its own
  }

  // x into the wave's slice of red (row r, piece p at r * 32 + (p ^ (r % 16))), then the
  // fragments: m-tile mt, group h, step s of lane (c, j) is row 16 mt + c, piece 16 h + 4 j + s
  u32x4_t* xs = reinterpret_cast<u32x4_t*>(&red[wave][0][0]);
#pragma unroll
  for (int i = 0; i < 8 * MT; ++i) {
    const int r = 2 * i + (lane >> 5);
    xs[r * 32 + ((lane & 31) ^ (r & 15))] = xl[i];
  }
  u32x4_t xf[MT][kXrGroups][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int h = 0; h < kXrGroups; ++h)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        xf[mt][h][s] = xs[(16 * mt + c) * 32 + 16 * h + ((GS == 128 ? 4 * j + s : 4 * s + j) ^ c)];
  // The wave's table: word r the scale pair of row r; then, when every zero of the wave lies in
  // [-2032, 1024] (one ballot), words kXrCols + r and 2 kXrCols + r the two groups' fp16 pair
  // (-(1024 + z), -(64 + z)) that rebuilds q - z exactly, else word kXrCols + r the zero pair
  // (the general route: exact q and z * sum x).
  //   With groups of 64 or 32 the table holds kGB scale words, then 2 kGB pair words (one per
  //   group) or kGB zero words; group gg of the wave is half gg % 2 of scale (zero) word gg / 2.
  uint32_t* sz = reinterpret_cast<uint32_t*>(&wsz[wave][0]);
  bool in_range = true;
#pragma unroll
  for (int u = 0; u < NT / 4; ++u)
#pragma unroll
    for (int gg = 0; gg < 2 * kGB; ++gg) {
      const float zf = half_bits_to_float((uint16_t)(zv[u][gg >> 1] >> (16 * (gg & 1))));
      in_range = in_range && zf >= -2032.0f && zf <= 1024.0f;
    }
  const bool fast = __builtin_amdgcn_ballot_w64(!in_range) == 0;
#pragma unroll
  for (int u = 0; u < NT / 4; ++u) {
#pragma unroll
    for (int w = 0; w < kGB; ++w) sz[w * kXrCols + lane + 64 * u] = sv[u][w];
    if (fast) {
#pragma unroll
      for (int gg = 0; gg < 2 * kGB; ++gg) {
        const _Float16 zh = __builtin_bit_cast(_Float16, (uint16_t)(zv[u][gg >> 1] >> (16 * (gg & 1))));
        const _Float16 clo = -((_Float16)1024.0f + zh), chi = -((_Float16)64.0f + zh);
        sz[(kGB + gg) * kXrCols + lane + 64 * u] =
            (uint32_t)__builtin_bit_cast(uint16_t, clo) | ((uint32_t)__builtin_bit_cast(uint16_t, chi) << 16);
      }
    } else {
#pragma unroll
      for (int w = 0; w < kGB; ++w) sz[(kGB + w) * kXrCols + lane + 64 * u] = zv[u][w];
    }
  }

  // (4) compute each n-tile as its codes land. Its two loads go to the stage: rows 0..7 to half
  //     A, rows 8..15 to half B, row r at (r % 8) * 8 + (p ^ ((r % 8) / 2 + 4 (r / 8))) for piece
  //     p; lane (c, j) reads row c, pieces j and 4 + j: words 4j .. 4j + 3 of each group, the B
  //     fragments of steps 0..3. A is the wave's last partial-tile slot and B the one before,
  //     both written after the last n-tile's stage reads; with one m-tile B is the next-to-last
  //     tile's own slot (written after its stage reads) and, for the last n-tile, the
  //     (scale, zero) area, whose pairs that tile has read by then.
  const u32x4_t ones_bits = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
  const half8_t ones = as_half8(ones_bits);
  u32x4_t* half_a = reinterpret_cast<u32x4_t*>(&red[wave][kSlotTiles * MT - 1][0]);
  u32x4_t* half_b = reinterpret_cast<u32x4_t*>(&red[wave][kSlotTiles * MT - 2][0]);
  auto tiles = [&](auto route) {
    constexpr bool FAST = decltype(route)::value;
#pragma unroll
  for (int tt = 0; tt < kXrTiles; ++tt) {
    const int row = 16 * tt + c;
    // scale words, then the pair words (fast route) or the zero words (general route)
    uint32_t sw[kGB], cws[2 * kGB];
#pragma unroll
    for (int w = 0; w < kGB; ++w) sw[w] = sz[w * kXrCols + row];
#pragma unroll
    for (int gg = 0; gg < 2 * kGB; ++gg) cws[gg] = FAST || gg < kGB ? sz[(kGB + gg) * kXrCols + row] : 0u;
    constexpr bool kBorrow = !kSpare && MT == 1;  // the last n-tile's half B is the table's area
    u32x4_t* hb = (kBorrow && tt == kXrTiles - 1) ? &wsz[wave][0] : half_b;
    // the table is read through another type than the stage is written with: keep the reads
    // first where they share the area
    if (kBorrow && tt == kXrTiles - 1) asm volatile("" ::: "memory");
    // groups of 64 or 32: word e of piece p goes to slot 4 (p / 4) + e, element p % 4, so that
    // lane (c, j) reads words j, 4 + j, 8 + j, 12 + j of each 128 inputs: step s then spans the
    // 32 inputs 32 s .. 32 s + 31 (x fragments read in the same order), one group or half of one
    if constexpr (GS != 128) asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = lane >> 3, swz = (r >> 1) | (i << 2);
      if constexpr (GS == 128) {
        (i ? hb : half_a)[r * 8 + ((lane & 7) ^ swz)] = q[tt][i];
      } else {
        uint32_t* dst = reinterpret_cast<uint32_t*>(i ? hb : half_a);
        const int pc = lane & 7;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(r * 8 + ((4 * (pc >> 2) + e) ^ swz)) * 4 + (pc & 3)] = q[tt][i][e];
      }
    }
    if constexpr (GS != 128) asm volatile("" ::: "memory");
    const int ci = c & 7, cb = c >> 3;
    const u32x4_t* hc = cb ? hb : half_a;
    const u32x4_t qc[2] = {hc[ci * 8 + (j ^ ((ci >> 1) | (cb << 2)))], hc[ci * 8 + ((4 + j) ^ ((ci >> 1) | (cb << 2)))]};
    float4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < kXrGroups; ++h)
#pragma unroll
      for (int gi = 0; gi < kGB; ++gi) {
      const int gg = h * kGB + gi;  // the wave's group; its steps are gi kSPG .. (gi + 1) kSPG - 1
      const float d = half_bits_to_float((uint16_t)(sw[gg >> 1] >> (16 * (gg & 1))));
      const uint32_t cw = FAST ? cws[gg] : 0xD400E400u;  // (-1024, -64): exact q
      const _Float16 clo = __builtin_bit_cast(_Float16, (uint16_t)(cw & 0xFFFFu));
      const _Float16 chi = __builtin_bit_cast(_Float16, (uint16_t)(cw >> 16));
      const half2_t c_lo = {clo, clo}, c_hi = {chi, chi};
      half8_t bq[kSPG];
#pragma unroll
      for (int s = 0; s < kSPG; ++s) bq[s] = dequant_word(qc[h][gi * kSPG + s], c_lo, c_hi);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        float4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kSPG; ++s)
          a = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(xf[mt][h][gi * kSPG + s]), bq[s], a, 0, 0, 0);
        if constexpr (FAST) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][i] = __builtin_fmaf(d, a[i], acc[mt][i]);
        } else {
          const float zf = half_bits_to_float((uint16_t)(cws[gg >> 1] >> (16 * (gg & 1))));
          float4_t sx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < kSPG; ++s)
            sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(xf[mt][h][gi * kSPG + s]), ones, sx, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][i] = __builtin_fmaf(d, __builtin_fmaf(-zf, sx[i], a[i]), acc[mt][i]);
        }
      }
    }
    // D fragment: lane (c, j) holds rows 16 mt + 4j + i of column n0 + 16 tt + c
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[wave][tt * MT + mt][lane] = acc[mt];
    if (tt == 0 && kLate < kXrTiles) {
      __builtin_amdgcn_sched_barrier(0);
      issue_codes(kXrTiles - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  };
  if (fast)
    tiles(std::true_type{});
  else
    tiles(std::false_type{});
  __syncthreads();

  // (5) the eight waves' tiles added in wave order; each thread takes whole D-fragment slots
  constexpr int kSlots = kXrTiles * MT * 64;
  float* p = DIRECT ? nullptr : part + (int64_t)range * M * N;
#pragma unroll
  for (int u0 = 0; u0 < kSlots; u0 += kXrThreads) {
    const int u = u0 + t;
    if (kSlots % kXrThreads != 0 && u >= kSlots) break;
    const int tile = u >> 6, ln = u & 63;
    float4_t sum = red[0][tile][ln];
#pragma unroll
    for (int w = 1; w < WV; ++w) sum += red[w][tile][ln];
    const int tt = tile / MT, mt = tile % MT;
    const int n = n0 + 16 * tt + (ln & 15);
    if (n < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * mt + 4 * (ln >> 4) + i;
        if (m < M) {
          if constexpr (DIRECT)
            y[(int64_t)m * N + n] = float_to_half_bits(sum[i]);
          else
            p[(int64_t)m * N + n] = sum[i];
        }
      }
    }
  }
}

template <int MT, int WV, int NT, int GS>
hipError_t launch_mt(const uint16_t* x, const uint32_t* qw, const uint16_t* sc, const uint16_t* zr, int64_t M,
                     int64_t N, int64_t K, float* workspace, uint16_t* y, hipStream_t stream) {
  const int S = (int)((K / 128 + WV * kXrGroups - 1) / (WV * kXrGroups));
  const int64_t items = ((N + 16 * NT - 1) / (16 * NT)) * S;
  if (S == 1)
    hipLaunchKernelGGL((xres_kernel<MT, WV, NT, GS, true>), dim3((unsigned)items), dim3(64 * WV), 0, stream, x, qw, sc,
                       zr, (int)M, (int)N, (int)K, 1, nullptr, y);
  else
    hipLaunchKernelGGL((xres_kernel<MT, WV, NT, GS, false>), dim3((unsigned)items), dim3(64 * WV), 0, stream, x, qw, sc,
                       zr, (int)M, (int)N, (int)K, S, workspace, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  return launch_splitk_reduce(workspace, M, N, S, y, stream);
}

}  // namespace

int xres_max_m() { return 32; }

// The workgroup shape: waves (two groups of 128 inputs each; a K range is 256 * waves inputs)
// and 16-column n-tiles per wave. From timings of the four shapes (graph-timed us, partials and
// reduction; waves x n-tiles):
// - one m-tile (M <= 16): four n-tiles (64 columns; 94 VGPRs and 36 or 72 KB of LDS, so 16
//   waves share a CU), eight waves where such workgroups come to at least 512, else four:
//   8192 -> 8192 at M = 16 13.3 (8 x 4) against 14.6 (8 x 8) and 13.8 (4 x 4); 22016 -> 8192
//   at M = 16 28.2 against 29.3; 8192 -> 28672 at M = 8 31.6 against 34.0; 8192 -> 1024 at
//   M = 16 6.8 (4 x 4) against 8.4 (8 x 4) and 12.2 (8 x 8); 4096 -> 11008 at M = 8 10.7 (4 x 4)
//   against 11.7 (8 x 4); 11008 -> 4096 at M = 16 13.1 against 13.7;
// - two m-tiles: eight n-tiles, four waves where eight-wave workgroups would come to at least
//   512 (two or more rounds of the chip: 68 KB of LDS, two per CU), else eight: 22016 -> 8192 at
//   M = 32 40.4 (4 x 8) against 45.0 (8 x 8), 8192 -> 28672 at M = 32 47.9 against 59.4;
//   8192 -> 8192 at M = 32 17.8 (8 x 8) against 18.7 (4 x 8) and 18.0 (4 x 4).
void xres_config(int64_t M, int64_t N, int64_t K, int* waves, int* tiles) {
  const int64_t ranges8 = (K / 128 + 15) / 16;
  if (M <= 16) {
    *tiles = 4;
    *waves = ((N + 63) / 64) * ranges8 >= 512 ? 8 : 4;
  } else {
    *tiles = 8;
    *waves = ((N + 127) / 128) * ranges8 >= 512 ? 4 : 8;
  }
}

int xres_waves(int64_t M, int64_t N, int64_t K) {
  int waves, tiles;
  xres_config(M, N, K, &waves, &tiles);
  return waves;
}

int xres_ranges(int64_t M, int64_t N, int64_t K) {
  const int64_t g = (int64_t)xres_waves(M, N, K) * kXrGroups;
  return (int)((K / 128 + g - 1) / g);
}

bool xres_supports(int64_t M, int64_t K) { return M >= 1 && M <= xres_max_m() && (K / 128) % 2 == 0; }

int64_t xres_workspace_floats(int64_t M, int64_t N, int64_t K) {
  const int S = xres_ranges(M, N, K);
  return S == 1 ? 0 : (int64_t)S * M * N;
}

hipError_t launch_xres_config(int waves, int tiles, int group, const uint16_t* x, const uint32_t* qweight,
                              const uint16_t* scales, const uint16_t* zeros, int64_t M, int64_t N, int64_t K,
                              float* workspace, uint16_t* y, hipStream_t stream) {
#define W4A16_XRES(MT, WV, NT) \
  if (waves == WV && tiles == NT) {                                                                                   \
    if (group == 128) return launch_mt<MT, WV, NT, 128>(x, qweight, scales, zeros, M, N, K, workspace, y, stream);  \
    if (group == 64) return launch_mt<MT, WV, NT, 64>(x, qweight, scales, zeros, M, N, K, workspace, y, stream);    \
    return hipErrorInvalidValue;                                                                                      \
  }
  // the shapes xres_config chooses
  if (M <= 16) {
    W4A16_XRES(1, 4, 4) W4A16_XRES(1, 8, 4)
  } else {
    W4A16_XRES(2, 8, 8) W4A16_XRES(2, 4, 8)
  }
#undef W4A16_XRES
  return hipErrorInvalidValue;
}

hipError_t launch_xres(int group, const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                       int64_t M, int64_t N, int64_t K, float* workspace, uint16_t* y, hipStream_t stream) {
  int waves, tiles;
  xres_config(M, N, K, &waves, &tiles);
  return launch_xres_config(waves, tiles, group, x, qweight, scales, zeros, M, N, K, workspace, y, stream);
}

}  // namespace w4a16
