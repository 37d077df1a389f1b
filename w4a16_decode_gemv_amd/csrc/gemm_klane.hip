// W4A16 GEMM for batches whose layers have few output tiles for the chip: K split
// into "K-lanes" inside each workgroup, so that a CU runs four waves per output tile
// without a global workspace.
//
// y[m][n] = sum_g d[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g])
//
// The fused dequantize + multiply of the other kernels ("MIT 6.5940 L13 LLM
// Deployment" guide, TinyChat kernel fusion); at large batch the layer is a dense
// contraction and belongs on the matrix cores ("CMU 11-868 Model Quantization"
// guide, "where the speed comes from"); dequantization in the GEMM main loop costs
// ALU time (L13 guide, QServe), so every rebuilt weight feeds four m-tiles of MFMAs.
//
// Shape, measured against the tiled kernel on the LLaMA projection shapes (it wins
// where the tiled kernel has one or two workgroups per CU and long rows, e.g. 11008 ->
// 4096 at M = 128: 37 against 57 us):
//   * a workgroup owns an output tile of BM = 16 MW rows by BN = 16 NW columns and
//     has KL waves, each a K-lane taking a contiguous range of the groups of 128
//     inputs; at the end the KL partial tiles are added in LDS in K-lane order
//     (reproducible) and rounded once to fp16;
//   * each wave computes its whole MW x NW grid of 16 x 16 tiles: per group it
//     rebuilds its NW n-tiles' codes (4 words per lane and n-tile) as exact fp16
//     (q - z), and every rebuilt B fragment feeds MW MFMAs (one per m-tile);
//   * x reaches the A fragments through a wave-private LDS area: whole 128-byte
//     lines are loaded (4 rows x 256 bytes per load), written to LDS, and read back
//     in fragment order (a fragment read straight from memory would take 16 half
//     lines per load). Codes go straight to registers, one 16-byte load per lane,
//     n-tile and group. Loads run R groups ahead, as range-checked buffer loads: rows
//     past M or N and groups past the K-lane's range read as zero, with no memory
//     traffic, so the stage sequence is a fixed pipeline;
//   * the group's scale is applied once per output element and group: the MFMAs of
//     the group's 4 steps accumulate sum x (q - z) exactly into P, then
//     acc += d * P (one FMA per element).
// A wave meeting a group whose zero lies outside [-2032, 1024] (possible only
// for one-signed groups) takes the general route for that group: exact q in the
// MFMA, and the zero applied as z * sum_k x, with sum_k x from MFMAs against ones.
//
// MFMA 16x16x32 f16 fragments: lane l holds A[m = l%16][8 k-slots of slot group
// l/16] and B[the same 8 k-slots][n = l%16]; D[m = 4(l/16) + i][n = l%16]. Step s
// of a group takes inputs 32s .. 32s+31, slot group j the 8 inputs 32s + 8j .. +8:
// code word 4s + j of the row. A lane's 16-byte code load brings words 4j .. 4j+3,
// so the four 16-lane rows exchange words with two levels of permlane swaps (a 4 x 4
// transpose) before the dequantization.
#include "device_utils.h"
#include "launchers.h"

namespace w4a16 {

namespace {

template <int MW, int NW>
struct KlaneStage {
  u32x4_t x[MW][4];  // A fragments: m-tile, step
  u32x4_t q[NW];     // the 4 code words (steps) of each n-tile
  uint32_t s[NW];    // fp16 scale bits
  uint32_t z[NW];    // fp16 zero bits
};

template <int MW, int NW, int KL, int R>
__global__ __launch_bounds__(64 * KL) __attribute__((amdgpu_waves_per_eu(2, 2))) void klane_kernel(const uint16_t* __restrict__ x,
                                                        const uint32_t* __restrict__ qw,
                                                        const uint16_t* __restrict__ scales,
                                                        const uint16_t* __restrict__ zeros, int M, int N, int K,
                                                        int TM, uint16_t* __restrict__ y) {
  constexpr int BM = 16 * MW, BN = 16 * NW;
  constexpr int kTile = MW * NW * 4;  // fp32 accumulator values per lane
  constexpr int kXBytes = KL * BM * 17 * 16;  // x areas: BM rows of 17 chunks per wave
  constexpr int kRedBytes = KL > 1 ? (KL - 1) * kTile * 64 * 4 : 4;
  __shared__ __align__(16) unsigned char smem[kXBytes > kRedBytes ? kXBytes : kRedBytes];
  float* red = reinterpret_cast<float*>(smem);
  // the K-lane is the wave's index: uniform over the wave, so every address derived from it
  // stays scalar (a per-lane buffer resource would need a waterfall loop around each load)
  const int lane = threadIdx.x & 63, kl = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane >> 4, c = lane & 15;
  const int item = xcd_contiguous_item(blockIdx.x, gridDim.x);
  const int tm = item % TM, tn = item / TM;  // the m-tiles of one weight tile run on one XCD
  const int m0 = tm * BM, n0 = tn * BN;
  const int G = K >> 7;
  // this K-lane's groups [g_begin, g_begin + gcount): the first G % KL lanes take one more
  const int base = G / KL, extra = G % KL;
  const int g_begin = kl * base + min(kl, extra);
  const int gcount = base + (kl < extra ? 1 : 0);

  const int64_t rows_m = min(M - m0, BM), rows_n = min(N - n0, BN);
  // this K-lane's first group in each tensor, and the bytes from there to the end of the tile's
  // rows; group g of the K-lane gets views that start g groups further on (scalar arithmetic,
  // so the per-load offsets below are fixed registers)
  const uint16_t* x0 = x + (int64_t)m0 * K + (int64_t)g_begin * 128;
  const uint32_t* q0 = qw + (int64_t)n0 * (K >> 3) + (int64_t)g_begin * 16;
  const uint16_t* s0 = scales + (int64_t)n0 * G + g_begin;
  const uint16_t* z0 = zeros + (int64_t)n0 * G + g_begin;
  const int64_t x_bytes = rows_m * K * 2 - (int64_t)g_begin * 256;
  const int64_t q_bytes = rows_n * (K >> 1) - (int64_t)g_begin * 64;
  const int64_t sz_bytes = rows_n * G * 2 - (int64_t)g_begin * 2;
  // x load u takes rows 4u .. 4u+3 of the m-block, 256 contiguous bytes (a group) each:
  // lane l row 4u + l/16 and 16-byte chunk l%16
  const int xo = (lane >> 4) * K * 2 + (lane & 15) * 16;
  const int qo = c * (K >> 1) + j * 16;  // lane's row within an n-tile, its 16 bytes of a group
  const int so = c * G * 2;

  using Stage = KlaneStage<MW, NW>;
  Stage set[R];
  // group g of this K-lane (0 .. gcount-1); groups past the range read as zero
  // x first: the LDS store of a group's x waits (in issue order) only for the loads issued
  // before its own, not for that group's codes, which come from HBM and are needed later
  auto issue = [&](int g, Stage& r) {
    // views of group g (empty past the K-lane's range: every load reads zero); each view
    // ends at the tile's last row, so rows past M or N read zero too
    const bool in = g < gcount;
    const __amdgpu_buffer_rsrc_t rx = rsrc(x0 + g * 128, in ? x_bytes - g * 256 : 0);
    const __amdgpu_buffer_rsrc_t rq = rsrc(q0 + g * 16, in ? q_bytes - g * 64 : 0);
    const __amdgpu_buffer_rsrc_t rs = rsrc(s0 + g, in ? sz_bytes - g * 2 : 0);
    const __amdgpu_buffer_rsrc_t rz = rsrc(z0 + g, in ? sz_bytes - g * 2 : 0);
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s) r.x[mt][s] = load16(rx, xo + (4 * mt + s) * 4 * K * 2);
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) {
      r.q[nt] = load16(rq, qo + nt * 16 * (K >> 1));
      r.s[nt] = __builtin_amdgcn_raw_buffer_load_b16(rs, so + nt * 16 * G * 2, 0, 0);
      r.z[nt] = __builtin_amdgcn_raw_buffer_load_b16(rz, so + nt * 16 * G * 2, 0, 0);
    }
  };
  // this wave's LDS area (rows padded to 17 chunks: the 16 lanes of one fragment read hit
  // distinct banks), written by the coalesced loads and read back as A fragments
  u32x4_t* xa = reinterpret_cast<u32x4_t*>(smem) + kl * BM * 17;
  auto stash = [&](const Stage& r) {
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s) xa[(4 * (4 * mt + s) + (lane >> 4)) * 17 + (lane & 15)] = r.x[mt][s];
  };
  // orders one wave's LDS stores and loads across its lanes (free at run time: a wave's LDS
  // accesses complete in order)
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  };

  float4_t acc[MW][NW];
#pragma unroll
  for (int mt = 0; mt < MW; ++mt)
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) acc[mt][nt] = (float4_t){0.f, 0.f, 0.f, 0.f};

  // One group: per step s the A fragments of every m-tile (from this wave's LDS area, or
  // from the stage registers) and the B fragments of every n-tile (rebuilt from one code
  // word each), then MW x NW independent MFMAs; the group's scale once per element.
  auto compute = [&](const Stage& r) {
    bool out = false;
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) {
      const float zf = half_bits_to_float((uint16_t)r.z[nt]);
      out |= !(zf >= -2032.0f && zf <= 1024.0f);
    }
    const bool fast = __builtin_amdgcn_ballot_w64(out) == 0;  // uniform over the wave
    // code words in step order: lane (j, n) holds words 4j + t (t = 0..3) of row n's group and
    // needs words 4s + j (s = 0..3), a 4 x 4 transpose across the four 16-lane rows
    uint32_t w[NW][4];
    half2_t c_lo[NW], c_hi[NW];
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) {
      const auto a01 = __builtin_amdgcn_permlane16_swap(r.q[nt].x, r.q[nt].y, false, false);
      const auto a23 = __builtin_amdgcn_permlane16_swap(r.q[nt].z, r.q[nt].w, false, false);
      const auto b02 = __builtin_amdgcn_permlane32_swap(a01[0], a23[0], false, false);
      const auto b13 = __builtin_amdgcn_permlane32_swap(a01[1], a23[1], false, false);
      w[nt][0] = b02[0];
      w[nt][1] = b13[0];
      w[nt][2] = b02[1];
      w[nt][3] = b13[1];
      // exact (q - z) on the usual route, exact q on the general one
      const _Float16 zh = __builtin_bit_cast(_Float16, (uint16_t)r.z[nt]);
      const _Float16 clo = fast ? -((_Float16)1024.0f + zh) : (_Float16)-1024.0f;
      const _Float16 chi = fast ? -((_Float16)64.0f + zh) : (_Float16)-64.0f;
      c_lo[nt] = (half2_t){clo, clo};
      c_hi[nt] = (half2_t){chi, chi};
    }
    float4_t p[MW][NW];
    float4_t sx[MW];
    const u32x4_t ones_bits = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t f[MW];
#pragma unroll
      for (int mt = 0; mt < MW; ++mt) f[mt] = xa[(16 * mt + c) * 17 + 4 * s + j];
      half8_t b[NW];
#pragma unroll
      for (int nt = 0; nt < NW; ++nt) b[nt] = dequant_word(w[nt][s], c_lo[nt], c_hi[nt]);
#pragma unroll
      for (int nt = 0; nt < NW; ++nt)
#pragma unroll
        for (int mt = 0; mt < MW; ++mt)
          p[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(f[mt]), b[nt],
                                                             s == 0 ? (float4_t){0.f, 0.f, 0.f, 0.f} : p[mt][nt], 0, 0, 0);
      if (!fast) {
#pragma unroll
        for (int mt = 0; mt < MW; ++mt)
          sx[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(f[mt]), as_half8(ones_bits),
                                                          s == 0 ? (float4_t){0.f, 0.f, 0.f, 0.f} : sx[mt], 0, 0, 0);
      }
    }
    if (!fast) {
      // the general route's zero term, -z * sum_k x, goes into the group's product first; only
      // this temporary differs between the routes, so the accumulators are updated in one place
#pragma unroll
      for (int nt = 0; nt < NW; ++nt) {
        const float zf = half_bits_to_float((uint16_t)r.z[nt]);
#pragma unroll
        for (int mt = 0; mt < MW; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) p[mt][nt][i] = __builtin_fmaf(-zf, sx[mt][i], p[mt][nt][i]);
      }
    }
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) {
      const float d = half_bits_to_float((uint16_t)r.s[nt]);
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][nt][i] = __builtin_fmaf(d, p[mt][nt][i], acc[mt][nt][i]);
    }
  };

#pragma unroll
  for (int r = 0; r < R; ++r) {
    issue(r, set[r]);
    __builtin_amdgcn_sched_barrier(0);  // stages stay in issue order: the waits count on it
  }
  stash(set[0]);
  wave_sync();
  for (int g0 = 0; g0 < gcount; g0 += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (g0 + r < gcount) compute(set[r]);
      wave_sync();  // the fragment reads come before the next group's stores
      __builtin_amdgcn_sched_barrier(0);
      issue(g0 + r + R, set[r]);
      __builtin_amdgcn_sched_barrier(0);
      stash(set[(r + 1) % R]);  // the next group's x
      wave_sync();
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load in flight at exit

  // K-lanes 1..KL-1 hand their partial tiles to K-lane 0 through LDS (lane-contiguous:
  // no bank conflicts), which adds them in K-lane order and stores y
  if constexpr (KL > 1) {
    __syncthreads();  // every wave is done with its x area, which the partials reuse
    if (kl > 0) {
      float* dst = red + (kl - 1) * kTile * 64 + lane;
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int nt = 0; nt < NW; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[((mt * NW + nt) * 4 + i) * 64] = acc[mt][nt][i];
    }
    __syncthreads();
    if (kl > 0) return;
#pragma unroll
    for (int w = 1; w < KL; ++w) {
      const float* src = red + (w - 1) * kTile * 64 + lane;
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int nt = 0; nt < NW; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][nt][i] += src[((mt * NW + nt) * 4 + i) * 64];
    }
  }
#pragma unroll
  for (int nt = 0; nt < NW; ++nt) {
    const int n = n0 + 16 * nt + c;
    if (n >= N) continue;
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 16 * mt + 4 * j + i;
        if (m < M) y[(int64_t)m * N + n] = float_to_half_bits(acc[mt][nt][i]);
      }
  }
}

// the one shape measured best on the LLaMA projection shapes: 64 x 32 tiles, four K-lanes,
// loads two groups ahead (sweeps of 33 <= M <= 512 over nine layer shapes). 64 x 64 tiles
// need AGPR spills of the accumulators; one group ahead was slower; with two waves per SIMD,
// eight K-lanes (4096 -> 4096 at M = 128: 18.0 against 15.8 us, slower on every shape) and
// 32 x 64 tiles (17.7 against 15.8 us; half the x reads per output, twice the dequant per
// MFMA) were slower too
constexpr int kMW = 4, kNW = 2, kKL = 4, kR = 2;

}  // namespace

int64_t klane_workgroups(int64_t M, int64_t N) { return ((M + 16 * kMW - 1) / (16 * kMW)) * ((N + 16 * kNW - 1) / (16 * kNW)); }

hipError_t launch_klane(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                        int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const int64_t TM = (M + 16 * kMW - 1) / (16 * kMW);
  hipLaunchKernelGGL((klane_kernel<kMW, kNW, kKL, kR>), dim3((unsigned)klane_workgroups(M, N)), dim3(64 * kKL), 0, stream,
                     x, qweight, scales, zeros, (int)M, (int)N, (int)K, (int)TM, y);
  return hipGetLastError();
}

}  // namespace w4a16
