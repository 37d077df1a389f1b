// W4A16 GEMM with K split across workgroups, for batches whose output has too few
// tiles to fill the chip (M = 128..256 against N = 4096..11008: 64-172 tiles of
// 64 x 128 for 256 CUs).
//
// y[m][n] = f16( sum_s P_s[m][n] ),  P_s[m][n] = sum_{g in split s} d[n][g] * sum_{k in g} x[m][k] (q[n][k] - z[n][g])
//
// The same fused dequantize + multiply as the other kernels ("MIT 6.5940 L13 LLM
// Deployment" guide, TinyChat kernel fusion; "CMU 11-868 Model Quantization"
// guide: at large batch the layer is compute-bound and belongs on the matrix
// cores). The K groups are split into S contiguous ranges; workgroup (tile, s)
// computes the float32 partial P_s of its 64 x 128 tile (32 x 128 for batches of at
// most 32 rows) over range s and writes it to the caller's workspace; a second
// kernel adds the S partials of every output in index order (reproducible) and
// rounds once to fp16. With one range the partial kernel writes y itself (same bits, no
// workspace, no second kernel).
//
// Partial kernel (same structure as the AWQ-search loss kernel): eight waves,
// each owning 16 output rows n and all 64 (or 32) rows m, one group per stage; the x tile
// is shared through LDS, a wave's codes and (scale, zero) stay in its registers;
// loads run two stages ahead in register sets, as buffer loads (rows past M or N
// and stages past the range read as zero, with no traffic), with an LDS-only
// barrier so loads stay in flight across it. B fragments are exact fp16 (q - z)
// while z lies in [-2032, 1024] (one FMA by the scale per output and group); a
// wave meeting another zero takes the general route for that stage (exact q and
// z * sum_k x with sum_k x from an MFMA against ones). The x fragments of the next
// m-tile are read from LDS while the current m-tile's MFMAs run (2-12 % faster on
// the LLaMA2-7B serving shapes than reading each fragment just before its MFMA).
#include <algorithm>
#include <mutex>

#include "device_utils.h"
#include "launchers.h"

// The split-K partials of w4a16_linear_splitk_noalloc, for callers that cannot
// allocate: one array per GPU the library runs on, held until the process ends.
// Host code never passes this name to a kernel (on the host it stands for no device
// address); it resolves the array's address on each device once, with
// hipGetSymbolAddress, and passes that address.
static __device__ __align__(256) float scratch[w4a16::kSplitkScratchFloats];

namespace w4a16 {

namespace {


constexpr int WAVES = 8;
constexpr int BN = 16 * WAVES;         // 128 rows n
constexpr int kThreads = 64 * WAVES;
constexpr int R = 2;                   // stages of loads in flight
constexpr int kMaxSplits = 16;




template <int XU>
struct Stage {
  u32x4_t x[XU];
  u32x4_t q;
  uint16_t s, z;
};

// grid: tiles_m * tiles_n * S items; item = (n-tile, split, m-tile) with m-tile fastest.
// MT 16-row MFMA tiles of m per workgroup: 4 (64 rows), or 2 (32 rows) for batches of at
// most 32 rows, where 64-row tiles would spend half their MFMA and LDS work on absent rows.
// DIRECT (one range, S = 1): the tile's sums are rounded to fp16 and written to y here, with
// no partials and no second kernel; the same bits as the partial plus a one-range reduction.
template <int MT, bool DIRECT = false>
__global__ __launch_bounds__(kThreads) void splitk_partial_kernel(const uint16_t* __restrict__ x,
                                                                 const uint32_t* __restrict__ qw,
                                                                 const uint16_t* __restrict__ scales,
                                                                 const uint16_t* __restrict__ zeros, int M, int N,
                                                                 int K, int S, int TM, float* __restrict__ part,
                                                                 uint16_t* __restrict__ y) {
  constexpr int BM = 16 * MT;              // rows m per workgroup
  constexpr int XU = BM * 16 / kThreads;   // 16-byte x chunks per thread per stage
  __shared__ u32x4_t lx[2][BM][17];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int j = lane >> 4, c = lane & 15;
  const int item = xcd_contiguous_item(blockIdx.x, gridDim.x);
  const int tm = item % TM;
  const int rest = item / TM;
  const int split = rest % S;
  const int tn = rest / S;
  const int m0 = tm * BM, n0 = tn * BN;
  const int G = K >> 7;
  // this split's groups [g_begin, g_end): the first G % S splits take one more
  const int base = G / S, extra = G % S;
  const int g_begin = split * base + min(split, extra);
  const int gcount = base + (split < extra ? 1 : 0);
  const int nl = wave * 16 + c;

  const int64_t rows_m = min(M - m0, BM), rows_n = min(N - n0, BN);
  const __amdgpu_buffer_rsrc_t rx = rsrc(x + (int64_t)m0 * K + (int64_t)g_begin * 128, rows_m * K * 2 - (int64_t)g_begin * 256);
  const __amdgpu_buffer_rsrc_t rq = rsrc(qw + (int64_t)n0 * (K >> 3) + (int64_t)g_begin * 16, rows_n * (K >> 1) - (int64_t)g_begin * 64);
  const __amdgpu_buffer_rsrc_t rs = rsrc(scales + (int64_t)n0 * G + g_begin, rows_n * G * 2 - (int64_t)g_begin * 2);
  const __amdgpu_buffer_rsrc_t rz = rsrc(zeros + (int64_t)n0 * G + g_begin, rows_n * G * 2 - (int64_t)g_begin * 2);
  int xoff[XU];
#pragma unroll
  for (int u = 0; u < XU; ++u) xoff[u] = ((t >> 4) + (kThreads / 16) * u) * K * 2 + (t & 15) * 16;
  const int qo = nl * (K >> 1) + j * 16;
  const int so = nl * G * 2;

  Stage<XU> set[R];
  // stage g of this split (0 .. gcount-1); stages past the split read as zero
  auto issue = [&](int g, Stage<XU>& r) {
    const int past = (int)(g >= gcount) * kOutOfRange;
#pragma unroll
    for (int u = 0; u < XU; ++u) r.x[u] = load16(rx, xoff[u] + g * 256 + past);
    r.q = load16(rq, qo + g * 64 + past);
    r.s = __builtin_amdgcn_raw_buffer_load_b16(rs, so + g * 2 + past, 0, 0);
    r.z = __builtin_amdgcn_raw_buffer_load_b16(rz, so + g * 2 + past, 0, 0);
  };
  auto store = [&](const Stage<XU>& r, int b) {
#pragma unroll
    for (int u = 0; u < XU; ++u) lx[b][(t >> 4) + (kThreads / 16) * u][t & 15] = r.x[u];
  };

  float4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = (float4_t){0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Stage<XU>& r, int b) {
    // x fragments one m-tile ahead: the next tile's LDS reads overlap this tile's MFMAs
    half8_t xa[2][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) xa[0][st] = as_half8(lx[b][c][4 * j + st]);
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
        for (int st = 0; st < 4; ++st) xa[(mt + 1) & 1][st] = as_half8(lx[b][16 * (mt + 1) + c][4 * j + st]);
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
  store(set[0], 0);
  lds_barrier();
  for (int g0 = 0; g0 < gcount; g0 += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int g = g0 + r;
      if (g < gcount) compute(set[r], r & 1);
      __builtin_amdgcn_sched_barrier(0);
      issue(g + R, set[r]);
      __builtin_amdgcn_sched_barrier(0);
      store(set[(r + 1) % R], (r + 1) & 1);
      lds_barrier();
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load in flight at exit

  const int n = n0 + nl;
  if constexpr (DIRECT) {
    if (n < N) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + 16 * mt + 4 * j + i;
          if (m < M) y[(int64_t)m * N + n] = float_to_half_bits(acc[mt][i]);
        }
    }
    return;
  }
  // the partial of this split: part[split][m][n]
  if (n < N) {
    float* p = part + (int64_t)split * M * N;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 16 * mt + 4 * j + i;
        if (m < M) p[(int64_t)m * N + n] = acc[mt][i];
      }
  }
}

// y[e] = f16( ((part[0][e] + part[1][e]) + ...) ), four outputs per thread. With the split
// count known at compile time (SC > 0) every partial's load is issued before the first add;
// a runtime count (SC = 0) keeps four loads in flight. A loop over a runtime count with one
// load per trip waited for each load in turn (one memory round trip per split).
template <int SC>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int64_t total, int S,
                                                           uint16_t* __restrict__ y) {
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e0 >= total) return;
  if (e0 + 4 <= total && (total & 3) == 0) {
    float4_t s;
    if constexpr (SC > 0) {
      float4_t v[SC];
#pragma unroll
      for (int k = 0; k < SC; ++k) v[k] = *reinterpret_cast<const float4_t*>(part + (int64_t)k * total + e0);
      s = v[0];
#pragma unroll
      for (int k = 1; k < SC; ++k) s += v[k];
    } else {
      s = *reinterpret_cast<const float4_t*>(part + e0);
      int k = 1;
      for (; k + 4 <= S; k += 4) {
        float4_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float4_t*>(part + (int64_t)(k + u) * total + e0);
#pragma unroll
        for (int u = 0; u < 4; ++u) s += v[u];
      }
      for (; k < S; ++k) s += *reinterpret_cast<const float4_t*>(part + (int64_t)k * total + e0);
    }
    const uint32_t lo = (uint32_t)float_to_half_bits(s[0]) | ((uint32_t)float_to_half_bits(s[1]) << 16);
    const uint32_t hi = (uint32_t)float_to_half_bits(s[2]) | ((uint32_t)float_to_half_bits(s[3]) << 16);
    if ((reinterpret_cast<uintptr_t>(y + e0) & 7) == 0) {
      *reinterpret_cast<uint2*>(y + e0) = make_uint2(lo, hi);
      return;
    }
    y[e0] = (uint16_t)(lo & 0xFFFFu);
    y[e0 + 1] = (uint16_t)(lo >> 16);
    y[e0 + 2] = (uint16_t)(hi & 0xFFFFu);
    y[e0 + 3] = (uint16_t)(hi >> 16);
    return;
  }
  for (int64_t e = e0; e < min(e0 + 4, total); ++e) {
    float s = part[e];
    for (int k = 1; k < S; ++k) s += part[(int64_t)k * total + e];
    y[e] = float_to_half_bits(s);
  }
}

// rows m per workgroup of the partial kernel for a batch of M rows
int64_t rows_per_tile(int64_t M) { return M <= 32 ? 32 : 64; }

int64_t tiles_of(int64_t M, int64_t N) {
  const int64_t bm = rows_per_tile(M);
  return ((M + bm - 1) / bm) * ((N + BN - 1) / BN);
}

}  // namespace

int splitk_max_splits() { return kMaxSplits; }

int64_t splitk_tiles(int64_t M, int64_t N) { return tiles_of(M, N); }

int splitk_default_splits(int64_t M, int64_t N, int64_t K) {
  // about two workgroups per CU, rounded up to a power of two (3 splits measured slower than
  // 4 on the 4096 -> 11008 layer at M = 128), at most 4 splits (more cost more in partial
  // traffic and pipeline fill than they gain: measured on the LLaMA2-7B serving shapes), and
  // at least four groups per split
  const int64_t tiles = tiles_of(M, N);
  const int64_t G = K / 128;
  const int64_t want = (512 + tiles - 1) / tiles;
  int64_t s = 1;
  while (s < want && s < 4) s <<= 1;
  s = std::min<int64_t>(s, std::max<int64_t>(1, G / 4));
  return (int)std::max<int64_t>(1, s);
}

int64_t splitk_workspace_floats(int64_t M, int64_t N, int splits) { return (int64_t)splits * M * N; }

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch[kMaxDevices];  // device address of `scratch` per device, resolved once
}  // namespace

hipError_t splitk_scratch(hipStream_t stream, float** ptr) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    int current = 0;
    e = hipGetDevice(&current);
    if (e != hipSuccess) return e;
    if (current != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = current != dev ? hipSetDevice(current) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

hipError_t launch_splitk(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                         int64_t M, int64_t N, int64_t K, int splits, float* workspace, uint16_t* y,
                         hipStream_t stream) {
  const int64_t bm = rows_per_tile(M);
  const int TM = (int)((M + bm - 1) / bm);
  const int64_t items = tiles_of(M, N) * splits;
  if (splits == 1) {
    // one range: the kernel writes y itself (the workspace is not touched)
    if (bm == 32)
      hipLaunchKernelGGL((splitk_partial_kernel<2, true>), dim3((unsigned)items), dim3(kThreads), 0, stream, x,
                         qweight, scales, zeros, (int)M, (int)N, (int)K, 1, TM, nullptr, y);
    else
      hipLaunchKernelGGL((splitk_partial_kernel<4, true>), dim3((unsigned)items), dim3(kThreads), 0, stream, x,
                         qweight, scales, zeros, (int)M, (int)N, (int)K, 1, TM, nullptr, y);
    return hipGetLastError();
  }
  if (bm == 32)
    hipLaunchKernelGGL(splitk_partial_kernel<2>, dim3((unsigned)items), dim3(kThreads), 0, stream, x, qweight, scales,
                       zeros, (int)M, (int)N, (int)K, splits, TM, workspace, nullptr);
  else
    hipLaunchKernelGGL(splitk_partial_kernel<4>, dim3((unsigned)items), dim3(kThreads), 0, stream, x, qweight, scales,
                       zeros, (int)M, (int)N, (int)K, splits, TM, workspace, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(workspace, M, N, splits, y, stream);
}

hipError_t launch_splitk_reduce(const float* part, int64_t M, int64_t N, int S, uint16_t* y, hipStream_t stream) {
  const int64_t total = M * N;
  const int64_t grid = (total + 1023) / 1024;
  switch (S) {
#define W4A16_REDUCE(SC)                                                                                      \
  case SC:                                                                                                     \
    hipLaunchKernelGGL(splitk_reduce_kernel<SC>, dim3((unsigned)grid), dim3(256), 0, stream, part, total, S, y); \
    break;
    W4A16_REDUCE(2)
    W4A16_REDUCE(4)
    W4A16_REDUCE(8)
    W4A16_REDUCE(16)
#undef W4A16_REDUCE
    default:
      hipLaunchKernelGGL(splitk_reduce_kernel<0>, dim3((unsigned)grid), dim3(256), 0, stream, part, total, S, y);
  }
  return hipGetLastError();
}

}  // namespace w4a16
