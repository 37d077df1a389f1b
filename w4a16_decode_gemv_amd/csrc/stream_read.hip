// A measurement aid, not part of the method: one launch that reads a buffer once,
// with the access pattern of the GEMV's code stream (each wave reads 1 KB of
// contiguous memory per 16-byte-per-lane load, non-temporal, all of a thread's loads
// issued before any is used), and does no other work. Timed beside the GEMV on the
// same number of bytes, it gives the single-launch floor of the weight stream on the
// machine at hand.
//
// The buffer is split into equal contiguous chunks, one per workgroup, over at least
// 1024 workgroups when there are enough bytes (four per CU, as the GEMV's 8192 x 8192
// launch has), so that no CU gets more than its share; thread t of a workgroup reads
// pieces t, t + 256, ... of its chunk. Nothing is written unless a thread's XOR of its
// words equals the magic value, so the loads cannot be optimised away and a test can
// check which workgroup read each piece.
#include <algorithm>

#include "device_utils.h"
#include "launchers.h"
#include "w4a16.h"

namespace w4a16 {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxLoads = 16;          // 16-byte loads per thread
constexpr int64_t kBlocksWanted = 1024;
constexpr uint32_t kMagic = W4A16_STREAM_READ_MAGIC;

struct Split {
  int64_t blocks, chunk;  // workgroups; pieces per workgroup (the last may have fewer)
  int loads;              // loads per thread
};

Split split_of(int64_t bytes) {
  const int64_t pieces = bytes / 16;
  int64_t blocks = std::min<int64_t>(kBlocksWanted, (pieces + kThreads - 1) / kThreads);
  blocks = std::max<int64_t>(blocks, (pieces + int64_t(kThreads) * kMaxLoads - 1) / (int64_t(kThreads) * kMaxLoads));
  const int64_t chunk = (pieces + blocks - 1) / blocks;
  return {(pieces + chunk - 1) / chunk, chunk, (int)((chunk + kThreads - 1) / kThreads)};
}

template <int U>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4_t* __restrict__ buf, int64_t pieces,
                                                               int64_t chunk, uint32_t* __restrict__ sink) {
  const int64_t begin = (int64_t)blockIdx.x * chunk;
  const int64_t end = begin + chunk < pieces ? begin + chunk : pieces;
  u32x4_t v[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int64_t p = begin + threadIdx.x + (int64_t)i * kThreads;
    v[i] = __builtin_nontemporal_load(&buf[p < end ? p : end - 1]);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int64_t p = begin + threadIdx.x + (int64_t)i * kThreads;
    if (p < end) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  if (acc == kMagic) sink[blockIdx.x] = acc;
}

template <int U>
hipError_t launch_u(const void* buf, int64_t pieces, const Split& sp, uint32_t* sink, hipStream_t stream) {
  if constexpr (U > kMaxLoads) {
    return hipErrorInvalidValue;
  } else {
    if (sp.loads > U) return launch_u<U + 1>(buf, pieces, sp, sink, stream);
    hipLaunchKernelGGL((stream_read_kernel<U>), dim3((unsigned)sp.blocks), dim3(kThreads), 0, stream,
                       static_cast<const u32x4_t*>(buf), pieces, sp.chunk, sink);
    return hipGetLastError();
  }
}

// A second read pattern that shares nothing with the GEMV's grid: a grid-stride
// read in tiles of THREADS x U pieces. Tile i is pieces [i T U, (i + 1) T U); thread t
// of the workgroup that takes it loads pieces i T U + t + j T (j < U), all U loads
// issued before any is used. Workgroup b takes tiles b, b + grid, b + 2 grid, ...
// (a persistent loop when the grid is smaller than the tile count).
template <int THREADS, int U>
__global__ __launch_bounds__(THREADS) void stream_read_grid_kernel(const u32x4_t* __restrict__ buf, int64_t pieces,
                                                                   uint32_t* __restrict__ sink) {
  constexpr int64_t kTile = (int64_t)THREADS * U;
  const int64_t tiles = (pieces + kTile - 1) / kTile;
  uint32_t acc = 0;
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int64_t base = tile * kTile + threadIdx.x;
    u32x4_t v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t p = base + (int64_t)j * THREADS;
      v[j] = __builtin_nontemporal_load(&buf[p < pieces ? p : pieces - 1]);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t p = base + (int64_t)j * THREADS;
      if (p < pieces) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
  }
  if (acc == kMagic) sink[blockIdx.x] = acc;
}

template <int THREADS>
hipError_t launch_grid_t(const void* buf, int64_t pieces, int blocks, int unroll, uint32_t* sink, hipStream_t stream) {
  const u32x4_t* b = static_cast<const u32x4_t*>(buf);
  switch (unroll) {
    case 1: hipLaunchKernelGGL((stream_read_grid_kernel<THREADS, 1>), dim3(blocks), dim3(THREADS), 0, stream, b, pieces, sink); break;
    case 2: hipLaunchKernelGGL((stream_read_grid_kernel<THREADS, 2>), dim3(blocks), dim3(THREADS), 0, stream, b, pieces, sink); break;
    case 4: hipLaunchKernelGGL((stream_read_grid_kernel<THREADS, 4>), dim3(blocks), dim3(THREADS), 0, stream, b, pieces, sink); break;
    case 8: hipLaunchKernelGGL((stream_read_grid_kernel<THREADS, 8>), dim3(blocks), dim3(THREADS), 0, stream, b, pieces, sink); break;
    case 16: hipLaunchKernelGGL((stream_read_grid_kernel<THREADS, 16>), dim3(blocks), dim3(THREADS), 0, stream, b, pieces, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int64_t stream_read_blocks(int64_t bytes) { return split_of(bytes).blocks; }

hipError_t launch_stream_read_grid(const void* buf, int64_t bytes, int threads, int blocks, int unroll, uint32_t* sink,
                                   hipStream_t stream) {
  const int64_t pieces = bytes / 16;
  switch (threads) {
    case 64: return launch_grid_t<64>(buf, pieces, blocks, unroll, sink, stream);
    case 128: return launch_grid_t<128>(buf, pieces, blocks, unroll, sink, stream);
    case 256: return launch_grid_t<256>(buf, pieces, blocks, unroll, sink, stream);
    case 512: return launch_grid_t<512>(buf, pieces, blocks, unroll, sink, stream);
    case 1024: return launch_grid_t<1024>(buf, pieces, blocks, unroll, sink, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  return launch_u<1>(buf, bytes / 16, split_of(bytes), sink, stream);
}

}  // namespace w4a16
