// Internal kernel launchers. Arguments are already validated by the C ABI
// (abi.hip); each launcher enqueues its kernel(s) on `stream` and returns the
// HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_utils.h"

namespace w4a16 {

hipError_t launch_channel_scale(const uint16_t* x_cal, int64_t T, int64_t K, double alpha, float* s,
                                hipStream_t stream);

hipError_t launch_scale_input(const uint16_t* x, const float* s, int64_t M, int64_t K, uint16_t* x_s,
                              hipStream_t stream);

hipError_t launch_rmsnorm_fold(const uint16_t* h, const uint16_t* gamma, const float* s, int64_t M, int64_t K,
                               double eps, uint16_t* x_s, hipStream_t stream);

// bits 3 or 4, group 32, 64 or 128 (validated by the caller)
hipError_t launch_quantize_pack(const uint16_t* w, const float* s, int64_t N, int64_t K, int bits, int group,
                                uint32_t* qweight, uint16_t* scales, uint16_t* zeros, hipStream_t stream);

// Symmetric absmax quantize-pack (codes q + 2^(b-1), zeros 2^(b-1)); bits 3 or 4, group 32, 64, 128.
hipError_t launch_quantize_pack_sym(const uint16_t* w, const float* s, int64_t N, int64_t K, int bits, int group,
                                    uint32_t* qweight, uint16_t* scales, uint16_t* zeros, hipStream_t stream);

// NF4 quantize-pack with the 16 fp16 codebook levels (ascending, two per word) in lut[8];
// block 32, 64 or 128; codes in layout v1, float32 absmax [N][K/block].
hipError_t launch_nf4_quantize_pack(const uint16_t* w, const float* s, int64_t N, int64_t K, int block,
                                    const uint32_t* lut, uint32_t* qweight, float* absmax, hipStream_t stream);

// GEMV kernel: needs M <= gemv_max_m() and gemv_supports(M, K).
int gemv_max_m();
bool gemv_supports(int64_t M, int64_t K);
// whether the GEMV takes narrow (4-row) tiles for this shape: M <= 2, one 32-input
// piece per thread, and fewer than 16 waves per CU with the default tiles
bool gemv_narrow(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemv(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                       const uint16_t* zeros, int64_t M, int64_t N, int64_t K, uint16_t* y,
                       hipStream_t stream);

// GEMV for the other code formats (bits 3 or 4, group 32, 64 or 128): needs
// gemv_variant_supports(M, K, group).
bool gemv_variant_supports(int64_t M, int64_t K, int group);
// whether launch_gemv_variant (bits 3 or 4) or launch_gemv_nf4 (bits 0) takes this shape,
// on whichever GEMV kernel it routes it to
bool gemv_format_supports(int bits, int group, int64_t M, int64_t N, int64_t K);
hipError_t launch_gemv_variant(int bits, int group, const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                               const uint16_t* zeros, int64_t M, int64_t N, int64_t K, uint16_t* y,
                               hipStream_t stream);

// Small-batch MFMA kernel: needs M <= skinny_max_m(). The variant takes 4-bit codes (layout
// v1) or 3-bit codes (the packed 3-bit layout) with groups of 32, 64 or 128 (scales and zeros
// 4-byte aligned below groups of 128), the NF4 entry point float32 absmax per block of 32, 64
// or 128.
int skinny_max_m();
hipError_t launch_skinny(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                         const uint16_t* zeros, int64_t M, int64_t N, int64_t K, uint16_t* y,
                         hipStream_t stream);
hipError_t launch_skinny_variant(int bits, int group, const uint16_t* x, const uint32_t* qweight,
                                 const uint16_t* scales, const uint16_t* zeros, int64_t M, int64_t N, int64_t K,
                                 uint16_t* y, hipStream_t stream);
hipError_t launch_skinny_nf4(const Nf4Table& table, int block, const uint16_t* x, const uint32_t* qweight,
                             const float* absmax, int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream);

// Split-K MFMA GEMM (4-bit, groups of 128): S partial tiles in a float32 workspace of
// splitk_workspace_floats(M, N, S) floats, then a fixed-order reduction into y. Needs 1 <= S <= K/128.
int splitk_max_splits();
int splitk_default_splits(int64_t M, int64_t N, int64_t K);
int64_t splitk_tiles(int64_t M, int64_t N);  // output tiles of the partial kernel (64 x 128)
int64_t splitk_workspace_floats(int64_t M, int64_t N, int splits);
hipError_t launch_splitk(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                         int64_t M, int64_t N, int64_t K, int splits, float* workspace, uint16_t* y,
                         hipStream_t stream);
// The library's own split-K partials for callers that cannot allocate: a static device
// array of kSplitkScratchFloats floats per GPU. splitk_scratch returns its address on the
// device of `stream` (resolved once per device; the first call on a device makes HIP calls).
constexpr int64_t kSplitkScratchFloats = int64_t(1) << 23;  // 32 MiB
hipError_t splitk_scratch(hipStream_t stream, float** ptr);

// The split-K reduction alone: y[m][n] = f16(sum over s = 0..S-1, in index order, of
// part[s][m][n]), part float32 [S][M][N].
hipError_t launch_splitk_reduce(const float* part, int64_t M, int64_t N, int S, uint16_t* y, hipStream_t stream);

// Small-batch MFMA kernel with x held in registers and K split into xres_ranges(M, N, K) ranges
// of 2048 or 1024 inputs (4-bit, groups of 128 or 64): needs xres_supports(M, K) (M <= 32, an even number of
// groups per row) and scales and zeros 4-byte aligned; with more than one range, a float32
// workspace of xres_workspace_floats(M, N, K) floats.
int xres_max_m();
// the workgroup shape launch_xres takes: waves (a K range is 256 * waves inputs) and 16-column
// n-tiles per wave
void xres_config(int64_t M, int64_t N, int64_t K, int* waves, int* tiles);
int xres_waves(int64_t M, int64_t N, int64_t K);
int xres_ranges(int64_t M, int64_t N, int64_t K);
bool xres_supports(int64_t M, int64_t K);
int64_t xres_workspace_floats(int64_t M, int64_t N, int64_t K);
hipError_t launch_xres(int group, const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                       int64_t M, int64_t N, int64_t K, float* workspace, uint16_t* y, hipStream_t stream);
// the same with 4 or 8 waves per workgroup (ranges of 1024 or 2048 inputs) and 4 n-tiles per
// wave (64 columns) for M <= 16, 8 (128 columns) above; the workspace holds the ranges of that
// choice; another shape or group returns hipErrorInvalidValue
hipError_t launch_xres_config(int waves, int tiles, int group, const uint16_t* x, const uint32_t* qweight,
                              const uint16_t* scales, const uint16_t* zeros, int64_t M, int64_t N, int64_t K,
                              float* workspace, uint16_t* y, hipStream_t stream);

// Tiled MFMA kernel: any M >= 1. mfma_workgroups: the workgroups launch_mfma starts (for M > 16).
int64_t mfma_workgroups(int64_t M, int64_t N);
hipError_t launch_mfma(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                       const uint16_t* zeros, int64_t M, int64_t N, int64_t K, uint16_t* y,
                       hipStream_t stream);

// K-lane MFMA kernel (4-bit, groups of 128): any M >= 1; klane_workgroups gives its grid.
int64_t klane_workgroups(int64_t M, int64_t N);
hipError_t launch_klane(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                        int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream);

// AWQ scale search: the original layer's output (float32), and the loss of one
// candidate scale (number of float64 partials it writes; loss kernel + fixed-order
// reduction).
hipError_t launch_output_reference(const uint16_t* x, const uint16_t* w, int64_t T, int64_t N, int64_t K, float* y,
                                   hipStream_t stream);
int64_t alpha_loss_partials(int64_t T, int64_t N);
hipError_t launch_alpha_loss(const uint16_t* x_s, const uint32_t* qweight, const uint16_t* scales,
                             const uint16_t* zeros, const float* y_ref, int64_t T, int64_t N, int64_t K,
                             double* partials, double* loss, hipStream_t stream);

// The search's choice on the device: best = first index of the smallest of `count` losses,
// alpha = best / (count - 1), and (when s is not NULL) s = s_all[best][0..K).
hipError_t launch_search_select(const double* losses, int count, const float* s_all, int64_t K, int32_t* best,
                                double* alpha, float* s, hipStream_t stream);

// Tiled MFMA kernel for the other code formats (bits 3 or 4, group 32, 64 or 128); any M >= 1.
hipError_t launch_mfma_variant(int bits, int group, const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                               const uint16_t* zeros, int64_t M, int64_t N, int64_t K, uint16_t* y,
                               hipStream_t stream);

// NF4 linear (codes in layout v1, float32 absmax per block of 32, 64 or 128): the GEMV kernel's
// NF4 variant (needs gemv_variant_supports(M, K, block)) and the tiled MFMA kernel's (any M).
hipError_t launch_gemv_nf4(const Nf4Table& table, int block, const uint16_t* x, const uint32_t* qweight,
                           const float* absmax, int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream);
hipError_t launch_mfma_nf4(const Nf4Table& table, int block, const uint16_t* x, const uint32_t* qweight,
                           const float* absmax, int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream);

// measurement aid: one read of a buffer with the GEMV's access pattern
int64_t stream_read_blocks(int64_t bytes);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);
// grid-stride read in tiles of threads x unroll pieces (threads 64..1024, unroll 1..16, powers of two)
hipError_t launch_stream_read_grid(const void* buf, int64_t bytes, int threads, int blocks, int unroll, uint32_t* sink,
                                   hipStream_t stream);

}  // namespace w4a16
