/*
 * w4a16.h - C ABI of the MI355X (gfx950) W4A16 group-quantized linear library.
 *
 * What it computes (pages cited by title and section):
 *   - AWQ, "MIT 6.5940 L13 LLM Deployment" reading guide, AWQ section (slides
 *     25-28): salient input channels of the weight are multiplied by
 *     s = s_X^alpha, where s_X is the mean activation magnitude; the matching
 *     input channel is divided by s (the 1/s is folded into the previous op);
 *     weights are quantized with Q(w) = Delta * Round(w / Delta), per group of
 *     128 input channels (QServe table: W4-A16, 4-bit per-group, group 128).
 *   - Zero-point (asymmetric) form: "CMU 11-868 Model Quantization" guide, L19
 *     "absmax and zero-point": scale from max - min (a zero range counts as 1),
 *     an integer zero offset, codes clipped to the integer range.
 *   - TinyChat, same L13 guide (slides 36-37): 4-bit codes reordered offline so
 *     that an AND and a shift unpack them, and dequantization fused into the
 *     matrix multiply so no dequantized weight is written to memory.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers (HIP device memory on the GPU the
 *     stream belongs to). The caller allocates and owns every buffer; the
 *     library never allocates, frees or keeps device memory, holds no mutable
 *     global state, and is safe to call from several host threads.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *     Calls are asynchronous and stream-ordered. A fault inside a kernel shows up
 *     at the caller's next synchronization, as for any HIP kernel.
 *   - Every argument check runs on the host before any HIP call; a failed check
 *     returns a nonzero status and launches nothing. w4a16_last_error() then
 *     describes the failure (thread-local text).
 *   - Outputs must not alias inputs. Inputs are assumed finite.
 *   - fp16 is IEEE binary16, little-endian; matrices are row-major, dense.
 *
 * Packed weight layout, version 1 (w4a16_layout_version() == 1):
 *   qweight: uint32 [N][K/8], row-major, K-contiguous. Word j of row n holds
 *   the codes of inputs k = 8j .. 8j+7: nibble i (bits 4i..4i+3, i = 0..3) is
 *   q[8j+2i] and nibble i+4 (bits 16+4i..16+4i+3) is q[8j+2i+1], so
 *   (word >> 4i) & 0x000F000F is the pair (q[8j+2i], q[8j+2i+1]) in the low and
 *   high 16-bit halves. Codes 0,1,...,7 pack to 0x75316420.
 *   scales, zeros: fp16 [N][K/group], row-major; group g of row n covers
 *   k = g*group .. g*group+group-1. The dequantized weight is
 *   w_hat[n][k] = (q[n][k] - zeros[n][g]) * scales[n][g]. Zeros are integers.
 *
 * Packed 3-bit layout (codes 0..7; "MIT 6.5940 Lab 4 + Lab 5" guide, Lab 4
 * setup: 3-bit weights with groups of 128; L13 AWQ section: INT3 g128):
 *   qweight: uint32 [N][3K/32]. The 32 inputs k = 32b .. 32b+31 of row n own
 *   words 3b, 3b+1, 3b+2. Word 3b+h (h = 0, 1) holds the low two bits of the
 *   codes of inputs 32b+16h .. 32b+16h+15: bits 2i..2i+1 (i = 0..7) are
 *   q[32b+16h+2i] & 3 and bits 16+2i..16+2i+1 are q[32b+16h+2i+1] & 3. Word
 *   3b+2 holds the high bits: bit i (i = 0..15) is q[32b+2i] >> 2 and bit 16+i
 *   is q[32b+2i+1] >> 2. So a pair of codes still ORs into an fp16 pair:
 *   ((lo >> 2i) & 0x00030003) | (((hi >> j) & 0x00010001) << 2), j = 8h + i.
 *   Codes 0..7, 0..7, 0..7, 0..7 pack to 0xDDDD8888, 0xDDDD8888, 0xCCCCCCCC.
 *   scales and zeros as above.
 *
 * Group sizes: 128 (the default; QServe table), 64 and 32 (Lab 5's kernel uses
 * groups of 32). Group 64 is this library's reading of the range between them.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4A16_OK = 0,
  W4A16_ERR_NULL = 1,        /* a required pointer is NULL                                  */
  W4A16_ERR_SHAPE = 2,       /* a size <= 0, K % group != 0, or a size beyond the limits    */
  W4A16_ERR_UNSUPPORTED = 3, /* an unsupported bits/group, or an unknown or unfit path        */
  W4A16_ERR_ALIGN = 4,       /* a pointer misses its alignment (stated per call)            */
  W4A16_ERR_HIP = 5,         /* the HIP runtime reported an error at launch                 */
  W4A16_ERR_ARG = 6          /* another invalid scalar argument (e.g. alpha)                */
} w4a16_status;

/* Limits (checked): K <= W4A16_MAX_K, N <= 2^24, M <= 2^16, T <= 2^20. */
#define W4A16_MAX_K 131072

/* Layout version of qweight/scales/zeros written and read by this library: 1. */
int32_t w4a16_layout_version(void);

/* Static English name of a status code ("ok", "null pointer", ...). */
const char* w4a16_status_str(int32_t status);

/* Text of the last failure on the calling host thread ("" if none). */
const char* w4a16_last_error(void);

/*
 * awq_channel_scale - the AWQ activation statistic (step "s = s_X^alpha").
 * L13 guide, AWQ section: s = s_X^alpha with s_X the mean magnitude of the
 * activation per input channel; "MIT 6.5940 Lab 4 + Lab 5" guide, Lab 4 setup:
 * forward hooks record the mean |input| per channel on calibration tokens.
 *
 *   s[k] = float32( (sum_t |x_cal[t][k]| / T) ^ alpha ),  computed in float64;
 *   a channel whose mean is 0 gets s[k] = 1. alpha = 0.5 uses sqrt.
 *
 * x_cal: fp16 [T][K]; s: float32 [K] (output). alpha in [0, 1].
 * Alignment: x_cal 2 bytes, s 4 bytes. The float64 sum is exact (hence
 * independent of order) while T * max|x| < 2^29.
 */
w4a16_status awq_channel_scale(const void* x_cal, int64_t T, int64_t K, double alpha, float* s,
                               void* stream);

/*
 * awq_scale_input - the 1/s folded into the layer input: x_s = f16(x / s).
 * L13 guide, AWQ section (the scaled channel's input is divided by s);
 * "Quantization for LLMs" chapter 11, section 11.3: Y = (X diag(s)^-1)(W diag(s))^T.
 *
 *   x_s[m][k] = f16_rne( float64(x[m][k]) / float64(s[k]) )   (one rounding)
 *
 * x: fp16 [M][K]; s: float32 [K], every s[k] > 0; x_s: fp16 [M][K] (output).
 * Alignment: x, x_s 2 bytes, s 4 bytes.
 */
w4a16_status awq_scale_input(const void* x, const float* s, int64_t M, int64_t K, void* x_s,
                             void* stream);

/*
 * awq_rmsnorm_fold - the RMSNorm in front of the scaled projections, with the
 * AWQ 1/s folded into it, so that it writes x_s directly and inference runs no
 * separate divide. "MIT 6.5940 Lab 4 + Lab 5" guide, AWQ skeleton part 2.3
 * (the scales are merged into the preceding LayerNorm or linear layer);
 * "Quantization for LLMs" chapter 11, AWQ section (the division by s is merged
 * into the LayerNorm in front). The LLaMA-shaped blocks use RMSNorm:
 *
 *   r[m]      = 1 / sqrt( sum_k h[m][k]^2 / K + eps )
 *   x_s[m][k] = f16_rne( ((h[m][k] * r[m]) * gamma[k]) / s[k] )
 *
 * every operation in float64 in that order (square root and division correctly
 * rounded), one float64 -> float16 rounding at the end; the sum of squares in a
 * fixed order (reproducible). s == NULL gives the plain RMSNorm output.
 * h: fp16 [M][K]; gamma: fp16 [K]; s: float32 [K] or NULL; eps: finite, > 0;
 * x_s: fp16 [M][K] (output; must not alias h). K % 8 == 0.
 * Alignment: h and x_s 16 bytes, gamma 2 bytes, s 4 bytes.
 * Errors: W4A16_ERR_NULL, W4A16_ERR_SHAPE (M, K <= 0, K % 8, limits),
 * W4A16_ERR_ARG (eps), W4A16_ERR_ALIGN, W4A16_ERR_HIP; checked before any HIP call.
 */
w4a16_status awq_rmsnorm_fold(const void* h, const void* gamma, const float* s, int64_t M, int64_t K,
                              double eps, void* x_s, void* stream);

/*
 * awq_quantize_pack - round-to-nearest group quantization and packing.
 * L13 guide, AWQ section: Q(w) = Delta * Round(w / Delta) on weights already
 * multiplied by s; CMU L19 zero-point quantizer (range max - min, integer zero,
 * clipped codes); QServe table: 4-bit weights, group 128; Lab 4 setup: 3-bit,
 * group 128; TinyChat packing.
 *
 * For every row n and group g (inputs k in [Gs g, Gs g + Gs), Gs = group), in
 * float64, with Q = 2^bits - 1:
 *   w   = float64(W[n][k]) * float64(s[k])      (exact; s == NULL means s = 1)
 *   R   = max w - min w, replaced by 1 when 0
 *   D   = R / Q                                  (IEEE division)
 *   z   = rint(-min w / D)                        (round half even, not clamped)
 *   q   = clamp(rint(w / D) + z, 0, Q)
 *   scales[n][g] = f16_rne(D), zeros[n][g] = f16_rne(z), qweight = layout v1
 *   (bits 4) or the 3-bit layout (bits 3).
 * Results are bit-identical to that definition.
 *
 * w: fp16 [N][K] (nn.Linear weight: rows are outputs); s: float32 [K] or NULL;
 * bits 3 or 4; group 32, 64 or 128; K % group == 0. Outputs: qweight uint32
 * [N][K/8] (bits 4) or [N][3K/32] (bits 3), scales and zeros fp16
 * [N][K/group]. Alignment: w and qweight 16 bytes, s 16 bytes, scales and
 * zeros 2 bytes.
 */
w4a16_status awq_quantize_pack(const void* w, const float* s, int64_t N, int64_t K, int32_t bits,
                               int32_t group, void* qweight, void* scales, void* zeros,
                               void* stream);

/*
 * w4a16_linear - the fused dequantize + matrix multiply of a W4A16 layer.
 * L13 guide, TinyChat kernel fusion (slide 37): dequantize inside the GEMV/GEMM
 * without writing weights back to memory; CMU guide, "where the speed comes
 * from": batch-1 decode is a memory-bound GEMV; QServe table: A16 (fp16 inputs).
 *
 *   y[m][n] = f16_rne( sum_k x[m][k] * (q[n][k] - zeros[n][g]) * scales[n][g] )
 *
 * accumulated in float32 (any summation order). Accuracy contract, with
 * B = sum_k |x[m][k] * w_hat[n][k]|: |y - exact| <= 1e-3 * B + 1e-5.
 * x: fp16 [M][K], the input after the 1/s fold; qweight/scales/zeros as written
 * by awq_quantize_pack with bits 4; y: fp16 [M][N] (output). group 32, 64 or
 * 128 (as quantized); K % 128 == 0.
 * Dispatch, group 128: M == 1, and M == 2 on layers with K <= 24576 or small
 * enough that the GEMV takes 4-row tiles (K <= 32768 and
 * ceil(N / 8) * ceil(K / 2048) < 4096 waves, under 16 per CU), run the
 * wave-tile GEMV kernel; other M <= 32 the small-batch
 * MFMA kernel (workgroups own whole rows of y, waves split K), except
 * 17 <= M <= 32 with K > 16384, which runs the K-lane kernel; M >= 256 the
 * one-range split-K kernel (w4a16_linear_path path 5) where its tiles
 * (ceil(M / 64) * ceil(N / 128)) are a multiple of 256 or at least 1280;
 * other M > 32 the K-lane MFMA kernel (K split over the four waves of a
 * workgroup) where the tiled MFMA kernel would start at most 256 workgroups (ceil(M / 32) *
 * ceil(N / 64) while ceil(M / 64) * ceil(N / 64) < 512, else the latter), or
 * where the K-lane grid (ceil(M / 64) * ceil(N / 32) workgroups) is at most
 * 512 with K >= 8192 or at most 768 with K > 8192; otherwise the small-batch
 * kernel twice (rows 0..31, then the rest) for M <= 64 on layers with
 * N <= 8192 and K <= 16384, and the tiled MFMA kernel for the rest.
 * Groups of 32 and 64: M == 1, and M == 2 with K <= 32768, run the GEMV
 * kernel (two or one 32-input pieces per group);
 * other M <= 32 the small-batch MFMA kernel (which needs scales and zeros
 * 4-byte aligned; otherwise the GEMV takes M <= 8 where it can), and
 * 33 <= M <= 64 the same two launches as for group 128 on the same layers;
 * other M the tiled MFMA kernel's variant (one (scale, zero) per 32-input MFMA
 * step).
 * Alignment: x and qweight 16 bytes, scales/zeros/y 2 bytes.
 */
w4a16_status w4a16_linear(const void* x, const void* qweight, const void* scales, const void* zeros,
                          int64_t M, int64_t N, int64_t K, int32_t group, void* y, void* stream);

/*
 * w4a16_linear_workspace - bytes of float32 workspace that w4a16_linear_ws may
 * use for this shape and group (0: it will run w4a16_linear's kernels and needs
 * none); -1 when the shape or group is not accepted. Host only.
 */
int64_t w4a16_linear_workspace(int64_t M, int64_t N, int64_t K, int32_t group);

/*
 * w4a16_linear_ws_splits - the number of K ranges w4a16_linear_ws splits this
 * shape into when given its workspace (0: no split, w4a16_linear's kernels);
 * -1 when the shape or group is not accepted. Host only.
 */
int32_t w4a16_linear_ws_splits(int64_t M, int64_t N, int64_t K, int32_t group);

/*
 * w4a16_linear_ws_kernel - the kernel w4a16_linear_ws runs for this shape when
 * given its workspace, with scales and zeros 4-byte aligned: 0 = w4a16_linear's
 * choice, 1 = the split-K kernels (w4a16_linear_ws_splits ranges), 2 = the
 * x-resident kernel (w4a16_linear_xres); -1 when the shape or group is not
 * accepted. Host only.
 */
int32_t w4a16_linear_ws_kernel(int64_t M, int64_t N, int64_t K, int32_t group);

/*
 * w4a16_linear_ws - w4a16_linear whose automatic choice may also take the
 * x-resident small-batch kernel (w4a16_linear_xres) and the
 * split-K kernels (w4a16_linear_splitk) when the caller lends a workspace, for
 * batched layers with too few output tiles to fill the chip (CMU guide: at
 * large batch the layer is compute-bound; L13 TinyChat kernel fusion). Same
 * formula, accuracy contract, arguments and alignment as w4a16_linear, plus
 * workspace: NULL (then exactly w4a16_linear), or device memory of
 * workspace_bytes >= w4a16_linear_workspace(M, N, K, group) bytes, 16-byte
 * aligned, overwritten (two calls in flight at once need two workspaces).
 * Dispatch with a workspace (from measured sweeps over the LLaMA projection
 * shapes), groups of 128 or 64: the x-resident kernel when K > 2048, K / 128 is even,
 * scales and zeros are 4-byte aligned and: for 4 <= M <= 16, N * K >= 2^27, or
 * M >= 8 with N * K >= 2^25 and N > K, or M >= 8 with ceil(N / 32) <= 64 and
 * K >= 8192, or M >= 12 with N * K >= 2^25; for 17 <= M <= 32, with
 * W = ceil(N / 128) * ceil(K / 2048), W >= 160; otherwise, groups of 128 only,
 * split-K: no split for M <= 16; else with G = K / 128 and T
 * the split-K kernel's tiles (ceil(N / 128) for M <= 32, else ceil(M / 64) *
 * ceil(N / 128)), for K >= 8192: no split up to M = 32 when K <= 16384 and
 * ceil(N / 32) is a multiple of 256 (the small-batch kernel's grid fills the
 * chip in whole rounds), else the largest S of 8, 4, 2 with S * T < 1024
 * (S * T <= 256 when T <= 64) and G / S >= 8, none if only S = 1 remains (the
 * automatic choice of w4a16_linear, which needs no workspace, covers those);
 * for 4096 <= K < 8192 from M = 21, S = 2 on 65..128 tiles and S = 4 on at
 * most 48 tiles at M > 32; otherwise no split
 * (w4a16_linear_ws_splits reports the split-K choice, w4a16_linear_ws_kernel
 * the kernel). With S > 0 the call launches the two split-K kernels, else
 * w4a16_linear's. Results are reproducible (fixed summation order for a given
 * shape).
 * Errors: those of w4a16_linear; W4A16_ERR_ARG (workspace too small for the
 * split chosen); W4A16_ERR_ALIGN (workspace). Checked before any HIP call.
 */
w4a16_status w4a16_linear_ws(const void* x, const void* qweight, const void* scales, const void* zeros,
                             int64_t M, int64_t N, int64_t K, int32_t group, void* workspace,
                             int64_t workspace_bytes, void* y, void* stream);

/*
 * w4a16_linear_path - w4a16_linear with the kernel chosen by the caller, for
 * measuring the GEMV/MFMA hand-off: path 0 = automatic (same as w4a16_linear),
 * 1 = GEMV kernel (needs M <= w4a16_gemv_max_m() and M * ceil(K / 16384) <= 8),
 * 2 = tiled MFMA kernel (any M), 3 = small-batch MFMA kernel (needs M <= 32;
 * with groups of 32 or 64, scales and zeros 4-byte aligned, else
 * W4A16_ERR_ALIGN), 4 = K-lane MFMA kernel (any M; groups of 128 only),
 * 5 = the split-K kernel with one K range, which writes fp16 y itself (no
 * workspace, one launch; any M; groups of 128 only). A path
 * that cannot take the shape returns W4A16_ERR_UNSUPPORTED before any HIP
 * call. Same contract otherwise.
 */
w4a16_status w4a16_linear_path(int32_t path, const void* x, const void* qweight, const void* scales,
                               const void* zeros, int64_t M, int64_t N, int64_t K, int32_t group,
                               void* y, void* stream);

/*
 * w4a16_linear_splitk_workspace - bytes of float32 workspace that
 * w4a16_linear_splitk needs for this shape and split count (splits 0 = the
 * library's choice); -1 when the shape or split count is not accepted.
 */
int64_t w4a16_linear_splitk_workspace(int64_t M, int64_t N, int64_t K, int32_t splits);

/*
 * w4a16_linear_splitk - w4a16_linear (4-bit, groups of 128) on the split-K
 * MFMA kernel (output tiles of 64 rows of y by 128 columns, 32 rows when
 * M <= 32), for batches whose output has too few tiles to fill the chip
 * (CMU guide: at large batch the layer is compute-bound; L13 TinyChat kernel
 * fusion). The K groups are split into `splits` contiguous ranges (0 = the
 * library's choice, else 1 <= splits <= min(16, K/128)); each range's float32
 * partial of every output goes to `workspace`, and a second kernel adds the
 * partials in index order and rounds once to fp16, so results are reproducible.
 * With one range the partial kernel rounds and writes y itself (the same bits,
 * one launch; the workspace is still required but not touched).
 * Same formula, accuracy contract, arguments and alignment as w4a16_linear,
 * plus workspace: device memory of workspace_bytes >=
 * w4a16_linear_splitk_workspace(M, N, K, splits) bytes, 16-byte aligned,
 * overwritten (two calls in flight at once need two workspaces).
 * Errors: those of w4a16_linear; W4A16_ERR_UNSUPPORTED (group != 128);
 * W4A16_ERR_NULL (workspace); W4A16_ERR_ARG (splits, workspace too small);
 * W4A16_ERR_ALIGN (workspace). Launches two kernels (one with one range).
 */
w4a16_status w4a16_linear_splitk(const void* x, const void* qweight, const void* scales, const void* zeros,
                                 int64_t M, int64_t N, int64_t K, int32_t group, int32_t splits,
                                 void* workspace, int64_t workspace_bytes, void* y, void* stream);

/*
 * w4a16_linear_xres_workspace - bytes of float32 workspace that
 * w4a16_linear_xres needs for this shape (S * M * N floats for its S K ranges,
 * 0 with one range); -1 when the shape is not accepted (M > 32, or an odd
 * number of groups of 128 per row).
 */
int64_t w4a16_linear_xres_workspace(int64_t M, int64_t N, int64_t K);

/*
 * w4a16_linear_xres - w4a16_linear (4-bit, groups of 128 or 64) for small batches,
 * 1 <= M <= 32, on the x-resident MFMA kernel: a workgroup owns 64 output
 * columns for M <= 16 (128 above) and one range of 256 inputs per wave (eight
 * waves, or four where M <= 16 and ceil(N / 64) * ceil(K / 2048) < 512, or
 * M > 16 and ceil(N / 128) * ceil(K / 2048) >= 512); each wave keeps the x
 * fragments of its 256 inputs in registers and streams the codes of the
 * workgroup's columns past them, so x crosses from L2 once per 64 or 128
 * columns instead of once per 32 (CMU guide, "where the speed comes from": small-batch
 * decode stays bound by the weight stream; L13 TinyChat kernel fusion). The S
 * ranges' float32 partials go to `workspace` and a second kernel adds them in
 * index order and rounds once to fp16 (reproducible); with one range the first
 * kernel writes y itself. Same formula, accuracy contract and arguments as
 * w4a16_linear, plus workspace: device memory of workspace_bytes >=
 * w4a16_linear_xres_workspace(M, N, K) bytes, 16-byte aligned, overwritten
 * (NULL allowed when that is 0; two calls in flight at once need two
 * workspaces). Needs (K / 128) even; scales and zeros 4-byte aligned. With
 * groups of 64 each MFMA step takes 32 contiguous inputs, so a group is two
 * steps and is scaled after them (groups of 128: four).
 * Errors: those of w4a16_linear; W4A16_ERR_UNSUPPORTED (group other than 128 or 64, M > 32,
 * odd group count); W4A16_ERR_NULL (workspace needed); W4A16_ERR_ARG
 * (workspace too small); W4A16_ERR_ALIGN (workspace, scales, zeros). Checked
 * before any HIP call.
 */
w4a16_status w4a16_linear_xres(const void* x, const void* qweight, const void* scales, const void* zeros,
                               int64_t M, int64_t N, int64_t K, int32_t group, void* workspace,
                               int64_t workspace_bytes, void* y, void* stream);

/*
 * w4a16_linear_splitk_noalloc - w4a16_linear_splitk for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels, launched with the same
 * arguments minus the workspace. The float32 partials go to the library's own
 * scratch, a static device array of 2^23 floats (32 MiB) on each GPU the library
 * runs on, held until the process ends; the call allocates and frees nothing.
 * Every call on one GPU uses that GPU's array and overwrites it (the kernels write
 * every partial they read, so nothing needs clearing): calls that overlap on one
 * GPU (other streams, other threads) race and must be serialised by the caller.
 * The first call on a device resolves the array's address there (HIP calls, no
 * allocation). Errors: those of w4a16_linear_splitk except the workspace ones;
 * W4A16_ERR_SHAPE when splits * M * N (splits after the library's choice for 0)
 * exceeds 2^23; checked before any HIP call.
 */
w4a16_status w4a16_linear_splitk_noalloc(const void* x, const void* qweight, const void* scales, const void* zeros,
                                         int64_t M, int64_t N, int64_t K, int32_t group, int32_t splits,
                                         void* y, void* stream);

/*
 * w3a16_linear - the fused dequantize + matrix multiply for 3-bit codes in the
 * packed 3-bit layout (awq_quantize_pack with bits 3). Lab 4 setup: 3-bit
 * weights, groups of 128; L13 TinyChat kernel fusion. Same formula, accuracy
 * contract, arguments and alignment as w4a16_linear; group 32, 64 or 128;
 * K % 128 == 0. Dispatch: M == 1 the GEMV kernel's 3-bit variant, and M == 2
 * too where K < N, where K == N with N * K >= 2^26, or where K <= 16384 with
 * N * K >= 2^27; other M <= 32 the small-batch MFMA kernel's (scales and zeros
 * 4-byte aligned below groups of 128, else the GEMV variant up to M = 8, M = 4
 * above K = 16384); 33 <= M <= 64 on layers with N <= 8192 and K <= 16384
 * two small-batch launches (rows 0..31, then the rest); other M the tiled MFMA
 * kernel's 3-bit variant.
 */
w4a16_status w3a16_linear(const void* x, const void* qweight, const void* scales, const void* zeros,
                          int64_t M, int64_t N, int64_t K, int32_t group, void* y, void* stream);

/*
 * w3a16_linear_path - w3a16_linear with the kernel chosen by the caller: path
 * 0 = automatic, 1 = GEMV variant (needs M <= 8, and M <= 4 above K = 16384,
 * K <= 32768), 2 = tiled MFMA variant (any M), 3 = small-batch MFMA variant
 * (M <= 32; W4A16_ERR_ALIGN when scales or zeros are not 4-byte aligned below
 * groups of 128). Other paths, or a shape the chosen kernel cannot take, return
 * W4A16_ERR_UNSUPPORTED before any HIP call.
 */
w4a16_status w3a16_linear_path(int32_t path, const void* x, const void* qweight, const void* scales,
                               const void* zeros, int64_t M, int64_t N, int64_t K, int32_t group,
                               void* y, void* stream);

/*
 * awq_alpha_loss_workspace - number of float64 values that awq_alpha_loss
 * needs in its workspace for T calibration rows and N outputs (one per 64 x 128
 * tile of the (t, n) plane); -1 when T or N is outside the limits.
 */
int64_t awq_alpha_loss_workspace(int64_t T, int64_t N);

/*
 * awq_output_reference - the original layer's output on the calibration
 * activations, the W X term of the AWQ scale-search loss. L13 guide, AWQ
 * section (slide 28): the loss compares the quantized layer's output with W X;
 * "Quantization for LLMs" chapter 11, AWQ section. It does not depend on the
 * candidate scale, so a search computes it once:
 *
 *   y_ref[t][n] = sum_k x[t][k] * w[n][k]      (float32 accumulation)
 *
 * x: fp16 [T][K]; w: fp16 [N][K] (nn.Linear weight); y_ref: float32 [T][N]
 * (output). K % 128 == 0. Alignment: x and w 16 bytes, y_ref 4 bytes.
 * Errors: W4A16_ERR_NULL; W4A16_ERR_SHAPE (a size <= 0, K % 128, T > 2^20,
 * N > 2^24, K > W4A16_MAX_K); W4A16_ERR_ALIGN; W4A16_ERR_HIP. Checked before
 * any HIP call.
 */
w4a16_status awq_output_reference(const void* x, const void* w, int64_t T, int64_t N, int64_t K,
                                  float* y_ref, void* stream);

/*
 * awq_alpha_loss - the output-error loss that the AWQ scale search minimises,
 * for one candidate scale s. L13 guide, AWQ section (slide 28): alpha is
 * chosen by a grid search minimising L(s) = || Q(W s)(s^-1 X) - W X || with
 * s = s_X^alpha, the error measured on the layer's output; "Quantization for
 * LLMs" chapter 11, AWQ section. Squared Frobenius norm:
 *
 *   loss = sum_{t,n} ( sum_k x_s[t][k] * w_hat[n][k] - y_ref[t][n] )^2
 *
 * where x_s = f16(x / s) (as awq_scale_input writes it), w_hat is the
 * dequantized layout-v1 weight of W * s (as awq_quantize_pack writes it) and
 * y_ref the original output (as awq_output_reference writes it). The product
 * is accumulated in float32 (a float32 dot product's rounding, far below the
 * quantization error being measured); the residual, its square and the sum
 * over (t, n) are float64, the sum in a fixed order, so the result is
 * reproducible run to run.
 * x_s: fp16 [T][K]; qweight uint32 [N][K/8], scales and zeros fp16 [N][K/128];
 * y_ref: float32 [T][N]; group must be 128. workspace: float64
 * [workspace_len], workspace_len >= awq_alpha_loss_workspace(T, N),
 * overwritten (two calls in flight at once need two workspaces); loss: one
 * float64 (output, device memory).
 * Alignment: x_s and qweight 16 bytes; scales and zeros 2 bytes; y_ref 4
 * bytes; workspace and loss 8 bytes.
 * Errors: W4A16_ERR_NULL; W4A16_ERR_SHAPE (a size <= 0, K % 128, T > 2^20,
 * N > 2^24, K > W4A16_MAX_K); W4A16_ERR_UNSUPPORTED (group); W4A16_ERR_ARG
 * (workspace too small); W4A16_ERR_ALIGN; W4A16_ERR_HIP. Checked before any
 * HIP call. Launches two kernels (the loss tiles, then the reduction).
 */
w4a16_status awq_alpha_loss(const void* x_s, const void* qweight, const void* scales, const void* zeros,
                            const float* y_ref, int64_t T, int64_t N, int64_t K, int32_t group,
                            double* workspace, int64_t workspace_len, double* loss, void* stream);

/* Points of the AWQ scale search's grid: alpha = i / 20, i = 0..20. */
#define W4A16_ALPHA_GRID_POINTS 21

/*
 * awq_search_alpha_workspace - bytes of device workspace that awq_search_alpha
 * needs for T calibration rows, N outputs and K inputs; -1 when the shape is
 * outside the limits (T <= 65536, N <= 2^24, K <= W4A16_MAX_K, K % 128 == 0).
 */
int64_t awq_search_alpha_workspace(int64_t T, int64_t N, int64_t K);

/*
 * awq_search_alpha - the whole AWQ scale search on the device. L13 guide, AWQ
 * section (slide 28): alpha* = argmin over alpha of || Q(W s)(s^-1 X) - W X ||
 * with s = s_X^alpha; "Quantization for LLMs" chapter 11, AWQ section. For the
 * grid alpha = i / 20 (i = 0..20) it computes, in stream order: the original
 * output W X once (awq_output_reference), then per grid point s =
 * awq_channel_scale(x_cal, alpha), x_s = awq_scale_input(x_cal, s),
 * awq_quantize_pack(w, s, bits 4, group 128) and the loss (awq_alpha_loss) into
 * losses[i]; finally the choice: best = the first index of the smallest loss
 * (equal losses keep the smaller alpha), alpha = best / 20, and s = the
 * candidate scale of that index. Results are bit-identical to running those
 * calls one by one (the same kernels on the same inputs).
 * x_cal: fp16 [T][K] calibration activations; w: fp16 [N][K] (nn.Linear
 * weight); workspace: device memory of workspace_bytes >=
 * awq_search_alpha_workspace(T, N, K) bytes, 256-byte aligned, overwritten (two
 * searches in flight at once need two workspaces). Outputs, device memory:
 * losses float64 [21], best int32 [1], alpha float64 [1], s float32 [K] (or
 * NULL: the chosen scale is not copied out). All launches are asynchronous on
 * `stream`; nothing is read back to the host.
 * Alignment: x_cal and w 16 bytes; losses and alpha 8; best and s 4.
 * Errors: W4A16_ERR_NULL; W4A16_ERR_SHAPE (a size <= 0, K % 128, T > 65536,
 * N > 2^24, K > W4A16_MAX_K); W4A16_ERR_ARG (workspace too small);
 * W4A16_ERR_ALIGN; W4A16_ERR_HIP. Checked before any HIP call.
 */
w4a16_status awq_search_alpha(const void* x_cal, const void* w, int64_t T, int64_t N, int64_t K,
                              void* workspace, int64_t workspace_bytes, double* losses, int32_t* best,
                              double* alpha, float* s, void* stream);

/*
 * awq_quantize_pack_sym - symmetric absmax group quantization into the same
 * packed layouts. "CMU 11-868 Model Quantization" guide, L19 "absmax and
 * zero-point" (the absmax quantizer: scale from the largest magnitude, values
 * mapped onto the symmetric integer range and rounded); L13 guide, AWQ section
 * (Q(w) = Delta * Round(w / Delta), Delta from max |w|). For every row n and
 * group g, in float64, with H = 2^(bits-1) - 1:
 *   w     = float64(W[n][k]) * float64(s[k])     (exact; s == NULL means s = 1)
 *   m     = max |w|, replaced by 1 when 0
 *   D     = m / H                                 (IEEE division)
 *   q     = clamp(rint(w / D), -H, H)
 *   stored code q + 2^(bits-1); scales[n][g] = f16_rne(D); zeros[n][g] = 2^(bits-1).
 * So w4a16_linear (bits 4) or w3a16_linear (bits 3) computes with these weights
 * unchanged. Arguments, layouts, alignment and errors as awq_quantize_pack.
 */
w4a16_status awq_quantize_pack_sym(const void* w, const float* s, int64_t N, int64_t K, int32_t bits,
                                   int32_t group, void* qweight, void* scales, void* zeros,
                                   void* stream);

/*
 * nf4_codebook - the 16 NormalFloat-4 levels as fp16 bit patterns, ascending
 * (host only; levels[7] is 0). "Quantization for LLMs" chapter 11, section 11.5:
 * 8 positive levels at standard normal quantiles of OFFSET - i (OFFSET - 1/2) / 8
 * (i = 0..7), 7 negative levels mirrored from OFFSET - i (OFFSET - 1/2) / 7
 * (i = 0..6), and 0, all divided by the largest; OFFSET = 0.9677083. Each level
 * is rounded once to fp16; these are the values the NF4 kernels multiply with.
 * levels: host array of 16 (NULL is ignored).
 */
void nf4_codebook(uint16_t* levels);

/*
 * nf4_quantize_pack - blockwise absmax NF4 quantization (chapter 11, section
 * 11.5: each block of 64 weights is divided by its largest magnitude and mapped
 * to the nearest of the 16 levels; the block keeps a float32 absmax). For every
 * row n and block b of `block` inputs:
 *   w = float64(W[n][k]) * float64(s[k])   (s == NULL means s = 1)
 *   a = f32_rne(max |w|)                    -> absmax[n][b]
 *   code = the index of the fp16 level nearest to w / float64(a) (the count of
 *          level midpoints at or below it, so an exact midpoint goes up); a
 *          block with a = 0 takes the code of level 0.
 * Codes are packed in layout v1. Bit-identical to that definition.
 * w: fp16 [N][K]; s: float32 [K] or NULL; block 32, 64 or 128 (64 on the page);
 * K % block == 0. Outputs: qweight uint32 [N][K/8], absmax float32 [N][K/block].
 * Alignment: w, qweight and s 16 bytes, absmax 4 bytes.
 * Errors: W4A16_ERR_NULL, W4A16_ERR_UNSUPPORTED (block), W4A16_ERR_SHAPE,
 * W4A16_ERR_ALIGN, W4A16_ERR_HIP; checked before any HIP call.
 */
w4a16_status nf4_quantize_pack(const void* w, const float* s, int64_t N, int64_t K, int32_t block,
                               void* qweight, float* absmax, void* stream);

/*
 * nf4_linear - the fused dequantize + matrix multiply for NF4 weights (chapter
 * 11, section 11.5: the NF4 weights are dequantized just before the multiply;
 * L13 TinyChat kernel fusion: in registers, never written back):
 *
 *   y[m][n] = f16_rne( sum_k x[m][k] * level[q[n][k]] * absmax[n][b] )
 *
 * with the fp16 codebook of nf4_codebook, float32 accumulation, and the
 * accuracy contract of w4a16_linear (B = sum_k |x * w_hat|). x: fp16 [M][K];
 * qweight, absmax as nf4_quantize_pack writes them; y: fp16 [M][N]; block 32,
 * 64 or 128; K % 128 == 0. Dispatch: M == 1 a GEMV kernel with the codebook
 * in LDS (on layers with N * K < 2^26 the tuned 4-bit GEMV's NF4 form, else
 * the per-piece GEMV's); other M <= 32 the small-batch MFMA kernel's, and
 * 33 <= M <= 64 on layers with N <= 8192 and K <= 16384 two small-batch
 * launches (rows 0..31, then the rest); other M the tiled MFMA kernel's.
 * Alignment: x and qweight 16 bytes, absmax 4, y 2.
 */
w4a16_status nf4_linear(const void* x, const void* qweight, const float* absmax, int64_t M, int64_t N,
                        int64_t K, int32_t block, void* y, void* stream);

/*
 * nf4_linear_path - nf4_linear with the kernel chosen: 0 auto, 1 GEMV (M <= 8,
 * M <= 4 above K = 16384, K <= 32768; or M == 1 with N * K < 2^26 and
 * K <= 131072, on the tuned kernel's NF4 form), 2 tiled MFMA (any M), 3 small-batch
 * MFMA (M <= 32). Other paths, or a shape the chosen kernel cannot take, return
 * W4A16_ERR_UNSUPPORTED before any HIP call.
 */
w4a16_status nf4_linear_path(int32_t path, const void* x, const void* qweight, const float* absmax,
                             int64_t M, int64_t N, int64_t K, int32_t block, void* y, void* stream);

/* Largest M that the GEMV kernel (w4a16_linear_path path 1) accepts. */
int32_t w4a16_gemv_max_m(void);

/*
 * w4a16_stream_read - a measurement aid, not part of the method. One launch reads
 * `bytes` of `buf` once, with the access pattern of the GEMV's weight stream (16-byte
 * non-temporal loads, 1 KB of contiguous memory per wave and load, every load of a
 * thread issued before any is used), and does no arithmetic beyond an XOR per thread.
 * Timed beside w4a16_linear on the same number of bytes, it gives the single-launch
 * floor of the weight stream on the machine at hand (the sources' point that decode is
 * bound by reading the weights: CMU guide, "where the speed comes from").
 * Split: with P = bytes / 16 pieces, W = max(min(1024, ceil(P / 256)), ceil(P / 4096)),
 * chunk = ceil(P / W); workgroup b (of ceil(P / chunk)) reads pieces
 * [b * chunk, min((b + 1) * chunk, P)), its 256 threads t, t + 256, ... of them.
 * buf: device memory, 16-byte aligned, bytes > 0 and a multiple of 16. sink: device
 * memory of w4a16_stream_read_sink_bytes(bytes) bytes, 4-byte aligned; workgroup b
 * writes sink[b] = W4A16_STREAM_READ_MAGIC only if the XOR of its thread's words equals
 * that value, and writes nothing otherwise. Errors: W4A16_ERR_NULL, W4A16_ERR_SHAPE
 * (bytes), W4A16_ERR_ALIGN, W4A16_ERR_HIP; checked before any HIP call.
 */
#define W4A16_STREAM_READ_MAGIC 0x5EAD5EADu
w4a16_status w4a16_stream_read(const void* buf, int64_t bytes, void* sink, void* stream);

/* Bytes of sink that w4a16_stream_read needs for `bytes` (-1 if bytes is not accepted). */
int64_t w4a16_stream_read_sink_bytes(int64_t bytes);

/*
 * w4a16_stream_read_grid - a measurement aid, not part of the method: a second read
 * pattern, independent of the GEMV's grid, to test whether the single-launch floor
 * belongs to the machine or to one access pattern. A grid-stride read of `bytes` of
 * `buf` in tiles of threads x unroll 16-byte pieces: tile i covers pieces
 * [i threads unroll, (i + 1) threads unroll); workgroup b (of `blocks`, each of
 * `threads` threads) takes tiles b, b + blocks, ...; its thread t loads pieces
 * i threads unroll + t + j threads (j < unroll) non-temporally, all before using any.
 * threads: 64, 128, 256, 512 or 1024; unroll: 1, 2, 4, 8 or 16; blocks in [1, 2^20].
 * sink: device memory of blocks 32-bit words, 4-byte aligned; workgroup b writes
 * sink[b] = W4A16_STREAM_READ_MAGIC only if the XOR of one of its thread's words over
 * all its tiles equals that value, and nothing otherwise. buf: device memory, 16-byte
 * aligned, bytes > 0 and a multiple of 16. Errors: W4A16_ERR_NULL, W4A16_ERR_SHAPE,
 * W4A16_ERR_ARG (threads, unroll, blocks), W4A16_ERR_ALIGN, W4A16_ERR_HIP; checked
 * before any HIP call.
 */
w4a16_status w4a16_stream_read_grid(const void* buf, int64_t bytes, int32_t threads, int32_t blocks, int32_t unroll,
                                    void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
