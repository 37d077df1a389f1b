// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32, round to nearest even
}

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// float64 -> binary16 with a single round-to-nearest-even step (no float32
// intermediate, which would round twice). Handles signed zero, subnormal
// results, overflow to infinity and NaN. Host and device.
__host__ __device__ inline uint16_t f64_to_f16_rne(double d) {
  const uint64_t b = __builtin_bit_cast(uint64_t, d);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
  if (a > 0x7FF0000000000000ull) return (uint16_t)(sign | 0x7E00u);  // NaN
  if (a >= 0x40EFFE0000000000ull) return (uint16_t)(sign | 0x7C00u); // >= 65520 rounds to inf
  const int e = (int)(a >> 52) - 1023;                                 // unbiased exponent
  if (e < -25) return sign;                                            // below half the least subnormal
  const uint64_t mant = (a & 0x000FFFFFFFFFFFFFull) | 0x0010000000000000ull;  // 53-bit significand
  // normal results keep 11 significant bits; subnormal results fewer
  const int shift = (e >= -14) ? 42 : 42 + (-14 - e);                  // 42 .. 53
  uint64_t r = mant >> shift;
  const uint64_t rem = mant & ((1ull << shift) - 1ull);
  const uint64_t halfway = 1ull << (shift - 1);
  if (rem > halfway || (rem == halfway && (r & 1ull))) ++r;
  uint32_t h;
  if (e >= -14)
    h = ((uint32_t)(e + 15) << 10) + (uint32_t)r - 1024u;  // a carry into the exponent is correct
  else
    h = (uint32_t)r;                                       // 1024 here is the least normal
  return (uint16_t)(sign | h);
}

// (a & mask) | bits in one v_and_or_b32. The compiler splits this into an AND
// and an OR because a gfx9 VOP3 instruction cannot carry literal constants; here
// the mask sits in an SGPR and the OR operand in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bits) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(mask), "v"(bits));
  return d;
}

// The NF4 codebook as kernels take it: the 16 fp16 levels in ascending order, two per
// word (low half first).
struct Nf4Table {
  uint32_t pairs[8];
};

// Sum over the 16 lanes of a DPP row; every lane of the row receives the sum.
__device__ __forceinline__ float dpp_row_sum16(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));  // row_half_mirror
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));  // row_mirror
  return v;
}

// Sum over all 64 lanes, valid in lane 63: four in-row DPP steps, then
// row_bcast15 (rows 1, 3) and row_bcast31 (rows 2, 3).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add_masked(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

__device__ __forceinline__ float wave_sum_lane63(float v) {
  v = dpp_add_masked<0xB1, 0xF>(v);   // quad_perm 1,0,3,2
  v = dpp_add_masked<0x4E, 0xF>(v);   // quad_perm 2,3,0,1
  v = dpp_add_masked<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_add_masked<0x140, 0xF>(v);  // row_mirror
  v = dpp_add_masked<0x142, 0xA>(v);  // row_bcast15
  v = dpp_add_masked<0x143, 0xC>(v);  // row_bcast31
  return v;
}

// Workgroups are dealt to the chip's eight XCDs round-robin by linear block id.
// Renumbering them so that each XCD takes a contiguous run of work items keeps
// neighbouring items (the m-tiles and K-splits of one weight tile) on one XCD, where
// they share its L2, instead of fetching the same codes once per XCD. A bijection on
// [0, nb) for any nb.
__device__ __forceinline__ int xcd_contiguous_item(int id, int nb) {
  const int xcd = id & 7, slot = id >> 3;
  const int per = nb >> 3, rem = nb & 7;
  return xcd * per + min(xcd, rem) + slot;
}

}  // namespace w4a16
