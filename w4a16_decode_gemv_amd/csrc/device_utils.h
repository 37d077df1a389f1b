// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3: raw 32-bit data, range-checked
constexpr int kOutOfRange = 1 << 30;      // added to an offset: past every buffer range used here
constexpr int kNonTemporal = 2;           // streaming hint for loads of data read once

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32, round to nearest even
}

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

__device__ __forceinline__ half8_t as_half8(u32x4_t v) { return __builtin_bit_cast(half8_t, v); }

__device__ __forceinline__ half8_t as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4_t v = {a, b, c, d};
  return __builtin_bit_cast(half8_t, v);
}

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

// The four exact fp16 pairs (q - z) of one layout-v1 code word, in the word's pair order
// (inputs 0,1 | 2,3 | 4,5 | 6,7): each nibble pair is OR-ed into the mantissa of 0x6400
// (fp16 1024), giving 1024 + q, or 1024 + 16 q for the upper nibble of a byte, which is
// rebased by 1/16. c_lo = -(1024 + z) and c_hi = -(64 + z); every step is exact for
// z in [-2032, 1024], and z = 0 gives the codes q themselves.
__device__ __forceinline__ half8_t dequant_word(uint32_t w, half2_t c_lo, half2_t c_hi) {
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w8 = w >> 8;
  const half2_t p0 = as_half2(and_or(w, 0x000F000Fu, 0x64006400u)) + c_lo;
  const half2_t p1 = __builtin_elementwise_fma(as_half2(and_or(w, 0x00F000F0u, 0x64006400u)), sixteenth, c_hi);
  const half2_t p2 = as_half2(and_or(w8, 0x000F000Fu, 0x64006400u)) + c_lo;
  const half2_t p3 = __builtin_elementwise_fma(as_half2(and_or(w8, 0x00F000F0u, 0x64006400u)), sixteenth, c_hi);
  return as_half8(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1), __builtin_bit_cast(uint32_t, p2),
                  __builtin_bit_cast(uint32_t, p3));
}

// the eight codes q of one code word as exact fp16, in k order
__device__ __forceinline__ half8_t codes_word(uint32_t w) {
  return dequant_word(w, (half2_t){(_Float16)-1024.0f, (_Float16)-1024.0f},
                      (half2_t){(_Float16)-64.0f, (_Float16)-64.0f});
}

// workgroup barrier that orders LDS only: global loads stay in flight across it
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// range-checked buffer resource over [base, base + bytes)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferFlags);
}

__device__ __forceinline__ u32x4_t load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// The NF4 codebook as kernels take it: the 16 fp16 levels in ascending order, two per
// word (low half first).
struct Nf4Table {
  uint32_t pairs[8];
};

// Sum of the two results of one permlane swap. clang has been seen to fold `p[0] + p[1]` of
// a single swap into twice its first result; the empty asm statement keeps the two apart.
__device__ __forceinline__ float swap_pair_sum(uint32_t a, uint32_t b) {
  asm volatile("" : "+v"(a), "+v"(b));
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// lane l < 32: a[l] + a[l + 32]; lane l >= 32: b[l - 32] + b[l] (the swap exchanges a's upper
// half with b's lower half)
__device__ __forceinline__ float permlane32_swap_sum(float a, float b) {
  const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                                  false, false);
  return swap_pair_sum(p[0], p[1]);
}

// lanes of 16-lane rows 0 and 2: a summed over rows (0, 1) and (2, 3) respectively; rows 1 and
// 3: b summed the same way (the swap exchanges a's odd rows with b's even rows)
__device__ __forceinline__ float permlane16_swap_sum(float a, float b) {
  const auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                                  false, false);
  return swap_pair_sum(p[0], p[1]);
}

// Last three steps of a wave sum, within each group of 8 lanes: lanes l ^ 1, then l ^ 2
// (quad perms), then j and 7 - j (row_half_mirror, which after the first two steps pairs the
// group's two quads). Every lane ends with its group's sum.
__device__ __forceinline__ float dpp_group8_sum(float s) {
  s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, true));
  s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x4E, 0xF, 0xF, true));
  s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x141, 0xF, 0xF, true));
  return s;
}

// s + s of lane l ^ 8 (row_ror:8 within each 16-lane row)
__device__ __forceinline__ float dpp_ror8_sum(float s) {
  return s + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x128, 0xF, 0xF, true));
}

// Sums over the wave of V values at once: out[j] = the sum of v[j] over the 64 lanes, stored
// by one lane per value. Eight values take three halving steps that leave value j in lanes
// 8j .. 8j + 7 (swaps across lane halves and 16-lane rows, then a DPP rotate by 8 that pairs
// lanes l and l ^ 8), then three DPP steps over those 8 lanes: 10 cross-lane adds for 8
// values, against 6 per value one at a time. Four values take the two swap steps (value j in
// row j), two take one (value j in lane half j) and a last one none; each then goes on the
// same way. Every value is summed in one order, pairs of lanes at distance 32, 16, 8, then
// 1, 2, 4, whatever V and its slot, so a row's result does not depend on how many rows share
// its wave, and results are deterministic.
template <int V>
__device__ __forceinline__ void wave_sums(const float* v, float* out, int lane) {
  constexpr int V8 = V / 8, V4 = (V % 8) / 4, V2 = (V % 4) / 2, V1 = V % 2;
#pragma unroll
  for (int b = 0; b < V8; ++b) {
    const float* w = v + 8 * b;
    float s4[4], s2[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) s4[j] = permlane32_swap_sum(w[j], w[j + 4]);  // value j + 4 (l >> 5)
#pragma unroll
    for (int j = 0; j < 2; ++j) s2[j] = permlane16_swap_sum(s4[j], s4[j + 2]);  // j + 2 ((l >> 4) & 1) + ...
    const bool up = (lane & 8) != 0;
    const float keep = up ? s2[1] : s2[0], give = up ? s2[0] : s2[1];
    const float s = dpp_group8_sum(keep + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                              __builtin_bit_cast(int, give), 0x128, 0xF, 0xF, true)));  // value l >> 3
    if ((lane & 7) == 0) out[8 * b + (lane >> 3)] = s;
  }
  int j = 8 * V8;
  if constexpr (V4) {
    const float* w = v + j;
    const float s2a = permlane32_swap_sum(w[0], w[2]), s2b = permlane32_swap_sum(w[1], w[3]);
    const float s = dpp_group8_sum(dpp_ror8_sum(permlane16_swap_sum(s2a, s2b)));  // value l >> 4
    if ((lane & 15) == 0) out[j + (lane >> 4)] = s;
    j += 4;
  }
  if constexpr (V2) {
    const float h = permlane32_swap_sum(v[j], v[j + 1]);  // value l >> 5
    const float s = dpp_group8_sum(dpp_ror8_sum(permlane16_swap_sum(h, h)));
    if ((lane & 31) == 0) out[j + (lane >> 5)] = s;
    j += 2;
  }
  if constexpr (V1) {
    const float h = permlane32_swap_sum(v[j], v[j]);
    const float s = dpp_group8_sum(dpp_ror8_sum(permlane16_swap_sum(h, h)));
    if (lane == 0) out[j] = s;
  }
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
