// Device helpers shared by the front-end kernels: fp16 widening, the
// round-to-nearest-even magic constant and the packing of eight 4-bit codes
// into one word (layout in include/rrs.h, "Packed codes").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rrs {
namespace {

// Adding 1.5 * 2^23 to 0 <= x < 2^22 rounds x to the nearest integer (ties
// to even, the default mode) and leaves it in the low mantissa bits: for a
// code magnitude (<= 7) the low 3 bits of the result are the magnitude.
constexpr float kMagic = 12582912.0f;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, false));
}

// Maximum over aligned groups of `lanes` lanes (1, 2, 4, ..., 64; the same
// in every lane, every lane active), left in every lane of its group, for
// non-negative floats as their bit patterns (whose integer order is the
// values' order, so an integer maximum gives the bits fmaxf would). Group
// widths 2 and 4 are quad permutes, 8 and 16 the half-row and row mirrors
// (once the smaller groups are reduced each pairs a lane with one of the
// other half of its group), 32 and 64 the gfx950 row swaps: VALU moves,
// where a lane shuffle is an LDS round trip per level.
__device__ __forceinline__ uint32_t lanes_max_u32(uint32_t x, int lanes) {
  if (lanes >= 2) x = max(x, dpp_u32<0xB1>(x));   // quad_perm [1, 0, 3, 2]
  if (lanes >= 4) x = max(x, dpp_u32<0x4E>(x));   // quad_perm [2, 3, 0, 1]
  if (lanes >= 8) x = max(x, dpp_u32<0x141>(x));  // row_half_mirror
  if (lanes >= 16) x = max(x, dpp_u32<0x140>(x)); // row_mirror
  if (lanes >= 32) {
    const auto s = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = max(static_cast<uint32_t>(s[0]), static_cast<uint32_t>(s[1]));
  }
  if (lanes >= 64) {
    const auto s = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    x = max(static_cast<uint32_t>(s[0]), static_cast<uint32_t>(s[1]));
  }
  return x;
}

__device__ __forceinline__ float lanes_max(float x, int lanes) {
  return __uint_as_float(lanes_max_u32(__float_as_uint(x), lanes));
}

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// Byte 0 (resp. byte 3) of four words, gathered into one word.
__device__ __forceinline__ uint32_t gather_b0(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3) {
  const uint32_t t01 = __builtin_amdgcn_perm(x1, x0, 0x0c0c0400u);
  const uint32_t t23 = __builtin_amdgcn_perm(x3, x2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(t23, t01, 0x05040100u);
}
__device__ __forceinline__ uint32_t gather_b3(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3) {
  const uint32_t t01 = __builtin_amdgcn_perm(x1, x0, 0x0c0c0703u);
  const uint32_t t23 = __builtin_amdgcn_perm(x3, x2, 0x0c0c0703u);
  return __builtin_amdgcn_perm(t23, t01, 0x05040100u);
}

// Eight codes -> one packed word. mag[i] holds |code i| in its low 3 bits,
// sgn[i] the float whose sign is the sign of code i. Layout (8 codes per
// little-endian word, a_j = code 2j, b_j = code 2j+1): byte j carries |a_j|
// in bits 0-2, |b_j| in bits 4-6 and sign(a_j) in bit 7; bit 3 of byte
// (j+1) mod 4 carries sign(b_j). With it, w & 0x87878787 and
// rotr(w, 4) & 0x87878787 are the a- and b-codes as fp8 e4m3 subnormals.
__device__ __forceinline__ uint32_t pack8(const uint32_t* mag, const uint32_t* sgn) {
  const uint32_t ma = gather_b0(mag[0], mag[2], mag[4], mag[6]);
  const uint32_t mb = gather_b0(mag[1], mag[3], mag[5], mag[7]);
  const uint32_t sa = gather_b3(sgn[0], sgn[2], sgn[4], sgn[6]);
  const uint32_t sb = gather_b3(sgn[7], sgn[1], sgn[3], sgn[5]);
  return ma | (mb << 4) | (sa & 0x80808080u) | ((sb >> 4) & 0x08080808u);
}

}  // namespace
}  // namespace rrs
