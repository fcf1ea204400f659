// Register-level INT4 unpack shared by the GFX950_B GEMM kernels.
//
// With q the int4 code, u = q + 8 its offset-binary nibble and B = 128 + u =
// q + 136 (exact in bf16: the bits 0x4300 | u; fp16 uses 1024 + u = q + 1032,
// bits 0x6400 | u), a code becomes a 16-bit MFMA operand with one byte permute
// and one three-input bit operation; the constant 136 (1032) times the row sum of x is removed
// after the contraction.
#pragma once

#include "wq_device.h"

namespace wq {

// bits: the magic exponent pattern of two 16-bit lanes (value 128 / 1024 at
// u = 0). xbits = bits with bit 3 of each lane's nibble set: one bitop3
// C ^ (M & p) then flips the code's sign bit (two's complement -> offset
// binary), keeps only the nibble, and inserts the exponent.
template <int ACT>
struct Magic;
template <>
struct Magic<ACT_BF16> {
  static constexpr uint32_t bits = 0x43004300u;
  static constexpr uint32_t xbits = 0x43084308u;
  static constexpr float bias = 136.f;
};
template <>
struct Magic<ACT_F16> {
  static constexpr uint32_t bits = 0x64006400u;
  static constexpr uint32_t xbits = 0x64086408u;
  static constexpr float bias = 1032.f;
};

constexpr uint32_t NIBBLE_MASK = 0x000F000Fu;   // the low nibble of each 16-bit lane

// c ^ (m & p) in one VALU op.
__device__ __forceinline__ uint32_t xor_and(uint32_t p, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(p, m, c, 0x6A);
}

// Eight int4 codes (one dword, K ascending from the low nibble, two's
// complement) -> eight 16-bit values (q + bias), dword j = codes (2j, 2j+1)
// in its (low, high) half. With m = NIBBLE_MASK and c = Magic::xbits;
// m = c = 0 gives zeros (a column whose group scale is zero).
__device__ __forceinline__ u32x4 unpack8(uint32_t w, uint32_t m, uint32_t c) {
  const uint32_t w4 = w >> 4;
  u32x4 r;
  r.x = xor_and(__builtin_amdgcn_perm(w4, w, 0x0C040C00u), m, c);
  r.y = xor_and(__builtin_amdgcn_perm(w4, w, 0x0C050C01u), m, c);
  r.z = xor_and(__builtin_amdgcn_perm(w4, w, 0x0C060C02u), m, c);
  r.w = xor_and(__builtin_amdgcn_perm(w4, w, 0x0C070C03u), m, c);
  return r;
}

}  // namespace wq
