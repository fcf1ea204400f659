// Register-level INT4 unpack shared by the GFX950_B GEMM kernels.
//
// With q the int4 code, u = q + 8 its offset-binary nibble and B = 128 + u =
// q + 136 (exact in bf16: the bits 0x4300 | u; fp16 uses 1024 + u = q + 1032,
// bits 0x6400 | u), a code becomes a 16-bit MFMA operand with one byte permute
// and one and-or; the constant 136 (1032) times the row sum of x is removed
// after the contraction.
#pragma once

#include "wq_device.h"

namespace wq {

template <int ACT>
struct Magic;
template <>
struct Magic<ACT_BF16> {
  static constexpr uint32_t bits = 0x43004300u;
  static constexpr float bias = 136.f;
};
template <>
struct Magic<ACT_F16> {
  static constexpr uint32_t bits = 0x64006400u;
  static constexpr float bias = 1032.f;
};

// (p & mask) | bits in one VALU op (the compiler emits and + or).
__device__ __forceinline__ uint32_t and_or(uint32_t p, uint32_t mask, uint32_t bits) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(p), "v"(mask), "v"(bits));
  return r;
}

// Eight int4 codes (one dword, K ascending from the low nibble) -> eight
// 16-bit values (q + bias), dword j = codes (2j, 2j+1) in (low, high) half.
// With mask = 0x000F000F and bits = the magic exponent pattern; mask = bits =
// 0 gives zeros (a column whose group scale is zero).
__device__ __forceinline__ u32x4 unpack8(uint32_t w, uint32_t mask, uint32_t bits) {
  const uint32_t u = w ^ 0x88888888u;        // two's complement -> offset binary
  const uint32_t u4 = u >> 4;
  u32x4 r;
  r.x = and_or(__builtin_amdgcn_perm(u4, u, 0x0C040C00u), mask, bits);
  r.y = and_or(__builtin_amdgcn_perm(u4, u, 0x0C050C01u), mask, bits);
  r.z = and_or(__builtin_amdgcn_perm(u4, u, 0x0C060C02u), mask, bits);
  r.w = and_or(__builtin_amdgcn_perm(u4, u, 0x0C070C03u), mask, bits);
  return r;
}

}  // namespace wq
