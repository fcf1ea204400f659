// Register-level INT4 unpack shared by the GFX950_B GEMM kernels.
//
// A code q (two's complement nibble) becomes the 16-bit MFMA operand
// B = q + 24, exact in both formats: with u = q + 8 its offset-binary nibble,
// B = 16 * (1 + u / 16), i.e. exponent 2^4 and the nibble in the top four
// mantissa bits (bf16: bits 3..6; fp16: bits 6..9). The constant 24 times
// the row sum of x is removed after the contraction. Putting the nibble in
// the top mantissa bits keeps that constant small: the float32 accumulator
// then carries 24 * sum(x) on top of the exact sum(x * q), instead of the
// 136 * sum(x) (bf16) or 1032 * sum(x) (fp16) of a nibble in the low
// mantissa bits, which loses up to 40x more accuracy when sum(x) is large
// (activations of one sign).
//
// Eight codes of one packed dword (K ascending from the low nibble) give
// four dwords; dword j holds codes (2j, 2j+1) in its (low, high) half. The
// work is split into a source step (once per packed dword) and one step per
// output dword, so that a kernel can interleave them with its MFMAs:
//   bf16: sources w << 3 and w >> 1 (byte j of each then holds nibble 2j
//         resp. 2j+1 in its bits 3..6); per dword one byte permute and one
//         bitop3 C ^ (M & p) that keeps bits 3..6, flips the nibble's sign
//         bit and inserts the exponent: 10 operations per 8 codes;
//   fp16: sources a = offset-binary low nibbles of the bytes, b = the high
//         ones (one bitop3 each, plus a shift); per dword one permute that
//         places a[j] and b[j] in the low byte of each half, then one
//         shift-or that moves them to bits 6..9 and inserts the exponent:
//         11 operations per 8 codes.
// Zeroed keys (a column whose group scale is zero) give zero operands.
#pragma once

#include "wq_device.h"

namespace wq {

// c ^ (m & p) in one VALU op.
__device__ __forceinline__ uint32_t xor_and(uint32_t p, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(p, m, c, 0x6A);
}

template <int ACT>
struct Unpack;

template <>
struct Unpack<ACT_BF16> {
  static constexpr float bias = 24.f;
  static constexpr uint32_t k1 = 0x00780078u;   // keep bits 3..6 of each half
  static constexpr uint32_t k2 = 0x41C041C0u;   // exponent 2^4 (0x4180) ^ the nibble's sign bit
  struct Src {
    uint32_t a, b;
  };
  __device__ static __forceinline__ Src src(uint32_t w, uint32_t, uint32_t) { return {w << 3, w >> 1}; }
  // dword j of the unpacked codes; (m, c) = (k1, k2), or (0, 0) for zeros
  template <int J>
  __device__ static __forceinline__ uint32_t dword(const Src& s, uint32_t m, uint32_t c) {
    return xor_and(__builtin_amdgcn_perm(s.b, s.a, 0x0C040C00u + 0x00010001u * J), m, c);
  }
};

template <>
struct Unpack<ACT_F16> {
  static constexpr float bias = 24.f;
  static constexpr uint32_t k1 = 0x0F0F0F0Fu;   // each byte's nibble ...
  static constexpr uint32_t k1c = 0x08080808u;  // ... with its sign bit flipped (offset binary)
  static constexpr uint32_t k2 = 0x4C004C00u;   // exponent 2^4
  struct Src {
    uint32_t a, b;
  };
  // (m, c) = (k1, k1c), or (0, 0) for zeros
  __device__ static __forceinline__ Src src(uint32_t w, uint32_t m, uint32_t c) {
    return {xor_and(w, m, c), xor_and(w >> 4, m, c)};
  }
  // e = k2, or 0 for zeros
  template <int J>
  __device__ static __forceinline__ uint32_t dword(const Src& s, uint32_t, uint32_t e) {
    return (__builtin_amdgcn_perm(s.b, s.a, 0x0C040C00u + 0x00010001u * J) << 6) | e;
  }
};

// The per-lane keys of one column: the constants, or zeros when the column's
// group scale is zero.
template <int ACT>
struct UnpackKeys {
  uint32_t m1, c1, m2, c2;
  __device__ __forceinline__ void set(bool on) {
    if constexpr (ACT == ACT_BF16) {
      m1 = c1 = 0u;
      m2 = on ? Unpack<ACT>::k1 : 0u;
      c2 = on ? Unpack<ACT>::k2 : 0u;
    } else {
      m1 = on ? Unpack<ACT>::k1 : 0u;
      c1 = on ? Unpack<ACT>::k1c : 0u;
      m2 = 0u;
      c2 = on ? Unpack<ACT>::k2 : 0u;
    }
  }
};

// Eight codes of one dword -> four dwords of (q + 24), unmasked.
template <int ACT>
__device__ __forceinline__ u32x4 unpack8(uint32_t w) {
  using U = Unpack<ACT>;
  const uint32_t m1 = ACT == ACT_BF16 ? 0u : Unpack<ACT_F16>::k1;
  const uint32_t c1 = ACT == ACT_BF16 ? 0u : Unpack<ACT_F16>::k1c;
  const uint32_t m2 = ACT == ACT_BF16 ? Unpack<ACT_BF16>::k1 : 0u;
  const typename U::Src s = U::src(w, m1, c1);
  u32x4 r;
  r.x = U::template dword<0>(s, m2, U::k2);
  r.y = U::template dword<1>(s, m2, U::k2);
  r.z = U::template dword<2>(s, m2, U::k2);
  r.w = U::template dword<3>(s, m2, U::k2);
  return r;
}

// Eight codes of one dword -> four dwords of (q + 136) (bf16) or (q + 1032)
// (fp16): the nibble in the low mantissa bits, one shift per dword and one
// permute plus one bitop3 per output dword (9 operations per 8 codes). The
// larger constant is harmless where the partial sums are folded into float32
// every 128 K values (the decode kernel); accumulators that run over many
// groups use the q + 24 form above.
template <int ACT>
struct UnpackLow {
  static constexpr float bias = ACT == ACT_BF16 ? 136.f : 1032.f;
  static constexpr uint32_t xbits = ACT == ACT_BF16 ? 0x43084308u : 0x64086408u;
};

template <int ACT>
__device__ __forceinline__ u32x4 unpack8_low(uint32_t w) {
  constexpr uint32_t m = 0x000F000Fu, c = UnpackLow<ACT>::xbits;
  const uint32_t w4 = w >> 4;
  u32x4 r;
  r.x = xor_and(__builtin_amdgcn_perm(w4, w, 0x0C040C00u), m, c);
  r.y = xor_and(__builtin_amdgcn_perm(w4, w, 0x0C050C01u), m, c);
  r.z = xor_and(__builtin_amdgcn_perm(w4, w, 0x0C060C02u), m, c);
  r.w = xor_and(__builtin_amdgcn_perm(w4, w, 0x0C070C03u), m, c);
  return r;
}

}  // namespace wq
