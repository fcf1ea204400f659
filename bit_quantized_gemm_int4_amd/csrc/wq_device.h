// Device helpers shared by the libwq kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef _Float16 f16x8 __attribute__((__vector_size__(16)));
typedef float f32x4 __attribute__((__vector_size__(16)));
typedef int i32x8 __attribute__((__vector_size__(32)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Act { ACT_F16 = 0, ACT_BF16 = 1 };

// ---- 16-bit float storage <-> float ------------------------------------
template <int ACT>
__device__ __forceinline__ float to_f32(uint16_t h) {
  if constexpr (ACT == ACT_BF16) {
    return __uint_as_float((uint32_t)h << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, h);
  }
}

// Round-to-nearest-even float -> 16-bit storage.
template <int ACT>
__device__ __forceinline__ uint16_t from_f32(float f) {
  if constexpr (ACT == ACT_BF16) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
  } else {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
  }
}

template <int ACT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)from_f32<ACT>(lo) | ((uint32_t)from_f32<ACT>(hi) << 16);
}

// Low / high 16-bit halves of a packed pair, as float.
template <int ACT>
__device__ __forceinline__ float lo_f32(uint32_t v) {
  if constexpr (ACT == ACT_BF16) return __uint_as_float(v << 16);
  else return to_f32<ACT>((uint16_t)(v & 0xFFFFu));
}
template <int ACT>
__device__ __forceinline__ float hi_f32(uint32_t v) {
  if constexpr (ACT == ACT_BF16) return __uint_as_float(v & 0xFFFF0000u);
  else return to_f32<ACT>((uint16_t)(v >> 16));
}

// ---- DPP reductions over the 16 lanes of a row -------------------------
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror:
// afterwards every lane of the row holds the row's result, combined in a
// fixed order.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return v;
}

__device__ __forceinline__ float quad_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  return v;
}

__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  return v;
}

__device__ __forceinline__ float row16_max(float v) {
  v = quad_max(v);
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return v;
}

// Whole-wavefront max (64 lanes) via cross-lane swizzles.
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// s_waitcnt that waits until at most N vector-memory operations are
// outstanding (they complete in issue order) and leaves the other counters
// alone. The compiler does not order LDS reads after an LDS DMA by itself.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The wave's index in its workgroup, in a scalar register (the compiler
// cannot infer that threadIdx.x / 64 is wave-uniform).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// Buffer resources: loads take a per-lane VGPR byte offset plus a
// wave-uniform SGPR offset, so no 64-bit address arithmetic runs per load.
// An offset at or past the resource's byte count reads zero; BUF_OOB is such
// an offset for every resource of at most 2 GiB.
// One float -> OCP E2M1 code, round to nearest even: count the rounding
// thresholds passed (ties go to the even code: 0, 1.0, 2.0, 4.0); a
// magnitude beyond 6 passes every threshold and saturates to 6; the sign bit
// is kept (-0.0 -> code 8). NaN has no code (outside every caller's contract).
__device__ __forceinline__ uint32_t e2m1(float v) {
  const float a = fabsf(v);
  uint32_t m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
               (a >= 3.5f) + (a > 5.0f);
  return m | ((__float_as_uint(v) >> 28) & 0x8u);
}

// Eight floats -> eight E2M1 codes in one word, the first lowest: the
// gfx950 converter (scale 1), which rounds as e2m1() does (nearest, ties to
// even, saturating, sign kept; checked on every grid value, tie, signed zero
// and infinity).
__device__ __forceinline__ uint32_t e2m1x8(const float (&v)[8]) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

constexpr uint32_t BUF_OOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// ---- MFMA (16x16x32, 16-bit inputs, fp32 accumulate) --------------------
// Operand layout for lane l: A row l%16, B column l%16, eight consecutive K
// values starting at 8*(l/16); D column l%16, rows 4*(l/16)+i.
template <int ACT>
__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, f32x4 c) {
  if constexpr (ACT == ACT_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

}  // namespace wq
