// Dynamic quantization (aclnnDynamicQuant page, Formula):
//   input = x * smooth;  scale = row_max(|input|) / dtypeMax;
//   y = round(input / scale)
// Per-token mode: one scale per row (INT8 / INT4 / INT32 outputs).
// MX mode: one power-of-two scale per (row, 32-long K block), E4M3 or E2M1
// codes, optionally stored transposed for the MX matmul's transposeX1 input.
//
// Both kernels are HBM-bound streams: 16-byte loads of eight 16-bit inputs
// per lane, row / block maxima reduced across lanes with DPP, codes decided
// in float32 exactly as the operator defines them (correctly rounded
// division for the per-token code, exact power-of-two scaling for MX).
#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

// ---------------------------------------------------------------------------
// Per-token. One 256-thread workgroup per row; the row is read twice (max,
// then codes); the second read is served by L2.
// ---------------------------------------------------------------------------
enum OutKind { OUT_INT8 = 0, OUT_NIBBLES = 1 };  // INT4 and INT32 share bytes

template <int ACT>
__device__ __forceinline__ void load8(const uint16_t* __restrict__ x, const uint16_t* __restrict__ sm,
                                      int64_t c, int64_t cols, bool vec, float v[8]) {
  if (vec) {
    const u32x4 xv = *reinterpret_cast<const u32x4*>(x + c);
    uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = lo_f32<ACT>(xw[i]);
      v[2 * i + 1] = hi_f32<ACT>(xw[i]);
    }
    if (sm) {
      const u32x4 sv = *reinterpret_cast<const u32x4*>(sm + c);
      uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] *= lo_f32<ACT>(sw[i]);
        v[2 * i + 1] *= hi_f32<ACT>(sw[i]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool in = c + i < cols;
      float t = in ? to_f32<ACT>(x[c + i]) : 0.f;
      if (sm) t *= in ? to_f32<ACT>(sm[c + i]) : 0.f;
      v[i] = t;
    }
  }
}

template <int ACT, int OUT>
__global__ __launch_bounds__(256) void quant_per_token_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ smooth, int64_t cols,
    float dmax, void* __restrict__ y, float* __restrict__ scale) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * cols;
  const bool vec = (cols & 7) == 0;
  const int t = threadIdx.x;

  float amax = 0.f;
  for (int64_t c = (int64_t)t * 8; c < cols; c += 256 * 8) {
    float v[8];
    load8<ACT>(xr, smooth, c, cols, vec, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max(amax);
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = amax / dmax;                 // correctly rounded fp32 divide
  if (t == 0) scale[row] = sc;

  for (int64_t c = (int64_t)t * 8; c < cols; c += 256 * 8) {
    float v[8];
    load8<ACT>(xr, smooth, c, cols, vec, v);
    int q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float r = sc == 0.f ? 0.f : __builtin_rintf(v[i] / sc);   // RNE of the fp32 quotient
      r = fminf(fmaxf(r, -dmax), dmax);
      q[i] = (int)r;
    }
    if constexpr (OUT == OUT_INT8) {
      int8_t* yr = reinterpret_cast<int8_t*>(y) + row * cols;
      if (vec) {
        u32x2 o;
        o.x = (q[0] & 0xFF) | ((q[1] & 0xFF) << 8) | ((q[2] & 0xFF) << 16) | ((uint32_t)(q[3] & 0xFF) << 24);
        o.y = (q[4] & 0xFF) | ((q[5] & 0xFF) << 8) | ((q[6] & 0xFF) << 16) | ((uint32_t)(q[7] & 0xFF) << 24);
        *reinterpret_cast<u32x2*>(yr + c) = o;
      } else {
        for (int i = 0; i < 8 && c + i < cols; ++i) yr[c + i] = (int8_t)q[i];
      }
    } else {
      // two codes per byte, even column in the low nibble (cols is even)
      uint8_t* yr = reinterpret_cast<uint8_t*>(y) + row * (cols / 2);
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) word |= (uint32_t)(q[i] & 0xF) << (4 * i);
      if (vec) {
        *reinterpret_cast<uint32_t*>(yr + c / 2) = word;
      } else {
        for (int i = 0; i < 4 && c + 2 * i < cols; ++i) yr[c / 2 + i] = (uint8_t)(word >> (8 * i));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MX block-32. A workgroup covers 128 rows x 64 columns; each thread owns 4
// rows x 8 columns, so one 32-block of a row spans a quad of lanes and its
// maximum is a two-step DPP reduction. Scale exponent from the block maximum
// by integer arithmetic on its float32 bits; codes = input * 2^-e converted
// with round-to-nearest-even.
// ---------------------------------------------------------------------------
enum MxFmt { MX_E4M3 = 0, MX_E2M1 = 1 };

// Smallest e with dmax * 2^e >= a (a > 0): dmax = 1.75 * 2^8 (E4M3) or
// 1.5 * 2^2 (E2M1); with a = 1.f * 2^E, e = E - 8 (or E - 2), plus one when
// the fraction exceeds dmax's.
template <int FMT>
__device__ __forceinline__ int mx_exponent(float a) {
  uint32_t b = __float_as_uint(a);
  int E;
  uint32_t frac;
  if ((b >> 23) == 0) {                          // float32 subnormal
    const int sh = __clz(b) - 8;
    frac = (b << sh) & 0x7FFFFFu;
    E = -126 - sh;
  } else {
    frac = b & 0x7FFFFFu;
    E = (int)(b >> 23) - 127;
  }
  int e = (FMT == MX_E4M3) ? E - 8 + (frac > 0x600000u ? 1 : 0)
                           : E - 2 + (frac > 0x400000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Two floats (|v| <= 448) -> two E4M3 codes in the low 16 bits, RNE, with
// the gfx950 OCP FP8 conversion.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// One float (|v| <= 6) -> E2M1 code, RNE: count the rounding thresholds
// passed (ties go to the even code: 0, 1.0, 2.0, 4.0).
__device__ __forceinline__ uint32_t e2m1(float v) {
  const float a = fabsf(v);
  uint32_t m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
               (a >= 3.5f) + (a > 5.0f);
  return m | ((__float_as_uint(v) >> 28) & 0x8u);
}

template <int ACT, int FMT, bool TRANS>
__global__ __launch_bounds__(256) void quant_mx_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ smooth, int64_t rows,
    int64_t cols, uint8_t* __restrict__ y, uint8_t* __restrict__ scale) {
  constexpr int LR = 128 + 4;                    // LDS row (one column), bytes
  __shared__ __attribute__((aligned(16))) uint8_t tile[TRANS ? 64 : 1][TRANS ? LR : 4];
  const int t = threadIdx.x;
  const int rg = t >> 3, cc = t & 7;
  const int64_t r0 = (int64_t)blockIdx.x * 128 + rg * 4;
  const int64_t c0 = (int64_t)blockIdx.y * 64 + cc * 8;
  const int64_t nb = (cols + 31) / 32;
  const bool vec = (cols & 7) == 0 && c0 + 8 <= cols;

  float sm[8];
  if (smooth) {
    float ones[8];
    load8<ACT>(smooth, nullptr, c0, cols, vec, ones);
#pragma unroll
    for (int i = 0; i < 8; ++i) sm[i] = ones[i];
  }
  uint32_t codes[4][2];                          // 4 rows x 8 codes (bytes or nibbles)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t row = r0 + r;
    float v[8];
    if (row < rows && c0 < cols) {
      load8<ACT>(x + row * cols, nullptr, c0, cols, vec, v);
      if (smooth) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= sm[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = quad_max(amax);                       // the 4 lanes of this 32-block
    const int e = amax > 0.f ? mx_exponent<FMT>(amax) : 0;
    if ((cc & 3) == 0 && row < rows && c0 < cols) scale[row * nb + c0 / 32] = (uint8_t)(e + 127);
    float s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = __builtin_ldexpf(v[i], -e);   // exact
    if constexpr (FMT == MX_E4M3) {
      codes[r][0] = e4m3x2(s[0], s[1]) | (e4m3x2(s[2], s[3]) << 16);
      codes[r][1] = e4m3x2(s[4], s[5]) | (e4m3x2(s[6], s[7]) << 16);
    } else {
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) w |= e2m1(s[i]) << (4 * i);
      codes[r][0] = w;
      codes[r][1] = 0;
    }
  }

  if constexpr (!TRANS) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = r0 + r;
      if (row >= rows || c0 >= cols) continue;
      if constexpr (FMT == MX_E4M3) {
        uint8_t* dst = y + row * cols + c0;
        if (vec) {
          u32x2 o;
          o.x = codes[r][0];
          o.y = codes[r][1];
          *reinterpret_cast<u32x2*>(dst) = o;
        } else {
          for (int i = 0; i < 8 && c0 + i < cols; ++i)
            dst[i] = (uint8_t)(codes[r][i >> 2] >> (8 * (i & 3)));
        }
      } else {
        uint8_t* dst = y + row * (cols / 2) + c0 / 2;
        if (vec) {
          *reinterpret_cast<uint32_t*>(dst) = codes[r][0];
        } else {
          for (int i = 0; 2 * i < 8 && c0 + 2 * i < cols; ++i) dst[i] = (uint8_t)(codes[r][0] >> (8 * i));
        }
      }
    }
  } else {
    // transpose through LDS: tile[col][row] bytes, one dword = 4 rows of a column
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t b0 = (codes[0][j >> 2] >> (8 * (j & 3))) & 0xFF;
      const uint32_t b1 = (codes[1][j >> 2] >> (8 * (j & 3))) & 0xFF;
      const uint32_t b2 = (codes[2][j >> 2] >> (8 * (j & 3))) & 0xFF;
      const uint32_t b3 = (codes[3][j >> 2] >> (8 * (j & 3))) & 0xFF;
      *reinterpret_cast<uint32_t*>(&tile[cc * 8 + j][rg * 4]) = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
    }
    __syncthreads();
    const int64_t rt = (int64_t)blockIdx.x * 128;
    const int64_t ct = (int64_t)blockIdx.y * 64;
    const bool rvec = (rows & 3) == 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = t + 256 * i;
      const int c = idx >> 5, dw = idx & 31;
      const int64_t col = ct + c, row = rt + dw * 4;
      if (col >= cols || row >= rows) continue;
      const uint32_t word = *reinterpret_cast<const uint32_t*>(&tile[c][dw * 4]);
      uint8_t* dst = y + col * rows + row;
      if (rvec) {
        *reinterpret_cast<uint32_t*>(dst) = word;
      } else {
        for (int b = 0; b < 4 && row + b < rows; ++b) dst[b] = (uint8_t)(word >> (8 * b));
      }
    }
  }
}

}  // namespace

hipError_t launch_quant_per_token(const void* x, bool bf16, int64_t rows, int64_t cols,
                                  const void* smooth, wq_dtype y_dtype, void* y,
                                  float* scale, hipStream_t s) {
  const float dmax = y_dtype == WQ_INT8 ? 127.f : 7.f;
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* sp = static_cast<const uint16_t*>(smooth);
  dim3 grid((unsigned)rows);
  if (y_dtype == WQ_INT8) {
    if (bf16) quant_per_token_kernel<ACT_BF16, OUT_INT8><<<grid, 256, 0, s>>>(xp, sp, cols, dmax, y, scale);
    else quant_per_token_kernel<ACT_F16, OUT_INT8><<<grid, 256, 0, s>>>(xp, sp, cols, dmax, y, scale);
  } else {
    if (bf16) quant_per_token_kernel<ACT_BF16, OUT_NIBBLES><<<grid, 256, 0, s>>>(xp, sp, cols, dmax, y, scale);
    else quant_per_token_kernel<ACT_F16, OUT_NIBBLES><<<grid, 256, 0, s>>>(xp, sp, cols, dmax, y, scale);
  }
  return hipGetLastError();
}

hipError_t launch_quant_mx(const void* x, bool bf16, int64_t rows, int64_t cols,
                           const void* smooth, wq_dtype y_dtype, bool transpose_y,
                           uint8_t* y, uint8_t* scale, hipStream_t s) {
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* sp = static_cast<const uint16_t*>(smooth);
  dim3 grid((unsigned)((rows + 127) / 128), (unsigned)((cols + 63) / 64));
#define WQ_MX_LAUNCH(A, F, T) quant_mx_kernel<A, F, T><<<grid, 256, 0, s>>>(xp, sp, rows, cols, y, scale)
  if (y_dtype == WQ_FP8_E4M3) {
    if (transpose_y) {
      if (bf16) WQ_MX_LAUNCH(ACT_BF16, MX_E4M3, true); else WQ_MX_LAUNCH(ACT_F16, MX_E4M3, true);
    } else {
      if (bf16) WQ_MX_LAUNCH(ACT_BF16, MX_E4M3, false); else WQ_MX_LAUNCH(ACT_F16, MX_E4M3, false);
    }
  } else {
    if (bf16) WQ_MX_LAUNCH(ACT_BF16, MX_E2M1, false); else WQ_MX_LAUNCH(ACT_F16, MX_E2M1, false);
  }
#undef WQ_MX_LAUNCH
  return hipGetLastError();
}

}  // namespace wq
