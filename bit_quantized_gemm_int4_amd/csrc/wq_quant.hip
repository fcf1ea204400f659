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
// Per-token: one workgroup per row (below). MX: one workgroup per 128 x 64
// tile (further down).
// ---------------------------------------------------------------------------
enum OutKind { OUT_INT8 = 0, OUT_NIBBLES = 1 };  // INT4 and INT32 share bytes

// Eight consecutive 16-bit values at byte offset `off` of a buffer, with no
// branch, so a caller can issue all of its loads before it uses any: an
// offset of BUF_OOB reads zeros. VEC: `off` is 16-byte aligned and the eight
// values are all in range or all out; otherwise only the first `lim` are
// read and the rest are zero.
template <bool VEC>
__device__ __forceinline__ u32x4 fetch8(__amdgpu_buffer_rsrc_t r, uint32_t off, int64_t lim) {
  if constexpr (VEC) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  } else {
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      h[i] = __builtin_amdgcn_raw_buffer_load_b16(r, i < lim ? off + 2 * i : BUF_OOB, 0, 0);
    return u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  }
}

template <int ACT>
__device__ __forceinline__ void widen8(const u32x4& raw, float v[8]) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = lo_f32<ACT>(w[i]);
    v[2 * i + 1] = hi_f32<ACT>(w[i]);
  }
}

// Row scale and its reciprocal. The code of v is RNE(fl(v / sc)), the
// correctly rounded fp32 quotient rounded to an integer. With |v| <= amax and
// sc = fl(amax / dmax), |v / sc| <= 128; both v * fl(1 / sc) and fl(v / sc)
// are within 2^-23 relative (so 2.4e-5 absolute) of the exact quotient, and
// the integer rounding of either one can only differ when the product lies
// that close to a half-integer. Such values, and rows whose reciprocal
// overflows (sc subnormal), take the division.
struct RowScale {
  float sc, inv;
  bool fast;
};

__device__ __forceinline__ RowScale row_scale(float sc) {
  const float inv = 1.f / sc;
  return {sc, inv, sc > 0.f && inv < 0x1p126f};
}

// Quantize 8 values with the row scale and store them at column c.
template <int OUT>
__device__ __forceinline__ void store_codes8(void* __restrict__ y, int64_t row, int64_t cols, int64_t c,
                                             bool vec, const RowScale& rs, float dmax, const float v[8]) {
  float qf[8];
  bool slow = !rs.fast;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    qf[i] = v[i] * rs.inv;
    const float fr = qf[i] - floorf(qf[i]);   // exact for |qf| < 2^23
    slow |= fabsf(fr - 0.5f) < 1e-4f;
  }
  if (slow) {                                 // rare: recompute with the division
#pragma unroll
    for (int i = 0; i < 8; ++i) qf[i] = rs.sc == 0.f ? 0.f : v[i] / rs.sc;
  }
  int q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float r = __builtin_rintf(qf[i]);
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

// One 256-thread workgroup per row, read in batches of PT_CACHE 8-column
// chunks per thread (all loads of a batch in flight together). The first
// batch (the whole row up to 8192 columns) stays in registers for the codes;
// later batches are read again.
constexpr int PT_CACHE = 4;
constexpr int PT_SPAN = PT_CACHE * 256 * 8;   // columns per batch

// x * smooth for the batch starting at column `base`, zero past the row.
template <int ACT, bool VEC, bool SMOOTH>
__device__ __forceinline__ void fetch_batch(__amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rs,
                                            int64_t base, int64_t cols, int t,
                                            float (&v)[PT_CACHE][8]) {
  u32x4 xr[PT_CACHE], sr[PT_CACHE];
#pragma unroll
  for (int j = 0; j < PT_CACHE; ++j) {
    const int64_t c = base + (j * 256 + t) * 8;
    const uint32_t off = c < cols ? (uint32_t)(c * 2) : BUF_OOB;
    xr[j] = fetch8<VEC>(rx, off, cols - c);
    if constexpr (SMOOTH) sr[j] = fetch8<VEC>(rs, off, cols - c);
  }
#pragma unroll
  for (int j = 0; j < PT_CACHE; ++j) {
    widen8<ACT>(xr[j], v[j]);
    if constexpr (SMOOTH) {
      float sm[8];
      widen8<ACT>(sr[j], sm);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[j][i] *= sm[i];
    }
  }
}

template <int ACT, int OUT, bool VEC, bool SMOOTH>
__global__ __launch_bounds__(256) void quant_per_token_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ smooth, int64_t cols,
    float dmax, void* __restrict__ y, float* __restrict__ scale) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const uint32_t row_bytes = (uint32_t)(cols * 2);
  const __amdgpu_buffer_rsrc_t rx = buf_rsrc(x + row * cols, row_bytes);
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(SMOOTH ? smooth : x, SMOOTH ? row_bytes : 0u);

  float vc[PT_CACHE][8];
  fetch_batch<ACT, VEC, SMOOTH>(rx, rs, 0, cols, t, vc);
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < PT_CACHE; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(vc[j][i]));
  for (int64_t base = PT_SPAN; base < cols; base += PT_SPAN) {
    float v[PT_CACHE][8];
    fetch_batch<ACT, VEC, SMOOTH>(rx, rs, base, cols, t, v);
#pragma unroll
    for (int j = 0; j < PT_CACHE; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[j][i]));
  }
  amax = wave_max(amax);
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = amax / dmax;                 // correctly rounded fp32 divide
  if (t == 0) scale[row] = sc;
  const RowScale rsc = row_scale(sc);

#pragma unroll
  for (int j = 0; j < PT_CACHE; ++j) {
    const int64_t c = (j * 256 + t) * 8;
    if (c < cols) store_codes8<OUT>(y, row, cols, c, VEC, rsc, dmax, vc[j]);
  }
  for (int64_t base = PT_SPAN; base < cols; base += PT_SPAN) {
    float v[PT_CACHE][8];
    fetch_batch<ACT, VEC, SMOOTH>(rx, rs, base, cols, t, v);
#pragma unroll
    for (int j = 0; j < PT_CACHE; ++j) {
      const int64_t c = base + (j * 256 + t) * 8;
      if (c < cols) store_codes8<OUT>(y, row, cols, c, VEC, rsc, dmax, v[j]);
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


template <int ACT, int FMT, bool TRANS, bool VEC, bool SMOOTH>
__global__ __launch_bounds__(256) void quant_mx_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ smooth, int64_t rows,
    int64_t cols, uint8_t* __restrict__ y, uint8_t* __restrict__ scale) {
  constexpr int LR = 128 + 4;                    // LDS row (one column), bytes
  __shared__ __attribute__((aligned(16))) uint8_t tile[TRANS ? 64 : 1][TRANS ? LR : 4];
  // A thread takes 8 columns of 4 rows. Transposed output: 8 threads along a
  // row, a 128-row x 64-column block (transposed through LDS). Row-major
  // output: 64 threads along a row, a 16-row x 512-column block, so a
  // wave's loads and stores each cover 512 consecutive columns of a row.
  constexpr int TCOLS = TRANS ? 8 : 64;
  constexpr int BR = 256 / TCOLS * 4, BC = TCOLS * 8;
  const int t = threadIdx.x;
  const int rg = t / TCOLS, cc = t % TCOLS;
  const int64_t r0 = (int64_t)blockIdx.x * BR + rg * 4;
  const int64_t c0 = (int64_t)blockIdx.y * BC + cc * 8;
  const int64_t nb = (cols + 31) / 32;
  // One resource over the workgroup's rows; block-relative byte offsets
  // stay below 2^31 for cols < 2^22. All loads are issued before any use.
  const __amdgpu_buffer_rsrc_t rx = buf_rsrc(x + (int64_t)blockIdx.x * BR * cols, 0x7FFFFFFFu);
  const bool cin = c0 < cols;
  u32x4 raw[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const bool ok = cin && r0 + r < rows;
    raw[r] = fetch8<VEC>(rx, ok ? (uint32_t)(((rg * 4 + r) * cols + c0) * 2) : BUF_OOB, cols - c0);
  }
  float sm[8];
  if constexpr (SMOOTH)
    widen8<ACT>(fetch8<VEC>(buf_rsrc(smooth, (uint32_t)(cols * 2)), cin ? (uint32_t)(c0 * 2) : BUF_OOB,
                            cols - c0), sm);
  uint32_t codes[4][2];                          // 4 rows x 8 codes (bytes or nibbles)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t row = r0 + r;
    float v[8];
    widen8<ACT>(raw[r], v);
    if constexpr (SMOOTH) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] *= sm[i];
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
      codes[r][0] = e2m1x8(s);
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
        if (VEC) {
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
        if (VEC) {
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

namespace {

hipError_t quant_per_token_rows(const void* x, bool bf16, int64_t rows, int64_t cols,
                                const void* smooth, wq_dtype y_dtype, void* y, float* scale,
                                hipStream_t s) {
  const float dmax = y_dtype == WQ_INT8 ? 127.f : 7.f;
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* sp = static_cast<const uint16_t*>(smooth);
  dim3 grid((unsigned)rows);
  const bool vec = (cols & 7) == 0;
#define WQ_PT_LAUNCH(A, O)                                                                        \
  do {                                                                                            \
    if (vec && sp) quant_per_token_kernel<A, O, true, true><<<grid, 256, 0, s>>>(xp, sp, cols, dmax, y, scale);   \
    else if (vec) quant_per_token_kernel<A, O, true, false><<<grid, 256, 0, s>>>(xp, sp, cols, dmax, y, scale);   \
    else if (sp) quant_per_token_kernel<A, O, false, true><<<grid, 256, 0, s>>>(xp, sp, cols, dmax, y, scale);    \
    else quant_per_token_kernel<A, O, false, false><<<grid, 256, 0, s>>>(xp, sp, cols, dmax, y, scale);           \
  } while (0)
  if (y_dtype == WQ_INT8) {
    if (bf16) WQ_PT_LAUNCH(ACT_BF16, OUT_INT8); else WQ_PT_LAUNCH(ACT_F16, OUT_INT8);
  } else {
    if (bf16) WQ_PT_LAUNCH(ACT_BF16, OUT_NIBBLES); else WQ_PT_LAUNCH(ACT_F16, OUT_NIBBLES);
  }
#undef WQ_PT_LAUNCH
  return hipGetLastError();
}

}  // namespace

// One workgroup per row: rows go in chunks of kRowChunk so that no grid
// exceeds the launch limit of 2^32 threads per dimension.
hipError_t launch_quant_per_token(const void* x, bool bf16, int64_t rows, int64_t cols,
                                  const void* smooth, wq_dtype y_dtype, void* y,
                                  float* scale, hipStream_t s) {
  const int64_t y_row = y_dtype == WQ_INT8 ? cols : cols / 2;     // bytes per output row
  for (int64_t r0 = 0; r0 < rows; r0 += kRowChunk) {
    const int64_t nr = rows - r0 < kRowChunk ? rows - r0 : kRowChunk;
    const hipError_t e = quant_per_token_rows(static_cast<const uint16_t*>(x) + r0 * cols, bf16, nr, cols,
                                              smooth, y_dtype, static_cast<uint8_t*>(y) + r0 * y_row,
                                              scale + r0, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

namespace {

hipError_t quant_mx_rows(const void* x, bool bf16, int64_t rows, int64_t cols,
                         const void* smooth, wq_dtype y_dtype, bool transpose_y,
                         uint8_t* y, uint8_t* scale, hipStream_t s) {
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* sp = static_cast<const uint16_t*>(smooth);
  // blocks of 128 x 64 (transposed output) or 16 x 512 (row-major output)
  dim3 grid = transpose_y ? dim3((unsigned)((rows + 127) / 128), (unsigned)((cols + 63) / 64))
                          : dim3((unsigned)((rows + 15) / 16), (unsigned)((cols + 511) / 512));
  const bool vec = (cols & 7) == 0;
#define WQ_MX_LAUNCH(A, F, T)                                                                     \
  do {                                                                                            \
    if (vec && sp) quant_mx_kernel<A, F, T, true, true><<<grid, 256, 0, s>>>(xp, sp, rows, cols, y, scale);   \
    else if (vec) quant_mx_kernel<A, F, T, true, false><<<grid, 256, 0, s>>>(xp, sp, rows, cols, y, scale);   \
    else if (sp) quant_mx_kernel<A, F, T, false, true><<<grid, 256, 0, s>>>(xp, sp, rows, cols, y, scale);    \
    else quant_mx_kernel<A, F, T, false, false><<<grid, 256, 0, s>>>(xp, sp, rows, cols, y, scale);           \
  } while (0)
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

}  // namespace

// The row-major output takes rows in chunks of kRowChunk (16-row blocks of
// 256 threads would pass 2^32 threads per grid dimension beyond 2^28 rows);
// the transposed output's grid (128-row blocks) always fits.
hipError_t launch_quant_mx(const void* x, bool bf16, int64_t rows, int64_t cols,
                           const void* smooth, wq_dtype y_dtype, bool transpose_y,
                           uint8_t* y, uint8_t* scale, hipStream_t s) {
  if (transpose_y) return quant_mx_rows(x, bf16, rows, cols, smooth, y_dtype, true, y, scale, s);
  const int64_t y_row = y_dtype == WQ_FP8_E4M3 ? cols : cols / 2, s_row = (cols + 31) / 32;
  for (int64_t r0 = 0; r0 < rows; r0 += kRowChunk) {
    const int64_t nr = rows - r0 < kRowChunk ? rows - r0 : kRowChunk;
    const hipError_t e = quant_mx_rows(static_cast<const uint16_t*>(x) + r0 * cols, bf16, nr, cols, smooth,
                                       y_dtype, false, y + r0 * y_row, scale + r0 * s_row, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
