// Weight-quantized matmul + residual add + RMSNorm
// (aclnnWeightQuantMatmulAllReduceAddRmsNorm page, Formula):
//   mm = x1 @ (x2 * antiquantScale + antiquantOffset) + bias
//   y = mm + residual;  normOut = y / sqrt(mean(y^2) + eps) * gamma
//
// Two launches on the caller's stream:
//   1. a GEMM kernel whose epilogue adds bias and residual, stores y and
//      writes partial sums of y^2 (float32 y) to the workspace: per (row,
//      32-column tile), row-major; the decode kernel per (workgroup, row);
//   2. rmsnorm_finish: sums a row's partials in a fixed order, forms
//      1/RMS and writes normOut = y * rstd * gamma.
// (When the INT8 tile splits K across workgroups, its launch writes float32
// sums to the workspace instead, and its own finish, w8_split_finish, forms
// y and normOut: still two launches.)
// GEMM kernels:
//   - gemm_decode (wq_gemm_decode.hip): m <= 32, INT4 GFX950_B, k a
//     multiple of 128, any group: a weight stream;
//   - gemm_b_wide (wq_gemm_fast.hip): the same weights at larger m, the
//     MFMA-bound tile;
//   - gemm_w8 (wq_gemm_w8.hip): INT8 weights, row-major or transposed, k a
//     multiple of 16: a 64 x 64 tile with loads two K steps ahead; also
//     INT4 GFX950_B weights where the two kernels above do not apply;
//   - gemm_generic: any weight layout (INT4 ND / ND transposed / GFX950_B,
//     INT8 ND / transposed), any group size, 64x64x32 tiles with both operands staged
//     in LDS; integer codes go to the MFMA and each group's scale and
//     offset are applied to its float32 partial sums.
#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

enum WFmt { W_I4_ND = 0, W_I4_B = 1, W_I8_ND = 2, W_I8_T = 3, W_I4_T = 4 };

struct GemmArgs {
  const uint16_t* x1;
  const uint8_t* x2;
  const uint16_t* scale;
  const uint16_t* offset;
  const uint16_t* bias;
  const uint16_t* residual;
  uint16_t* y;
  float* partial;        // [m][ceil(n/32)]
  int64_t m, k, n, np;   // np: padded N of the GFX950_B layout
  int64_t group, s_row, s_col;
};

// Epilogue for one 16x16 MFMA tile held by a wave: y = acc + bias + residual
// (no residual: zero), stored rounded; returns the float32 y values (0
// outside the matrix).
template <int ACT>
__device__ __forceinline__ void epilogue_tile(const GemmArgs& a, const f32x4& acc, int64_t row0,
                                              int64_t col, float yv[4]) {
  const int lane = threadIdx.x & 63;
  const bool cin = col < a.n;
  const float b = (cin && a.bias) ? to_f32<ACT>(a.bias[col]) : 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row0 + 4 * (lane >> 4) + i;
    float v = 0.f;
    if (cin && row < a.m) {
      const int64_t idx = row * a.n + col;
      v = acc[i] + b + (a.residual ? to_f32<ACT>(a.residual[idx]) : 0.f);
      a.y[idx] = from_f32<ACT>(v);
    }
    yv[i] = v;
  }
}

constexpr int GB_M = 64, GB_N = 64, GB_K = 32, G_LDS = GB_K + 8;

// One K step of 32 covers a single quantization group (G is a multiple of 32),
// so each 16x16x32 MFMA sums x1 * q for one group. The codes enter the MFMA
// exactly (|q| <= 127 fits both 16-bit formats); the group's scale and offset
// are applied to the float32 partial when the group ends:
//   acc += s[g, n] * sum_k x1[r, k] q[k, n] + o[g, n] * sum_k x1[r, k]
// with the row sums from one more MFMA against a fragment of ones.
template <int ACT, int WF>
__global__ __launch_bounds__(256) void gemm_generic(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[GB_M][G_LDS];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[GB_N][G_LDS];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.x * GB_M;
  const int64_t n0 = (int64_t)blockIdx.y * GB_N;
  const bool avec = (a.k & 7) == 0;
  const uint32_t one2 = pack2<ACT>(1.f, 1.f);
  const u32x4 ones = {one2, one2, one2, one2};
  f32x4 acc[2][2] = {}, part[2][2] = {}, rsum[2] = {};

  for (int64_t k0 = 0; k0 < a.k; k0 += GB_K) {
    // ---- A tile: thread -> row t/4, 8 consecutive k ----
    {
      const int r = t >> 2, kc = (t & 3) * 8;
      const int64_t row = m0 + r, kk = k0 + kc;
      u32x4 v = {0, 0, 0, 0};
      if (row < a.m) {
        const uint16_t* src = a.x1 + row * a.k + kk;
        if (avec && kk + 8 <= a.k) {
          v = *reinterpret_cast<const u32x4*>(src);
        } else {
          uint16_t e[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) e[i] = (kk + i < a.k) ? src[i] : (uint16_t)0;
          v.x = e[0] | ((uint32_t)e[1] << 16);
          v.y = e[2] | ((uint32_t)e[3] << 16);
          v.z = e[4] | ((uint32_t)e[5] << 16);
          v.w = e[6] | ((uint32_t)e[7] << 16);
        }
      }
      *reinterpret_cast<u32x4*>(&As[r][kc]) = v;
    }
    // ---- B tile: integer codes as 16-bit floats, stored [n][k] ----
    if constexpr (WF == W_I4_B || WF == W_I8_T || WF == W_I4_T) {
      // thread -> column t/4, 8 consecutive k
      const int c = t >> 2, kc = (t & 3) * 8;
      const int64_t col = n0 + c, kk = k0 + kc;
      int q[8];
      if constexpr (WF == W_I4_B) {
        uint32_t word = 0;
        if (col < a.np)
          word = *reinterpret_cast<const uint32_t*>(
              a.x2 + ((kk / 128) * a.np + col) * 64 + ((kk / 32) % 4) * 16 + (kk % 32) / 2);
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = ((int)(word << (28 - 4 * i))) >> 28;
      } else if constexpr (WF == W_I4_T) {
        // (n, k) with k packed two per byte, even k in the low nibble (k even)
        const uint8_t* src = a.x2 + col * (a.k / 2) + kk / 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int b = (col < a.n && kk + 2 * i < a.k) ? (int)src[i] : 0;
          q[2 * i] = ((int)(b << 28)) >> 28;
          q[2 * i + 1] = ((int)(b << 24)) >> 28;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          q[i] = (col < a.n && kk + i < a.k) ? (int)(int8_t)a.x2[col * a.k + kk + i] : 0;
      }
      u32x4 v;
      v.x = pack2<ACT>((float)q[0], (float)q[1]);
      v.y = pack2<ACT>((float)q[2], (float)q[3]);
      v.z = pack2<ACT>((float)q[4], (float)q[5]);
      v.w = pack2<ACT>((float)q[6], (float)q[7]);
      *reinterpret_cast<u32x4*>(&Bs[c][kc]) = v;
    } else {
      // row-major (k, n): thread -> k row t/8, 8 consecutive columns
      const int r = t >> 3, nc = (t & 7) * 8;
      const int64_t kk = k0 + r;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t col = n0 + nc + i;
        int q = 0;
        if (kk < a.k && col < a.n) {
          if constexpr (WF == W_I4_ND) {
            const uint8_t b = a.x2[kk * (a.n / 2) + col / 2];
            q = (col & 1) ? ((int)(int8_t)b >> 4) : (((int)(int8_t)(b << 4)) >> 4);
          } else {
            q = (int)(int8_t)a.x2[kk * a.n + col];
          }
        }
        Bs[nc + i][r] = from_f32<ACT>((float)q);
      }
    }
    __syncthreads();
    // ---- MFMA: each wave 32x32 = 2x2 tiles of 16x16, one group's partial ----
    const int kq = (lane >> 4) * 8;
    u32x4 af[2], bf[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      af[i] = *reinterpret_cast<const u32x4*>(&As[wr * 32 + i * 16 + (lane & 15)][kq]);
      bf[i] = *reinterpret_cast<const u32x4*>(&Bs[wc * 32 + i * 16 + (lane & 15)][kq]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j) part[i][j] = mfma16<ACT>(af[i], bf[j], part[i][j]);
      if (a.offset) rsum[i] = mfma16<ACT>(af[i], ones, rsum[i]);
    }
    // ---- group end: fold scale and offset into the float32 accumulator ----
    const int64_t g = k0 / a.group;
    if ((k0 + GB_K) % a.group == 0 || k0 + GB_K >= a.k) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + wc * 32 + j * 16 + (lane & 15);
        float sv = 0.f, ov = 0.f;
        if (col < a.n) {
          const int64_t si = g * a.s_row + col * a.s_col;
          sv = to_f32<ACT>(a.scale[si]);
          if (a.offset) ov = to_f32<ACT>(a.offset[si]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            acc[i][j][r] = fmaf(sv, part[i][j][r], acc[i][j][r]);
            if (a.offset) acc[i][j][r] = fmaf(ov, rsum[i][r], acc[i][j][r]);
            part[i][j][r] = 0.f;
          }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) rsum[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();
  }

  // ---- epilogue: y, and the wave's per-row sum of y^2 over its 32 columns ----
  float ss[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float y0[4], y1[4];
    const int64_t row0 = m0 + wr * 32 + i * 16;
    epilogue_tile<ACT>(a, acc[i][0], row0, n0 + wc * 32 + (lane & 15), y0);
    epilogue_tile<ACT>(a, acc[i][1], row0, n0 + wc * 32 + 16 + (lane & 15), y1);
#pragma unroll
    for (int r = 0; r < 4; ++r) ss[i][r] = row16_sum(y0[r] * y0[r] + y1[r] * y1[r]);
  }
  const int64_t tile32 = (n0 + wc * 32) / 32;
  if ((lane & 15) == 0 && n0 + wc * 32 < a.n) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wr * 32 + i * 16 + 4 * (lane >> 4) + r;
        if (row < a.m) a.partial[row * ((a.n + 31) / 32) + tile32] = ss[i][r];
      }
  }
}

// ---------------------------------------------------------------------------
// RMSNorm finish: grid (m rows, column chunks). Every workgroup of a row sums
// the same partials in the same order, so all of them agree on rstd. Partial
// (tile i, row r) sits at i * ts + r * rstride.
// ---------------------------------------------------------------------------
template <int ACT>
__global__ __launch_bounds__(256) void rmsnorm_finish(const uint16_t* __restrict__ y,
                                                      const float* __restrict__ partial,
                                                      int64_t tiles, int64_t ts, int64_t rstride,
                                                      const uint16_t* __restrict__ gamma,
                                                      uint16_t* __restrict__ out, int64_t m, int64_t n,
                                                      float eps, int64_t chunk) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t c_begin = (int64_t)blockIdx.y * chunk;
  const int64_t c_end = c_begin + chunk < n ? c_begin + chunk : n;
  const uint16_t* yr = y + row * n;
  uint16_t* orow = out + row * n;
  const bool vec = (n & 7) == 0 && chunk <= 256 * 8;
  // y and gamma do not depend on the row's sum: fetch them first (vector
  // case: one 8-column group per thread), then reduce the partials.
  u32x4 yv = {0u, 0u, 0u, 0u}, gv = {0u, 0u, 0u, 0u};
  const int64_t cv = c_begin + t * 8;
  if (vec && cv < c_end) {
    yv = *reinterpret_cast<const u32x4*>(yr + cv);
    gv = *reinterpret_cast<const u32x4*>(gamma + cv);
  }
  float s = 0.f;
  for (int64_t i = t; i < tiles; i += 256) s += partial[i * ts + row * rstride];
  s = wave_sum(s);
  if ((t & 63) == 0) red[t >> 6] = s;
  __syncthreads();
  s = (red[0] + red[1]) + (red[2] + red[3]);
  const float rstd = 1.0f / sqrtf(s / (float)n + eps);
  if (vec) {
    if (cv < c_end) {
      uint32_t yw[4] = {yv.x, yv.y, yv.z, yv.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w}, ow[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ow[i] = pack2<ACT>(lo_f32<ACT>(yw[i]) * rstd * lo_f32<ACT>(gw[i]),
                           hi_f32<ACT>(yw[i]) * rstd * hi_f32<ACT>(gw[i]));
      u32x4 o;
      o.x = ow[0];
      o.y = ow[1];
      o.z = ow[2];
      o.w = ow[3];
      *reinterpret_cast<u32x4*>(orow + cv) = o;
    }
  } else {
    for (int64_t c = c_begin + t; c < c_end; c += 256)
      orow[c] = from_f32<ACT>(to_f32<ACT>(yr[c]) * rstd * to_f32<ACT>(gamma[c]));
  }
}

template <int ACT>
hipError_t launch_generic(const WqProblem& p, const GemmArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((p.m + GB_M - 1) / GB_M), (unsigned)((p.n + GB_N - 1) / GB_N));
  prof_begin(s);
  if (p.w_bits == 4) {
    if (p.layout == WQ_LAYOUT_GFX950_B) gemm_generic<ACT, W_I4_B><<<grid, 256, 0, s>>>(a);
    else if (p.transpose_x2) gemm_generic<ACT, W_I4_T><<<grid, 256, 0, s>>>(a);
    else gemm_generic<ACT, W_I4_ND><<<grid, 256, 0, s>>>(a);
  } else {
    if (p.transpose_x2) gemm_generic<ACT, W_I8_T><<<grid, 256, 0, s>>>(a);
    else gemm_generic<ACT, W_I8_ND><<<grid, 256, 0, s>>>(a);
  }
  prof_end(s);
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_finish(const WqProblem& p, const GemmArgs& a, int64_t tiles, int64_t ts,
                         int64_t rstride, hipStream_t s) {
  // one 8-column group per thread (256 x 8 = 2048 columns per workgroup);
  // narrower chunks for few rows so that the grid still spreads over the CUs
  int64_t chunk = 2048;
  if (p.m < 64) chunk = 512;
  if (chunk > p.n) chunk = p.n;
  dim3 grid((unsigned)p.m, (unsigned)((p.n + chunk - 1) / chunk));
  rmsnorm_finish<ACT><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(p.y), a.partial, tiles, ts,
                                           rstride,
                                           static_cast<const uint16_t*>(p.gamma),
                                           static_cast<uint16_t*>(p.norm_out), p.m, p.n, p.eps, chunk);
  return hipGetLastError();
}

}  // namespace

namespace {
// room for one partial per (16-column tile, row): the finest granularity any
// GEMM kernel writes
size_t partial_bytes(int64_t m, int64_t n) {
  const int64_t tiles = (n + 15) / 16;
  return ((size_t)(tiles * m) * sizeof(float) + 255) & ~(size_t)255;
}
}  // namespace

// Workspace: per-(32-column tile, row) partial sums of y^2, then (fast path)
// per-group row sums of x1 and per-group column corrections as bf16 splits;
// or, for the decode kernel, its per-(workgroup, row) sums. Rows run in
// chunks of kRowChunk, so the workspace covers one chunk. No call needs
// initial contents: each writes what it reads.
size_t wq_workspace_bytes(int64_t m, int64_t k, int64_t n) {
  // the last chunk's rows, which may take the INT8 tile's K split where a
  // full chunk does not
  const int64_t tail = m > kRowChunk && m % kRowChunk ? m % kRowChunk : 0;
  if (m > kRowChunk) m = kRowChunk;
  size_t tiled = partial_bytes(m, n) + fast_rowsum_bytes(m, k) + fast_corr_bytes(n, k);
  const size_t dec = decode_partial_bytes(n);
  const size_t split = w8_split_bytes(m, k, n), split_tail = w8_split_bytes(tail, k, n);
  if (dec > tiled) tiled = dec;
  if (split > tiled) tiled = split;
  if (split_tail > tiled) tiled = split_tail;
  return tiled + 256;
}

namespace {

hipError_t wq_rows(const WqProblem& p, hipStream_t s) {
  GemmArgs a;
  a.x1 = static_cast<const uint16_t*>(p.x1);
  a.x2 = static_cast<const uint8_t*>(p.x2);
  a.scale = static_cast<const uint16_t*>(p.scale);
  a.offset = static_cast<const uint16_t*>(p.offset);
  a.bias = static_cast<const uint16_t*>(p.bias);
  a.residual = static_cast<const uint16_t*>(p.residual);
  a.y = static_cast<uint16_t*>(p.y);
  a.partial = static_cast<float*>(p.workspace);
  a.m = p.m;
  a.k = p.k;
  a.n = p.n;
  a.np = 16 * ((p.n + 15) / 16);
  a.group = p.group;
  a.s_row = p.s_row;
  a.s_col = p.s_col;
  hipError_t e;
  // partials: [row][tile] with 32-column tiles, or the decode kernel's
  // [row][workgroup]: partial i of row r at i * ts + r * rstride
  int64_t tiles = (p.n + 31) / 32, ts = 1, rstride = tiles;
  if (decode_ok(p)) {
    tiles = decode_grid(p);
    rstride = tiles;
    e = launch_decode(p, a.partial, s);
  } else if (fast_path_ok(p)) {
    uint8_t* ws = reinterpret_cast<uint8_t*>(a.partial);
    uint16_t* rs = reinterpret_cast<uint16_t*>(ws + partial_bytes(p.m, p.n));
    uint16_t* corr = reinterpret_cast<uint16_t*>(ws + partial_bytes(p.m, p.n) +
                                                 fast_rowsum_bytes(p.m, p.k));
    e = launch_prefill(p, a.partial, rs, corr, s);
  } else if (w8_ok(p)) {
    bool finished = false;
    e = launch_w8(p, a.partial, s, finished);
    if (e != hipSuccess || finished) return e;
  } else {
    e = p.bf16 ? launch_generic<ACT_BF16>(p, a, s) : launch_generic<ACT_F16>(p, a, s);
  }
  if (e != hipSuccess) return e;
  if (!p.norm_out) return hipSuccess;                 // the standalone matmul: no norm
  return p.bf16 ? launch_finish<ACT_BF16>(p, a, tiles, ts, rstride, s)
                : launch_finish<ACT_F16>(p, a, tiles, ts, rstride, s);
}

}  // namespace

// Rows are independent: taller inputs run as chunks of kRowChunk rows, one
// after the other on the stream (the workspace is reused), so that no grid
// over rows passes the launch limit after an earlier kernel has written.
hipError_t launch_wq_matmul_add_rmsnorm(const WqProblem& p, hipStream_t s) {
  for (int64_t r0 = 0; r0 < p.m; r0 += kRowChunk) {
    WqProblem c = p;
    c.m = p.m - r0 < kRowChunk ? p.m - r0 : kRowChunk;
    c.x1 = static_cast<const uint16_t*>(p.x1) + r0 * p.k;
    if (p.residual) c.residual = static_cast<const uint16_t*>(p.residual) + r0 * p.n;
    c.y = static_cast<uint16_t*>(p.y) + r0 * p.n;
    if (p.norm_out) c.norm_out = static_cast<uint16_t*>(p.norm_out) + r0 * p.n;
    const hipError_t e = wq_rows(c, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
