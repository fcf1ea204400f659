// AddRmsNorm, the second half of the unfused chain that replaces the fused
// operator (aclnnWeightQuantMatmulAllReduceAddRmsNorm page: deprecation note;
// Formula, its last two lines):
//   y = x + residual;  normOut = y / sqrt(mean over the row of y^2 + eps) * gamma
// x, residual, y and normOut are (rows, d) row-major in one activation dtype,
// gamma (d). As in the fused operator, the sum of squares uses the float32 y
// and normOut scales the stored (rounded) y.
//
// One workgroup of 256 threads per row. Vector path (d a multiple of 8):
// thread t takes the 16-byte chunks c = t, t + 256, ...; the first ARN_CACHE
// of them stay in registers as float32 y, the rest are read back from the
// stored y after the reduction (the thread's own stores, so y may alias x or
// residual). Element path otherwise. The row's sum is reduced in a fixed
// order (wave sums, then the four waves in index order).
#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int ARN_THREADS = 256;
constexpr int ARN_CACHE = 8;          // chunks of 8 per thread kept in registers (d <= 16384)

__device__ __forceinline__ float arn_block_sum(float s, float* red) {
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

template <int ACT>
__global__ __launch_bounds__(ARN_THREADS) void add_rmsnorm_vec(const uint16_t* x,
                                                               const uint16_t* res,
                                                               const uint16_t* __restrict__ gamma,
                                                               uint16_t* y, uint16_t* __restrict__ out,
                                                               int64_t d, float eps) {
  __shared__ float red[4];
  const int t = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * d;
  const int64_t chunks = d / 8;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + base);
  const u32x4* rr = reinterpret_cast<const u32x4*>(res + base);
  u32x4* yr = reinterpret_cast<u32x4*>(y + base);
  float yc[ARN_CACHE][8];
  float ss = 0.f;
  // y = x + residual: every load of the cached chunks first, then the sums
  u32x4 xv[ARN_CACHE], rv[ARN_CACHE];
#pragma unroll
  for (int j = 0; j < ARN_CACHE; ++j) {
    const int64_t c = t + (int64_t)j * ARN_THREADS;
    if (c < chunks) {
      xv[j] = xr[c];
      rv[j] = rr[c];
    }
  }
#pragma unroll
  for (int j = 0; j < ARN_CACHE; ++j) {
    const int64_t c = t + (int64_t)j * ARN_THREADS;
    if (c < chunks) {
      const uint32_t xw[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
      const uint32_t rw[4] = {rv[j].x, rv[j].y, rv[j].z, rv[j].w};
      uint32_t yw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a0 = lo_f32<ACT>(xw[e]) + lo_f32<ACT>(rw[e]);
        const float a1 = hi_f32<ACT>(xw[e]) + hi_f32<ACT>(rw[e]);
        ss = fmaf(a0, a0, ss);
        ss = fmaf(a1, a1, ss);
        yw[e] = pack2<ACT>(a0, a1);
        yc[j][2 * e] = lo_f32<ACT>(yw[e]);          // the stored (rounded) y
        yc[j][2 * e + 1] = hi_f32<ACT>(yw[e]);
      }
      yr[c] = (u32x4){yw[0], yw[1], yw[2], yw[3]};
    }
  }
  for (int64_t c = t + (int64_t)ARN_CACHE * ARN_THREADS; c < chunks; c += ARN_THREADS) {
    const u32x4 xa = xr[c], ra = rr[c];
    const uint32_t xw[4] = {xa.x, xa.y, xa.z, xa.w};
    const uint32_t rw[4] = {ra.x, ra.y, ra.z, ra.w};
    uint32_t yw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a0 = lo_f32<ACT>(xw[e]) + lo_f32<ACT>(rw[e]);
      const float a1 = hi_f32<ACT>(xw[e]) + hi_f32<ACT>(rw[e]);
      ss = fmaf(a0, a0, ss);
      ss = fmaf(a1, a1, ss);
      yw[e] = pack2<ACT>(a0, a1);
    }
    yr[c] = (u32x4){yw[0], yw[1], yw[2], yw[3]};
  }
  const float rstd = 1.0f / sqrtf(arn_block_sum(ss, red) / (float)d + eps);

  const u32x4* gr = reinterpret_cast<const u32x4*>(gamma);
  u32x4* orow = reinterpret_cast<u32x4*>(out + base);
  auto emit = [&](int64_t c, const float (&v)[8]) {
    const u32x4 ga = gr[c];
    const uint32_t gw[4] = {ga.x, ga.y, ga.z, ga.w};
    uint32_t ow[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      ow[e] = pack2<ACT>(v[2 * e] * rstd * lo_f32<ACT>(gw[e]), v[2 * e + 1] * rstd * hi_f32<ACT>(gw[e]));
    orow[c] = (u32x4){ow[0], ow[1], ow[2], ow[3]};
  };
#pragma unroll
  for (int j = 0; j < ARN_CACHE; ++j) {
    const int64_t c = t + (int64_t)j * ARN_THREADS;
    if (c < chunks) emit(c, yc[j]);
  }
  for (int64_t c = t + (int64_t)ARN_CACHE * ARN_THREADS; c < chunks; c += ARN_THREADS) {
    const u32x4 ya = yr[c];
    const uint32_t yw[4] = {ya.x, ya.y, ya.z, ya.w};
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = lo_f32<ACT>(yw[e]);
      v[2 * e + 1] = hi_f32<ACT>(yw[e]);
    }
    emit(c, v);
  }
}

template <int ACT>
__global__ __launch_bounds__(ARN_THREADS) void add_rmsnorm_elem(const uint16_t* x,
                                                                const uint16_t* res,
                                                                const uint16_t* __restrict__ gamma,
                                                                uint16_t* y, uint16_t* __restrict__ out,
                                                                int64_t d, float eps) {
  __shared__ float red[4];
  const int64_t base = (int64_t)blockIdx.x * d;
  float ss = 0.f;
  for (int64_t c = threadIdx.x; c < d; c += ARN_THREADS) {
    const float a = to_f32<ACT>(x[base + c]) + to_f32<ACT>(res[base + c]);
    ss = fmaf(a, a, ss);
    y[base + c] = from_f32<ACT>(a);
  }
  const float rstd = 1.0f / sqrtf(arn_block_sum(ss, red) / (float)d + eps);
  for (int64_t c = threadIdx.x; c < d; c += ARN_THREADS)
    out[base + c] = from_f32<ACT>(to_f32<ACT>(y[base + c]) * rstd * to_f32<ACT>(gamma[c]));
}

}  // namespace

hipError_t launch_add_rmsnorm(const void* x, const void* residual, const void* gamma, int64_t rows,
                              int64_t d, bool bf16, float eps, void* y, void* norm_out, hipStream_t s) {
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* rp = static_cast<const uint16_t*>(residual);
  const auto* gp = static_cast<const uint16_t*>(gamma);
  auto* yp = static_cast<uint16_t*>(y);
  auto* op = static_cast<uint16_t*>(norm_out);
  // one workgroup per row, rows in chunks of kRowChunk (launch limit)
  for (int64_t r0 = 0; r0 < rows; r0 += kRowChunk) {
    const int64_t nr = rows - r0 < kRowChunk ? rows - r0 : kRowChunk;
    const int64_t o = r0 * d;
    const dim3 grid((unsigned)nr);
    if (d % 8 == 0) {
      if (bf16) add_rmsnorm_vec<ACT_BF16><<<grid, ARN_THREADS, 0, s>>>(xp + o, rp + o, gp, yp + o, op + o, d, eps);
      else add_rmsnorm_vec<ACT_F16><<<grid, ARN_THREADS, 0, s>>>(xp + o, rp + o, gp, yp + o, op + o, d, eps);
    } else {
      if (bf16) add_rmsnorm_elem<ACT_BF16><<<grid, ARN_THREADS, 0, s>>>(xp + o, rp + o, gp, yp + o, op + o, d, eps);
      else add_rmsnorm_elem<ACT_F16><<<grid, ARN_THREADS, 0, s>>>(xp + o, rp + o, gp, yp + o, op + o, d, eps);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
