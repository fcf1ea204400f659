// MX block-32 quantized matmul with in-place add
// (aclnnQuantBatchMatmulInplaceAdd page, Formula, mx quantization):
//   y[m,n] += sum_j (sum_{k in slice j} x1[m,k] x2[k,n]) * scale1[m,j] * scale2[j,n]
// x1: E4M3 codes stored (K, M) (transposeX1); x2: E2M1 codes in the
// GFX950_B layout; scales: E8M0 codes, scale1 (M, K/32), scale2 (K/32, N).
//
// gfx950's scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4 computes a 16x16
// tile over 128 K with one E8M0 scale per (row, 32-block) of A and per
// (column, 32-block) of B: exactly the page's block-scaled sum. Lane l
// supplies row/column l%16 and the scale byte of 32-block l/16. Operand
// order, measured on the device with one-hot and random probes: the B lane
// (E2M1) holds the 32 K values of block l/16 as 16 bytes, low nibble first;
// the A lane (E4M3) holds K 16*(l/16) .. +16 in bytes 0..15 and
// K 64 + 16*(l/16) .. +16 in bytes 16..31.
// Since GFX950_B stores each column's 32-deep block as 16 contiguous bytes,
// a B fragment is one dwordx4 load straight from global memory. A arrives
// K-major, so the workgroup transposes its A tile into LDS ([m][k] bytes).
#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int MX_BM = 64, MX_BN = 64, MX_BK = 128, MX_LDS = MX_BK + 16;

__global__ __launch_bounds__(256) void mx_gemm_kernel(const uint8_t* __restrict__ x1t,
                                                      const uint8_t* __restrict__ x2,
                                                      const uint8_t* __restrict__ s1,
                                                      const uint8_t* __restrict__ s2,
                                                      float* __restrict__ y, int64_t M, int64_t K,
                                                      int64_t N, int64_t Np) {
  __shared__ __attribute__((aligned(16))) uint8_t As[MX_BM][MX_LDS];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * MX_BM;
  const int64_t n0 = (int64_t)blockIdx.x * MX_BN;
  const int64_t KB = (K + 31) / 32;
  f32x4 acc[2][2] = {};

  for (int64_t k0 = 0; k0 < K; k0 += MX_BK) {
    // ---- A tile transpose: thread -> k row t/2, 32 consecutive m ----
    {
      const int kr = t >> 1, mc = (t & 1) * 32;
      const int64_t kk = k0 + kr;
#pragma unroll 4
      for (int i = 0; i < 32; ++i) {
        const int64_t mm = m0 + mc + i;
        As[mc + i][kr] = (kk < K && mm < M) ? x1t[kk * M + mm] : (uint8_t)0;
      }
    }
    __syncthreads();
    const int kbl = lane >> 4;                 // this lane's 32-block in the 128 slab
    const int64_t kb = k0 / 32 + kbl;
    i32x8 af[2], bf[2];
    int sa[2], sb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wr * 32 + i * 16 + (lane & 15);
      const u32x4 lo = *reinterpret_cast<const u32x4*>(&As[r][kbl * 16]);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(&As[r][64 + kbl * 16]);
      af[i] = (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                      (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const int64_t row = m0 + r;
      sa[i] = (row < M && kb < KB) ? (int)s1[row * KB + kb] : 127;
      const int64_t col = n0 + wc * 32 + i * 16 + (lane & 15);
      u32x4 bv = {0, 0, 0, 0};
      if (col < Np) bv = *reinterpret_cast<const u32x4*>(x2 + ((kb / 4) * Np + col) * 64 + (kb % 4) * 16);
      bf[i] = (i32x8){(int)bv.x, (int)bv.y, (int)bv.z, (int)bv.w, 0, 0, 0, 0};
      sb[i] = (col < N && kb < KB) ? (int)s2[kb * N + col] : 127;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            af[i], bf[j], acc[i][j], 0 /*A: E4M3*/, 4 /*B: E2M1*/, 0, sa[i], 0, sb[j]);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wc * 32 + j * 16 + (lane & 15);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wr * 32 + i * 16 + 4 * (lane >> 4) + r;
        if (row < M) y[row * N + col] += acc[i][j][r];
      }
    }
}

}  // namespace

hipError_t launch_mx_matmul(const MxProblem& p, hipStream_t s) {
  const int64_t Np = 16 * ((p.n + 15) / 16);
  dim3 grid((unsigned)((p.n + MX_BN - 1) / MX_BN), (unsigned)((p.m + MX_BM - 1) / MX_BM));
  mx_gemm_kernel<<<grid, 256, 0, s>>>(p.x1, p.x2, p.s1, p.s2, p.y, p.m, p.k, p.n, Np);
  return hipGetLastError();
}

}  // namespace wq
