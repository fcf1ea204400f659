// INT8 quantized matmul with in-place add: the aclnnQuantBatchMatmulInplaceAdd
// page's Formula read for INT8 operands with one K group, a per-token scale for
// x1 (DynamicQuant's per-token output) and a per-channel scale for x2:
//   y[m,n] = (sum_k x1[m,k] * x2[n,k]) * (scale1[m] * scale2[n]) + y[m,n]
// x1 is (M, K) row-major, x2 is stored (N, K) (each output column's K values
// contiguous), both int8; the sums are exact int32 (v_mfma_i32_16x16x64_i8)
// and the float part is rounded step by step in float32:
// s = fl(scale1 * scale2), t = fl(fl(acc) * s), y = fl(y + t).
//
// Tile: 256 (m) x 256 (n) per workgroup of 8 waves, each wave 64 x 128 (4 x 8
// MFMA tiles), two waves per SIMD. Per 128-deep K step the workgroup moves
// 32 KiB of x1 and 32 KiB of x2 into LDS by buffer->LDS DMA, double-buffered;
// both operands are K-contiguous rows, so every MFMA operand is one 16-byte
// LDS read and nothing is unpacked. The accumulators need no VALU work inside
// the K loop and live wherever the compiler puts them.
#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int I8_BM = 256, I8_BN = 256, I8_BK = 128;
constexpr int I8_SLAB = 256 * I8_BK;   // one operand's LDS stage: 32 KiB

// LDS rows are 128 bytes (one K step of one row / column), 16-byte chunks.
// Chunk c of row r sits at position c ^ ((r >> 1) & 7): two rows share a
// 256-byte bank row, so the 16 rows of one MFMA operand read (one chunk) land
// in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int i8_pos(int r, int c) { return c ^ ((r >> 1) & 7); }

// One operand stage (256 rows x 128 K bytes) by 32 DMA instructions of 1 KiB
// (8 rows); wave w issues 4w + j, lane l fills row 8 (4w + j) + l / 8 at
// position l % 8, fetching logical chunk (l % 8) ^ ((row >> 1) & 7). Rows
// past `rows` and chunks past k read zeros (offset BUF_OOB): they add nothing.
__device__ __forceinline__ void i8_dma(__amdgpu_buffer_rsrc_t rs, int rows, int64_t k, int64_t k0,
                                       uint8_t* buf) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 8 * (4 * wave + j) + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    const int64_t kk = k0 + 16 * c;
    const uint32_t off = row < rows && kk < k ? (uint32_t)(row * k + kk) : BUF_OOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(buf + (4 * wave + j) * 1024), 16, off, 0, 0, 0);
  }
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(512, 1) void i8_gemm_tile(const int8_t* __restrict__ x1,
                                                       const int8_t* __restrict__ x2t,
                                                       const float* __restrict__ s1,
                                                       const float* __restrict__ s2,
                                                       float* __restrict__ y, int64_t M, int64_t K,
                                                       int64_t N, int64_t tiles_m, int64_t tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t a0[I8_SLAB], a1[I8_SLAB];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[I8_SLAB], b1[I8_SLAB];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave & 3, wn = wave >> 2;       // 64-row and 128-column blocks of the tile

  // XCD-major tile order: workgroup b runs on XCD b % 8; each XCD gets a
  // contiguous run of tiles, so tiles sharing x1 rows share an L2
  int64_t id = blockIdx.x;
  const int64_t T = tiles_m * tiles_n;
  if ((T & 7) == 0) id = (id & 7) * (T >> 3) + (id >> 3);
  const int64_t m0 = (int64_t)__builtin_amdgcn_readfirstlane((int)(id / tiles_n)) * I8_BM;
  const int64_t n0 = (int64_t)__builtin_amdgcn_readfirstlane((int)(id % tiles_n)) * I8_BN;
  const int rows_a = (int)(M - m0 < I8_BM ? M - m0 : I8_BM);
  const int rows_b = (int)(N - n0 < I8_BN ? N - n0 : I8_BN);
  // tile-relative offsets stay below 2^31: 256 rows of at most 65535 bytes
  const __amdgpu_buffer_rsrc_t ra = buf_rsrc(x1 + m0 * K, (uint32_t)(rows_a * K));
  const __amdgpu_buffer_rsrc_t rb = buf_rsrc(x2t + n0 * K, (uint32_t)(rows_b * K));
  const int steps = (int)((K + I8_BK - 1) / I8_BK);

  i32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = (i32x4){0, 0, 0, 0};

  i8_dma(ra, rows_a, K, 0, a0);
  i8_dma(rb, rows_b, K, 0, b0);
  wait_vm<0>();
  __syncthreads();

  // lane roles of the 16x16x64 MFMA: operand row / column l % 16, lane group
  // g = l / 16 takes 16 K bytes; substep h of a step covers K 64h .. 64h + 63,
  // so group g reads logical chunk 4h + g of its row. A and B use the same
  // assignment, so every K index of the step is multiplied exactly once.
  const int g = lane >> 4, r16 = lane & 15;
  auto step = [&](int s, const uint8_t* acur, uint8_t* anxt, const uint8_t* bcur, uint8_t* bnxt) {
    if (s + 1 < steps) {
      i8_dma(ra, rows_a, K, (int64_t)(s + 1) * I8_BK, anxt);
      i8_dma(rb, rows_b, K, (int64_t)(s + 1) * I8_BK, bnxt);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      i32x4 av[4], bv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 64 * wm + 16 * i + r16;
        av[i] = *reinterpret_cast<const i32x4*>(acur + r * I8_BK + 16 * i8_pos(r, 4 * h + g));
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 128 * wn + 16 * j + r16;
        bv[j] = *reinterpret_cast<const i32x4*>(bcur + r * I8_BK + 16 * i8_pos(r, 4 * h + g));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    wait_vm<0>();            // this wave's DMA into the next buffers has landed
    __syncthreads();
  };
  for (int s = 0; s < steps; s += 2) {
    step(s, a0, a1, b0, b1);
    if (s + 1 < steps) step(s + 1, a1, a0, b1, b0);
  }

  // epilogue: lane holds rows 4 g + r (r = 0..3) of column r16 in each 16x16
  // tile; y, the row scales and the column scales through buffer resources
  // (rows / columns past M / N read zeros and are not stored). Each float
  // step rounds on its own (the file is built without multiply-add contraction).
  // y element (row, c) of the tile sits at (row * N + c) past the tile origin
  const __amdgpu_buffer_rsrc_t ry = buf_rsrc(y + m0 * N + n0, (uint32_t)(((rows_a - 1) * N + rows_b) * 4));
  const __amdgpu_buffer_rsrc_t rs1 = buf_rsrc(s1 + m0, (uint32_t)(rows_a * 4));
  const __amdgpu_buffer_rsrc_t rs2 = buf_rsrc(s2 + n0, (uint32_t)(rows_b * 4));
  float sc2[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = 128 * wn + 16 * j + r16;
    sc2[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs2, c < rows_b ? (uint32_t)(c * 4) : BUF_OOB, 0, 0));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float sc1[4], yv[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 64 * wm + 16 * i + 4 * g + r;
      sc1[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs1, row < rows_a ? (uint32_t)(row * 4) : BUF_OOB, 0, 0));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = 128 * wn + 16 * j + r16;
        const bool ok = row < rows_a && c < rows_b;
        yv[r][j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            ry, ok ? (uint32_t)((row * N + c) * 4) : BUF_OOB, 0, 0));
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 64 * wm + 16 * i + 4 * g + r;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = 128 * wn + 16 * j + r16;
        const bool ok = row < rows_a && c < rows_b;
        const float sc = __fmul_rn(sc1[r], sc2[j]);
        const float t = __fmul_rn((float)acc[i][j][r], sc);
        const float out = __fadd_rn(yv[r][j], t);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out), ry, ok ? (uint32_t)((row * N + c) * 4) : BUF_OOB, 0, 0);
      }
    }
  }
}

}  // namespace

hipError_t launch_i8_matmul(const I8Problem& p, hipStream_t s) {
  const int64_t tm = (p.m + I8_BM - 1) / I8_BM, tn = (p.n + I8_BN - 1) / I8_BN;
  prof_begin(s);
  i8_gemm_tile<<<dim3((unsigned)(tm * tn)), 512, 0, s>>>(p.x1, p.x2t, p.s1, p.s2, p.y, p.m, p.k, p.n,
                                                         tm, tn);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace wq
