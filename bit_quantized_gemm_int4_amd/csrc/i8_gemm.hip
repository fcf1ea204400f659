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
// MFMA tiles), two waves per SIMD. K advances 64 bytes per step; each step's
// operands (16 KiB of x1 and 16 KiB of x2) come into LDS by buffer->LDS DMA
// into a ring of four stages, issued about two and a half steps ahead so the
// fetch latency hides behind the MFMAs of the steps between. Both operands are K-contiguous rows, so
// every MFMA operand is one 16-byte LDS read and nothing is unpacked; each
// step's operands are read into registers during the second half of the
// previous step's MFMAs.
#include "i8_ring.h"
#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int I8_BM = 256, I8_BN = 256;

__global__ __launch_bounds__(512, 1) void i8_gemm_tile(const int8_t* __restrict__ x1,
                                                       const int8_t* __restrict__ x2t,
                                                       const float* __restrict__ s1,
                                                       const float* __restrict__ s2,
                                                       float* __restrict__ y, int64_t M, int64_t K,
                                                       int64_t N, int64_t tiles_m, int64_t tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t a0[I8_STAGE], a1[I8_STAGE], a2[I8_STAGE], a3[I8_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[I8_STAGE], b1[I8_STAGE], b2[I8_STAGE], b3[I8_STAGE];
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
  const I8Dma da = i8_dma_setup(rows_a, K), db = i8_dma_setup(rows_b, K);
  // steps rounded up to a multiple of the ring length; steps past K read
  // zero stages and add nothing
  const int steps = (int)((K + 4 * I8_BK - 1) / (4 * I8_BK)) * 4;

  i32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = (i32x4){0, 0, 0, 0};

  // lane roles of the 16x16x64 MFMA: operand row / column l % 16, lane group
  // g = l / 16 takes 16 K bytes, logical chunk g of its row. A and B use the
  // same assignment, so every K index of the step is multiplied exactly once.
  // The rows a lane reads differ by multiples of 16, so its chunk position is
  // the same for all of them.
  const int g = lane >> 4, r16 = lane & 15;
  const int lds_off = r16 * I8_BK + 16 * i8_pos(r16, g);
  // operand t of a step: t = 0 is A block 0, 1..8 B blocks 0..7, 9..11 A
  // blocks 1..3 (the order the next step's MFMAs consume them)
  auto read_op = [&](int t, const uint8_t* abuf, const uint8_t* bbuf, i32x4 (&av)[4], i32x4 (&bv)[8]) {
    if (t == 0 || t >= 9) {
      const int i = t == 0 ? 0 : t - 8;
      av[i] = *reinterpret_cast<const i32x4*>(abuf + (64 * wm + 16 * i) * I8_BK + lds_off);
    } else {
      const int j = t - 1;
      bv[j] = *reinterpret_cast<const i32x4*>(bbuf + (128 * wn + 16 * j) * I8_BK + lds_off);
    }
  };
  auto mfma = [&](int i, int j, const i32x4 (&av)[4], const i32x4 (&bv)[8]) {
    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[i], bv[j], acc[i][j], 0, 0, 0);
  };

  // prologue: stages 0..2 in flight; stage 0 landed everywhere; its operands
  // in registers
#pragma unroll
  for (int st = 0; st < 3; ++st) {
    uint8_t* ab = st == 0 ? a0 : st == 1 ? a1 : a2;
    uint8_t* bb = st == 0 ? b0 : st == 1 ? b1 : b2;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      i8_dma(ra, da, j, st * I8_BK, ab);
      i8_dma(rb, db, j, st * I8_BK, bb);
    }
  }
  wait_vm<8>();                      // this wave's stage 0 (in-order completion)
  lds_barrier();
  i32x4 pa[4], pb[8], qa[4], qb[8];
#pragma unroll
  for (int t = 0; t < 12; ++t) read_op(t, a0, b0, pa, pb);

  // step s: the operands of stage s are in registers (cur); stage s + 3's
  // buffers were last read before the previous barrier. The first half of the
  // MFMAs carries the DMA of stage s + 3 (one instruction per slot, so no wave
  // stalls on a full memory queue with MFMAs waiting behind it); then wait for
  // this wave's DMA of stage s + 1 (stages s + 1 .. s + 3 are in flight, four
  // instructions each, completing in order); the barrier makes stage s + 1
  // visible; the second half carries the twelve reads of stage s + 1's
  // operands (nxt). Every slot is fixed by a scheduling barrier.
  auto step = [&](int s, uint8_t* adma, uint8_t* bdma, const uint8_t* anxt, const uint8_t* bnxt,
                  const i32x4 (&ca)[4], const i32x4 (&cb)[8], i32x4 (&na)[4], i32x4 (&nb)[8]) {
    const int kd = (s + 3) * I8_BK;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      mfma(t >> 3, t & 7, ca, cb);
      if (t == 1) i8_dma(ra, da, 0, kd, adma);
      if (t == 3) i8_dma(rb, db, 0, kd, bdma);
      if (t == 5) i8_dma(ra, da, 1, kd, adma);
      if (t == 7) i8_dma(rb, db, 1, kd, bdma);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm<8>();
    lds_barrier();
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      mfma(2 + (t >> 3), t & 7, ca, cb);
      if (t < 12) read_op(t, anxt, bnxt, na, nb);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int s = 0; s < steps; s += 4) {
    step(s, a3, b3, a1, b1, pa, pb, qa, qb);
    step(s + 1, a0, b0, a2, b2, qa, qb, pa, pb);
    step(s + 2, a1, b1, a3, b3, pa, pb, qa, qb);
    step(s + 3, a2, b2, a0, b0, qa, qb, pa, pb);
  }
  wait_vm<0>();                      // the DMA of the stages past the end

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

// Rows in chunks of kRowChunk (independent row blocks), so that the grid
// stays within the launch limit for every m the call accepts.
hipError_t launch_i8_matmul(const I8Problem& p, hipStream_t s) {
  for (int64_t r0 = 0; r0 < p.m; r0 += kRowChunk) {
    const int64_t m = p.m - r0 < kRowChunk ? p.m - r0 : kRowChunk;
    const int64_t tm = (m + I8_BM - 1) / I8_BM, tn = (p.n + I8_BN - 1) / I8_BN;
    prof_begin(s);
    i8_gemm_tile<<<dim3((unsigned)(tm * tn)), 512, 0, s>>>(p.x1 + r0 * p.k, p.x2t, p.s1 + r0, p.s2,
                                                           p.y + r0 * p.n, m, p.k, p.n, tm, tn);
    prof_end(s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
