// MXFP4 x MXFP4 quantized matmul with in-place add: the
// aclnnQuantBatchMatmulInplaceAdd page's Formula (mx quantization) with both
// operands E2M1:
//   y[m,n] += sum_j (sum_{k in 32-slice j} x1[m,k] x2[k,n]) * scale1[m,j] * scale2[j,n]
// x1: E2M1 codes stored (M, K), two per byte along K, even k in the low
// nibble (the block-32 dynamic quant's E2M1 output); x2: E2M1 codes in the
// GFX950_B layout; scales: E8M0 codes, scale1 (M, ceil(K/32)), scale2
// (ceil(K/32), N); y: fp32 (M, N).
//
// gfx950's scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4 with both formats
// E2M1 runs at the FP4 rate. Lane l supplies row (column) l % 16 and the 32
// K values of 32-slice l / 16 as 16 bytes, low nibble first, for A and for B
// alike, plus one E8M0 scale byte for that (row, slice) / (slice, column),
// picked out of a 32-bit register by the instruction's byte select.
//
// Tile: 256 (m) x 256 (n) per workgroup of 8 waves, each wave 64 x 128 (4 x 8
// MFMA tiles), two waves per SIMD. K advances 128 values (64 bytes of a row,
// one GFX950_B column record) per step. A step's x1 rows, weight records and
// scales move by buffer->LDS DMA into a ring of four stages, issued about two
// and a half steps ahead, one DMA instruction per MFMA slot. In LDS a 64-byte
// row keeps 16-byte chunk c at position c ^ ((row >> 1) & 3), the INT8
// tile's swizzle (the fastest of those timed for these reads). The
// accumulators start as y, so the in-place add needs no extra pass over y.
//
// Scales: a pre-pass writes them in the order the lanes use them (the byte
// select is one immediate for all lanes): per (m tile, step), one dword per
// (row block wm, lane) holding the scale bytes of row blocks i = 0..3 of the
// lane's row and slice; per (n tile, step), one dword per (column block wn,
// half h, lane) holding those of column blocks 4h .. 4h + 3. Rows, columns
// and slices past the matrix get code 127 (1.0: their data is zero).
#include <type_traits>

#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int F4_BM = 256, F4_BN = 256, F4_BK = 128;   // K values per step
constexpr int F4_ROW = F4_BK / 2;                       // bytes per row per step
constexpr int F4_OPS = 256 * F4_ROW;                    // one operand's stage: 16 KiB
constexpr int F4_SC = 2048;                             // a stage's scale dwords

__device__ __forceinline__ int f4_pos(int r, int c) { return c ^ ((r >> 1) & 3); }

__global__ __launch_bounds__(256) void mx4_scale_prep(const uint8_t* __restrict__ s1,
                                                      const uint8_t* __restrict__ s2,
                                                      uint32_t* __restrict__ sa,
                                                      uint32_t* __restrict__ sb, int64_t M,
                                                      int64_t N, int64_t KB, int64_t steps,
                                                      int64_t tiles_m) {
  const int t = threadIdx.x, lane = t & 63, r16 = lane & 15, g = lane >> 4;
  int64_t blk = blockIdx.x;
  uint32_t word = 0;
  if (blk < tiles_m * steps) {
    // (m tile, step): thread t = (wm, lane)
    const int64_t tm = blk / steps, s = blk % steps, kb = 4 * s + g;
    const int wm = t >> 6;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = tm * F4_BM + 64 * wm + 16 * i + r16;
      const uint32_t c = row < M && kb < KB ? s1[row * KB + kb] : 127u;
      word |= c << (8 * i);
    }
    sa[blk * 256 + t] = word;
  } else {
    // (n tile, step): thread t = (wn, h, lane)
    blk -= tiles_m * steps;
    const int64_t tn = blk / steps, s = blk % steps, kb = 4 * s + g;
    const int wn = t >> 7, h = (t >> 6) & 1;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int64_t col = tn * F4_BN + 128 * wn + 16 * (4 * h + jj) + r16;
      const uint32_t c = col < N && kb < KB ? s2[kb * N + col] : 127u;
      word |= c << (8 * jj);
    }
    sb[blk * 256 + t] = word;
  }
}

// Per-lane DMA addressing of one operand stage: 256 rows x 64 bytes by 16
// DMA instructions of 1 KiB (16 rows); wave w issues 2w + j, lane l fills
// row 16 (2w + j) + l / 4 at position l % 4, fetching logical chunk
// (l % 4) ^ ((row >> 1) & 3). `base` is the byte offset of that chunk at step
// 0 (BUF_OOB for rows past the operand), `lim` bounds the step offset.
struct F4Dma {
  uint32_t base[2];
  int lim[2];
};

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>) in order:
// the MFMA's byte selects must be constants.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// acc[I][J] += A block I x B block J over one 128-deep step; the scale bytes
// of row block I and column block J sit in byte I of sa and byte J % 4 of
// sb[J / 4].
template <int I, int J>
__device__ __forceinline__ void mx4_mfma(f32x4 (&acc)[4][8], const i32x4 (&a)[4], const i32x4 (&b)[8],
                                         int sa, const int (&sb)[2]) {
  const i32x8 a8 = {a[I].x, a[I].y, a[I].z, a[I].w, 0, 0, 0, 0};
  const i32x8 b8 = {b[J].x, b[J].y, b[J].z, b[J].w, 0, 0, 0, 0};
  acc[I][J] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[I][J], 4 /*A: E2M1*/,
                                                               4 /*B: E2M1*/, I, sa, J & 3, sb[J >> 2]);
}

__device__ __forceinline__ void f4_dma(__amdgpu_buffer_rsrc_t rs, const F4Dma& d, int j,
                                       uint32_t step_off, int k0, uint8_t* buf) {
  const uint32_t off = k0 < d.lim[j] ? d.base[j] + step_off : BUF_OOB;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(buf + (2 * wave_id() + j) * 1024), 16, off, 0, 0, 0);
}

// A workgroup barrier ordering LDS accesses only: the buffer->LDS DMA of
// later stages stays in flight across it (each wave has waited for its own).
__device__ __forceinline__ void f4_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(512, 1) void mx4_gemm_tile(const uint8_t* __restrict__ x1,
                                                        const uint8_t* __restrict__ x2,
                                                        const uint32_t* __restrict__ sa,
                                                        const uint32_t* __restrict__ sb,
                                                        float* __restrict__ y, int64_t M, int64_t K,
                                                        int64_t N, int64_t Np, int64_t tiles_m,
                                                        int64_t tiles_n, int64_t steps_real) {
  __shared__ __attribute__((aligned(1024))) uint8_t a0[F4_OPS], a1[F4_OPS], a2[F4_OPS], a3[F4_OPS];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[F4_OPS], b1[F4_OPS], b2[F4_OPS], b3[F4_OPS];
  __shared__ __attribute__((aligned(256))) uint8_t c0[F4_SC], c1[F4_SC], c2[F4_SC], c3[F4_SC];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave & 3, wn = wave >> 2;

  // XCD-major tile order: workgroup b runs on XCD b % 8; each XCD gets a
  // contiguous run of tiles, so tiles sharing x1 rows share an L2
  int64_t id = blockIdx.x;
  const int64_t T = tiles_m * tiles_n;
  if ((T & 7) == 0) id = (id & 7) * (T >> 3) + (id >> 3);
  const int64_t tm = __builtin_amdgcn_readfirstlane((int)(id / tiles_n));
  const int64_t tn = __builtin_amdgcn_readfirstlane((int)(id % tiles_n));
  const int64_t m0 = tm * F4_BM, n0 = tn * F4_BN;
  const int rows_a = (int)(M - m0 < F4_BM ? M - m0 : F4_BM);
  const int64_t kbytes = K / 2;                          // x1 row bytes
  // steps rounded up to the ring length; steps past K read zero stages
  const int steps = (int)((steps_real + 3) / 4) * 4;

  // x1 rows of the tile: chunk c of row r at r * kbytes + 16 c + 64 s
  const __amdgpu_buffer_rsrc_t ra = buf_rsrc(x1 + m0 * kbytes, (uint32_t)(rows_a * kbytes));
  // the whole weight: column record (n0 + r) of step s at (s * Np + n0 + r) * 64
  const __amdgpu_buffer_rsrc_t rb = buf_rsrc(x2, (uint32_t)(steps_real * Np * 64));
  // the pre-arranged scales of this tile's rows and columns
  const __amdgpu_buffer_rsrc_t rsa = buf_rsrc(sa + tm * steps_real * 256, (uint32_t)(steps_real * 1024));
  const __amdgpu_buffer_rsrc_t rsb = buf_rsrc(sb + tn * steps_real * 256, (uint32_t)(steps_real * 1024));
  F4Dma da, db;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 16 * (2 * wave + j) + (lane >> 2);
    const int c = f4_pos(row, lane & 3);
    da.base[j] = row < rows_a ? (uint32_t)(row * kbytes + 16 * c) : BUF_OOB;
    da.lim[j] = (int)kbytes - 16 * c;                    // chunk inside the row: step bytes < lim
    db.base[j] = n0 + row < Np ? (uint32_t)((n0 + row) * 64 + 16 * c) : BUF_OOB;
    db.lim[j] = (int)(steps_real * 64);                  // real steps only
  }
  // scale piece of this wave: waves 0..3 the row dwords of block wm, waves
  // 4..7 the column dwords of (wn, h) = ((w - 4) / 2, (w - 4) % 2)
  const __amdgpu_buffer_rsrc_t rsc = wave < 4 ? rsa : rsb;
  const uint32_t sc_lane = (uint32_t)((wave & 3) * 256 + lane * 4);
  auto dma_stage_part = [&](int part, int s, uint8_t* ab, uint8_t* bb, uint8_t* cb) {
    const int k0 = s * F4_ROW;                          // step offset in a row, bytes
    if (part < 2) {
      f4_dma(ra, da, part, (uint32_t)k0, k0, ab);
    } else if (part < 4) {
      f4_dma(rb, db, part - 2, (uint32_t)(s * Np * 64), k0, bb);
    } else {
      const uint32_t off = s < steps_real ? sc_lane + (uint32_t)(s * 1024) : BUF_OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, (lds_void*)(cb + wave * 256), 4, off, 0, 0, 0);
    }
  };

  // accumulators start as y (the in-place add): lane holds rows 4 g + r of
  // column l % 16 in each 16 x 16 tile
  const int g = lane >> 4, r16 = lane & 15;
  const int rows_b = (int)(N - n0 < F4_BN ? N - n0 : F4_BN);
  const __amdgpu_buffer_rsrc_t ry = buf_rsrc(y + m0 * N + n0, (uint32_t)(((rows_a - 1) * N + rows_b) * 4));
  auto y_off = [&](int i, int j, int r) -> uint32_t {
    const int row = 64 * wm + 16 * i + 4 * g + r, col = 128 * wn + 16 * j + r16;
    return row < rows_a && col < rows_b ? (uint32_t)((row * N + col) * 4) : BUF_OOB;
  };
  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[i][j][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ry, y_off(i, j, r), 0, 0));

  const int lds_off = r16 * F4_ROW + 16 * f4_pos(r16, g);
  // operand t of a step: t = 0 is A block 0, 1..8 B blocks 0..7, 9..11 A
  // blocks 1..3, 12 the row scales, 13..14 the column scales
  auto read_op = [&](int t, const uint8_t* ab, const uint8_t* bb, const uint8_t* cb, i32x4 (&av)[4],
                     i32x4 (&bv)[8], int& sav, int (&sbv)[2]) {
    if (t == 0 || (t >= 9 && t < 12)) {
      const int i = t == 0 ? 0 : t - 8;
      av[i] = *reinterpret_cast<const i32x4*>(ab + (64 * wm + 16 * i) * F4_ROW + lds_off);
    } else if (t < 9) {
      const int j = t - 1;
      bv[j] = *reinterpret_cast<const i32x4*>(bb + (128 * wn + 16 * j) * F4_ROW + lds_off);
    } else if (t == 12) {
      sav = *reinterpret_cast<const int*>(cb + wm * 256 + lane * 4);
    } else {
      sbv[t - 13] = *reinterpret_cast<const int*>(cb + 1024 + (2 * wn + (t - 13)) * 256 + lane * 4);
    }
  };

  // prologue: stages 0..2 in flight (five instructions each), stage 0 landed
  // everywhere, its operands and scales in registers
#pragma unroll
  for (int st = 0; st < 3; ++st) {
    uint8_t* ab = st == 0 ? a0 : st == 1 ? a1 : a2;
    uint8_t* bb = st == 0 ? b0 : st == 1 ? b1 : b2;
    uint8_t* cb = st == 0 ? c0 : st == 1 ? c1 : c2;
#pragma unroll
    for (int part = 0; part < 5; ++part) dma_stage_part(part, st, ab, bb, cb);
  }
  wait_vm<10>();                     // this wave's stage 0 (in-order completion)
  f4_barrier();
  i32x4 pa[4], pb[8], qa[4], qb[8];
  int psa, psb[2], qsa, qsb[2];
#pragma unroll
  for (int t = 0; t < 15; ++t) read_op(t, a0, b0, c0, pa, pb, psa, psb);

  // step s (the INT8 tile's schedule): the first 16 MFMAs carry the five
  // DMA instructions of stage s + 3 (its buffers were last read before the
  // previous barrier); wait for this wave's stage s + 1 (stages s + 1 .. s + 3
  // in flight, five instructions each, completing in order); the barrier
  // makes stage s + 1 visible; the last 16 MFMAs carry the fifteen reads of
  // stage s + 1's operands and scales.
  auto step = [&](int s, uint8_t* adma, uint8_t* bdma, uint8_t* cdma, const uint8_t* anxt,
                  const uint8_t* bnxt, const uint8_t* cnxt, const i32x4 (&ca)[4], const i32x4 (&cb)[8],
                  const int csa, const int (&csb)[2], i32x4 (&na)[4], i32x4 (&nb)[8], int& nsa,
                  int (&nsb)[2]) {
    static_for<16>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      mx4_mfma<(t >> 3), (t & 7)>(acc, ca, cb, csa, csb);
      if (t == 1) dma_stage_part(0, s + 3, adma, bdma, cdma);
      if (t == 3) dma_stage_part(2, s + 3, adma, bdma, cdma);
      if (t == 5) dma_stage_part(1, s + 3, adma, bdma, cdma);
      if (t == 7) dma_stage_part(3, s + 3, adma, bdma, cdma);
      if (t == 9) dma_stage_part(4, s + 3, adma, bdma, cdma);
      __builtin_amdgcn_sched_barrier(0);
    });
    wait_vm<10>();
    f4_barrier();
    static_for<16>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      mx4_mfma<(2 + (t >> 3)), (t & 7)>(acc, ca, cb, csa, csb);
      if (t < 15) read_op(t, anxt, bnxt, cnxt, na, nb, nsa, nsb);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  for (int s = 0; s < steps; s += 4) {
    step(s, a3, b3, c3, a1, b1, c1, pa, pb, psa, psb, qa, qb, qsa, qsb);
    step(s + 1, a0, b0, c0, a2, b2, c2, qa, qb, qsa, qsb, pa, pb, psa, psb);
    step(s + 2, a1, b1, c1, a3, b3, c3, pa, pb, psa, psb, qa, qb, qsa, qsb);
    step(s + 3, a2, b2, c2, a0, b0, c0, qa, qb, qsa, qsb, pa, pb, psa, psb);
  }
  wait_vm<0>();                      // the DMA of the stages past the end

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), ry, y_off(i, j, r), 0, 0);
}

}  // namespace

// Rows run in chunks of kRowChunk (the launch limit), so the workspace covers
// one chunk.
size_t mx4_workspace_bytes(int64_t m, int64_t k, int64_t n) {
  if (m > kRowChunk) m = kRowChunk;
  const int64_t steps = (k + F4_BK - 1) / F4_BK;
  return (size_t)(((m + F4_BM - 1) / F4_BM + (n + F4_BN - 1) / F4_BN) * steps * 1024);
}

hipError_t launch_mx4_matmul(const Mx4Problem& p, hipStream_t s) {
  const int64_t steps = (p.k + F4_BK - 1) / F4_BK, kb = (p.k + 31) / 32;
  const int64_t np = 16 * ((p.n + 15) / 16);
  for (int64_t r0 = 0; r0 < p.m; r0 += kRowChunk) {
    const int64_t m = p.m - r0 < kRowChunk ? p.m - r0 : kRowChunk;
    const int64_t tm = (m + F4_BM - 1) / F4_BM, tn = (p.n + F4_BN - 1) / F4_BN;
    uint32_t* sa = static_cast<uint32_t*>(p.workspace);
    uint32_t* sb = sa + tm * steps * 256;
    mx4_scale_prep<<<dim3((unsigned)((tm + tn) * steps)), 256, 0, s>>>(p.s1 + r0 * kb, p.s2, sa, sb, m, p.n,
                                                                       kb, steps, tm);
    prof_begin(s);
    mx4_gemm_tile<<<dim3((unsigned)(tm * tn)), 512, 0, s>>>(p.x1 + r0 * (p.k / 2), p.x2, sa, sb,
                                                            p.y + r0 * p.n, m, p.k, p.n, np, tm, tn, steps);
    prof_end(s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
