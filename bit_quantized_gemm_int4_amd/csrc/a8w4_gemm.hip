// INT8 (or INT4) x INT4 quantized matmul with in-place add: the
// aclnnQuantBatchMatmulInplaceAdd page's Formula read for an INT8 x1 (the
// per-token output of the aclnnDynamicQuant page) and an INT4 weight packed by
// the aclnnConvertWeightToINT4Pack page's operator, with one K group, a
// per-token scale for x1 and a per-channel scale for x2:
//   y[m,n] = (sum_k x1[m,k] * q[k,n]) * (scale1[m] * scale2[n]) + y[m,n]
// x1 is (M, K) int8 row-major; the codes q in [-8, 7] come in the GFX950_B
// layout. The sums are exact int32 and the float part is rounded step by
// step in float32: s = fl(scale1 * scale2), t = fl(fl(acc) * s), y = fl(y + t).
//
// The weight enters the 8-bit MFMA (v_mfma_i32_16x16x64_i8) as 16 * q: a
// code moved to the high nibble of its byte is that signed byte exactly, so
// the unpack is a byte permute and a mask per four codes, with no sign
// extension and no row-sum correction. The accumulator holds 16 * sum, which
// stays inside int32 (16 * 65535 * 128 * 8 < 2^31); an arithmetic shift by 4
// recovers the exact sum.
//
// Tile: 256 (m) x 256 (n) per workgroup of 8 waves, each wave 128 x 64 (8 x 4
// MFMA tiles), two waves per SIMD: an unpacked weight fragment feeds eight
// MFMAs. K advances 64 values per step through the INT8 tile's ring of four
// stages (i8_ring.h): 16 KiB of x1 rows and 8 KiB of weight (the 32 bytes of
// each column's GFX950_B record that hold the step's 64 codes), three DMA
// instructions per wave per stage, issued about two and a half steps ahead.
// The A4 variant takes INT4 activations (see the kernel's comment): its x1
// stage is 8 KiB, two DMA instructions per wave per stage.
#include "i8_ring.h"
#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int W4_BM = 256, W4_BN = 256;
constexpr int W4_BSTAGE = 256 * 32;      // weight stage: 256 columns x 32 bytes

// Four int4 codes (two packed bytes: b0 = codes 0, 1; b1 = codes 2, 3, even
// code in the low nibble) -> four int8 bytes 16 * q in code order. w4 = w << 4
// puts the even codes in the high nibbles; the permute picks byte 0 of w4,
// byte 0 of w, byte 1 of w4, byte 1 of w (selector 0x01050004; 0x03070206
// for bytes 2 and 3), and the mask clears the other codes' bits.
__device__ __forceinline__ void w4_unpack(uint2 raw, i32x4& out) {
  const uint32_t w0 = raw.x, w1 = raw.y;
  const uint32_t s0 = w0 << 4, s1 = w1 << 4;
  out[0] = (int)(__builtin_amdgcn_perm(s0, w0, 0x01050004u) & 0xF0F0F0F0u);
  out[1] = (int)(__builtin_amdgcn_perm(s0, w0, 0x03070206u) & 0xF0F0F0F0u);
  out[2] = (int)(__builtin_amdgcn_perm(s1, w1, 0x01050004u) & 0xF0F0F0F0u);
  out[3] = (int)(__builtin_amdgcn_perm(s1, w1, 0x03070206u) & 0xF0F0F0F0u);
}

// A4: x1 holds INT4 codes (M, K/2) bytes (the per-token quant's INT4 output,
// even k in the low nibble) and enters the MFMA as 16 * a too: the
// accumulator holds 256 * sum (256 * 65504 * 8 * 8 < 2^31), shifted back by 8.
template <bool A4>
__global__ __launch_bounds__(512, 1) void a8w4_gemm_tile(const uint8_t* __restrict__ x1,
                                                         const uint8_t* __restrict__ x2,
                                                         const float* __restrict__ s1,
                                                         const float* __restrict__ s2,
                                                         float* __restrict__ y, int64_t M, int64_t K,
                                                         int64_t N, int64_t Np, uint32_t x2_bytes,
                                                         int64_t tiles_m, int64_t tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t a0[I8_STAGE], a1[I8_STAGE], a2[I8_STAGE], a3[I8_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[W4_BSTAGE], b1[W4_BSTAGE], b2[W4_BSTAGE], b3[W4_BSTAGE];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave & 1, wn = wave >> 1;       // 128-row and 64-column blocks of the tile

  // XCD-major tile order, as in the INT8 tile
  int64_t id = blockIdx.x;
  const int64_t T = tiles_m * tiles_n;
  if ((T & 7) == 0) id = (id & 7) * (T >> 3) + (id >> 3);
  const int64_t m0 = (int64_t)__builtin_amdgcn_readfirstlane((int)(id / tiles_n)) * W4_BM;
  const int64_t n0 = (int64_t)__builtin_amdgcn_readfirstlane((int)(id % tiles_n)) * W4_BN;
  const int rows_a = (int)(M - m0 < W4_BM ? M - m0 : W4_BM);
  const int cols_b = (int)(N - n0 < W4_BN ? N - n0 : W4_BN);
  // x1: INT8 rows through the INT8 ring's addressing; INT4 rows (K / 2 bytes)
  // like the weight, one instruction per wave and stage: lane l fills row
  // 32 w + l / 2, bytes 16 (l % 2) of the step's 32
  const int64_t arow_bytes = A4 ? K / 2 : K;
  const __amdgpu_buffer_rsrc_t ra = buf_rsrc(x1 + m0 * arow_bytes, (uint32_t)(rows_a * arow_bytes));
  const I8Dma da = i8_dma_setup(rows_a, K);
  const int arow4 = 32 * wave + (lane >> 1);
  const uint32_t abase4 = (uint32_t)(arow4 * arow_bytes + 16 * (lane & 1));
  auto dma_a = [&](int s, uint8_t* buf) {
    if constexpr (A4) {
      const bool ok = arow4 < rows_a && (int64_t)s * 32 + 16 * (lane & 1) < arow_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(buf + wave * 1024), 16,
                                               ok ? abase4 + 32u * (uint32_t)s : BUF_OOB, 0, 0, 0);
    } else {
      i8_dma(ra, da, 0, s * I8_BK, buf);
      i8_dma(ra, da, 1, s * I8_BK, buf);
    }
  };
  // DMA instructions per wave and stage: x1 (2, or 1 for INT4) + weight (1)
  constexpr int DMA_N = A4 ? 2 : 3;
  // weight DMA: one instruction per wave and stage; lane l fills column
  // 32 w + l / 2 (16 bytes, half l % 2) of the stage, from the column's
  // record of 128-block s / 2, bytes 32 (s % 2) + 16 (l % 2). Columns past the
  // padded width and steps past the padded K read zeros.
  const __amdgpu_buffer_rsrc_t rb = buf_rsrc(x2, x2_bytes);
  const int64_t bcol = n0 + 32 * wave + (lane >> 1);
  const bool bcol_ok = bcol < Np;
  const uint32_t bbase = bcol_ok ? (uint32_t)(bcol * 64 + 16 * (lane & 1)) : 0u;
  const int bsteps = (int)(2 * ((K + 127) / 128));          // 64-code steps of the padded K
  const uint32_t kb_stride = (uint32_t)(Np * 64);           // bytes per 128-block of all columns
  auto dma_b = [&](int s, uint8_t* buf) {
    const uint32_t off = (bcol_ok && s < bsteps)
                             ? bbase + (uint32_t)(s >> 1) * kb_stride + 32u * (uint32_t)(s & 1)
                             : BUF_OOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(buf + wave * 1024), 16, off, 0, 0, 0);
  };
  const int steps = (int)((K + 4 * I8_BK - 1) / (4 * I8_BK)) * 4;

  i32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (i32x4){0, 0, 0, 0};

  // lane roles of the 16x16x64 MFMA: row / column l % 16; lane group g = l / 16
  // takes K values 16 g .. 16 g + 15 of the step, for x1 the 16-byte logical
  // chunk g of its row, for the weight bytes 8 g .. 8 g + 7 of its column's
  // 32 (codes 16 g .. 16 g + 15 in order). Byte i of both operands is K 16 g + i.
  const int g = lane >> 4, r16 = lane & 15;
  const int a_off = A4 ? (128 * wm + r16) * 32 + 8 * g : (128 * wm + r16) * I8_BK + 16 * i8_pos(r16, g);
  const int b_off = (64 * wn + r16) * 32 + 8 * g;
  uint2 araw[8];
  auto read_a = [&](int i, const uint8_t* buf, i32x4 (&av)[8]) {
    if constexpr (A4) araw[i] = *reinterpret_cast<const uint2*>(buf + a_off + 16 * i * 32);
    else av[i] = *reinterpret_cast<const i32x4*>(buf + a_off + 16 * i * I8_BK);
  };
  auto read_b = [&](int j, const uint8_t* buf, uint2 (&raw)[4]) {
    raw[j] = *reinterpret_cast<const uint2*>(buf + b_off + 16 * j * 32);
  };
  auto mfma = [&](int i, int j, const i32x4 (&av)[8], const i32x4 (&bv)[4]) {
    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[i], bv[j], acc[i][j], 0, 0, 0);
  };

  // prologue: stages 0..2 in flight; stage 0 landed everywhere; its operands
  // in registers
#pragma unroll
  for (int st = 0; st < 3; ++st) {
    uint8_t* ab = st == 0 ? a0 : st == 1 ? a1 : a2;
    uint8_t* bb = st == 0 ? b0 : st == 1 ? b1 : b2;
    dma_a(st, ab);
    dma_b(st, bb);
  }
  wait_vm<2 * DMA_N>();              // this wave's stage 0 (in-order completion)
  lds_barrier();
  i32x4 pa[8], qa[8], pb[4], qb[4];
  uint2 raw[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) read_a(i, a0, pa);
#pragma unroll
  for (int j = 0; j < 4; ++j) read_b(j, b0, raw);
#pragma unroll
  for (int j = 0; j < 4; ++j) w4_unpack(raw[j], pb[j]);
  if constexpr (A4) {
#pragma unroll
    for (int i = 0; i < 8; ++i) w4_unpack(araw[i], pa[i]);
  }

  // step s: stage s's operands are in registers (ca, cb); stage s + 3's
  // buffers were last read before the previous barrier. The first sixteen
  // MFMAs carry the DMA of stage s + 3 (slots 1, 3, 5); then wait for this
  // wave's DMA of stage s + 1 (stages s + 1 .. s + 3 in flight, three
  // instructions each, completing in order) and meet at the barrier, which
  // makes stage s + 1 visible. The last sixteen carry its reads into the other
  // register set: the four weight fragments (slots 0..3), the eight x1
  // fragments (slots 4..11) and the weight unpacks (odd slots 9..15). Every
  // read of a stage is consumed before the barrier of the step after, and
  // the DMA that reuses its buffer comes after that barrier.
  auto step = [&](int s, uint8_t* adma, uint8_t* bdma, const uint8_t* anxt, const uint8_t* bnxt,
                  const i32x4 (&ca)[8], const i32x4 (&cb)[4], i32x4 (&na)[8], i32x4 (&nb)[4]) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      mfma(t >> 2, t & 3, ca, cb);
      if constexpr (A4) {
        if (t == 1) dma_a(s + 3, adma);
        if (t == 3) dma_b(s + 3, bdma);
      } else {
        if (t == 1) i8_dma(ra, da, 0, (s + 3) * I8_BK, adma);
        if (t == 3) i8_dma(ra, da, 1, (s + 3) * I8_BK, adma);
        if (t == 5) dma_b(s + 3, bdma);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm<2 * DMA_N>();
    lds_barrier();
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      mfma(4 + (t >> 2), t & 3, ca, cb);
      if (t < 4) read_b(t, bnxt, raw);
      else if (t < 12) read_a(t - 4, anxt, na);
      if (t >= 9 && (t & 1)) w4_unpack(raw[(t - 9) >> 1], nb[(t - 9) >> 1]);
      if constexpr (A4) {
        if (t >= 6 && t < 14) w4_unpack(araw[t - 6], na[t - 6]);
      }
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
  // tile; y and the scales through buffer resources (rows / columns past M /
  // N read zeros and are not stored); each float step rounds on its own (no
  // multiply-add contraction in this file)
  const __amdgpu_buffer_rsrc_t ry = buf_rsrc(y + m0 * N + n0, (uint32_t)(((rows_a - 1) * N + cols_b) * 4));
  const __amdgpu_buffer_rsrc_t rs1 = buf_rsrc(s1 + m0, (uint32_t)(rows_a * 4));
  const __amdgpu_buffer_rsrc_t rs2 = buf_rsrc(s2 + n0, (uint32_t)(cols_b * 4));
  float sc2[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = 64 * wn + 16 * j + r16;
    sc2[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs2, c < cols_b ? (uint32_t)(c * 4) : BUF_OOB, 0, 0));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float sc1[4], yv[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 128 * wm + 16 * i + 4 * g + r;
      sc1[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs1, row < rows_a ? (uint32_t)(row * 4) : BUF_OOB, 0, 0));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 64 * wn + 16 * j + r16;
        const bool ok = row < rows_a && c < cols_b;
        yv[r][j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            ry, ok ? (uint32_t)((row * N + c) * 4) : BUF_OOB, 0, 0));
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 128 * wm + 16 * i + 4 * g + r;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 64 * wn + 16 * j + r16;
        const bool ok = row < rows_a && c < cols_b;
        const float sc = __fmul_rn(sc1[r], sc2[j]);
        const float t = __fmul_rn((float)(acc[i][j][r] >> (A4 ? 8 : 4)), sc);
        const float out = __fadd_rn(yv[r][j], t);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out), ry, ok ? (uint32_t)((row * N + c) * 4) : BUF_OOB, 0, 0);
      }
    }
  }
}

}  // namespace

// Rows in chunks of kRowChunk (independent row blocks), so that the grid
// stays within the launch limit for every m the call accepts.
hipError_t launch_a8w4_matmul(const A8W4Problem& p, hipStream_t s) {
  const int64_t np = 16 * ((p.n + 15) / 16);
  const uint32_t x2_bytes = (uint32_t)(((p.k + 127) / 128) * np * 64);
  const int64_t row_bytes = p.x1_int4 ? p.k / 2 : p.k;
  for (int64_t r0 = 0; r0 < p.m; r0 += kRowChunk) {
    const int64_t m = p.m - r0 < kRowChunk ? p.m - r0 : kRowChunk;
    const int64_t tm = (m + W4_BM - 1) / W4_BM, tn = (p.n + W4_BN - 1) / W4_BN;
    const uint8_t* x1 = p.x1 + r0 * row_bytes;
    float* y = p.y + r0 * p.n;
    prof_begin(s);
    if (p.x1_int4)
      a8w4_gemm_tile<true><<<dim3((unsigned)(tm * tn)), 512, 0, s>>>(x1, p.x2, p.s1 + r0, p.s2, y, m, p.k,
                                                                     p.n, np, x2_bytes, tm, tn);
    else
      a8w4_gemm_tile<false><<<dim3((unsigned)(tm * tn)), 512, 0, s>>>(x1, p.x2, p.s1 + r0, p.s2, y, m,
                                                                      p.k, p.n, np, x2_bytes, tm, tn);
    prof_end(s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
