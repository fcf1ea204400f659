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
// a B fragment is one 16-byte load. A arrives K-major.
//
// Two kernels:
//   - mx_gemm_tile: M, N multiples of 256 and K a multiple of 128 (RG: any
//     M a multiple of 16, N and K, through bounded buffer resources). A
//     256 x 256 workgroup tile, 8 waves of 64 (m) x 128 (n). Per 128-deep
//     step the x1 tile (128 k-rows x 256 m bytes), the weight slab (256
//     columns x 64 bytes) and both scale tiles move by direct global->LDS DMA,
//     double-buffered. A operands come out of LDS with the gfx950 transpose
//     read ds_read_b64_tr_b8: in each group of 16 lanes, lane i receives
//     byte c of the 8 bytes that in-group lane 2b + h fetched, as byte b,
//     where i = 8h + c. Pointing in-group lane j at k-row k0 + j/2, m column
//     m0 + 8 (j%2) therefore hands lane i the 8 consecutive K values of row
//     m0 + i. The x1 rows' 16-byte chunks are XOR-swizzled by k so that the
//     32 rows one such read touches spread over all LDS banks. The
//     accumulators start as y, so the in-place add costs no extra pass.
//   - mx_gemm_kernel: the shapes the tile does not take (M not a multiple of
//     16 without a workspace for a padded x1 copy, offsets past 2 GiB); a
//     small 64 x 64 tile that transposes A byte-wise.
#include <utility>

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
                                                      int64_t N, int64_t Np, int64_t mb, int64_t nb,
                                                      int64_t ne) {
  __shared__ __attribute__((aligned(16))) uint8_t As[MX_BM][MX_LDS];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  // the grid covers rows [mb, M) and columns [nb, ne) of the (M, N) output
  const int64_t m0 = mb + (int64_t)blockIdx.y * MX_BM;
  const int64_t n0 = nb + (int64_t)blockIdx.x * MX_BN;
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
      sb[i] = (col < ne && kb < KB) ? (int)s2[kb * N + col] : 127;
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
      if (col >= ne) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wr * 32 + i * 16 + 4 * (lane >> 4) + r;
        if (row < M) y[row * N + col] += acc[i][j][r];
      }
    }
}


// ---------------------------------------------------------------------------
// Tiled kernel
// ---------------------------------------------------------------------------
constexpr int MF_BM = 256, MF_BN = 256, MF_BK = 128;
constexpr int MF_ABYTES = MF_BK * MF_BM;   // 32 KiB: 128 k-rows x 256 m
constexpr int MF_BBYTES = MF_BN * 64;      // 16 KiB: 256 columns x (128 K / 2)
constexpr int MF_SBYTES = 1024;            // 256 x 4 scale bytes

// physical 16-byte chunk of logical chunk c in k-row r: c ^ swz(r). The 32
// rows of one transpose read, {off + 16 g + u : g < 4, u < 8} with off a
// multiple of 8 below 128, hit each value of (r & 7) | ((r & 16) >> 1) twice.
__device__ __forceinline__ int mf_swz(int r) { return (r & 7) | ((r & 16) >> 1); }

// position of 32-deep block g inside weight record slot jl (mod 16): g ^ mf_bswz(jl)
__device__ __forceinline__ int mf_bswz(int jl) { return (jl >> 1) & 2; }

struct MfBufs {
  uint8_t* a;
  uint8_t* b;
  uint8_t* s1;
  uint8_t* s2;
};

// The tile's global inputs. With RG (a ragged shape: K not a multiple of 128,
// or M, N not multiples of 256) every input goes through a buffer resource
// (a read past the tensor returns zero).
struct MfSrc {
  const uint8_t* x1t;
  const uint8_t* x2;
  const uint8_t* s1;
  const uint8_t* s2;
  __amdgpu_buffer_rsrc_t rx, rw, rs1, rs2;
};

__device__ __forceinline__ void mf_dma16(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void mf_dma4(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, voff, 0, 0, 0);
}

// DMA of one 128-deep step into the given buffers: 7 instructions per wave
// (x1: 4 KiB in four 1 KiB pieces; weights: 2 KiB; one 256-byte scale row).
// With RG, waves 0..3 read their scale1 bytes with byte loads instead (issued
// first, so that their wait does not cover the DMA) and return them packed;
// the caller writes them to LDS before the step's closing barrier. With ON
// (N not a multiple of 4: scale2 rows not 4-byte aligned) waves 4..7 do the
// same for their scale2 bytes.
template <bool RG, bool ON>
__device__ __forceinline__ uint32_t mf_dma(const MfSrc& src, const MfBufs& bf, int64_t Mx, int64_t N,
                                           int64_t Np, int64_t KB, int64_t m0, int64_t n0, int step,
                                           int wave, int lane) {
  const int64_t k0 = (int64_t)step * MF_BK;
  uint32_t s1w = 0;
  if constexpr (RG) {
    if (wave < 4) {
      const int64_t row = m0 + 64 * wave + lane;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t blk = 4 * (int64_t)step + b;
        const uint32_t off = blk < KB ? (uint32_t)(row * KB + blk) : BUF_OOB;
        s1w |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(src.rs1, off, 0, 0) << (8 * b);
      }
    } else if (ON) {
      const int64_t blk = 4 * (int64_t)step + (wave - 4);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t col = n0 + 4 * lane + b;
        const uint32_t off = blk < KB && col < N ? (uint32_t)(blk * N + col) : BUF_OOB;
        s1w |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(src.rs2, off, 0, 0) << (8 * b);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = 4 * wave + i;                 // k-rows 4q .. 4q + 3
    const int r = 4 * q + (lane >> 4);
    const int c = (lane & 15) ^ mf_swz(r);      // logical chunk for this physical slot
    if constexpr (RG)
      mf_dma16(src.rx, bf.a + q * 1024, (uint32_t)((k0 + r) * Mx + m0 + 16 * c));
    else
      __builtin_amdgcn_global_load_lds((glb_void*)(src.x1t + (k0 + r) * Mx + m0 + 16 * c),
                                       (lds_void*)(bf.a + q * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    // 64-byte record slot sl = 128 wn + 16 j + jl holds the tile's column
    // 128 wn + 8 jl + j, so that a lane's eight columns (j = 0..7) are
    // consecutive: their scales are one 8-byte read and their y one 32-byte run.
    // Inside slot jl (mod 16) the 16-byte 32-deep blocks sit at position
    // g ^ mf_bswz(jl): the fragment reads then take no bank-conflict cycles
    // (unswizzled: 4 per read; picked with the SQ_LDS_BANK_CONFLICT counter
    // of an LDS probe of these reads). Four lanes still fetch one record.
    const int q = 2 * wave + i;
    const int sl = 16 * q + (lane >> 2);
    const int col = (sl & 128) + 8 * (sl & 15) + ((sl >> 4) & 7);
    const int blk = (lane & 3) ^ mf_bswz(lane >> 2);
    if constexpr (RG)
      mf_dma16(src.rw, bf.b + q * 1024, (uint32_t)(((int64_t)step * Np + n0 + col) * 64 + 16 * blk));
    else
      __builtin_amdgcn_global_load_lds((glb_void*)(src.x2 + ((int64_t)step * Np + n0 + col) * 64 + 16 * blk),
                                       (lds_void*)(bf.b + q * 1024), 16, 0, 0);
  }
  if (wave < 4) {   // scale1 rows m0 + 64 wave + lane, blocks 4 step .. 4 step + 3
    if constexpr (!RG)
      __builtin_amdgcn_global_load_lds((glb_void*)(src.s1 + (m0 + 64 * wave + lane) * KB + 4 * step),
                                       (lds_void*)(bf.s1 + wave * 256), 4, 0, 0);
  } else {          // scale2 block row 4 step + (wave - 4), columns n0 .. n0 + 255
    if constexpr (ON)
      ;                // byte loads above
    else if constexpr (RG)
      mf_dma4(src.rs2, bf.s2 + (wave - 4) * 256, (uint32_t)((4 * (int64_t)step + (wave - 4)) * N + n0 + 4 * lane));
    else
      __builtin_amdgcn_global_load_lds((glb_void*)(src.s2 + (4 * (int64_t)step + (wave - 4)) * N + n0 + 4 * lane),
                                       (lds_void*)(bf.s2 + (wave - 4) * 256), 4, 0, 0);
  }
  return s1w;
}

// The eight MFMAs of one A fragment (row block i) against the weight
// fragments j = 0..7: weight fragment j's scale is byte j % 4 of sbw[j / 4]
// (the instruction's byte select is an immediate).
template <int... J>
__device__ __forceinline__ void mf_row(f32x4 (&acc)[8], const i32x8& af, const u32x4 (&bv)[8], int sa,
                                       const uint2& sbw, std::integer_sequence<int, J...>) {
  ((acc[J] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        af, (i32x8){(int)bv[J].x, (int)bv[J].y, (int)bv[J].z, (int)bv[J].w, 0, 0, 0, 0}, acc[J],
        0 /*A: E4M3*/, 4 /*B: E2M1*/, 0, sa, J & 3, (int)(J < 4 ? sbw.x : sbw.y))), ...);
}

// The tiles cover the (M, N) output, all of K; x1's rows are Mx >= M bytes
// apart (Mx = M, or M padded to 16 in a workspace copy).
template <bool RG, bool ON>
__global__ __launch_bounds__(512, 1) void mx_gemm_tile(const uint8_t* __restrict__ x1t,
                                                       const uint8_t* __restrict__ x2,
                                                       const uint8_t* __restrict__ s1,
                                                       const uint8_t* __restrict__ s2,
                                                       float* __restrict__ y, int64_t M, int64_t Mx,
                                                       int64_t K, int64_t N, int64_t Np, int64_t tiles_m,
                                                       int64_t tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t a0[MF_ABYTES], a1[MF_ABYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[MF_BBYTES], b1[MF_BBYTES];
  __shared__ __attribute__((aligned(256))) uint8_t s10[MF_SBYTES], s11[MF_SBYTES];
  __shared__ __attribute__((aligned(256))) uint8_t s20[MF_SBYTES], s21[MF_SBYTES];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave & 3, wn = wave >> 2;      // 64-row and 128-column blocks of the tile

  // tiles in XCD-major order: workgroup b runs on XCD b % 8; give each XCD a
  // contiguous run of tiles so that the tiles sharing x1 rows share an L2
  int64_t id = blockIdx.x;
  const int64_t T = tiles_m * tiles_n;
  if ((T & 7) == 0) id = (id & 7) * (T >> 3) + (id >> 3);
  const int64_t m0 = (id / tiles_n) * MF_BM, n0 = (id % tiles_n) * MF_BN;
  const int64_t KB = (K + 31) / 32;
  const int steps = (int)((K + MF_BK - 1) / MF_BK);
  MfSrc src;
  src.x1t = x1t;
  src.x2 = x2;
  src.s1 = s1;
  src.s2 = s2;
  if constexpr (RG) {
    src.rx = buf_rsrc(x1t, (uint32_t)(K * Mx));
    src.rw = buf_rsrc(x2, (uint32_t)((int64_t)steps * Np * 64));
    src.rs1 = buf_rsrc(s1, (uint32_t)(M * KB));
    src.rs2 = buf_rsrc(s2, (uint32_t)(KB * N));
  }
  MfBufs buf0, buf1;
  buf0.a = a0; buf0.b = b0; buf0.s1 = s10; buf0.s2 = s20;
  buf1.a = a1; buf1.b = b1; buf1.s1 = s11; buf1.s2 = s21;

  // accumulators start as y (the in-place add). y goes through a buffer
  // resource: a per-lane offset, a uniform row offset and an immediate column
  // offset, so no per-element address is kept across the K loop.
  // Lane l holds rows 4 (l / 16) + r of each 16-row block and the tile
  // columns 128 wn + 8 (l % 16) + j, j = 0..7: two 16-byte runs per row.
  const __amdgpu_buffer_rsrc_t ry = buf_rsrc(y, (uint32_t)(M * N * 4));
  const uint32_t yl = (uint32_t)((4 * (lane >> 4)) * N + 8 * (lane & 15)) * 4u;
  const uint32_t yw = (uint32_t)(((m0 + 64 * wm) * N + n0 + 128 * wn) * 4);
  // with a ragged shape, rows past M and 4-column runs past N (N % 4 == 0;
  // otherwise ON, below) are neither read nor written: out-of-range offsets
  auto y_ok = [&](int i, int r, int h) {
    return m0 + 64 * wm + 16 * i + 4 * (lane >> 4) + r < M && n0 + 128 * wn + 8 * (lane & 15) + 4 * h < N;
  };
  // ON: y rows are only 4-byte aligned. A 4-column run inside the row still
  // moves as one 16-byte access (dword-aligned multi-dword buffer accesses
  // are supported on this target); the run that crosses N moves element by
  // element. Every access is issued, the ones not taken with an
  // out-of-range offset (no traffic), so no lane branches.
  auto y_el_ok = [&](int i, int r, int c) {
    return m0 + 64 * wm + 16 * i + 4 * (lane >> 4) + r < M && n0 + 128 * wn + 8 * (lane & 15) + c < N;
  };
  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t so = yw + (uint32_t)((16 * i + r) * N * 4);
      if constexpr (ON) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool full = y_el_ok(i, r, 4 * h + 3);
          const u32x4 v = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(ry, full ? yl + 16u * h : BUF_OOB, so, 0));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t vo = !full && y_el_ok(i, r, 4 * h + e) ? yl + 16u * h + 4u * e : BUF_OOB;
            const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(ry, vo, so, 0);
            acc[i][4 * h + e][r] = __uint_as_float(full ? v[e] : w);
          }
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t vo = RG && !y_ok(i, r, h) ? BUF_OOB : yl + 16u * h;
          const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ry, vo, so, 0));
          acc[i][4 * h + 0][r] = __uint_as_float(v.x);
          acc[i][4 * h + 1][r] = __uint_as_float(v.y);
          acc[i][4 * h + 2][r] = __uint_as_float(v.z);
          acc[i][4 * h + 3][r] = __uint_as_float(v.w);
        }
      }
    }

  // (the byte-loaded scale words go to LDS: scale1 rows for waves 0..3, with
  // ON the scale2 rows for waves 4..7)
  auto put_sw = [&](const MfBufs& b, uint32_t w) {
    if (RG && wave < 4) *reinterpret_cast<uint32_t*>(b.s1 + wave * 256 + 4 * lane) = w;
    if (ON && wave >= 4) *reinterpret_cast<uint32_t*>(b.s2 + (wave - 4) * 256 + 4 * lane) = w;
  };
  {
    const uint32_t s1w = mf_dma<RG, ON>(src, buf0, Mx, N, Np, KB, m0, n0, 0, wave, lane);
    wait_vm<0>();
    put_sw(buf0, s1w);
  }
  __syncthreads();

  // per-lane LDS read offsets (independent of the step)
  const int g = lane >> 4, jl = lane & 15;
  // transpose read tt of A fragment i: k-row r(tt), logical chunk 4 wm + i;
  // the four rows differ by multiples of 8 below 128, so they share
  // (r & 7) | ((r & 16) >> 1) and one swizzle value serves all four reads
  const int r0 = 16 * g + (jl >> 1);
  const int swz = mf_swz(r0);
  const int abase = r0 * 256 + 8 * (jl & 1);
  const int boff = (128 * wn + jl) * 64 + 16 * (g ^ mf_bswz(jl));   // + 1024 j
  const int s1off = (64 * wm + jl) * 4 + g;             // + 64 i
  const int s2off = g * 256 + 128 * wn + 8 * jl;        // columns 8 jl .. 8 jl + 7

  // One 128-deep step on buffer `cur` while the next step streams into
  // `nxt`. The single barrier at the end both publishes every wave's DMA into
  // `nxt` and frees `cur`, which the next step's DMA refills.
  auto do_step = [&](int step, const MfBufs& cur, const MfBufs& nxt) {
    uint32_t s1w = 0;
    if (step + 1 < steps) s1w = mf_dma<RG, ON>(src, nxt, Mx, N, Np, KB, m0, n0, step + 1, wave, lane);
    u32x4 bv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) bv[j] = *reinterpret_cast<const u32x4*>(cur.b + boff + 1024 * j);
    const uint2 sbw = *reinterpret_cast<const uint2*>(cur.s2 + s2off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      typedef int v2i __attribute__((ext_vector_type(2)));
      v2i p[4];
      const int achunk = 16 * ((4 * wm + i) ^ swz);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        p[tt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(
            cur.a + abase + achunk + ((tt & 1) * 8 + (tt >> 1) * 64) * 256));
      const i32x8 af = {p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
      const int sa = cur.s1[s1off + 64 * i];
      mf_row(acc[i], af, bv, sa, sbw, std::make_integer_sequence<int, 8>{});
    }
    wait_vm<0>();            // this wave's DMA into `nxt` has landed
    if (step + 1 < steps) put_sw(nxt, s1w);
    __syncthreads();
  };
  for (int step = 0; step < steps; step += 2) {
    do_step(step, buf0, buf1);
    if (step + 1 < steps) do_step(step + 1, buf1, buf0);
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t so = yw + (uint32_t)((16 * i + r) * N * 4);
      if constexpr (ON) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool full = y_el_ok(i, r, 4 * h + 3);
          u32x4 v;
          v.x = __float_as_uint(acc[i][4 * h + 0][r]);
          v.y = __float_as_uint(acc[i][4 * h + 1][r]);
          v.z = __float_as_uint(acc[i][4 * h + 2][r]);
          v.w = __float_as_uint(acc[i][4 * h + 3][r]);
          __builtin_amdgcn_raw_buffer_store_b128(v, ry, full ? yl + 16u * h : BUF_OOB, so, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t vo = !full && y_el_ok(i, r, 4 * h + e) ? yl + 16u * h + 4u * e : BUF_OOB;
            __builtin_amdgcn_raw_buffer_store_b32(v[e], ry, vo, so, 0);
          }
        }
        continue;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 v;
        v.x = __float_as_uint(acc[i][4 * h + 0][r]);
        v.y = __float_as_uint(acc[i][4 * h + 1][r]);
        v.z = __float_as_uint(acc[i][4 * h + 2][r]);
        v.w = __float_as_uint(acc[i][4 * h + 3][r]);
        const uint32_t vo = RG && !y_ok(i, r, h) ? BUF_OOB : yl + 16u * h;
        __builtin_amdgcn_raw_buffer_store_b128(v, ry, vo, so, 0);
      }
    }
}

// x1 (K, M) -> (K, Mx) with zero columns past M: one 16-byte output chunk per
// thread (its source bytes read one by one: rows of x1 need not be aligned).
__global__ __launch_bounds__(256) void mx_pad_x1(const uint8_t* __restrict__ x1t, uint8_t* __restrict__ out,
                                                 int64_t K, int64_t M, int64_t Mx) {
  const int64_t chunks = Mx / 16;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= K * chunks) return;
  const int64_t k = i / chunks, c = i - k * chunks;
  const uint8_t* src = x1t + k * M + 16 * c;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int b = 0; b < 16; ++b)
    if (16 * c + b < M) w[b >> 2] |= (uint32_t)src[b] << (8 * (b & 3));
  *reinterpret_cast<u32x4*>(out + k * Mx + 16 * c) = (u32x4){w[0], w[1], w[2], w[3]};
}

// The 256 x 256 tile takes x1 rows of 16-byte chunks (Mx % 16) and y below
// 2 GiB (one buffer resource); a ragged shape also needs every input, and
// every offset its last step and its last tile row and column form past the
// inputs, below 2 GiB. N not a multiple of 4 (scale2 and y rows not 4- and
// 16-byte aligned) runs the ragged tile's ON form: scale2 by byte loads, y
// in dword-aligned 16-byte runs and element by element where a run crosses N.
bool mx_tile_ok(int64_t m, int64_t mx, int64_t k, int64_t n) {
  const int64_t lim = int64_t(1) << 31;
  const int64_t Np = 16 * ((n + 15) / 16);
  const int64_t KB = (k + 31) / 32, steps = (k + MF_BK - 1) / MF_BK;
  const bool aligned = m % MF_BM == 0 && n % MF_BN == 0 && k % MF_BK == 0 && mx == m;
  return mx % 16 == 0 && m * n * 4 < lim &&
         (aligned || ((steps + 1) * MF_BK * mx < lim && (m + MF_BM) * KB < lim && (KB + 8) * n < lim &&
                      steps * Np * 64 < lim));
}

}  // namespace

size_t mx_x1pad_bytes(int64_t m, int64_t k, int64_t n) {
  if (m <= 0 || k <= 0 || n <= 0 || m % 16 == 0) return 0;
  const int64_t mx = 16 * ((m + 15) / 16);
  if (!mx_tile_ok(m, mx, k, n)) return 0;
  return ((size_t)(k * mx) + 255) & ~(size_t)255;
}

hipError_t launch_mx_matmul(const MxProblem& p, hipStream_t s) {
  const int64_t Np = 16 * ((p.n + 15) / 16);
  const int64_t tm = (p.m + MF_BM - 1) / MF_BM, tn = (p.n + MF_BN - 1) / MF_BN;
  const bool aligned = p.m % MF_BM == 0 && p.n % MF_BN == 0 && p.k % MF_BK == 0;
  // x1 rows not 16-byte aligned: with a workspace, the tile runs on a padded copy
  const bool pad = p.m % 16 != 0 && p.x1pad != nullptr && mx_x1pad_bytes(p.m, p.k, p.n) > 0;
  const int64_t mx = pad ? 16 * ((p.m + 15) / 16) : p.m;
  const uint8_t* x1 = pad ? p.x1pad : p.x1;
  prof_begin(s);
  if (pad) {
    const int64_t threads = p.k * (mx / 16);
    mx_pad_x1<<<dim3((unsigned)((threads + 255) / 256)), 256, 0, s>>>(p.x1, p.x1pad, p.k, p.m, mx);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (mx_tile_ok(p.m, mx, p.k, p.n) && aligned && !pad) {
    mx_gemm_tile<false, false><<<dim3((unsigned)(tm * tn)), 512, 0, s>>>(x1, p.x2, p.s1, p.s2, p.y, p.m, mx,
                                                                       p.k, p.n, Np, tm, tn);
  } else if (mx_tile_ok(p.m, mx, p.k, p.n) && p.n % 4 == 0) {
    mx_gemm_tile<true, false><<<dim3((unsigned)(tm * tn)), 512, 0, s>>>(x1, p.x2, p.s1, p.s2, p.y, p.m, mx,
                                                                      p.k, p.n, Np, tm, tn);
  } else if (mx_tile_ok(p.m, mx, p.k, p.n)) {
    mx_gemm_tile<true, true><<<dim3((unsigned)(tm * tn)), 512, 0, s>>>(x1, p.x2, p.s1, p.s2, p.y, p.m, mx,
                                                                     p.k, p.n, Np, tm, tn);
  } else {
    dim3 grid((unsigned)((p.n + MX_BN - 1) / MX_BN), (unsigned)((p.m + MX_BM - 1) / MX_BM));
    mx_gemm_kernel<<<grid, 256, 0, s>>>(p.x1, p.x2, p.s1, p.s2, p.y, p.m, p.k, p.n, Np, 0, 0, p.n);
  }
  prof_end(s);
  return hipGetLastError();
}

}  // namespace wq
