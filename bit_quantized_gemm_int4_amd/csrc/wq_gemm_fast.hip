// Fast weight-quantized GEMM for INT4 weights in the GFX950_B layout when the
// quantization group is a multiple of 128 along K (or per channel / per
// tensor) and k is a multiple of 128. Same operator as wq_gemm.hip
// (aclnnWeightQuantMatmulAllReduceAddRmsNorm page, Formula); this file holds
// the MFMA-bound tile used for large m.
//
// Arithmetic. With q the int4 code, u = q + 8 its offset-binary nibble and
// B = 128 + u = q + 136 (exact in bf16: the bits 0x4300 | u; fp16 uses
// 1024 + u = q + 1032, bits 0x6400 | u), no weight is ever dequantized:
//   sum_k x[r,k] (q s + o) = s * sum_k x B  +  (o - 136 s) * sum_k x
// The MFMAs sum x * B straight into the float32 accumulator, kept in units of
// the current group's scale (rescaled by s_prev / s_g at each group start: one
// multiply per element per group; a zero scale zeroes that column's weight
// operand instead). The rank-1 remainder sum_g rowsum_g(x) (o_g - 136 s_g) is
// added at the end with MFMAs over the group axis on bf16 hi/lo splits of
// both factors (three products; relative error ~2^-16 of a term that is a
// small multiple of the result). Two pre-passes produce those factors: the
// per-group row sums of x1 and the per-group column corrections, both stored
// in MFMA operand order.
//
// Tile: 128 (m) x 512 (n) per workgroup of 8 waves, each wave 128 x 64 (8 x 4
// MFMA 16x16x32 tiles), two waves per SIMD. Wide N because the 4-bit weight is
// a quarter of the bf16 activation's bytes: per 128-deep slab the workgroup
// moves 32 KiB of x1 and 32 KiB of packed weight from L2 into LDS by direct
// global->LDS DMA, double-buffered. A lane's weight fragment is one 16-byte
// LDS read: column l%16 and the 32 K values of block l/16 of the slab; dword c
// of it feeds MFMA c, whose A operand is x1[row][32*(l/16) + 8c ...].
// The epilogue stages the accumulators through LDS so that residual loads and
// y stores are 16-byte, row-contiguous accesses.
#include "wq_device.h"
#include "wq_internal.h"
#include "wq_unpack.h"

namespace wq {
namespace {

// bf16 hi/lo split of a float: v ~= hi + lo with |v - hi - lo| <= 2^-16 |v|.
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = from_f32<ACT_BF16>(v);
  lo = from_f32<ACT_BF16>(v - to_f32<ACT_BF16>(hi));
}


struct FastArgs {
  const uint16_t* x1;
  const uint8_t* x2;
  const uint16_t* scale;
  const uint16_t* bias;
  const uint16_t* residual;
  uint16_t* y;
  float* partial;          // [m][ceil(n/32)]
  const uint16_t* rs;      // [m][2][gp]  per-group row sums of x1, bf16 hi then lo
  const uint16_t* corr;    // [np][2][gp] per-group o - bias*s per column, hi then lo
  int64_t m, k, n, np;
  int64_t group;           // K length of a group (multiple of 128, or >= k)
  int64_t s_row, s_col;
  int64_t groups, gp;      // groups = ceil(k / group); gp = 32 * ceil(groups / 32)
};

// ---------------------------------------------------------------------------
// Pre-pass 1: per-group row sums of x1, written as bf16 hi/lo (zero padded to
// gp groups). One workgroup per row; eight-element chunk sums in LDS, then
// each group summed in a fixed order.
// ---------------------------------------------------------------------------
template <int ACT>
__global__ __launch_bounds__(256) void group_rowsum_kernel(const uint16_t* __restrict__ x1, int64_t k,
                                                           int64_t group, int64_t groups, int64_t gp,
                                                           uint16_t* __restrict__ rs) {
  extern __shared__ float chunk_sum[];        // k / 8 floats
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x1 + row * k;
  const int64_t chunks = k / 8;
  for (int64_t c = threadIdx.x; c < chunks; c += 256) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xr + 8 * c);
    float s = lo_f32<ACT>(v.x) + hi_f32<ACT>(v.x);
    s += lo_f32<ACT>(v.y) + hi_f32<ACT>(v.y);
    s += lo_f32<ACT>(v.z) + hi_f32<ACT>(v.z);
    s += lo_f32<ACT>(v.w) + hi_f32<ACT>(v.w);
    chunk_sum[c] = s;
  }
  __syncthreads();
  const int64_t per = group / 8;               // chunks per group
  for (int64_t g = threadIdx.x; g < gp; g += 256) {
    float s = 0.f;
    if (g < groups) {
      const int64_t c1 = (g + 1) * per < chunks ? (g + 1) * per : chunks;
      for (int64_t c = g * per; c < c1; ++c) s += chunk_sum[c];
    }
    uint16_t hi, lo;
    split_bf16(s, hi, lo);
    rs[row * 2 * gp + g] = hi;
    rs[row * 2 * gp + gp + g] = lo;
  }
}

// ---------------------------------------------------------------------------
// Pre-pass 2: per-group column corrections o[g][n] - bias * s[g][n] (zero for
// padding), written [np][2][gp] as bf16 hi/lo. One thread per (column, group).
// ---------------------------------------------------------------------------
template <int ACT>
__global__ __launch_bounds__(256) void group_corr_kernel(const uint16_t* __restrict__ scale,
                                                         const uint16_t* __restrict__ offset,
                                                         int64_t n, int64_t np, int64_t groups,
                                                         int64_t gp, int64_t s_row, int64_t s_col,
                                                         uint16_t* __restrict__ corr) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= np * gp) return;
  const int64_t col = idx / gp, g = idx % gp;
  float c = 0.f;
  if (col < n && g < groups) {
    const int64_t si = g * s_row + col * s_col;
    const float sv = to_f32<ACT>(scale[si]);
    const float ov = offset ? to_f32<ACT>(offset[si]) : 0.f;
    c = ov - Magic<ACT>::bias * sv;
  }
  uint16_t hi, lo;
  split_bf16(c, hi, lo);
  corr[col * 2 * gp + g] = hi;
  corr[col * 2 * gp + gp + g] = lo;
}

// ---------------------------------------------------------------------------
// Main tile
// ---------------------------------------------------------------------------
constexpr int WD_BM = 128, WD_BN = 512, WD_KS = 128;
constexpr int WD_LROW = WD_KS * 2;                 // LDS bytes per x1 row
constexpr int WD_ABUF = WD_BM * WD_LROW;           // x1 slab: 32 KiB
constexpr int WD_BBUF = WD_BN * 64;                // weight slab: 32 KiB
constexpr int WD_EROW = (64 + 4) * 4;              // epilogue staging row (fp32, padded)
static_assert(32 * WD_EROW <= 16384, "epilogue staging must fit a wave's 16 KiB region");

// x1 slab (128 rows x 128 K) -> LDS: 32 DMA instructions of 1 KiB (4 rows);
// wave w issues 4w + j: rows 4*(4w + j) + lane/16. LDS rows are 256 bytes; the
// 16-byte chunk j of row r sits at position j ^ (r & 15), so the A-fragment
// reads of 16 lanes (16 rows, one K chunk) hit 16 distinct bank groups.
// off[j] is the lane's element offset of instruction j from the tile's first
// row (row and swizzled chunk); k0 advances it by slab.
__device__ __forceinline__ void wd_dma_a(const uint16_t* xblk, const uint32_t (&off)[4], uint32_t k0,
                                         uint8_t* buf) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    __builtin_amdgcn_global_load_lds((glb_void*)(xblk + (off[j] + k0)),
                                     (lds_void*)(buf + (4 * wave + j) * 4 * WD_LROW), 16, 0, 0);
}

// Weight slab for the tile's 512 columns (64 bytes per column in GFX950_B
// order): 32 DMA instructions of 1 KiB (16 columns); wave w issues chunks
// 4w + j, lane l the 16 bytes of column 16*chunk + l/4, block l%4; bsrc[j] is
// the lane's byte offset from the tile's first column (clamped to the padded
// width; columns past n are computed but never stored).
__device__ __forceinline__ void wd_dma_b(const uint8_t* xslab, const int32_t (&bsrc)[4], uint8_t* buf) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    __builtin_amdgcn_global_load_lds((glb_void*)(xslab + bsrc[j]),
                                     (lds_void*)(buf + (4 * wave + j) * 1024), 16, 0, 0);
}

// One 128-deep slab accumulated into acc: acc[i][f] += sum over the slab of
// x1 * (q + bias), the MFMAs accumulating in place. Per K step c: the eight
// A-fragment reads, the four weight fragments unpacked, 32 MFMAs.
template <int ACT>
__device__ __forceinline__ void wd_slab(const uint8_t* abuf, const uint8_t* wbuf,
                                        const uint32_t (&mk)[4], const uint32_t (&mg)[4],
                                        f32x4 (&acc)[8][4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t b[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(
        wbuf + (wave * 64 + 16 * f + (lane & 15)) * 64 + (lane >> 4) * 16);
    b[f][0] = v.x;
    b[f][1] = v.y;
    b[f][2] = v.z;
    b[f][3] = v.w;
  }
  const uint8_t* arow = abuf + (lane & 15) * WD_LROW;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int pos = ((4 * (lane >> 4) + c) ^ (lane & 15)) * 16;
    u32x4 av[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) av[i] = *reinterpret_cast<const u32x4*>(arow + i * 16 * WD_LROW + pos);
    u32x4 bf[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) bf[f] = unpack8(b[f][c], mk[f], mg[f]);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[i][f] = mfma16<ACT>(av[i], bf[f], acc[i][f]);
  }
}

template <int ACT>
__global__ __launch_bounds__(512, 1) void gemm_b_wide(FastArgs a, int64_t tiles_m, int64_t tiles_n) {
  // Four LDS objects (two x1 slabs, two weight slabs): the compiler then sees
  // that the DMA filling one buffer does not alias reads of the other.
  __shared__ __attribute__((aligned(16))) uint8_t abuf0[WD_ABUF];
  __shared__ __attribute__((aligned(16))) uint8_t abuf1[WD_ABUF];
  __shared__ __attribute__((aligned(16))) uint8_t wbuf0[WD_BBUF];
  __shared__ __attribute__((aligned(16))) uint8_t wbuf1[WD_BBUF];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

  // XCD-aware tile order: consecutive workgroups land on different XCDs, so
  // give each XCD a contiguous range of tiles, walked two tile-rows at a time.
  const int64_t T = tiles_m * tiles_n;
  int64_t id = blockIdx.x;
  if ((T & 7) == 0) id = (id & 7) * (T >> 3) + (id >> 3);
  const int64_t band = id / (2 * tiles_n);
  const int64_t rem = id % (2 * tiles_n);
  int64_t tm = band * 2 + (rem & 1);
  int64_t tn = rem >> 1;
  if (band * 2 + 1 >= tiles_m && (tiles_m & 1)) {  // last odd band: one tile-row
    tm = band * 2;
    tn = rem;
  }
  const int64_t m0 = tm * WD_BM;
  const int64_t n0 = tn * WD_BN;
  const int64_t ncol0 = n0 + wave * 64;             // the wave's first column
  const int slabs = (int)(a.k / WD_KS);
  const uint32_t k = (uint32_t)a.k;

  // ---- DMA sources ----
  const uint16_t* xblk = a.x1 + m0 * a.k;
  const int rows_left = (int)(a.m - m0 < WD_BM ? a.m - m0 : WD_BM);
  uint32_t aoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (4 * wave + j) * 4 + (lane >> 4);
    const int cj = (lane & 15) ^ (row & 15);
    const int r = row < rows_left ? row : rows_left - 1;   // rows past m: never stored
    aoff[j] = (uint32_t)r * k + 8 * cj;
  }
  const uint8_t* xw = a.x2 + n0 * 64;
  const int64_t slab_bytes = a.np * 64;
  int32_t bsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int64_t col = n0 + 16 * (4 * wave + j) + (lane >> 2);
    col = col < a.np ? col : a.np - 1;
    bsrc[j] = (int32_t)((col - n0) * 64 + (lane & 3) * 16);
  }
  // scale offsets of the wave's 4 column tiles (clamped; columns past n get scale 0)
  uint32_t soff[4];
  float cmask[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int64_t col = ncol0 + 16 * f + (lane & 15);
    soff[f] = (uint32_t)((col < a.n ? col : a.n - 1) * a.s_col);
    cmask[f] = col < a.n ? 1.f : 0.f;
  }
  const int spg = (int)(a.group / WD_KS);              // slabs per group (>= 1)

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[i][f] = (f32x4){0.f, 0.f, 0.f, 0.f};

  wd_dma_a(xblk, aoff, 0, abuf0);
  wd_dma_b(xw, bsrc, wbuf0);
  // raw scales of the current group and of the next one; the next group's
  // are loaded one step ahead, before that step's DMA, and used only after
  // the step's barrier, so waiting for them never waits for the DMA.
  uint16_t scur[4], snxt[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) scur[f] = a.scale[soff[f]];
  __syncthreads();

  // acc holds the running sum in units of the current group's scale cs:
  // true sum = cs * acc. At a group with scale s: acc *= cs / s, then the
  // MFMAs add that group's x1 * (q + bias) to acc, and cs = s. A zero scale
  // zeroes the column's weight operand and leaves acc and cs unchanged.
  float cs[4] = {0.f, 0.f, 0.f, 0.f};
  uint32_t mk[4], mg[4];
  int gpos = 0;                                        // slab index within its group
  const uint16_t* srow_next = a.scale + a.s_row;       // scale row of the next group
  auto step = [&](int s, const uint8_t* acur, uint8_t* anxt, const uint8_t* wcur, uint8_t* wnxt) {
    const bool more = s + 1 < slabs;
    if (more && gpos == spg - 1) {                     // next slab starts a group
#pragma unroll
      for (int f = 0; f < 4; ++f) snxt[f] = srow_next[soff[f]];
      srow_next += a.s_row;
    }
    if (more) {
      wd_dma_a(xblk, aoff, (uint32_t)(s + 1) * WD_KS, anxt);
      wd_dma_b(xw + (s + 1) * slab_bytes, bsrc, wnxt);
    }
    if (gpos == 0) {                                   // group start
      float ratio[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const float sg = to_f32<ACT>(scur[f]) * cmask[f];
        const bool z = sg == 0.f;
        ratio[f] = (z || cs[f] == 0.f) ? 1.f : cs[f] / sg;
        cs[f] = z ? cs[f] : sg;
        mk[f] = z ? 0u : 0x000F000Fu;
        mg[f] = z ? 0u : Magic<ACT>::bits;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][f][r] *= ratio[f];
    }
    wd_slab<ACT>(acur, wcur, mk, mg, acc);
    if (++gpos == spg) {
      gpos = 0;
#pragma unroll
      for (int f = 0; f < 4; ++f) scur[f] = snxt[f];
    }
    __syncthreads();
  };
  for (int s = 0; s < slabs; s += 2) {
    step(s, abuf0, abuf1, wbuf0, wbuf1);
    if (s + 1 < slabs) step(s + 1, abuf1, abuf0, wbuf1, wbuf0);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][f][r] *= cs[f];

  // ---- rank-1 remainder: acc += sum_g rowsum_g(x) * corr_g over the group
  //      axis, three bf16 MFMA products per 32 groups ----
  for (int64_t g0 = 0; g0 < a.gp; g0 += 32) {
    u32x4 chi[4], clo[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      int64_t col = ncol0 + 16 * f + (lane & 15);
      col = col < a.np ? col : a.np - 1;
      const uint16_t* p = a.corr + col * 2 * a.gp + g0 + 8 * (lane >> 4);
      chi[f] = *reinterpret_cast<const u32x4*>(p);
      clo[f] = *reinterpret_cast<const u32x4*>(p + a.gp);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int64_t row = m0 + 16 * i + (lane & 15);
      row = row < a.m ? row : a.m - 1;
      const uint16_t* p = a.rs + row * 2 * a.gp + g0 + 8 * (lane >> 4);
      const u32x4 rhi = *reinterpret_cast<const u32x4*>(p);
      const u32x4 rlo = *reinterpret_cast<const u32x4*>(p + a.gp);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        acc[i][f] = mfma16<ACT_BF16>(rhi, chi[f], acc[i][f]);
        acc[i][f] = mfma16<ACT_BF16>(rhi, clo[f], acc[i][f]);
        acc[i][f] = mfma16<ACT_BF16>(rlo, chi[f], acc[i][f]);
      }
    }
  }

  // ---- epilogue, four quarters of 32 rows: stage the wave's 32 x 64 fp32
  //      block in LDS (32 rows x 272 bytes of its 16 KiB region), then each
  //      lane takes 8 consecutive columns of a row: y = acc + bias + residual
  //      with 16-byte loads/stores, and the row's sum of y^2 over each
  //      32-column half of the wave's columns ----
  uint8_t* stage = (wave < 2 ? abuf0 : wave < 4 ? abuf1 : wave < 6 ? wbuf0 : wbuf1) + (wave & 1) * 16384;
  const int lr = lane >> 3, lc = (lane & 7) * 8;       // row within 8, first column
  const int64_t col = ncol0 + lc;
  const bool vec = (a.n & 7) == 0 && col + 8 <= a.n;
  float bv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) bv[e] = (a.bias && col + e < a.n) ? to_f32<ACT>(a.bias[col + e]) : 0.f;
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * i + 4 * (lane >> 4) + r;          // 0..31
          *reinterpret_cast<float*>(stage + row * WD_EROW + (16 * f + (lane & 15)) * 4) = acc[2 * qt + i][f][r];
        }
    __syncthreads();
#pragma unroll 2
    for (int st = 0; st < 4; ++st) {
      const int rl = 8 * st + lr;                                // 0..31
      const int64_t row = m0 + 32 * qt + rl;
      const float* sp = reinterpret_cast<const float*>(stage + rl * WD_EROW + lc * 4);
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(sp);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(sp + 4);
      const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      float ss = 0.f;
      if (row < a.m) {
        const int64_t idx = row * a.n + col;
        if (vec) {
          const u32x4 rv = *reinterpret_cast<const u32x4*>(a.residual + idx);
          const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
          uint32_t yw[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float y0 = v[2 * e] + bv[2 * e] + lo_f32<ACT>(rw[e]);
            const float y1 = v[2 * e + 1] + bv[2 * e + 1] + hi_f32<ACT>(rw[e]);
            ss = fmaf(y0, y0, ss);
            ss = fmaf(y1, y1, ss);
            yw[e] = pack2<ACT>(y0, y1);
          }
          *reinterpret_cast<u32x4*>(a.y + idx) = (u32x4){yw[0], yw[1], yw[2], yw[3]};
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (col + e < a.n) {
              const float yv = v[e] + bv[e] + to_f32<ACT>(a.residual[idx + e]);
              ss = fmaf(yv, yv, ss);
              a.y[idx + e] = from_f32<ACT>(yv);
            }
          }
        }
      }
      ss = quad_sum(ss);                               // the 4 lanes of 32 columns
      const int64_t c32 = ncol0 + (lc & 32);
      if ((lane & 3) == 0 && row < a.m && c32 < a.n) a.partial[row * ((a.n + 31) / 32) + c32 / 32] = ss;
    }
    __syncthreads();
  }
}

template <int ACT>
hipError_t launch_wide_t(const WqProblem& p, float* partial, uint16_t* rs, uint16_t* corr,
                         hipStream_t s) {
  FastArgs a;
  a.x1 = static_cast<const uint16_t*>(p.x1);
  a.x2 = static_cast<const uint8_t*>(p.x2);
  a.scale = static_cast<const uint16_t*>(p.scale);
  a.bias = static_cast<const uint16_t*>(p.bias);
  a.residual = static_cast<const uint16_t*>(p.residual);
  a.y = static_cast<uint16_t*>(p.y);
  a.partial = partial;
  a.rs = rs;
  a.corr = corr;
  a.m = p.m;
  a.k = p.k;
  a.n = p.n;
  a.np = 16 * ((p.n + 15) / 16);
  a.group = p.group >= p.k ? p.k : p.group;       // k is a multiple of 128 here
  a.s_row = p.s_row;
  a.s_col = p.s_col;
  a.groups = (p.k + a.group - 1) / a.group;
  a.gp = 32 * ((a.groups + 31) / 32);
  group_rowsum_kernel<ACT><<<dim3((unsigned)p.m), 256, (size_t)(p.k / 8) * sizeof(float), s>>>(
      a.x1, p.k, a.group, a.groups, a.gp, rs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t cells = a.np * a.gp;
  group_corr_kernel<ACT><<<dim3((unsigned)((cells + 255) / 256)), 256, 0, s>>>(
      a.scale, static_cast<const uint16_t*>(p.offset), p.n, a.np, a.groups, a.gp, p.s_row,
      p.s_col, corr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t tm = (p.m + WD_BM - 1) / WD_BM, tn = (p.n + WD_BN - 1) / WD_BN;
  gemm_b_wide<ACT><<<dim3((unsigned)(tm * tn)), 512, 0, s>>>(a, tm, tn);
  return hipGetLastError();
}

}  // namespace

bool fast_path_ok(const WqProblem& p) {
  if (p.w_bits != 4 || p.layout != WQ_LAYOUT_GFX950_B) return false;
  if (p.k % 128 != 0) return false;
  return p.group >= p.k || p.group % 128 == 0;
}

// per-group row sums (m rows) and column corrections (np columns), worst case
// over group sizes: groups = ceil(k / 128)
size_t fast_rowsum_bytes(int64_t m, int64_t k) {
  const int64_t groups = (k + 127) / 128;
  const int64_t gp = 32 * ((groups + 31) / 32);
  return ((size_t)(m * 2 * gp * 2) + 255) & ~(size_t)255;
}
size_t fast_corr_bytes(int64_t n, int64_t k) {
  const int64_t groups = (k + 127) / 128;
  const int64_t gp = 32 * ((groups + 31) / 32);
  const int64_t np = 16 * ((n + 15) / 16);
  return ((size_t)(np * 2 * gp * 2) + 255) & ~(size_t)255;
}

hipError_t launch_prefill(const WqProblem& p, float* partial, uint16_t* rs, uint16_t* corr,
                          hipStream_t s) {
  return p.bf16 ? launch_wide_t<ACT_BF16>(p, partial, rs, corr, s)
                : launch_wide_t<ACT_F16>(p, partial, rs, corr, s);
}

}  // namespace wq
