// Fast weight-quantized GEMM for INT4 weights in the GFX950_B layout when the
// quantization group is a multiple of 128 along K (or per channel / per
// tensor). Same operator as wq_gemm.hip (aclnnWeightQuantMatmulAllReduceAddRmsNorm
// page, Formula); this file holds the MFMA-bound tile used for large m.
//
// Arithmetic. With q the int4 code, u = q + 8 its offset-binary nibble and
// B = 128 + u = q + 136 (exact in bf16: the bits 0x4300 | u; fp16 uses
// 1024 + u = q + 1032, bits 0x6400 | u), a 128-deep K slab needs no per-element
// dequantization at all:
//   sum_k x[r,k] (q s + o) = s * sum_k x B  +  (o - 136 s) * sum_k x
// so the MFMAs sum x * B straight into the float32 accumulator, kept in units
// of the current group's scale (rescaled by s_prev / s_g at each group
// start: one multiply per element per group), and the rank-1 remainder
// sum_g rowsum_g(x) (o_g - 136 s_g) is added once at the end with MFMAs on
// bf16 hi/lo splits of both factors (three products; relative error ~2^-16
// of a term that is a small multiple of the result). The row sums come from
// a pre-pass (group_rowsum_kernel) that reads x1 once.
//
// Tile: 256 (m) x 128 (n) per workgroup, 4 waves as 2 x 2, 128 x 64 per wave
// = 8 x 4 MFMA 16x16x32 tiles. x1 slabs (256 x 128) are double-buffered in
// LDS, filled by direct global->LDS DMA (k a multiple of 128); the packed weight goes straight from global memory to registers: one
// dwordx4 per lane gives lane l column l%16 and the 32 K values of block
// l/16 of a 128-deep slab, and dword c of it feeds MFMA c of the slab, whose
// A operand is the matching 8 K values x1[row][32*(l/16) + 8c ...].
#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

template <int ACT>
struct Magic;
template <>
struct Magic<ACT_BF16> {
  static constexpr uint32_t bits = 0x43004300u;
  static constexpr float bias = 136.f;
};
template <>
struct Magic<ACT_F16> {
  static constexpr uint32_t bits = 0x64006400u;
  static constexpr float bias = 1032.f;
};

// (p & mask) | bits in one VALU op (the compiler emits and + or).
__device__ __forceinline__ uint32_t and_or(uint32_t p, uint32_t mask, uint32_t bits) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(p), "v"(mask), "v"(bits));
  return r;
}

// Eight int4 codes (one dword, K ascending from the low nibble) -> eight
// 16-bit values (q + bias), dword j = codes (2j, 2j+1) in (low, high) half.
// With mask = 0x000F000F and bits = the magic exponent pattern; mask = bits =
// 0 gives zeros (a column whose group scale is zero).
__device__ __forceinline__ u32x4 unpack8(uint32_t w, uint32_t mask, uint32_t bits) {
  const uint32_t u = w ^ 0x88888888u;        // two's complement -> offset binary
  const uint32_t u4 = u >> 4;
  u32x4 r;
  r.x = and_or(__builtin_amdgcn_perm(u4, u, 0x0C040C00u), mask, bits);
  r.y = and_or(__builtin_amdgcn_perm(u4, u, 0x0C050C01u), mask, bits);
  r.z = and_or(__builtin_amdgcn_perm(u4, u, 0x0C060C02u), mask, bits);
  r.w = and_or(__builtin_amdgcn_perm(u4, u, 0x0C070C03u), mask, bits);
  return r;
}

// bf16 hi/lo split of a float: v ~= hi + lo with |v - hi - lo| <= 2^-16 |v|.
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = from_f32<ACT_BF16>(v);
  lo = from_f32<ACT_BF16>(v - to_f32<ACT_BF16>(hi));
}

struct FastArgs {
  const uint16_t* x1;
  const uint8_t* x2;
  const uint16_t* scale;
  const uint16_t* offset;
  const uint16_t* bias;
  const uint16_t* residual;
  uint16_t* y;
  float* partial;          // [ceil(n/32)][m]
  const uint16_t* rs;      // [m][2][gp] bf16: row sums per group, hi then lo
  int64_t m, k, n, np;
  int64_t group;           // K length of a group (multiple of 128, or >= k)
  int64_t s_row, s_col;
  int64_t groups, gp;      // groups = ceil(k / group); gp = 32 * ceil(groups / 32)
};

// ---------------------------------------------------------------------------
// Pre-pass: per-group row sums of x1, written as bf16 hi/lo (zero padded to
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

constexpr int PF_BM = 256, PF_BN = 128, PF_KS = 128;
constexpr int PF_LROW = PF_KS * 2;                 // LDS bytes per x1 row
constexpr int PF_LBUF = PF_BM * PF_LROW;           // one slab buffer (64 KiB)
constexpr size_t PF_LDS = 2 * (size_t)PF_LBUF;     // double buffer

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// x1 slab (256 rows x 128 K) -> LDS by direct global->LDS DMA, 16 bytes per
// lane, 1 KiB (4 rows) per wave instruction. LDS rows are 256 bytes; the
// 16-byte chunk j of row r sits at position j ^ (r & 15), so the A-fragment
// reads of 16 lanes (16 rows, one K chunk) hit 16 distinct bank groups.
// Wave w, instruction j covers tile rows 4*(16w + j) + (lane / 16); its
// element offset from the tile's first row is off[j & 3] + (j & ~3) * 4k,
// with off[] the per-lane offsets of instructions 0..3 (the chunk swizzle
// depends on the row only through j & 3). Rows past m are
// clamped to m - 1 in a separate (uniform) path: their results are never
// stored. k is a multiple of 128, so there is no K tail.
struct ADma {
  uint32_t off[4];      // lane offset (elements) of instructions j = 0..3 (mod 4)
};

__device__ __forceinline__ void pf_dma_a(const uint16_t* xblk, const ADma& d, uint32_t k4,
                                         uint32_t k0, uint8_t* buf) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint16_t* src = xblk + (d.off[j & 3] + (uint32_t)(j & ~3) * k4 + k0);
    __builtin_amdgcn_global_load_lds((glb_void*)src,
                                     (lds_void*)(buf + (wave * 16 + j) * 4 * PF_LROW), 16, 0, 0);
  }
}

// Ragged last row block: rows past m read row m - 1.
__device__ __forceinline__ void pf_dma_a_clamped(const uint16_t* xblk, int rows_left, uint32_t k,
                                                 uint32_t k0, uint8_t* buf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = (wave * 16 + j) * 4 + (lane >> 4);
    const int cj = (lane & 15) ^ (row & 15);
    const int r = row < rows_left ? row : rows_left - 1;
    const uint16_t* src = xblk + ((uint32_t)r * k + k0 + 8 * cj);
    __builtin_amdgcn_global_load_lds((glb_void*)src,
                                     (lds_void*)(buf + (wave * 16 + j) * 4 * PF_LROW), 16, 0, 0);
  }
}

// Packed weight of one slab for the wave's 64 columns: xs points at the
// slab's first column block of this wave; boff[f] is the lane's byte offset
// (column clamped to the padded width; columns past n are never stored).
__device__ __forceinline__ void pf_load_b(const uint8_t* xs, const int32_t (&boff)[4],
                                          uint32_t (&b)[4][4]) {
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xs + boff[f]);
    b[f][0] = v.x;
    b[f][1] = v.y;
    b[f][2] = v.z;
    b[f][3] = v.w;
  }
}

// One 128-deep slab accumulated into acc: acc[i][f] += sum over the slab of
// x1 * (q + bias), the MFMAs accumulating in place.
template <int ACT>
__device__ __forceinline__ void pf_slab(const uint8_t* buf, int wr, const uint32_t (&b)[4][4],
                                        const uint32_t (&mk)[4], const uint32_t (&mg)[4],
                                        f32x4 (&acc)[8][4]) {
  const int lane = threadIdx.x & 63;
  const uint8_t* arow = buf + (wr * 128 + (lane & 15)) * PF_LROW;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u32x4 bf[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) bf[f] = unpack8(b[f][c], mk[f], mg[f]);
    const int pos = ((4 * (lane >> 4) + c) ^ (lane & 15)) * 16;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 av = *reinterpret_cast<const u32x4*>(arow + i * 16 * PF_LROW + pos);
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[i][f] = mfma16<ACT>(av, bf[f], acc[i][f]);
    }
  }
}

template <int ACT>
__global__ __launch_bounds__(256, 1) void gemm_b_prefill(FastArgs a, int64_t tiles_m, int64_t tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wr = wave >> 1, wc = wave & 1;

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
  const int64_t m0 = tm * PF_BM;
  const int64_t n0 = tn * PF_BN;
  const int64_t ncol0 = n0 + wc * 64;
  const int slabs = (int)(a.k / PF_KS);
  const uint32_t k = (uint32_t)a.k;

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[i][f] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // x1 DMA offsets
  const uint16_t* xblk = a.x1 + m0 * a.k;
  const int rows_left = (int)(a.m - m0 < PF_BM ? a.m - m0 : PF_BM);
  const bool full_rows = rows_left == PF_BM;
  ADma dma;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (wave * 16 + j) * 4 + (lane >> 4);
    const int cj = (lane & 15) ^ (row & 15);
    dma.off[j] = (uint32_t)row * k + 8 * cj;
  }
  auto dma_a = [&](int slab, uint8_t* buf) {
    if (full_rows) pf_dma_a(xblk, dma, 4 * k, (uint32_t)slab * PF_KS, buf);
    else pf_dma_a_clamped(xblk, rows_left, k, (uint32_t)slab * PF_KS, buf);
  };
  // packed weight offsets (bytes from the wave's column block of a slab)
  const uint8_t* xw = a.x2 + ncol0 * 64;
  const int64_t slab_bytes = a.np * 64;
  int32_t boff[4];                                     // may be negative: the
#pragma unroll                                        // clamped column can lie
  for (int f = 0; f < 4; ++f) {                        // before ncol0
    int64_t col = ncol0 + 16 * f + (lane & 15);
    col = col < a.np ? col : a.np - 1;
    boff[f] = (int32_t)((col - ncol0) * 64 + (lane >> 4) * 16);
  }
  // scale offsets of the wave's 4 columns (clamped; columns past n get scale 0)
  uint32_t soff[4];
  float cmask[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int64_t col = ncol0 + 16 * f + (lane & 15);
    soff[f] = (uint32_t)((col < a.n ? col : a.n - 1) * a.s_col);
    cmask[f] = col < a.n ? 1.f : 0.f;
  }
  const int spg = (int)(a.group / PF_KS);              // slabs per group (>= 1)

  uint32_t bcur[4][4], bnext[4][4];
  dma_a(0, smem);
  pf_load_b(xw, boff, bcur);
  float svn[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) svn[f] = to_f32<ACT>(a.scale[soff[f]]) * cmask[f];
  __syncthreads();

  // acc holds the running sum in units of the current group's scale cs:
  // true sum = cs * acc. At a group with scale s: acc *= cs / s, then the
  // MFMAs add that group's x1 * (q + bias) to acc, and cs = s. A zero scale
  // zeroes the column's weight operand and leaves acc and cs unchanged.
  float cs[4] = {0.f, 0.f, 0.f, 0.f};
  uint32_t mk[4], mg[4];
  int gpos = 0;                                        // slab index within its group
  const uint16_t* srow_next = a.scale + a.s_row;       // scale row of the next group
  for (int s = 0; s < slabs; ++s) {
    const uint8_t* cur = smem + (s & 1) * PF_LBUF;
    const bool more = s + 1 < slabs;
    if (more) {
      dma_a(s + 1, smem + ((s + 1) & 1) * PF_LBUF);
      pf_load_b(xw + (s + 1) * slab_bytes, boff, bnext);
    }
    if (gpos == 0) {                                   // group start
      float ratio[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const float sg = svn[f];
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
    if (++gpos == spg) {                               // next slab starts a group
      gpos = 0;
      if (more) {
#pragma unroll
        for (int f = 0; f < 4; ++f) svn[f] = to_f32<ACT>(srow_next[soff[f]]) * cmask[f];
        srow_next += a.s_row;
      }
    }
    pf_slab<ACT>(cur, wr, bcur, mk, mg, acc);
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int c = 0; c < 4; ++c) bcur[f][c] = bnext[f][c];
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][f][r] *= cs[f];

  // ---- rank-1 remainder: acc += rowsum_g(x) * (o_g - bias * s_g) over groups,
  //      as MFMAs over the group axis on bf16 hi/lo splits ----
  for (int64_t g0 = 0; g0 < a.gp; g0 += 32) {
    // B operand: corr[g][col] for g = g0 + 8*(lane/16) .. +8, hi and lo
    u32x4 chi[4], clo[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int64_t col = ncol0 + 16 * f + (lane & 15);
      uint16_t h[8], l[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t g = g0 + 8 * (lane >> 4) + e;
        float corr = 0.f;
        if (col < a.n && g < a.groups) {
          const int64_t si = g * a.s_row + col * a.s_col;
          const float sv = to_f32<ACT>(a.scale[si]);
          const float ov = a.offset ? to_f32<ACT>(a.offset[si]) : 0.f;
          corr = ov - Magic<ACT>::bias * sv;
        }
        split_bf16(corr, h[e], l[e]);
      }
      chi[f] = (u32x4){h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                       h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16)};
      clo[f] = (u32x4){l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16),
                       l[4] | ((uint32_t)l[5] << 16), l[6] | ((uint32_t)l[7] << 16)};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t row = m0 + wr * 128 + 16 * i + (lane & 15);
      u32x4 rhi = {0u, 0u, 0u, 0u}, rlo = {0u, 0u, 0u, 0u};
      if (row < a.m) {
        const uint16_t* p = a.rs + row * 2 * a.gp + g0 + 8 * (lane >> 4);
        rhi = *reinterpret_cast<const u32x4*>(p);
        rlo = *reinterpret_cast<const u32x4*>(p + a.gp);
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        acc[i][f] = mfma16<ACT_BF16>(rhi, chi[f], acc[i][f]);
        acc[i][f] = mfma16<ACT_BF16>(rhi, clo[f], acc[i][f]);
        acc[i][f] = mfma16<ACT_BF16>(rlo, chi[f], acc[i][f]);
      }
    }
  }

  // ---- epilogue: y = acc + bias + residual; per-row sum of y^2 per 32 columns ----
  const int64_t t32 = ncol0 / 32;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float ss[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) ss[i][r] = 0.f;
#pragma unroll
    for (int f = 2 * h; f < 2 * h + 2; ++f) {
      const int64_t col = ncol0 + 16 * f + (lane & 15);
      const bool cin = col < a.n;
      const float bv = (cin && a.bias) ? to_f32<ACT>(a.bias[col]) : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t row = m0 + wr * 128 + 16 * i + 4 * (lane >> 4) + r;
          if (cin && row < a.m) {
            const int64_t idx = row * a.n + col;
            const float v = acc[i][f][r] + bv + to_f32<ACT>(a.residual[idx]);
            a.y[idx] = from_f32<ACT>(v);
            ss[i][r] = fmaf(v, v, ss[i][r]);
          }
        }
    }
    const bool valid = ncol0 + 32 * h < a.n;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = row16_sum(ss[i][r]);
        const int64_t row = m0 + wr * 128 + 16 * i + 4 * (lane >> 4) + r;
        if (valid && (lane & 15) == 0 && row < a.m) a.partial[(t32 + h) * a.m + row] = v;
      }
  }
}

template <int ACT>
hipError_t launch_prefill_t(const WqProblem& p, float* partial, uint16_t* rs, hipStream_t s) {
  FastArgs a;
  a.x1 = static_cast<const uint16_t*>(p.x1);
  a.x2 = static_cast<const uint8_t*>(p.x2);
  a.scale = static_cast<const uint16_t*>(p.scale);
  a.offset = static_cast<const uint16_t*>(p.offset);
  a.bias = static_cast<const uint16_t*>(p.bias);
  a.residual = static_cast<const uint16_t*>(p.residual);
  a.y = static_cast<uint16_t*>(p.y);
  a.partial = partial;
  a.rs = rs;
  a.m = p.m;
  a.k = p.k;
  a.n = p.n;
  a.np = 16 * ((p.n + 15) / 16);
  a.group = p.group >= p.k ? 128 * ((p.k + 127) / 128) : p.group;
  a.s_row = p.s_row;
  a.s_col = p.s_col;
  a.groups = (p.k + a.group - 1) / a.group;
  a.gp = 32 * ((a.groups + 31) / 32);
  group_rowsum_kernel<ACT><<<dim3((unsigned)p.m), 256, (size_t)(p.k / 8) * sizeof(float), s>>>(
      a.x1, p.k, a.group, a.groups, a.gp, rs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  static bool attr_set[2] = {false, false};
  if (!attr_set[ACT]) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_b_prefill<ACT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)PF_LDS);
    if (e != hipSuccess) return e;
    attr_set[ACT] = true;
  }
  const int64_t tm = (p.m + PF_BM - 1) / PF_BM, tn = (p.n + PF_BN - 1) / PF_BN;
  gemm_b_prefill<ACT><<<dim3((unsigned)(tm * tn)), 256, PF_LDS, s>>>(a, tm, tn);
  return hipGetLastError();
}

}  // namespace

bool fast_path_ok(const WqProblem& p) {
  if (p.w_bits != 4 || p.layout != WQ_LAYOUT_GFX950_B) return false;
  if (p.k % 128 != 0) return false;
  return p.group >= p.k || p.group % 128 == 0;
}

size_t fast_rowsum_bytes(int64_t m, int64_t k) {
  // worst case over group sizes: groups = ceil(k / 128)
  const int64_t groups = (k + 127) / 128;
  const int64_t gp = 32 * ((groups + 31) / 32);
  return (size_t)(m * 2 * gp * 2);
}

hipError_t launch_prefill(const WqProblem& p, float* partial, uint16_t* rs, hipStream_t s) {
  return p.bf16 ? launch_prefill_t<ACT_BF16>(p, partial, rs, s)
                : launch_prefill_t<ACT_F16>(p, partial, rs, s);
}

}  // namespace wq
