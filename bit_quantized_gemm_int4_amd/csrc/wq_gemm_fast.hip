// Fast weight-quantized GEMM for INT4 weights in the GFX950_B layout when the
// quantization group is a multiple of 128 along K (or per channel / per
// tensor) and k is a multiple of 128. Same operator as wq_gemm.hip
// (aclnnWeightQuantMatmulAllReduceAddRmsNorm page, Formula); this file holds
// the MFMA-bound tile used for large m.
//
// Arithmetic. With q the int4 code and B = q + 24 its exact 16-bit operand
// (wq_unpack.h), no weight is ever dequantized:
//   sum_k x[r,k] (q s + o) = s * sum_k x B  +  (o - 24 s) * sum_k x
// The MFMAs sum x * B straight into the float32 accumulator, kept in units of
// the current group's scale (rescaled by s_prev / s_g at each group start: one
// multiply per element per group; a zero scale zeroes that column's weight
// operand instead). The rank-1 remainder sum_g rowsum_g(x) (o_g - 24 s_g) is
// added at the end with MFMAs over the group axis on bf16 splits of both
// factors: the corrections in two parts (hi, lo), the row sums in three
// (hi, mid, lo). Groups of 128 take the three products hi*hi, hi*lo, mid*hi
// (relative error ~2^-16 per group, of independent sign across the many
// groups); larger groups, whose row sums are larger and fewer, add mid*lo
// and lo*hi (~2^-24): with activations of one sign a per-channel group's
// 24 * rowsum * s is many times the result. One pre-pass launch produces
// those factors:
// the per-group row sums of x1 and the per-group column corrections, both
// stored in MFMA operand order.
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

// three-part split: v ~= hi + mid + lo with |v - hi - mid - lo| <= 2^-24 |v|
// (each remainder is exact in float32)
__device__ __forceinline__ void split3_bf16(float v, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = from_f32<ACT_BF16>(v);
  const float r = v - to_f32<ACT_BF16>(hi);
  mid = from_f32<ACT_BF16>(r);
  lo = from_f32<ACT_BF16>(r - to_f32<ACT_BF16>(mid));
}


struct FastArgs {
  const uint16_t* x1;
  const uint8_t* x2;
  const uint16_t* scale;
  const uint16_t* bias;
  const uint16_t* residual;
  uint16_t* y;
  float* partial;          // [m][ceil(n/32)]
  const uint16_t* rs;      // [m][3][gp]  per-group row sums of x1, bf16 hi, mid, lo
  const uint16_t* corr;    // [np][2][gp] per-group o - bias*s per column, hi then lo
  int64_t m, k, n, np;
  int64_t group;           // K length of a group (multiple of 128, or >= k)
  int64_t s_row, s_col;
  int64_t groups, gp;      // groups = ceil(k / group); gp = 32 * ceil(groups / 32)
  uint32_t s_bytes;        // extent of the scale tensor in bytes
  const uint32_t* zflag;   // [ceil(np / 64)][ngb] nonzero: a zero scale in that 64-column x 32-group tile
  int ngb;                 // group tiles: gp / 32
};

// ---------------------------------------------------------------------------
// Pre-pass (one launch): the per-group row sums of x1 and the per-group
// column corrections, both written as bf16 hi/lo in MFMA operand order.
//   blocks [0, nct), nct = ncb * ngb: a tile of 64 columns x 32 groups of
//     o[g][n] - bias * s[g][n] (zero for padding), [np][2][gp]: read along the
//     columns (coalesced), transposed through LDS, written along the groups.
//     The tile also writes one word, nonzero when one of its scales is zero
//     (zflag[ci * ngb + gi]); the main tile ORs the words of its strip;
//   blocks [nct, nct + m): row b - nct's sums, [m][3][gp] (zero padded to gp
//     groups): eight-element chunk sums in LDS (each thread's loads issued
//     together), then each group summed in a fixed order.
// ---------------------------------------------------------------------------
constexpr int PC_COLS = 64, PC_GROUPS = 32;

template <int ACT>
__global__ __launch_bounds__(256) void prefill_prep(const uint16_t* __restrict__ x1, int64_t m, int64_t k,
                                                    int64_t group, int64_t groups, int64_t gp,
                                                    uint16_t* __restrict__ rs,
                                                    const uint16_t* __restrict__ scale,
                                                    const uint16_t* __restrict__ offset, int64_t n,
                                                    int64_t np, int64_t s_row, int64_t s_col, int ngb,
                                                    uint16_t* __restrict__ corr,
                                                    uint32_t* __restrict__ zflag) {
  extern __shared__ float sh[];               // max(k / 8 + k / 128, 32 * 65) floats
  const int t = threadIdx.x;
  // the correction tiles take the first blocks, so that the row blocks,
  // which only stream x1, make up the last round of workgroups
  const int64_t nct = ((np + PC_COLS - 1) / PC_COLS) * ngb;
  const int64_t b = blockIdx.x;
  if (b >= nct) {
    const int64_t row = b - nct;
    const uint16_t* xr = x1 + row * k;
    const int64_t chunks = k / 8;
    for (int64_t c0 = 0; c0 < chunks; c0 += 1024) {
      u32x4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t c = c0 + t + 256 * i;
        v[i] = c < chunks ? *reinterpret_cast<const u32x4*>(xr + 8 * c) : (u32x4){0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t c = c0 + t + 256 * i;
        float s = lo_f32<ACT>(v[i].x) + hi_f32<ACT>(v[i].x);
        s += lo_f32<ACT>(v[i].y) + hi_f32<ACT>(v[i].y);
        s += lo_f32<ACT>(v[i].z) + hi_f32<ACT>(v[i].z);
        s += lo_f32<ACT>(v[i].w) + hi_f32<ACT>(v[i].w);
        if (c < chunks) sh[c + (c >> 4)] = s;   // one pad float per 16 chunks
      }
    }
    __syncthreads();
    // chunks per group: a multiple of 16, so with the padding thread g's
    // reads start 17 * per / 16 floats after thread g - 1's (an odd stride
    // for groups of 128: the 64 lanes read 64 distinct banks)
    const int64_t per = group / 8;
    for (int64_t g = t; g < gp; g += 256) {
      float s = 0.f;
      if (g < groups) {
        const int64_t c1 = (g + 1) * per < chunks ? (g + 1) * per : chunks;
        for (int64_t c = g * per; c < c1; ++c) s += sh[c + (c >> 4)];
      }
      uint16_t hi, mid, lo;
      split3_bf16(s, hi, mid, lo);
      rs[row * 3 * gp + g] = hi;
      rs[row * 3 * gp + gp + g] = mid;
      rs[row * 3 * gp + 2 * gp + g] = lo;
    }
    return;
  }
  const int64_t cb = b;
  const int64_t ci = cb / ngb, gi = cb % ngb;
  float (*tile)[PC_COLS + 1] = reinterpret_cast<float (*)[PC_COLS + 1]>(sh);
  int zero = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int gl = t / PC_COLS + 4 * i, cl = t % PC_COLS;
    const int64_t col = ci * PC_COLS + cl, g = gi * PC_GROUPS + gl;
    float c = 0.f;
    if (col < n && g < groups) {
      const int64_t si = g * s_row + col * s_col;
      const float sv = to_f32<ACT>(scale[si]);
      const float ov = offset ? to_f32<ACT>(offset[si]) : 0.f;
      c = ov - Unpack<ACT>::bias * sv;
      zero |= sv == 0.f;
    }
    tile[gl][cl] = c;
  }
  zero = __syncthreads_or(zero);
  if (t == 0) zflag[cb] = zero ? 1u : 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = t + 256 * i;
    const int cl = idx / PC_GROUPS, gl = idx % PC_GROUPS;
    const int64_t col = ci * PC_COLS + cl, g = gi * PC_GROUPS + gl;
    if (col < np) {
      uint16_t hi, lo;
      split_bf16(tile[gl][cl], hi, lo);
      corr[col * 2 * gp + g] = hi;
      corr[col * 2 * gp + gp + g] = lo;
    }
  }
}

// ---------------------------------------------------------------------------
// Main tile
// ---------------------------------------------------------------------------
constexpr int WD_BM = 128, WD_BN = 512, WD_KS = 128;
constexpr int WD_GM = 4;                           // tile-rows per group of the tile order
constexpr int WD_LROW = WD_KS * 2;                 // LDS bytes per x1 row
constexpr int WD_ABUF = WD_BM * WD_LROW;           // x1 slab: 32 KiB
constexpr int WD_BBUF = WD_BN * 64;                // weight slab: 32 KiB
constexpr int WD_EROW = (64 + 4) * 4;              // epilogue staging row (fp32, padded)
static_assert(32 * WD_EROW <= 16384, "epilogue staging must fit a wave's 16 KiB region");

// x1 slab (128 rows x 128 K) -> LDS: 32 DMA instructions of 1 KiB (4 rows);
// wave w issues 4w + j: rows 16w + 4j + lane/16. LDS rows are 256 bytes; the
// 16-byte chunk of row r at position p holds logical chunk p ^ h(r & 15),
// with h linear over the bits of r: h(1) = 8, h(2) = 3, h(4) = 0, h(8) = 1.
// The 16-byte A-fragment reads (16 rows; in lane group g, K chunk 4g + d)
// then take no bank-conflict cycles: this map was picked from 200 random
// linear maps by the SQ_LDS_BANK_CONFLICT counter of an LDS probe on
// gfx950 that reads exactly these fragments (the earlier (r mod 4) * 4 +
// r / 4, like most maps tried, cost 2 cycles per read; the read cost does
// not follow a plain bank-count model). With r & 15 = 4j + lane/16 and h
// linear, h(r) = h(lane/16) ^ h(4j), so the lane's source chunk is
// c0 ^ h(4j), c0 = (lane & 15) ^ h(lane / 16), and its byte offset is
// (v0 ^ 16 h(4j)) + 8jk with v0 = (16w + lane/16) * 2k + 16 c0 (2k is a
// multiple of 256, so the XOR only touches the chunk bits). The buffer
// resource starts at the slab and ends after the tile's last row: rows past
// m read 0.
__host__ __device__ constexpr int wd_swz(int r) {
  return ((r & 1) ? 8 : 0) ^ ((r & 2) ? 3 : 0) ^ ((r & 8) ? 1 : 0);
}

__device__ __forceinline__ void wd_dma_a1(__amdgpu_buffer_rsrc_t ra, uint32_t v0, uint32_t k, uint8_t* buf,
                                          int j) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(buf + (4 * wave_id() + j) * 4 * WD_LROW), 16,
                                           (v0 ^ (16u * (uint32_t)wd_swz(4 * j))) + 8u * j * k, 0, 0, 0);
}

__device__ __forceinline__ void wd_dma_a(__amdgpu_buffer_rsrc_t ra, uint32_t v0, uint32_t k, uint8_t* buf) {
#pragma unroll
  for (int j = 0; j < 4; ++j) wd_dma_a1(ra, v0, k, buf, j);
}

// Weight slab for the tile's 512 columns (64 bytes per column in GFX950_B
// order) in 32 chunks of 16 columns (1 KiB), one DMA instruction each: wave
// w issues chunks 4w + j. Inside a chunk, 16-byte slot p holds column p / 4,
// K block b = (p % 4) ^ (p / 16), i.e. slot 4c + (b ^ (c / 4)) for column c:
// with the per-step dword rotation of wd_slab, every 64-lane 4-byte read of
// the weight fragments then hits 64 distinct banks. Lane l fetches slot l:
// byte v0 + 1024 j of the tile's slab row, v0 = 4096 w + 64 (l / 4) +
// 16 ((l % 4) ^ (l / 16)). The resource ends at the padded width: columns
// past it read 0 (never stored).
__device__ __forceinline__ uint32_t wd_b_v0(int wave, int lane) {
  return 4096u * wave + 64u * (lane >> 2) + 16u * ((lane & 3) ^ (lane >> 4));
}

__device__ __forceinline__ void wd_dma_b1(__amdgpu_buffer_rsrc_t rb, uint32_t v0, uint8_t* buf, int j) {
  // (the instruction's immediate offset would also move the LDS address, so
  // the 1 KiB step goes into the per-lane offset)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(buf + wave_id() * 4096 + 1024 * j), 16,
                                           v0 + 1024u * j, 0, 0, 0);
}

__device__ __forceinline__ void wd_dma_b(__amdgpu_buffer_rsrc_t rb, uint32_t v0, uint8_t* buf) {
#pragma unroll
  for (int j = 0; j < 4; ++j) wd_dma_b1(rb, v0, buf, j);
}

// One 128-deep slab accumulated into acc: acc[i][f] += sum over the slab of
// x1 * (q + bias), the MFMAs accumulating in place. The slab runs as four
// 32-deep K steps; a step is four passes (column tile f) of eight MFMAs (row
// tile i). The instruction order is fixed by hand (a scheduling barrier
// after every MFMA slot) so that each operand is held once and every load
// and unpack hides behind MFMAs:
//  - pass f of step c unpacks one weight fragment in five pieces between its
//    MFMAs: pass 0 fragment 3 of step c, pass f > 0 fragment f - 1 of step
//    c + 1 (the registers of a fragment are free once its pass is done);
//  - the packed dwords are read a step ahead: tiles 0..2 at the step start,
//    tile 3 in pass 1 (after pass 0 consumed the previous one);
//  - pass 3 refills A fragment i for step c + 1 right after its last MFMA;
//  - FIRST (the slab starts a quantization group): accumulator (i, f) is
//    rescaled by ratio[f] = old scale / new scale one MFMA slot before its
//    first MFMA of the slab;
//  - dma(n), n = 0..7, issues the n-th DMA instruction of the next slab in
//    slots 5 and 7 of the passes of step 0: spread between MFMAs, no wave
//    stalls on a full memory queue with its MFMAs waiting behind the loads.
// MASKED: per-lane masks mk / mc zero the weight operand of columns whose
// group scale is zero (otherwise the unpack constants apply).
template <int ACT, bool FIRST, bool MASKED, typename Dma>
__device__ __forceinline__ void wd_slab(const uint8_t* abuf, const uint8_t* wbuf,
                                        const UnpackKeys<ACT> (&keys)[4],
                                        const float (&ratio)[4], f32x4 (&acc)[8][4], const Dma& dma) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  // Step c gives lane group g = lane / 16 the 8 K values of dword
  // d = (c + g) % 4 of its 32-deep block (A chunk 4g + d), a rotation that
  // makes the weight reads conflict-free; each group still covers its block
  // once over the four steps.
  const int g = lane >> 4, cl = lane & 15;
  const int hcl = wd_swz(cl);                             // the row swizzle h(cl)
  const uint8_t* arow = abuf + cl * WD_LROW;
  const uint8_t* brow = wbuf + wave * 4096 + 16 * (4 * cl + (g ^ (cl >> 2)));
  auto a_at = [&](int i, int c) {
    return *reinterpret_cast<const u32x4*>(arow + i * 16 * WD_LROW + (((4 * g + ((c + g) & 3)) ^ hcl) * 16));
  };
  auto b_at = [&](int f, int c) {
    return *reinterpret_cast<const uint32_t*>(brow + f * 1024 + 4 * ((c + g) & 3));
  };
  auto rescale = [&](int i, int f) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[i][f][r] *= ratio[f];
  };
  using U = Unpack<ACT>;
  typename U::Src us;
  // piece p (0..4) of unpacking dword w of column tile f into out: the
  // sources, then one output dword per piece
  auto unpack_piece = [&](int p, uint32_t w, int f, u32x4& out) {
    UnpackKeys<ACT> kk;
    if (MASKED) kk = keys[f];
    else kk.set(true);
    if (p == 0) us = U::src(w, kk.m1, kk.c1);
    if (p == 1) out.x = U::template dword<0>(us, kk.m2, kk.c2);
    if (p == 2) out.y = U::template dword<1>(us, kk.m2, kk.c2);
    if (p == 3) out.z = U::template dword<2>(us, kk.m2, kk.c2);
    if (p == 4) out.w = U::template dword<3>(us, kk.m2, kk.c2);
  };

  uint32_t rw[4];
  u32x4 av[8], bf[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) rw[f] = b_at(f, 0);
#pragma unroll
  for (int i = 0; i < 8; ++i) av[i] = a_at(i, 0);
#pragma unroll
  for (int f = 0; f < 3; ++f)
#pragma unroll
    for (int p = 0; p < 5; ++p) unpack_piece(p, rw[f], f, bf[f]);
#pragma unroll
  for (int f = 0; f < 3; ++f) rw[f] = b_at(f, 1);
  if (FIRST) rescale(0, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (c > 0 && c + 1 < 4) {
#pragma unroll
      for (int f = 0; f < 3; ++f) rw[f] = b_at(f, c + 1);
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      // the fragment this pass unpacks: tile 3 of this step, or tile f - 1
      // of the next one
      const int uf = f == 0 ? 3 : f - 1;
      const bool unpacking = f == 0 || c + 1 < 4;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[i][f] = mfma16<ACT>(av[i], bf[f], acc[i][f]);
        if (FIRST && c == 0) {
          if (i < 7) rescale(i + 1, f);
          else if (f < 3) rescale(0, f + 1);
        }
        if (unpacking && i < 5) unpack_piece(i, rw[uf], uf, bf[uf]);
        if (f == 1 && i == 5 && c + 1 < 4) rw[3] = b_at(3, c + 1);
        if (f == 3 && c + 1 < 4) av[i] = a_at(i, c + 1);
        if (c == 0 && (i == 5 || i == 7)) dma(2 * f + (i == 7));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// The tile's K loop, rank-1 remainder and epilogue. EVERY: every slab starts
// a quantization group (group = 128), so each slab rescales inside its MFMA
// stream; otherwise the rescale runs before the first slab of a group.
template <int ACT, bool EVERY, bool MASKED>
__device__ __forceinline__ void wide_body(const FastArgs& a, int64_t m0, int64_t n0, uint8_t* abuf0,
                                          uint8_t* abuf1, uint8_t* wbuf0, uint8_t* wbuf1) {
  const int t = threadIdx.x, lane = t & 63, wave = wave_id();
  const int64_t ncol0 = n0 + wave * 64;             // the wave's first column
  const int slabs = (int)(a.k / WD_KS);
  const uint32_t k = (uint32_t)a.k;

  // ---- DMA sources: one base offset per lane and operand; the buffer
  //      resources are rebuilt per slab in scalar registers ----
  const int rows_left = (int)(a.m - m0 < WD_BM ? a.m - m0 : WD_BM);
  const uint32_t a_v0 = (uint32_t)(16 * wave + (lane >> 4)) * 2u * k +
                        16u * (uint32_t)((lane & 15) ^ wd_swz(lane >> 4));
  const uint32_t b_v0 = wd_b_v0(wave, lane);
  const int64_t slab_bytes = a.np * 64;
  // (the slab after the last one gets empty resources: its DMA, issued
  // unconditionally inside the last slab's MFMA stream, reads zeros and
  // touches no memory)
  auto rsrc_a = [&](int sl) {
    return buf_rsrc(a.x1 + m0 * a.k + (int64_t)sl * WD_KS,
                    sl < slabs ? (uint32_t)(rows_left * 2 * a.k - (int64_t)sl * 2 * WD_KS) : 0u);
  };
  auto rsrc_b = [&](int sl) {
    return buf_rsrc(a.x2 + sl * slab_bytes + n0 * 64, sl < slabs ? (uint32_t)((a.np - n0) * 64) : 0u);
  };
  // Scales: lane's column of tile f is ncol0 + 16 f + lane % 16; a column
  // past n reads scale 0 (its weight operand is then zeroed and it is never
  // stored). Raw 16-bit scales are kept two to a register.
  const __amdgpu_buffer_rsrc_t rscale = buf_rsrc(a.scale, a.s_bytes);
  auto load_scales = [&](int64_t g, uint32_t (&dst)[2]) {
    uint32_t v[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int64_t col = ncol0 + 16 * f + (lane & 15);
      v[f] = __builtin_amdgcn_raw_buffer_load_b16(
          rscale, col < a.n ? (uint32_t)(col * a.s_col * 2) : BUF_OOB, (uint32_t)(g * a.s_row * 2), 0);
    }
    dst[0] = v[0] | (v[1] << 16);
    dst[1] = v[2] | (v[3] << 16);
  };
  auto scale_of = [](const uint32_t (&sc)[2], int f) -> uint16_t {
    return (uint16_t)(sc[f >> 1] >> (16 * (f & 1)));
  };
  const int spg = (int)(a.group / WD_KS);              // slabs per group (>= 1)

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[i][f] = (f32x4){0.f, 0.f, 0.f, 0.f};

  wd_dma_a(rsrc_a(0), a_v0, k, abuf0);
  wd_dma_b(rsrc_b(0), b_v0, wbuf0);
  // raw scales of the current group and of the next one; the next group's
  // are loaded one step ahead, before that step's DMA, and used only after
  // the step's barrier, so waiting for them never waits for the DMA.
  uint32_t scur[2], snxt[2];
  load_scales(0, scur);
  __syncthreads();

  // acc holds the running sum in units of the current group's scale cs:
  // true sum = cs * acc. At a group with scale s: acc *= cs / s, then the
  // MFMAs add that group's x1 * (q + bias) to acc, and cs = s. A zero scale
  // zeroes the column's weight operand and leaves acc and cs unchanged.
  float cs[4] = {0.f, 0.f, 0.f, 0.f};
  float ratio[4];
  UnpackKeys<ACT> keys[4];                             // MASKED: per-lane unpack keys
  int gpos = 0;                                        // slab index within its group
  int64_t gnext = 1;                                   // the next group
  auto step = [&](int s, const uint8_t* acur, uint8_t* anxt, const uint8_t* wcur, uint8_t* wnxt) {
    const bool more = s + 1 < slabs;
    if (more && gpos == spg - 1) load_scales(gnext++, snxt);   // next slab starts a group
    const __amdgpu_buffer_rsrc_t ra_n = rsrc_a(s + 1), rb_n = rsrc_b(s + 1);
    auto dma = [&](int n) {
      if (n < 4) wd_dma_a1(ra_n, a_v0, k, anxt, n);
      else wd_dma_b1(rb_n, b_v0, wnxt, n - 4);
    };
    if (gpos == 0) {                                   // group start
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const float sg = to_f32<ACT>(scale_of(scur, f));
        const bool z = sg == 0.f;
        ratio[f] = (z || cs[f] == 0.f) ? 1.f : cs[f] * __builtin_amdgcn_rcpf(sg);   // ~2 ulp
        cs[f] = z ? cs[f] : sg;
        if (MASKED) keys[f].set(!z);
      }
      if (!EVERY) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][f][r] *= ratio[f];
      }
    }
    wd_slab<ACT, EVERY, MASKED>(acur, wcur, keys, ratio, acc, dma);
    if (++gpos == spg) {
      gpos = 0;
      scur[0] = snxt[0];
      scur[1] = snxt[1];
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

  // Residual rows for the epilogue, prefetched a quarter (32 rows) ahead so
  // their HBM latency hides behind the remainder MFMAs and the previous
  // quarter: lane (lr, lc) of quarter qt, pass st reads row 32 qt + 8 st + lr,
  // columns ncol0 + lc .. + 7. Rows past m and lanes outside the 16-byte path
  // read zeros (the latter use the element path below).
  const int lr = lane >> 3, lc = (lane & 7) * 8;       // row within 8, first column
  const int64_t col = ncol0 + lc;
  const bool vec = (a.n & 7) == 0 && col + 8 <= a.n;
  const int rows_here = (int)(a.m - m0 < WD_BM ? a.m - m0 : WD_BM);
  // (no residual: an empty resource, every lane reads zeros)
  const __amdgpu_buffer_rsrc_t rres = a.residual ? buf_rsrc(a.residual + m0 * a.n, (uint32_t)(rows_here * a.n * 2))
                                                 : buf_rsrc(a.x1, 0u);
  auto load_res = [&](int qt, u32x4 (&rr)[4]) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int rl = 32 * qt + 8 * st + lr;
      rr[st] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
          rres, vec && rl < rows_here ? (uint32_t)((rl * a.n + col) * 2) : BUF_OOB, 0, 0));
    }
  };
  u32x4 res_cur[4];
  // (the larger-group variant's five remainder products need the registers:
  // it fetches the first quarter after them)
  if (EVERY) load_res(0, res_cur);

  // ---- rank-1 remainder: acc += sum_g rowsum_g(x) * corr_g over the group
  //      axis, three (group 128) or five bf16 MFMA products per 32 groups ----
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
      const uint16_t* p = a.rs + row * 3 * a.gp + g0 + 8 * (lane >> 4);
      const u32x4 rhi = *reinterpret_cast<const u32x4*>(p);
      const u32x4 rmid = *reinterpret_cast<const u32x4*>(p + a.gp);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        acc[i][f] = mfma16<ACT_BF16>(rhi, chi[f], acc[i][f]);
        acc[i][f] = mfma16<ACT_BF16>(rhi, clo[f], acc[i][f]);
        acc[i][f] = mfma16<ACT_BF16>(rmid, chi[f], acc[i][f]);
      }
    }
    if (!EVERY) {
      // second pass (fewer operands live at once): mid * lo and lo * hi
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int64_t row = m0 + 16 * i + (lane & 15);
        row = row < a.m ? row : a.m - 1;
        const uint16_t* p = a.rs + row * 3 * a.gp + g0 + 8 * (lane >> 4);
        const u32x4 rmid = *reinterpret_cast<const u32x4*>(p + a.gp);
        const u32x4 rlo = *reinterpret_cast<const u32x4*>(p + 2 * a.gp);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          acc[i][f] = mfma16<ACT_BF16>(rmid, clo[f], acc[i][f]);
          acc[i][f] = mfma16<ACT_BF16>(rlo, chi[f], acc[i][f]);
        }
      }
    }
  }
  if (!EVERY) load_res(0, res_cur);

  // ---- epilogue, four quarters of 32 rows: stage the wave's 32 x 64 fp32
  //      block in LDS (32 rows x 272 bytes of its 16 KiB region), then each
  //      lane takes 8 consecutive columns of a row: y = acc + bias + residual
  //      with 16-byte loads/stores, and the row's sum of y^2 over each
  //      32-column half of the wave's columns ----
  uint8_t* stage = (wave < 2 ? abuf0 : wave < 4 ? abuf1 : wave < 6 ? wbuf0 : wbuf1) + (wave & 1) * 16384;
  float bv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) bv[e] = (a.bias && col + e < a.n) ? to_f32<ACT>(a.bias[col + e]) : 0.f;
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    u32x4 res_nxt[4];
    if (qt + 1 < 4) load_res(qt + 1, res_nxt);
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
#pragma unroll
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
          const u32x4 rv = res_cur[st];
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
              const float yv = v[e] + bv[e] + (a.residual ? to_f32<ACT>(a.residual[idx + e]) : 0.f);
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
    if (qt + 1 < 4) {
#pragma unroll
      for (int st = 0; st < 4; ++st) res_cur[st] = res_nxt[st];
    }
  }
}

template <int ACT, bool EVERY>
__global__ __launch_bounds__(512, 1) void gemm_b_wide(FastArgs a, int64_t tiles_m, int64_t tiles_n) {
  // Four LDS objects (two x1 slabs, two weight slabs): the compiler then sees
  // that the DMA filling one buffer does not alias reads of the other.
  __shared__ __attribute__((aligned(16))) uint8_t abuf0[WD_ABUF];
  __shared__ __attribute__((aligned(16))) uint8_t abuf1[WD_ABUF];
  __shared__ __attribute__((aligned(16))) uint8_t wbuf0[WD_BBUF];
  __shared__ __attribute__((aligned(16))) uint8_t wbuf1[WD_BBUF];
  const int t = threadIdx.x, lane = t & 63, wave = wave_id();

  // XCD-aware tile order: consecutive workgroups land on different XCDs, so
  // give each XCD a contiguous range of tiles. The range is walked in groups
  // of WD_GM tile-rows, down each group's rows and then across its columns:
  // the 32 tiles an XCD runs at once then span 4 tile-rows x 8 weight strips
  // (per 128-deep slab 4 x 32 KiB of x1 + 8 x 32 KiB of weight through its
  // L2), not 2 rows x 16 strips (2 x 32 + 16 x 32 KiB).
  const int64_t T = tiles_m * tiles_n;
  int64_t id = blockIdx.x;
  if ((T & 7) == 0) id = (id & 7) * (T >> 3) + (id >> 3);
  const int64_t grp = id / (WD_GM * tiles_n);
  const int64_t rows_g = tiles_m - grp * WD_GM < WD_GM ? tiles_m - grp * WD_GM : WD_GM;
  const int64_t rem = id - grp * WD_GM * tiles_n;
  const int64_t tm = grp * WD_GM + rem % rows_g;
  const int64_t tn = rem / rows_g;
  // wave-uniform by construction; readfirstlane lets the compiler keep the
  // tile origin (and the buffer resources built from it) in scalar registers
  const int64_t m0 = (int64_t)__builtin_amdgcn_readfirstlane((int)tm) * WD_BM;
  const int64_t n0 = (int64_t)__builtin_amdgcn_readfirstlane((int)tn) * WD_BN;
  // A tile with a zero group scale somewhere in its columns (flagged by the
  // correction pre-pass) or with columns past n runs the masked variant;
  // the branch is taken once, outside the K loop.
  uint32_t zf = 0;
  const int64_t c_end = (a.np + PC_COLS - 1) / PC_COLS;
  for (int64_t ci = n0 / PC_COLS; ci < n0 / PC_COLS + WD_BN / PC_COLS && ci < c_end; ++ci)
    for (int gi = 0; gi < a.ngb; ++gi) zf |= a.zflag[ci * a.ngb + gi];
  const bool masked = n0 + WD_BN > a.n || zf != 0;
  if (masked) wide_body<ACT, EVERY, true>(a, m0, n0, abuf0, abuf1, wbuf0, wbuf1);
  else wide_body<ACT, EVERY, false>(a, m0, n0, abuf0, abuf1, wbuf0, wbuf1);
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
  a.s_bytes = (uint32_t)(((a.groups - 1) * p.s_row + (p.n - 1) * p.s_col + 1) * 2);
  a.ngb = (int)(a.gp / PC_GROUPS);
  uint32_t* zflag = reinterpret_cast<uint32_t*>(corr + a.np * 2 * a.gp);
  a.zflag = zflag;
  const int64_t ncb = (a.np + PC_COLS - 1) / PC_COLS;
  const int64_t blocks = p.m + ncb * a.ngb;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int64_t row_floats = p.k / 8 + p.k / 128;    // chunk sums, one pad float per 16
  const int64_t sh_floats = row_floats > PC_GROUPS * (PC_COLS + 1) ? row_floats : PC_GROUPS * (PC_COLS + 1);
  prefill_prep<ACT><<<dim3((unsigned)blocks), 256, (size_t)sh_floats * sizeof(float), s>>>(
      a.x1, p.m, p.k, a.group, a.groups, a.gp, rs, a.scale, static_cast<const uint16_t*>(p.offset),
      p.n, a.np, p.s_row, p.s_col, a.ngb, corr, zflag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t tm = (p.m + WD_BM - 1) / WD_BM, tn = (p.n + WD_BN - 1) / WD_BN;
  prof_begin(s);
  if (a.group == WD_KS) gemm_b_wide<ACT, true><<<dim3((unsigned)(tm * tn)), 512, 0, s>>>(a, tm, tn);
  else gemm_b_wide<ACT, false><<<dim3((unsigned)(tm * tn)), 512, 0, s>>>(a, tm, tn);
  prof_end(s);
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
  return ((size_t)(m * 3 * gp * 2) + 255) & ~(size_t)255;
}
// ... followed by the zero-scale flags of the 64-column x 32-group tiles
size_t fast_corr_bytes(int64_t n, int64_t k) {
  const int64_t groups = (k + 127) / 128;
  const int64_t gp = 32 * ((groups + 31) / 32);
  const int64_t np = 16 * ((n + 15) / 16);
  const int64_t flags = (np + PC_COLS - 1) / PC_COLS * (gp / PC_GROUPS);
  return ((size_t)(np * 2 * gp * 2 + flags * 4) + 255) & ~(size_t)255;
}

hipError_t launch_prefill(const WqProblem& p, float* partial, uint16_t* rs, uint16_t* corr,
                          hipStream_t s) {
  return p.bf16 ? launch_wide_t<ACT_BF16>(p, partial, rs, corr, s)
                : launch_wide_t<ACT_F16>(p, partial, rs, corr, s);
}

}  // namespace wq
