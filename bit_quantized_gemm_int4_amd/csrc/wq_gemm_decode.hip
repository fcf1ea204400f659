// Decode-shaped weight-quantized GEMM (m <= 32) for INT4 weights in the
// GFX950_B layout or INT8 weights stored transposed (n, k), any group the
// pages allow (a multiple of 32 along K, or per channel / per tensor), k a
// multiple of 128. Same operator as wq_gemm.hip
// (aclnnWeightQuantMatmulAllReduceAddRmsNorm page, Formula); the RMSNorm
// finish runs as the next launch (rmsnorm_finish), which on this GPU costs
// less than any in-kernel grid synchronization: every cross-XCD handoff
// through memory (a write-through store's acknowledgement, an atomic on one
// address from every workgroup, a poll, a re-read) costs about as much as a
// kernel boundary's one cache release, and a grid-wide finish needs several.
//
// Weight stream. At small m the packed weight is almost all of the bytes.
// Every byte of x2 is read once, 16 bytes per lane per load; the 1 KiB a
// wave loads per instruction is one 128-deep K block of 16 columns (the
// GFX950_B unit), contiguous in memory.
//
// Work split. A workgroup (16 waves) owns CTW column tiles of 16 over all of
// K; CTW grows with n so that up to n = 12288 the grid stays within one
// workgroup per CU. Its waves split K: wave w takes 128-deep blocks
// [w*kpw, (w+1)*kpw), two blocks in flight: the loads of block b + 1
// (weights first, then the x1 rows by buffer -> LDS DMA into one of the
// wave's two LDS slots, one instruction per four rows of the launch, then
// the scales and offsets) are issued before block b is multiplied. The
// waves' sums meet in LDS and are added in a fixed wave order.
//
// Arithmetic per 128-deep block: the codes enter the MFMA as 16-bit
// B = q + 136 (fp16: q + 1032; wq_unpack.h, unpack8_low), one more MFMA
// against a ones fragment gives the row sums of x, and each group's share of
// the block is folded into the float32 result as
//   acc += s * sum_k x B  +  (o - 136 s) * sum_k x
// with s, o that group's scale and offset for the column: the constant
// cancels within one fold, so the cheaper unpack costs no accuracy here.
//
// Groups shorter than 128 (SPG = 32-deep K steps per fold: 1 for a group
// that is an odd multiple of 32, 2 for an odd multiple of 64, 4 otherwise).
// The GFX950_B load gives lane row R (lanes 16R .. 16R + 15) the four dwords
// of 32-deep sub-block R, so one MFMA step would mix all four sub-blocks.
// Two rounds of cross-row lane swaps (v_permlane32_swap, then
// v_permlane16_swap) transpose the 4 x 4 dwords: afterwards step j holds
// sub-block j in every row, i.e. K values 128 kb + 32 j .. + 31, which lie in
// one group, and the x1 fragments are fetched to match (row R, K values
// 32 j + 8 R .. + 7). Each fold unit accumulates into one of two MFMA
// accumulator sets and is folded while the next unit's MFMAs run; its scale
// and offset, loaded by the lanes of one row, reach the other rows by the
// same swaps.
//
// INT8 weights (W8, the transposed (n, k) layout: each column's K values
// contiguous) take the same path with 32 bytes per lane and block: lane row
// R loads K values 32 R .. + 31 of its column (two 16-byte loads), i.e. the
// layout of a GFX950_B sub-block at one byte per code, and step j uses its
// dwords 2 j and 2 j + 1. fp16 codes enter as q + 1152 (the byte with its
// sign bit flipped under the exponent byte 0x64: 1024 + q + 128, exact), the
// constant folded per block like the INT4 one; bf16 codes enter as q
// (converted through float32, exact for |q| <= 128).
//
// Epilogue: y = acc + bias + residual (stored rounded to the activation
// dtype) and, per (workgroup, row), the sum of the float32 y^2 over the
// workgroup's columns: partial[row][workgroup], so that the finish reads a
// row's sums as one contiguous run.
#include "wq_device.h"
#include "wq_internal.h"
#include "wq_unpack.h"

namespace wq {
namespace {

constexpr int DC_WAVES = 16;

struct DecodeArgs {
  const uint16_t* x1;
  const uint8_t* x2;
  const uint16_t* scale;
  const uint16_t* offset;    // the scale array when there is no offset (omul = 0)
  const uint16_t* bias;      // may be null
  const uint16_t* residual;  // may be null (the standalone matmul)
  uint16_t* y;
  float* partial;            // [m][grid]: sum of y^2 per (row, workgroup); null: none
  int64_t m, k, n, np, nct;  // nct = np / 16 column tiles
  int64_t row0;              // first of the 16 rows this launch computes
  int64_t s_row, s_col;      // scale element (g, n) at g * s_row + n * s_col
  uint32_t x1_bytes, x2_bytes, s_bytes, res_bytes;
  int32_t kpw;               // 128-deep K blocks per wave
  int32_t bpg;               // 128-deep K blocks per quantization group (SPG = 4)
  float upg_rcp;             // 1 / (fold units per group) (SPG < 4)
  float omul;                // 1 with an offset, 0 without
};

// fold units per 128-deep block, and MFMA accumulator sets (two for short
// groups: one unit accumulates while the previous one is folded)
template <int SPG>
constexpr int fold_units() { return 4 / SPG; }
template <int SPG>
constexpr int acc_sets() { return SPG == 4 ? 1 : 2; }

template <int CTW, int XD>
struct DecodeLane {
  __amdgpu_buffer_rsrc_t w, x, s, o;
  uint32_t woff[CTW];        // lane's first weight byte in block 0, per column tile
  uint32_t xoff[XD];         // x1 bytes the lane fetches in DMA d of a block (BUF_OOB past m)
  uint32_t soff[CTW];        // scale element per tile (SPG = 4: [0] only, tile of the lane row)
};

// One 128-deep block's register loads (its x1 fragments go to LDS).
template <int CTW, bool W8>
struct DecodeBatch {
  u32x4 w[W8 ? 2 * CTW : CTW];   // INT4: dword w4 of tile c feeds K step w4; INT8: tile c in w[2c], w[2c + 1]
  uint32_t s[CTW], o[CTW];       // raw 16-bit scale and offset
};

// vector-memory instructions one batch issues: weights, XD x1 DMAs, scales
// and offsets (SPG = 4: one of each, lane row R holding tile R's)
template <int CTW, int SPG, bool W8, int XD>
constexpr int batch_loads() { return (W8 ? 2 : 1) * CTW + XD + (SPG == 4 ? 2 : 2 * CTW); }

// The constant the 16-bit operand adds to a code: INT4 q + 136 / q + 1032
// (unpack8_low), INT8 q + 1152 in fp16, q itself in bf16.
template <int ACT, bool W8>
constexpr float code_bias() {
  return W8 ? (ACT == ACT_F16 ? 1152.f : 0.f) : UnpackLow<ACT>::bias;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Eight INT8 codes (lo: K 0..3, hi: K 4..7, K ascending from the low byte)
// -> the MFMA operand of one step.
template <int ACT>
__device__ __forceinline__ u32x4 i8_operand(uint32_t lo, uint32_t hi) {
  if constexpr (ACT == ACT_F16) {
    const uint32_t ul = lo ^ 0x80808080u, uh = hi ^ 0x80808080u;
    return (u32x4){__builtin_amdgcn_perm(0x64646464u, ul, 0x04010400u),
                   __builtin_amdgcn_perm(0x64646464u, ul, 0x04030402u),
                   __builtin_amdgcn_perm(0x64646464u, uh, 0x04010400u),
                   __builtin_amdgcn_perm(0x64646464u, uh, 0x04030402u)};
  } else {
    auto pair = [](uint32_t w, int j) {
      const f32x2 f = {(float)(int)(int8_t)(w >> (8 * j)), (float)(int)(int8_t)(w >> (8 * j + 8))};
      return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
    };
    return (u32x4){pair(lo, 0), pair(lo, 2), pair(hi, 0), pair(hi, 2)};
  }
}

// Loop-carried MFMA accumulators of a wave: the block's partial sums per
// column tile and the block's row sums of x. Every MFMA updates them in
// place (cleared in place by a multiply with zero at each block start), so
// each MFMA's destination is exactly its accumulator source and never
// overlaps its A or B operand.
template <int CTW, int NS>
struct DecodeAcc {
  f32x4 part[NS][CTW];       // per accumulator set
  f32x4 rs[NS];
};

// One buffer -> LDS DMA instruction: 16 bytes per lane, written to dst in
// lane order.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, soff, 0, 0);
}

// x1 staging. A block's x1 slot holds row r's 128 K values (sixteen 16-byte
// chunks, chunk j = K values 8 j .. + 7) at xs + 256 r, chunk j in slot
// j ^ r, which spreads the sixteen rows of one MFMA operand read over the
// banks (the bank-conflict counter still shows about four cycles per read,
// a few hundredths of a microsecond per wave).
// DMA d fetches rows 4 d .. 4 d + 3 (a DMA instruction writes its 64 lanes'
// 16 bytes in lane order: lane i lands in row 4 d + i/16, slot i%16, so it
// fetches chunk (i%16) ^ row). XD = ceil(rows / 4) DMAs: rows past the
// launch's last are not fetched, and their MFMA output rows are discarded.
//
// K step w4 pairs the weight dword w4 of lane l (K values 32 (l/16) + 8 w4
// .. + 7 of its column: the lane's GFX950_B sub-block) with the same eight K
// values of x1 row l%16: chunk 4 (l/16) + w4. With SPG < 4 the weights are
// transposed across lane rows and step w4 takes chunk 4 w4 + l/16.
//
// Scales: with SPG = 4 lane row R loads tile min(R, CTW - 1)'s scale and
// offset, broadcast to the other rows at the fold. With SPG < 4 lane row R
// loads the scale and offset of fold unit R / SPG for every tile: group
// floor((unit + 1/2) / upg) with upg fold units per group, exact in float32
// for every unit index below 2^11 (k < 2^16).
template <int CTW, int SPG, bool W8, int XD>
__device__ __forceinline__ void issue_batch(const DecodeArgs& a, const DecodeLane<CTW, XD>& ln, int kb,
                                            uint8_t* xs, DecodeBatch<CTW, W8>& b) {
  if constexpr (W8) {
    const uint32_t wso = (uint32_t)kb * 128u;
#pragma unroll
    for (int c = 0; c < CTW; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        b.w[2 * c + h] =
            __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ln.w, ln.woff[c] + 16u * h, wso, 0));
  } else {
    const uint32_t wso = (uint32_t)kb * (uint32_t)a.np * 64u;
#pragma unroll
    for (int c = 0; c < CTW; ++c)
      b.w[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ln.w, ln.woff[c], wso, 0));
  }
#pragma unroll
  for (int d = 0; d < XD; ++d) dma16(ln.x, xs + 1024 * d, ln.xoff[d], (uint32_t)kb * 256u);
  if constexpr (SPG == 4) {
    const uint32_t sso = (uint32_t)((kb / a.bpg) * a.s_row) * 2u;
    b.s[0] = __builtin_amdgcn_raw_buffer_load_b16(ln.s, ln.soff[0], sso, 0);
    b.o[0] = __builtin_amdgcn_raw_buffer_load_b16(ln.o, ln.soff[0], sso, 0);
  } else {
    const int unit = kb * fold_units<SPG>() + (int)((threadIdx.x & 63) >> 4) / SPG;
    const uint32_t g = (uint32_t)(((float)unit + 0.5f) * a.upg_rcp);
    const uint32_t vso = g * (uint32_t)a.s_row * 2u;
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
      b.s[c] = __builtin_amdgcn_raw_buffer_load_b16(ln.s, ln.soff[c] + vso, 0u, 0);
      b.o[c] = __builtin_amdgcn_raw_buffer_load_b16(ln.o, ln.soff[c] + vso, 0u, 0);
    }
  }
}

// Byte offset of lane l's x1 fragment for K step w4 in a block's slot.
template <int SPG>
__device__ __forceinline__ uint32_t x1_frag(int lane, int w4) {
  const int r = lane & 15, kq = lane >> 4;
  const int j = SPG == 4 ? 4 * kq + w4 : 4 * w4 + kq;
  return (uint32_t)(256 * r + 16 * (j ^ r));
}

// Cross-row lane swaps (rows of 16 lanes, r0 .. r3), in the layout of the
// gfx950 instructions:
//   v_permlane32_swap(a, b): a' = [a0, a1, b0, b1], b' = [a2, a3, b2, b3]
//   v_permlane16_swap(a, b): a' = [a0, b0, a2, b2], b' = [a1, b1, a3, b3]
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

// 4 x 4 transpose of (lane row, register): register j of row R <- register
// R of row j.
__device__ __forceinline__ u32x4 transpose_rows(u32x4 d) {
  uint32_t d0 = d[0], d1 = d[1], d2 = d[2], d3 = d[3];
  swap32(d0, d2);
  swap32(d1, d3);
  swap16(d0, d1);
  swap16(d2, d3);
  return (u32x4){d0, d1, d2, d3};
}

// Row U * SPG of v (the value that lane row loaded for fold unit U) to
// every row.
template <int SPG, int U>
__device__ __forceinline__ float bcast_unit(float v) {
  uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
  swap32(a, b);                              // a = [r0, r1, r0, r1], b = [r2, r3, r2, r3]
  uint32_t x = (U * SPG) < 2 ? a : b;
  if constexpr (SPG == 1) {
    uint32_t y = x;
    swap16(x, y);                            // x = [x0, x0, x0, x0], y = [x1, x1, x1, x1]
    x = (U & 1) ? y : x;
  }
  return __builtin_bit_cast(float, x);
}

// The per-step weight words of one tile: INT4 one dword per step (src.x ..
// src.w), INT8 two (lo[j], hi[j]); with short groups transposed across lane
// rows so that step j holds 32-deep sub-block j in every row.
template <bool W8>
struct StepWords {
  u32x4 lo, hi;    // hi unused for INT4
};

template <int SPG, bool W8>
__device__ __forceinline__ StepWords<W8> step_words(const u32x4* w) {
  StepWords<W8> r;
  if constexpr (W8) {
    r.lo = (u32x4){w[0].x, w[0].z, w[1].x, w[1].z};
    r.hi = (u32x4){w[0].y, w[0].w, w[1].y, w[1].w};
    if constexpr (SPG < 4) {
      r.lo = transpose_rows(r.lo);
      r.hi = transpose_rows(r.hi);
    }
  } else {
    r.lo = SPG == 4 ? w[0] : transpose_rows(w[0]);
  }
  return r;
}

template <int ACT, bool W8>
__device__ __forceinline__ u32x4 step_operand(const StepWords<W8>& sw, int j) {
  if constexpr (W8) return i8_operand<ACT>(sw.lo[j], sw.hi[j]);
  else return unpack8_low<ACT>(sw.lo[j]);
}

template <int ACT, int CTW, int SPG, bool W8>
__device__ __forceinline__ void mma_batch(const DecodeArgs& a, const DecodeBatch<CTW, W8>& b, const uint8_t* xs,
                                          DecodeAcc<CTW, acc_sets<SPG>()>& ma, f32x4 (&acc)[CTW]) {
  constexpr int U = fold_units<SPG>();
  constexpr int WPT = W8 ? 2 : 1;            // weight registers per tile
  constexpr float BIAS = code_bias<ACT, W8>();
  const int lane = threadIdx.x & 63;
  const uint32_t one2 = pack2<ACT>(1.f, 1.f);
  const u32x4 ones = {one2, one2, one2, one2};
  StepWords<W8> w[CTW];
#pragma unroll
  for (int c = 0; c < CTW; ++c) w[c] = step_words<SPG, W8>(&b.w[WPT * c]);
  if constexpr (SPG == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ma.rs[0][i] *= 0.f;
#pragma unroll
    for (int c = 0; c < CTW; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) ma.part[0][c][i] *= 0.f;
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      const u32x4 av = *reinterpret_cast<const u32x4*>(xs + x1_frag<SPG>(lane, w4));
      ma.rs[0] = mfma16<ACT>(av, ones, ma.rs[0]);
#pragma unroll
      for (int c = 0; c < CTW; ++c) ma.part[0][c] = mfma16<ACT>(av, step_operand<ACT, W8>(w[c], w4), ma.part[0][c]);
      // one K step's operands at a time (bounds the live unpacked fragments)
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane row R loaded tile min(R, CTW - 1)'s scale and offset
    const float s_r = to_f32<ACT>((uint16_t)b.s[0]);
    const float o_r = to_f32<ACT>((uint16_t)b.o[0]) * a.omul;
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
      float s = s_r, o = o_r;
      if constexpr (CTW > 1) {
        switch (c) {   // unrolled: a constant row index
          case 0: s = bcast_unit<1, 0>(s_r); o = bcast_unit<1, 0>(o_r); break;
          case 1: s = bcast_unit<1, 1>(s_r); o = bcast_unit<1, 1>(o_r); break;
          default: s = bcast_unit<1, 2>(s_r); o = bcast_unit<1, 2>(o_r); break;
        }
      }
      const float cc = o - BIAS * s;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[c][i] = fmaf(s, ma.part[0][c][i], fmaf(cc, ma.rs[0][i], acc[c][i]));
    }
  } else {
    // lane row R holds the scale and folded offset of unit R / SPG
    float sr[CTW], cr[CTW];
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
      sr[c] = to_f32<ACT>((uint16_t)b.s[c]);
      cr[c] = to_f32<ACT>((uint16_t)b.o[c]) * a.omul - BIAS * sr[c];
    }
    // unit u accumulates into set u % 2 and is folded after unit u + 1's
    // MFMAs are issued, so the fold does not wait on its own MFMAs
#pragma unroll
    for (int u = 0; u <= U; ++u) {
      if (u < U) {
        const int st = u & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) ma.rs[st][i] *= 0.f;
#pragma unroll
        for (int c = 0; c < CTW; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) ma.part[st][c][i] *= 0.f;
#pragma unroll
        for (int w4 = u * SPG; w4 < (u + 1) * SPG; ++w4) {
          const u32x4 av = *reinterpret_cast<const u32x4*>(xs + x1_frag<SPG>(lane, w4));
          ma.rs[st] = mfma16<ACT>(av, ones, ma.rs[st]);
#pragma unroll
          for (int c = 0; c < CTW; ++c)
            ma.part[st][c] = mfma16<ACT>(av, step_operand<ACT, W8>(w[c], w4), ma.part[st][c]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (u > 0) {
        const int ps = (u - 1) & 1;
#pragma unroll
        for (int c = 0; c < CTW; ++c) {
          float su, cu;
          switch (u - 1) {   // unrolled: a constant unit index
            case 0: su = bcast_unit<SPG, 0>(sr[c]); cu = bcast_unit<SPG, 0>(cr[c]); break;
            case 1: su = bcast_unit<SPG, 1>(sr[c]); cu = bcast_unit<SPG, 1>(cr[c]); break;
            case 2: su = bcast_unit<SPG, 2>(sr[c]); cu = bcast_unit<SPG, 2>(cr[c]); break;
            default: su = bcast_unit<SPG, 3>(sr[c]); cu = bcast_unit<SPG, 3>(cr[c]); break;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[c][i] = fmaf(su, ma.part[ps][c][i], fmaf(cu, ma.rs[ps][i], acc[c][i]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

template <int ACT, int CTW, int SPG, bool W8, int XD>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4, 4))) void gemm_decode(DecodeArgs a) {
  constexpr int RS = CTW * 16 + 4;                  // reduction row stride (floats)
  // per wave: two 4 KiB x1 slots, reused after the K loop for the wave's
  // share of the cross-wave sum
  __shared__ __attribute__((aligned(16))) uint8_t xlds[DC_WAVES][2][4096];
  static_assert(16 * RS * 4 <= 2 * 4096, "reduction rows must fit a wave's slots");
  __shared__ float sq[16 * CTW * 8];                // per-thread sums of y^2
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);      // uniform: K ranges are scalar
  const int col = lane & 15, kq = lane >> 4;
  const int64_t ct0 = (int64_t)blockIdx.x * CTW;
  const int64_t n0 = ct0 * 16;
  const int64_t ctn = a.nct - ct0 < CTW ? a.nct - ct0 : CTW;   // tiles this workgroup stores

  // Lane offsets: weight column 16 * tile + l%16 (tile clamped to the last
  // one; a partial last workgroup discards the repeats), 32-deep sub-block
  // l/16; x1 row row0 + 4 d + l/16 of DMA d, chunk (l%16) ^ that local row
  // (rows >= m read zeros); scale column clamped to n - 1. Every offset a
  // valid lane uses stays inside its buffer.
  DecodeLane<CTW, XD> ln;
  ln.w = buf_rsrc(a.x2, a.x2_bytes);
  ln.x = buf_rsrc(a.x1, a.x1_bytes);
  ln.s = buf_rsrc(a.scale, a.s_bytes);
  ln.o = buf_rsrc(a.offset, a.s_bytes);
#pragma unroll
  for (int d = 0; d < XD; ++d) {
    const int q = 4 * d + kq;                       // local row 0..15
    const int64_t xrow = a.row0 + q;
    ln.xoff[d] = xrow < a.m ? (uint32_t)(xrow * a.k * 2 + 16 * (col ^ q)) : BUF_OOB;
  }
  auto scol = [&](int c) { return n0 + 16 * c + col < a.n ? n0 + 16 * c + col : a.n - 1; };
#pragma unroll
  for (int c = 0; c < CTW; ++c) {
    const int64_t ct = ct0 + c < a.nct ? ct0 + c : a.nct - 1;
    // INT4: the GFX950_B record's sub-block kq; INT8: 32 bytes of column
    // row (n, k), past n out of the weight (reads zeros)
    ln.woff[c] = W8 ? (uint32_t)((ct * 16 + col) * a.k + kq * 32) : (uint32_t)((ct * 16 + col) * 64 + kq * 16);
    ln.soff[c] = (uint32_t)(scol(c) * a.s_col * 2);
  }
  if constexpr (SPG == 4) ln.soff[0] = (uint32_t)(scol(kq < CTW ? kq : CTW - 1) * a.s_col * 2);

  // Epilogue mapping (two adjacent columns of one row per thread, TPR threads
  // per row); its residual and bias values are fetched before the K loop so
  // that they arrive while the weights stream.
  constexpr int TPR = CTW * 8;
  const bool epi = t < 16 * TPR;
  const int r = t / TPR, cp = t % TPR, c = 2 * cp;
  const int64_t col0 = n0 + c;
  const bool tile_ok = epi && (c >> 4) < ctn;
  const bool c0ok = tile_ok && col0 < a.n, c1ok = tile_ok && col0 + 1 < a.n;
  const int64_t orow = a.row0 + r;
  const bool rok = epi && orow < a.m;
  const bool pair = (a.n & 1) == 0 && c1ok;       // y rows start 4-byte aligned
  const int64_t idx = orow * a.n + col0;
  // Unconditional buffer loads (an invalid element reads zero; no bias is a
  // zero-size buffer, as is no residual), so nothing forces a wait before the
  // stream is issued.
  const __amdgpu_buffer_rsrc_t rres = buf_rsrc(a.residual ? a.residual : a.x1, a.residual ? a.res_bytes : 0u);
  const __amdgpu_buffer_rsrc_t rbias = buf_rsrc(a.bias ? a.bias : a.x1, a.bias ? (uint32_t)(a.n * 2) : 0u);
  const uint32_t r0 = __builtin_amdgcn_raw_buffer_load_b16(rres, rok && c0ok ? (uint32_t)(idx * 2) : BUF_OOB, 0, 0);
  const uint32_t r1 = __builtin_amdgcn_raw_buffer_load_b16(rres, rok && c1ok ? (uint32_t)(idx * 2 + 2) : BUF_OOB, 0, 0);
  const uint32_t b0 = __builtin_amdgcn_raw_buffer_load_b16(rbias, c0ok ? (uint32_t)(col0 * 2) : BUF_OOB, 0, 0);
  const uint32_t b1 = __builtin_amdgcn_raw_buffer_load_b16(rbias, c1ok ? (uint32_t)(col0 * 2 + 2) : BUF_OOB, 0, 0);

  // ---- weight stream: blocks [kb0, kb1), two in flight ----
  const int kbs = (int)(a.k / 128);
  const int kb0 = wave * a.kpw;
  const int kb1 = kb0 + a.kpw < kbs ? kb0 + a.kpw : kbs;
  f32x4 acc[CTW];
  DecodeAcc<CTW, acc_sets<SPG>()> ma;
#pragma unroll
  for (int u = 0; u < acc_sets<SPG>(); ++u) {
    ma.rs[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < CTW; ++i) ma.part[u][i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < CTW; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // Batch b's loads complete in issue order, so once no more than the next
  // batch's loads are outstanding, b's weights, DMA and scales have landed
  // (the explicit wait also orders the LDS reads after the DMA, which the
  // compiler does not do by itself). The scheduling barriers keep every load
  // ahead of the first use.
  uint8_t* xa = xlds[wave][0];
  uint8_t* xb = xlds[wave][1];
  DecodeBatch<CTW, W8> ba, bb;
  if (kb0 < kb1) issue_batch<CTW, SPG, W8, XD>(a, ln, kb0, xa, ba);
  for (int kb = kb0; kb < kb1; kb += 2) {
    if (kb + 1 < kb1) issue_batch<CTW, SPG, W8, XD>(a, ln, kb + 1, xb, bb);
    __builtin_amdgcn_sched_barrier(0);
    if (kb + 1 < kb1) wait_vm<batch_loads<CTW, SPG, W8, XD>()>();
    else wait_vm<0>();
    __builtin_amdgcn_sched_barrier(0);
    mma_batch<ACT, CTW, SPG, W8>(a, ba, xa, ma, acc);
    __builtin_amdgcn_sched_barrier(0);
    if (kb + 1 >= kb1) break;
    if (kb + 2 < kb1) issue_batch<CTW, SPG, W8, XD>(a, ln, kb + 2, xa, ba);
    __builtin_amdgcn_sched_barrier(0);
    if (kb + 2 < kb1) wait_vm<batch_loads<CTW, SPG, W8, XD>()>();
    else wait_vm<0>();
    __builtin_amdgcn_sched_barrier(0);
    mma_batch<ACT, CTW, SPG, W8>(a, bb, xb, ma, acc);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- combine the waves' K slices in a fixed order ----
  // (the wave's own LDS reads are complete: their values fed its MFMAs)
  float* myred = reinterpret_cast<float*>(xlds[wave][0]);
#pragma unroll
  for (int i = 0; i < CTW; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) myred[(4 * kq + e) * RS + i * 16 + col] = acc[i][e];
  __syncthreads();

  // ---- epilogue: y = acc + bias + residual; sums of y^2 ----
  float ss = 0.f;
  if (epi) {
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int w = 0; w < DC_WAVES; ++w) {
      const float* rw = reinterpret_cast<const float*>(xlds[w][0]);
      v0 += rw[r * RS + c];
      v1 += rw[r * RS + c + 1];
    }
    if (rok) {
      float y0 = v0 + to_f32<ACT>((uint16_t)b0) + to_f32<ACT>((uint16_t)r0);
      float y1 = v1 + to_f32<ACT>((uint16_t)b1) + to_f32<ACT>((uint16_t)r1);
      const uint32_t o2 = pack2<ACT>(y0, y1);
      if (pair) {
        *reinterpret_cast<uint32_t*>(a.y + idx) = o2;
      } else {
        if (c0ok) a.y[idx] = (uint16_t)(o2 & 0xFFFFu);
        if (c1ok) a.y[idx + 1] = (uint16_t)(o2 >> 16);
      }
      y0 = c0ok ? y0 : 0.f;                 // the sum of squares uses float32 y
      y1 = c1ok ? y1 : 0.f;
      ss = y0 * y0 + y1 * y1;
    }
    sq[t] = ss;
  }
  if (!a.partial) return;                   // the standalone matmul: no norm
  __syncthreads();
  if (t < 16 && a.row0 + t < a.m) {
    float s = 0.f;
    for (int i = 0; i < TPR; ++i) s += sq[t * TPR + i];
    a.partial[(a.row0 + t) * gridDim.x + blockIdx.x] = s;
  }
}

template <int ACT, bool W8, int XD>
void launch_spg4(const DecodeArgs& a, int ctw, unsigned grid, hipStream_t s) {
  switch (ctw) {
    case 1: gemm_decode<ACT, 1, 4, W8, XD><<<dim3(grid), 1024, 0, s>>>(a); break;
    case 2: gemm_decode<ACT, 2, 4, W8, XD><<<dim3(grid), 1024, 0, s>>>(a); break;
    default:
      if constexpr (!W8) gemm_decode<ACT, 3, 4, W8, XD><<<dim3(grid), 1024, 0, s>>>(a);
      break;
  }
}

// xd: x1 DMAs per block, 1, 2 or 4 for at most 4, 8 or 16 rows in the launch
// (short groups always take 4)
template <int ACT, bool W8>
void launch_fmt(const DecodeArgs& a, int spg, int ctw, int xd, unsigned grid, hipStream_t s) {
  if (spg == 4) {
    if (xd == 1) launch_spg4<ACT, W8, 1>(a, ctw, grid, s);
    else if (xd == 2) launch_spg4<ACT, W8, 2>(a, ctw, grid, s);
    else launch_spg4<ACT, W8, 4>(a, ctw, grid, s);
  } else if (spg == 2) {
    if (W8 || ctw == 1) gemm_decode<ACT, 1, 2, W8, 4><<<dim3(grid), 1024, 0, s>>>(a);
    else if constexpr (!W8) gemm_decode<ACT, 2, 2, W8, 4><<<dim3(grid), 1024, 0, s>>>(a);
  } else {
    if (W8 || ctw == 1) gemm_decode<ACT, 1, 1, W8, 4><<<dim3(grid), 1024, 0, s>>>(a);
    else if constexpr (!W8) gemm_decode<ACT, 2, 1, W8, 4><<<dim3(grid), 1024, 0, s>>>(a);
  }
}

template <int ACT>
void launch_act(const DecodeArgs& a, bool w8, int spg, int ctw, int xd, unsigned grid, hipStream_t s) {
  prof_begin(s);
  if (w8) launch_fmt<ACT, true>(a, spg, ctw, xd, grid, s);
  else launch_fmt<ACT, false>(a, spg, ctw, xd, grid, s);
  prof_end(s);
}

// 32-deep K steps per fold: a group (>= 32, a multiple of 32) that is not a
// multiple of 128 folds every 64 (an even multiple of 32) or every 32 K.
int decode_spg(const WqProblem& p) {
  if (p.group >= p.k || p.group % 128 == 0) return 4;
  return p.group % 64 == 0 ? 2 : 1;
}

// column tiles per workgroup: keep the grid within one workgroup per CU up to
// 768 tiles (n = 12288); wider layers take more workgroups of 3. Within the
// register budget of 16 waves per CU, the second accumulator set of short
// groups caps the tiles at 2, the INT8 weights' doubled registers at 2, both
// together at 1.
int decode_ctw(int64_t nct, int spg, bool w8) {
  const int ctw = nct <= 256 ? 1 : nct <= 512 ? 2 : 3;
  const int cap = spg == 4 ? (w8 ? 2 : 3) : (w8 ? 1 : 2);
  return ctw < cap ? ctw : cap;
}

bool decode_w8(const WqProblem& p) { return p.w_bits == 8; }

}  // namespace

// INT4 in the GFX950_B layout or INT8 stored (n, k), k a multiple of 128,
// m <= 32. The weight stream addresses the weight through one buffer
// resource whose out-of-range offset is 2^31: the weight (with the INT8
// columns of a partial last tile) must stay below 2 GiB.
bool decode_ok(const WqProblem& p) {
  if (p.k % 128 != 0 || p.m > 32) return false;
  if (p.group < p.k && p.group % 32 != 0) return false;
  const int64_t np = 16 * ((p.n + 15) / 16);
  if (p.w_bits == 4 && p.layout == WQ_LAYOUT_GFX950_B) return (p.k / 128) * np * 64 < (int64_t(1) << 31);
  if (p.w_bits == 8 && p.transpose_x2) return np * p.k < (int64_t(1) << 31);
  return false;
}

// Per-(row, workgroup) sums of y^2 of the decode kernel: [32][grid] at most.
int64_t decode_grid(const WqProblem& p) {
  const int64_t nct = (p.n + 15) / 16;
  const int ctw = decode_ctw(nct, decode_spg(p), decode_w8(p));
  return (nct + ctw - 1) / ctw;
}
size_t decode_partial_bytes(int64_t n) {
  // the largest grid over the fold shapes and weight formats
  const int64_t nct = (n + 15) / 16;
  int64_t grid = 0;
  for (int w8 = 0; w8 < 2; ++w8)
    for (int spg = 1; spg <= 4; spg *= 2) {
      const int ctw = decode_ctw(nct, spg, w8 != 0);
      const int64_t g = (nct + ctw - 1) / ctw;
      grid = g > grid ? g : grid;
    }
  return (size_t)(grid * 32 * 4);
}

hipError_t launch_decode(const WqProblem& p, float* partial, hipStream_t s) {
  DecodeArgs a;
  a.x1 = static_cast<const uint16_t*>(p.x1);
  a.x2 = static_cast<const uint8_t*>(p.x2);
  a.scale = static_cast<const uint16_t*>(p.scale);
  a.offset = static_cast<const uint16_t*>(p.offset ? p.offset : p.scale);
  a.omul = p.offset ? 1.f : 0.f;
  a.bias = static_cast<const uint16_t*>(p.bias);
  a.residual = static_cast<const uint16_t*>(p.residual);
  a.y = static_cast<uint16_t*>(p.y);
  a.partial = p.norm_out ? partial : nullptr;
  a.m = p.m;
  a.k = p.k;
  a.n = p.n;
  a.np = 16 * ((p.n + 15) / 16);
  a.nct = a.np / 16;
  const int64_t group = p.group >= p.k ? p.k : p.group;
  const int64_t groups = (p.k + group - 1) / group;
  const int spg = decode_spg(p);
  a.bpg = (int32_t)(group / 128);
  a.upg_rcp = 1.f / (float)(group / (32 * spg));
  a.s_row = p.s_row;
  a.s_col = p.s_col;
  a.x1_bytes = (uint32_t)(p.m * p.k * 2);
  const bool w8 = decode_w8(p);
  a.x2_bytes = w8 ? (uint32_t)(p.n * p.k) : (uint32_t)(p.k / 128 * a.np * 64);
  a.s_bytes = (uint32_t)(((groups - 1) * p.s_row + (p.n - 1) * p.s_col + 1) * 2);
  a.res_bytes = (uint32_t)(p.m * p.n * 2);
  const int64_t kbs = p.k / 128;
  a.kpw = (int32_t)((kbs + DC_WAVES - 1) / DC_WAVES);
  const int ctw = decode_ctw(a.nct, spg, w8);
  const unsigned grid = (unsigned)decode_grid(p);
  // one launch per 16 rows (m <= 32: at most two; the second finds the
  // weights in the last-level cache)
  for (a.row0 = 0; a.row0 < p.m; a.row0 += 16) {
    const int64_t rows = p.m - a.row0;
    const int xd = rows <= 4 ? 1 : rows <= 8 ? 2 : 4;
    if (p.bf16) launch_act<ACT_BF16>(a, w8, spg, ctw, xd, grid, s);
    else launch_act<ACT_F16>(a, w8, spg, ctw, xd, grid, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
