// Decode-shaped weight-quantized GEMM (m <= 32) for INT4 weights in the
// GFX950_B layout, group a multiple of 128 along K (or per channel / per
// tensor), k a multiple of 128. Same operator as wq_gemm.hip
// (aclnnWeightQuantMatmulAllReduceAddRmsNorm page, Formula).
//
// At small m the packed weight is almost all of the bytes, so the kernel is a
// weight stream: every byte of x2 is read once, 16 bytes per lane per load,
// and the 1 KiB a wave loads per instruction is one 128-deep K block of 16
// columns (the GFX950_B unit), contiguous in memory.
//
// Work split. A workgroup (8 waves) owns CTW column tiles of 16 over all of K;
// CTW grows with n so that the grid stays within one wave of workgroups on the
// 256 compute units. Its waves split K: wave w takes k-blocks [w*kpw,
// (w+1)*kpw) and issues every load of a batch (weights, x1 fragments, one
// scale/offset pair per column and block) before its first MFMA. The
// per-wave sums meet in LDS and are added in a fixed wave order.
//
// Arithmetic per 128-deep block: the codes enter the MFMA as 16-bit B = q + 136
// (fp16: q + 1032, see wq_unpack.h), one more MFMA against a ones fragment
// gives the row sums of x, and the block is folded into the float32 result as
//   acc += s * sum_k x B  +  (o - 136 s) * sum_k x
// with s, o the block's group scale and offset for the column.
//
// Epilogue: y = acc + bias + residual (stored rounded to the activation
// dtype) and per-(row, 16-column tile) sums of the float32 y^2 for the
// RMSNorm finish.
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
  const uint16_t* residual;
  uint16_t* y;
  float* partial;            // [m][np / 16]
  int64_t m, k, n, np, nct;  // nct = np / 16 column tiles
  int64_t row0;              // first of the 16 rows this launch computes
  int64_t s_row, s_col;      // scale element (g, n) at g * s_row + n * s_col
  uint32_t x1_bytes, x2_bytes, s_bytes;
  int32_t kpw;               // 128-deep K blocks per wave
  int32_t bpg;               // 128-deep K blocks per quantization group
  float omul;                // 1 with an offset, 0 without
};

template <int CTW>
struct DecodeLane {
  __amdgpu_buffer_rsrc_t w, x, s, o;
  uint32_t woff[CTW];        // lane's 16 weight bytes in a K block, per column tile
  uint32_t xoff;             // x1 row l%16 + 32-deep sub-block l/16 (BUF_OOB for rows >= m)
  uint32_t soff[CTW];        // lane's scale element per tile (columns clamped to n - 1)
};

// Loop-carried MFMA accumulators of a wave: the block's partial sums per
// column tile and the block's row sums of x. They live across the whole K
// loop and every MFMA updates them in place (cleared in place by a multiply
// with zero at each block start), so each MFMA's destination is exactly its
// accumulator source and never overlaps its A or B operand.
template <int CTW>
struct DecodeAcc {
  f32x4 part[CTW];
  f32x4 rs;
};



// Vector-memory loads decode_blocks issues after block j's four x1 DMAs.
constexpr int loads_after_dma(int nb, int ctw, int j) {
  return j < nb ? 4 * (nb - 1 - j) + 3 * nb * ctw : 0;
}

// NB consecutive 128-deep K blocks starting at kb. Every load is issued
// first, in the order of use: the wave's x1 fragments go by DMA into its LDS
// slice xs (fragment (j, w4) of lane l at xs + 1024 (4j + w4) + 16 l: the
// lane reads back exactly what it loaded), then the weights, then scales and
// offsets into registers. Rows >= m read zeros; columns >= n read valid bytes
// whose results are never stored.
template <int ACT, int CTW, int NB>
__device__ __forceinline__ void decode_blocks(const DecodeArgs& a, const DecodeLane<CTW>& ln,
                                              uint8_t* xs, int kb, DecodeAcc<CTW>& ma,
                                              f32x4 (&acc)[CTW]) {
  static_assert(NB == 1 || NB == 2, "the DMA waits are written for one or two blocks");
  const int lane = threadIdx.x & 63;
  const uint32_t kslab = (uint32_t)a.np * 64u;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ln.x, (lds_void*)(xs + 1024 * (4 * j + w4)), 16,
                                               ln.xoff + 16u * w4, (uint32_t)(kb + j) * 256u, 0, 0);
  // the DMAs stay first: the waits below count the loads issued after them
  __builtin_amdgcn_sched_barrier(0);
  u32x4 wv[NB][CTW];
  uint32_t sr[NB][CTW], orw[NB][CTW];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const uint32_t wso = (uint32_t)(kb + j) * kslab;
#pragma unroll
    for (int c = 0; c < CTW; ++c)
      wv[j][c] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ln.w, ln.woff[c], wso, 0));
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const uint32_t sso = (uint32_t)(((kb + j) / a.bpg) * a.s_row) * 2u;
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
      sr[j][c] = __builtin_amdgcn_raw_buffer_load_b16(ln.s, ln.soff[c], sso, 0);
      orw[j][c] = __builtin_amdgcn_raw_buffer_load_b16(ln.o, ln.soff[c], sso, 0);
    }
  }
  // keep every load of the batch ahead of the first use (the scheduler would
  // otherwise sink loads next to their uses and serialize their latencies)
  __builtin_amdgcn_sched_barrier(0);
  const uint32_t one2 = pack2<ACT>(1.f, 1.f);
  const u32x4 ones = {one2, one2, one2, one2};
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    // block j's x1 DMAs are done once no more than the loads issued after
    // them (later blocks' DMAs, all weights, scales and offsets) remain
    if (j == 0) wait_vm<loads_after_dma(NB, CTW, 0)>();
    else wait_vm<loads_after_dma(NB, CTW, 1)>();
#pragma unroll
    for (int i = 0; i < 4; ++i) ma.rs[i] *= 0.f;
#pragma unroll
    for (int c = 0; c < CTW; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) ma.part[c][i] *= 0.f;
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      const u32x4 av = *reinterpret_cast<const u32x4*>(xs + 1024 * (4 * j + w4) + 16 * lane);
      ma.rs = mfma16<ACT>(av, ones, ma.rs);
#pragma unroll
      for (int c = 0; c < CTW; ++c) {
        const u32x4 b = unpack8(wv[j][c][w4], NIBBLE_MASK, Magic<ACT>::xbits);
        ma.part[c] = mfma16<ACT>(av, b, ma.part[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
      const float s = to_f32<ACT>((uint16_t)sr[j][c]);
      const float o = to_f32<ACT>((uint16_t)orw[j][c]) * a.omul;
      const float cc = o - Magic<ACT>::bias * s;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[c][i] = fmaf(s, ma.part[c][i], fmaf(cc, ma.rs[i], acc[c][i]));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int ACT, int CTW, int KBB>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4, 4))) void gemm_decode(DecodeArgs a) {
  // per wave: its x1 fragments (KBB blocks), reused at the end for its share
  // of the cross-wave sum
  __shared__ __attribute__((aligned(16))) uint8_t xlds[DC_WAVES][KBB * 4096];
  static_assert(16 * (CTW * 16 + 4) * 4 <= KBB * 4096, "reduction rows must fit a wave's slice");
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);      // uniform: K ranges are scalar
  const int col = lane & 15, kq = lane >> 4;
  const int64_t ct0 = (int64_t)blockIdx.x * CTW;
  const int64_t n0 = ct0 * 16;
  const int64_t ctn = a.nct - ct0 < CTW ? a.nct - ct0 : CTW;   // tiles this workgroup stores

  // Lane offsets: weight column 16 * tile + l%16 (tile clamped to the last
  // one; a partial last workgroup discards the repeats), 32-deep sub-block
  // l/16; x1 row row0 + l%16 (rows >= m read zeros); scale column clamped to
  // n - 1. Every offset a valid lane uses stays inside its buffer.
  DecodeLane<CTW> ln;
  ln.w = buf_rsrc(a.x2, a.x2_bytes);
  ln.x = buf_rsrc(a.x1, a.x1_bytes);
  ln.s = buf_rsrc(a.scale, a.s_bytes);
  ln.o = buf_rsrc(a.offset, a.s_bytes);
  const int64_t row = a.row0 + col;
  ln.xoff = row < a.m ? (uint32_t)(row * a.k * 2 + kq * 64) : BUF_OOB;
#pragma unroll
  for (int c = 0; c < CTW; ++c) {
    const int64_t ct = ct0 + c < a.nct ? ct0 + c : a.nct - 1;
    ln.woff[c] = (uint32_t)((ct * 16 + col) * 64 + kq * 16);
    const int64_t sc = n0 + 16 * c + col < a.n ? n0 + 16 * c + col : a.n - 1;
    ln.soff[c] = (uint32_t)(sc * a.s_col * 2);
  }

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
  const __amdgpu_buffer_rsrc_t rres = buf_rsrc(a.residual ? a.residual : a.x1, a.residual ? (uint32_t)(a.m * a.n * 2) : 0u);
  const __amdgpu_buffer_rsrc_t rbias = buf_rsrc(a.bias ? a.bias : a.residual, a.bias ? (uint32_t)(a.n * 2) : 0u);
  const uint32_t r0 = __builtin_amdgcn_raw_buffer_load_b16(rres, rok && c0ok ? (uint32_t)(idx * 2) : BUF_OOB, 0, 0);
  const uint32_t r1 = __builtin_amdgcn_raw_buffer_load_b16(rres, rok && c1ok ? (uint32_t)(idx * 2 + 2) : BUF_OOB, 0, 0);
  const uint32_t b0 = __builtin_amdgcn_raw_buffer_load_b16(rbias, c0ok ? (uint32_t)(col0 * 2) : BUF_OOB, 0, 0);
  const uint32_t b1 = __builtin_amdgcn_raw_buffer_load_b16(rbias, c1ok ? (uint32_t)(col0 * 2 + 2) : BUF_OOB, 0, 0);

  const int kbs = (int)(a.k / 128);
  const int kb0 = wave * a.kpw;
  const int kb1 = kb0 + a.kpw < kbs ? kb0 + a.kpw : kbs;
  f32x4 acc[CTW];
  DecodeAcc<CTW> ma;
  ma.rs = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < CTW; ++i) {
    acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    ma.part[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  int kb = kb0;
  uint8_t* xs = xlds[wave];
  for (; kb + KBB <= kb1; kb += KBB) decode_blocks<ACT, CTW, KBB>(a, ln, xs, kb, ma, acc);
  for (; kb < kb1; ++kb) decode_blocks<ACT, CTW, 1>(a, ln, xs, kb, ma, acc);

  // ---- combine the waves' K slices in a fixed order ----
  // (the wave's own x1 reads are complete: their values fed its MFMAs)
  constexpr int RS = CTW * 16 + 4;                 // reduction row stride (floats)
  float* red = reinterpret_cast<float*>(xs);
#pragma unroll
  for (int i = 0; i < CTW; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[(4 * kq + e) * RS + i * 16 + col] = acc[i][e];
  __syncthreads();

  // ---- epilogue: y = acc + bias + residual, sums of y^2 per 16-column tile ----
  if (!epi) return;
  float v0 = 0.f, v1 = 0.f;
#pragma unroll
  for (int w = 0; w < DC_WAVES; ++w) {
    const float* rw = reinterpret_cast<const float*>(xlds[w]);
    v0 += rw[r * RS + c];
    v1 += rw[r * RS + c + 1];
  }
  float y0 = 0.f, y1 = 0.f;
  if (rok) {
    y0 = v0 + to_f32<ACT>((uint16_t)b0) + to_f32<ACT>((uint16_t)r0);
    y1 = v1 + to_f32<ACT>((uint16_t)b1) + to_f32<ACT>((uint16_t)r1);
    const uint32_t o2 = pack2<ACT>(y0, y1);
    if (pair) {
      *reinterpret_cast<uint32_t*>(a.y + idx) = o2;
    } else {
      if (c0ok) a.y[idx] = (uint16_t)(o2 & 0xFFFFu);
      if (c1ok) a.y[idx + 1] = (uint16_t)(o2 >> 16);
    }
    y0 = c0ok ? y0 : 0.f;                 // the sum of squares uses float32 y
    y1 = c1ok ? y1 : 0.f;
  }
  // sum of y^2 over the 16 columns of the tile: 8 aligned lanes
  float ss = y0 * y0 + y1 * y1;
  ss = quad_sum(ss);
  ss += dpp_f32<0x141>(ss);
  if ((cp & 7) == 0 && rok && tile_ok) a.partial[orow * a.nct + ct0 + (c >> 4)] = ss;
}

template <int ACT, int CTW>
void launch_ct(const DecodeArgs& a, unsigned grid, hipStream_t s) {
  prof_begin(s);
  gemm_decode<ACT, CTW, 2><<<dim3(grid), 1024, 0, s>>>(a);
  prof_end(s);
}

template <int ACT>
void launch_act(const DecodeArgs& a, int ctw, unsigned grid, hipStream_t s) {
  switch (ctw) {
    case 1: launch_ct<ACT, 1>(a, grid, s); break;
    case 2: launch_ct<ACT, 2>(a, grid, s); break;
    default: launch_ct<ACT, 3>(a, grid, s); break;
  }
}

}  // namespace

int64_t decode_tiles(int64_t n) { return (n + 15) / 16; }

// The weight stream addresses the packed weight through one buffer resource
// whose out-of-range offset is 2^31: the weight must stay below 2 GiB.
bool decode_ok(const WqProblem& p) {
  return p.m <= 32 && (p.k / 128) * (16 * ((p.n + 15) / 16)) * 64 < (int64_t(1) << 31);
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
  a.partial = partial;
  a.m = p.m;
  a.k = p.k;
  a.n = p.n;
  a.np = 16 * ((p.n + 15) / 16);
  a.nct = a.np / 16;
  const int64_t group = p.group >= p.k ? p.k : p.group;
  const int64_t groups = (p.k + group - 1) / group;
  a.bpg = (int32_t)(group / 128);
  a.s_row = p.s_row;
  a.s_col = p.s_col;
  a.x1_bytes = (uint32_t)(p.m * p.k * 2);
  a.x2_bytes = (uint32_t)(p.k / 128 * a.np * 64);
  a.s_bytes = (uint32_t)(((groups - 1) * p.s_row + (p.n - 1) * p.s_col + 1) * 2);
  const int64_t kbs = p.k / 128;
  a.kpw = (int32_t)((kbs + DC_WAVES - 1) / DC_WAVES);
  // column tiles per workgroup: keep the grid within one workgroup per CU
  // up to 768 tiles (n = 12288); wider layers take more workgroups of 3
  const int ctw = a.nct <= 256 ? 1 : a.nct <= 512 ? 2 : 3;
  const unsigned grid = (unsigned)((a.nct + ctw - 1) / ctw);
  // one launch per 16 rows (m <= 32: at most two; the second finds the
  // weights in the last-level cache)
  for (a.row0 = 0; a.row0 < p.m; a.row0 += 16) {
    if (p.bf16) launch_act<ACT_BF16>(a, ctw, grid, s);
    else launch_act<ACT_F16>(a, ctw, grid, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
