// INT8-weight tile of the weight-quantized matmul + AddRmsNorm
// (aclnnWeightQuantMatmulAllReduceAddRmsNorm page, Formula; x2 int8 (k, n)
// or its transpose (n, k), Constraints section), also run on INT4 weights
// (B4): the GFX950_B layout, for the groups and K the prefill tile does not
// take, and the ND layout, transposed ((n, k / 2) bytes, each column's K
// codes contiguous) or row-major ((k, n / 2) bytes, staged like a row-major
// INT8 weight). Same operator and numerics
// as wq_gemm.hip: the codes enter the MFMA as exact 16-bit values q, each
// group's scale and offset are applied to its float32 partial sums, the
// epilogue writes y = acc + bias + residual and per-(row, 32-column tile)
// sums of y^2 for the rmsnorm_finish launch.
//
// Tile: 64 x 64 outputs per workgroup, K in steps of 64 (two 32-deep MFMA
// steps). The workgroup's 16 waves form four K slices of four waves (each
// wave 32 x 32 outputs, 2 x 2 MFMA tiles of 16 x 16); slice q multiplies a
// contiguous quarter of the steps and the slices' sums are added in LDS in
// slice order at the end. One wave per SIMD would leave every latency
// (LDS round trips, conversions, MFMA dependencies, barriers) exposed at
// small m; four slices keep four waves on each SIMD. Both operands are
// staged through LDS in 16-bit form, so every code is converted once per
// slice:
//   - x1: 16 halves per thread and step (two 16-byte loads), copied;
//   - x2 transposed (n, k): 16 consecutive K bytes of one column per
//     thread (one 16-byte load);
//   - x2 row-major (k, n): four K rows x four columns per thread (four
//     4-byte loads), transposed in registers with byte permutes.
// Loads run two K steps ahead of the MFMAs (two register stages, LDS double
// buffer, one barrier per step): at small m the tile is latency-bound, and
// two steps in flight halve the exposed load latency.
// A small grid over a long K also splits K across workgroups (up to four
// per output tile, within one workgroup per CU): each writes its float32
// sums to the workspace, and w8_split_finish adds them per row and forms y
// and normOut in place of the tile's epilogue and the norm finish.
//
// Conversion to exact 16-bit values:
//   fp16: u = q + 128 (sign bit flipped) placed under the exponent byte 0x64
//         gives 1024 + u = q + 1152 exactly (ulp 1 on [1024, 2048)); one
//         packed half subtraction of 1152 leaves q;
//   bf16: each signed byte to float32 (byte-select conversions), two per
//         packed bf16 conversion (|q| <= 128 has at most 8 significant
//         bits: exact).
#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int W8_BM = 64, W8_BN = 64, W8_BK = 64, W8_KS = 4;
constexpr int W8_LDS = W8_BK + 8;   // halves per LDS row: 144 bytes, conflict-free 16-byte reads

struct W8Args {
  const uint16_t* x1;
  const uint8_t* x2;        // INT8 (k, n) or (n, k); or INT4 (B4): GFX950_B, or ND transposed (n, k / 2)
  const uint16_t* scale;
  const uint16_t* offset;   // may be null
  const uint16_t* bias;     // may be null
  const uint16_t* residual;  // may be null (the standalone matmul)
  uint16_t* y;
  float* partial;           // [m][ceil(n / 32)]
  int64_t m, k, n, s_row, s_col;
  int64_t np;               // B4: the padded width of the GFX950_B layout; 0 for ND transposed
  int upg;                  // 32-deep units per group; INT32_MAX: one group over all of K
  uint32_t s_bytes;
  // K split across workgroups: workgroup z takes K values [z kz, (z + 1) kz)
  // (kz a multiple of the step) and writes its float32 sums to ypart[z]
  // ((m, n) row-major) for w8_split_finish; ypart null: one workgroup over
  // all of K (kz >= k) and the epilogue in the tile.
  float* ypart;
  int64_t kz;
};

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two 16-bit values in one dword: fp16 (1024 + u) for the bytes u of the
// two selected positions, minus 1152 -> q.
__device__ __forceinline__ uint32_t f16_pair(uint32_t u, uint32_t sel) {
  const uint32_t biased = __builtin_amdgcn_perm(0x64646464u, u, sel);
  const f16x2 v = __builtin_bit_cast(f16x2, biased) - (f16x2){(_Float16)1152.f, (_Float16)1152.f};
  return __builtin_bit_cast(uint32_t, v);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// signed byte j of w -> float q
__device__ __forceinline__ float sbyte(uint32_t w, int j) { return (float)(int)(int8_t)(w >> (8 * j)); }

// two floats -> one dword of two bf16 (one packed conversion; the values
// here are exact in bf16)
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// 16 consecutive K codes of one column (four dwords, K ascending from the
// low byte) -> eight dwords of 16-bit q, K ascending.
template <int ACT>
__device__ __forceinline__ void convert_k16(const u32x4& w, u32x4& lo, u32x4& hi) {
  uint32_t o[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    if constexpr (ACT == ACT_F16) {
      const uint32_t u = w[d] ^ 0x80808080u;
      o[2 * d] = f16_pair(u, 0x04010400u);      // bytes 0, 1
      o[2 * d + 1] = f16_pair(u, 0x04030402u);  // bytes 2, 3
    } else {
      o[2 * d] = bf16_pair(sbyte(w[d], 0), sbyte(w[d], 1));
      o[2 * d + 1] = bf16_pair(sbyte(w[d], 2), sbyte(w[d], 3));
    }
  }
  lo = (u32x4){o[0], o[1], o[2], o[3]};
  hi = (u32x4){o[4], o[5], o[6], o[7]};
}

// 16 consecutive K codes of one column as INT4 nibbles (w0: K 0..7, w1:
// K 8..15, low nibble first; the GFX950_B byte order) -> eight dwords of
// 16-bit q, K ascending. u = n ^ 8 = q + 8 in [0, 15]: fp16 places u under
// the exponent byte 0x64 (1024 + u) and subtracts 1032 with one packed half
// subtraction per pair; bf16 converts each byte to float32 and subtracts 8
// (exact), two per packed bf16 conversion.
template <int ACT>
__device__ __forceinline__ void convert_n16(uint32_t w0, uint32_t w1, u32x4& lo4, u32x4& hi4) {
  uint32_t o[8];
  const uint32_t w[2] = {w0, w1};
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const uint32_t u = w[d] ^ 0x88888888u;
    const uint32_t ev = u & 0x0F0F0F0Fu, od = (u >> 4) & 0x0F0F0F0Fu;   // K 0, 2, 4, 6 / K 1, 3, 5, 7
    const uint32_t p0 = __builtin_amdgcn_perm(od, ev, 0x05010400u);    // K 0..3 as bytes
    const uint32_t p1 = __builtin_amdgcn_perm(od, ev, 0x07030602u);    // K 4..7
    if constexpr (ACT == ACT_F16) {
      const f16x2 bias = {(_Float16)1032.f, (_Float16)1032.f};
      auto pair = [&](uint32_t b, uint32_t sel) {
        const uint32_t h = __builtin_amdgcn_perm(0x64646464u, b, sel);
        return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, h) - bias);
      };
      o[4 * d] = pair(p0, 0x04010400u);
      o[4 * d + 1] = pair(p0, 0x04030402u);
      o[4 * d + 2] = pair(p1, 0x04010400u);
      o[4 * d + 3] = pair(p1, 0x04030402u);
    } else {
      auto q = [](uint32_t b, int j) { return (float)((b >> (8 * j)) & 0xFFu) - 8.f; };
      o[4 * d] = bf16_pair(q(p0, 0), q(p0, 1));
      o[4 * d + 1] = bf16_pair(q(p0, 2), q(p0, 3));
      o[4 * d + 2] = bf16_pair(q(p1, 0), q(p1, 1));
      o[4 * d + 3] = bf16_pair(q(p1, 2), q(p1, 3));
    }
  }
  lo4 = (u32x4){o[0], o[1], o[2], o[3]};
  hi4 = (u32x4){o[4], o[5], o[6], o[7]};
}

// Four K rows of four INT4 columns (r[i] = row i, nibble j = column j, the
// ND byte order) -> per column j the four K values as 16-bit q:
// out[j] = {rows 0-1, rows 2-3}; u = n ^ 8 = q + 8 as in convert_n16.
template <int ACT>
__device__ __forceinline__ void convert_rows4_n(const uint32_t (&r)[4], u32x2 (&out)[4]) {
  uint32_t u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = r[i] ^ 0x8888u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    auto nib = [&](int i) { return (u[i] >> (4 * j)) & 0xFu; };
    if constexpr (ACT == ACT_F16) {
      const f16x2 bias = {(_Float16)1032.f, (_Float16)1032.f};
      auto pair = [&](int i0, int i1) {
        const uint32_t h = (0x6400u | nib(i0)) | ((0x6400u | nib(i1)) << 16);   // 1024 + u, two halves
        return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, h) - bias);
      };
      out[j] = (u32x2){pair(0, 1), pair(2, 3)};
    } else {
      auto q = [&](int i) { return (float)nib(i) - 8.f; };
      out[j] = (u32x2){bf16_pair(q(0), q(1)), bf16_pair(q(2), q(3))};
    }
  }
}

// Four K rows of four columns (r[i] = row i, byte j = column j) -> per
// column j the four K values as 16-bit q: out[j] = {rows 0-1, rows 2-3}.
template <int ACT>
__device__ __forceinline__ void convert_rows4(const uint32_t (&r)[4], u32x2 (&out)[4]) {
  if constexpr (ACT == ACT_F16) {
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = r[i] ^ 0x80808080u;
    // pair rows (0, 1) and (2, 3) byte by byte: p01l = [u0.b0, u1.b0, u0.b1,
    // u1.b1], p01h = the same for bytes 2, 3
    const uint32_t p01l = __builtin_amdgcn_perm(u[1], u[0], 0x05010400u);
    const uint32_t p01h = __builtin_amdgcn_perm(u[1], u[0], 0x07030602u);
    const uint32_t p23l = __builtin_amdgcn_perm(u[3], u[2], 0x05010400u);
    const uint32_t p23h = __builtin_amdgcn_perm(u[3], u[2], 0x07030602u);
    out[0] = (u32x2){f16_pair(p01l, 0x04010400u), f16_pair(p23l, 0x04010400u)};
    out[1] = (u32x2){f16_pair(p01l, 0x04030402u), f16_pair(p23l, 0x04030402u)};
    out[2] = (u32x2){f16_pair(p01h, 0x04010400u), f16_pair(p23h, 0x04010400u)};
    out[3] = (u32x2){f16_pair(p01h, 0x04030402u), f16_pair(p23h, 0x04030402u)};
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      out[j] = (u32x2){bf16_pair(sbyte(r[0], j), sbyte(r[1], j)), bf16_pair(sbyte(r[2], j), sbyte(r[3], j))};
  }
}

// One K step's register stage: raw x1 halves, raw weight bytes, and (threads
// t < 128) the scale / offset of column t % 64 for the group that 32-deep
// half t / 64 closes. The scales go to LDS with the tiles, so that no value
// loaded for a later step is held across the loop's back edge in registers
// the compiler would have to copy (and wait for).
struct W8Stage {
  u32x4 a0, a1;
  u32x4 b;                  // transposed: 16 K bytes of one column; row-major: 4 rows x 4 columns
  uint32_t sv, ov;
};

struct W8Lane {
  __amdgpu_buffer_rsrc_t x, w, s, o;
  int rows, cols;           // valid rows / columns of the workgroup's tile
};

// Place of a 32-deep unit of K in its group: the unit's index within the
// group and the group. Units are visited in order, so moving to the next is
// a compare and an add on scalars (no division in the loop).
struct FoldPos {
  int pos, g;
  __device__ __forceinline__ FoldPos next(int upg) const {
    return pos + 1 == upg ? FoldPos{0, g + 1} : FoldPos{pos + 1, g};
  }
};

// A 32-deep half at unit position f starting at K value kh closes a group
// when it holds K values of the slice (which ends at kend) and it is its
// group's last unit or the slice's last (a group split between slices is
// folded by each with the same scale and offset).
__device__ __forceinline__ bool closes_group(const W8Args& a, int kend, int kh, FoldPos f) {
  return (kh < kend) & ((f.pos == a.upg - 1) | (kh + 32 >= kend));
}

// The loads of one step of one slice: K values [k0, k0 + 64) below kend.
template <bool ND, bool B4>
__device__ __forceinline__ void load_stage(const W8Args& a, const W8Lane& ln, int64_t n0, int kend, int k0,
                                           FoldPos& fp, W8Stage& st) {
  const int t = threadIdx.x & 255, lane = t & 63;
  {
    const int r = t >> 2, kc = (t & 3) * 16;
    const uint32_t v = (r < ln.rows) & (k0 + kc < kend) ? (uint32_t)((r * (int)a.k + k0 + kc) * 2) : BUF_OOB;
    st.a0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ln.x, v, 0, 0));
    st.a1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ln.x, v + 16u, 0, 0));
  }
  if constexpr (B4 && !ND) {
    // column c's K values kk .. kk + 15: 8 bytes of its GFX950_B record
    // (the 32-deep block kk / 32 of 128-deep block kk / 128), or of its ND
    // row of k / 2 bytes; the resource starts at the workgroup's first column
    const int c = t >> 2, kk = k0 + (t & 3) * 16;
    const uint32_t at = a.np ? (uint32_t)((((int64_t)(kk >> 7) * a.np + c) * 64) + ((kk >> 5) & 3) * 16 + ((kk & 31) >> 1))
                             : (uint32_t)(c * (a.k >> 1) + (kk >> 1));
    const uint32_t v = (c < ln.cols) & (kk < kend) ? at : BUF_OOB;
    const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(ln.w, v, 0, 0));
    st.b = (u32x4){w.x, w.y, 0u, 0u};
  } else if constexpr (!ND) {
    const int c = t >> 2, kc = (t & 3) * 16;
    const uint32_t v = (c < ln.cols) & (k0 + kc < kend) ? (uint32_t)(c * (int)a.k + k0 + kc) : BUF_OOB;
    st.b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ln.w, v, 0, 0));
  } else if constexpr (B4) {
    // INT4 ND (k, n / 2) bytes: K row kk's columns c4 .. c4 + 3 are 2 bytes
    const int rg = t >> 4, c4 = (t & 15) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t kk = k0 + 4 * rg + i;
      const uint32_t v = (c4 < ln.cols) & (kk < kend) ? (uint32_t)(kk * (a.n >> 1) + (c4 >> 1)) : BUF_OOB;
      st.b[i] = __builtin_amdgcn_raw_buffer_load_b16(ln.w, v, 0, 0);
    }
  } else {
    const int rg = t >> 4, c4 = (t & 15) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t kk = k0 + 4 * rg + i;
      const uint32_t v = (c4 < ln.cols) & (kk < kend) ? (uint32_t)(kk * a.n + c4) : BUF_OOB;
      st.b[i] = __builtin_amdgcn_raw_buffer_load_b32(ln.w, v, 0, 0);
    }
  }
  // the scale and offset of a half that closes a group (else, or for
  // t >= 128, an out-of-range offset: the load reads nothing). Every load of
  // a stage is issued on every path, so the compiler's wait before a stage's
  // first use counts only the loads issued after it.
  {
    const FoldPos f0 = fp, f1 = fp.next(a.upg);
    fp = f1.next(a.upg);
    const bool fold0 = closes_group(a, kend, k0, f0), fold1 = closes_group(a, kend, k0 + 32, f1);
    const bool h = (t >> 6) & 1;
    const bool fold = (h ? fold1 : fold0) & (t < 128);
    const int64_t g = h ? f1.g : f0.g;              // < groups when fold
    int64_t col = n0 + lane;
    col = col < a.n ? col : a.n - 1;
    const uint32_t so = fold ? (uint32_t)((g * a.s_row + col * a.s_col) * 2) : BUF_OOB;
    st.sv = __builtin_amdgcn_raw_buffer_load_b16(ln.s, so, 0, 0);
    st.ov = __builtin_amdgcn_raw_buffer_load_b16(ln.o, so, 0, 0);
  }
}

// Scales and offsets of one buffer: [half][column] raw 16-bit values.
struct W8Scales {
  uint16_t s[2][W8_BN], o[2][W8_BN];
};

template <int ACT, bool ND, bool B4>
__device__ __forceinline__ void store_stage(const W8Stage& st, uint16_t* As, uint16_t* Bs, W8Scales& ss) {
  const int t = threadIdx.x & 255;
  if (t < 128) {
    ss.s[t >> 6][t & 63] = (uint16_t)st.sv;
    ss.o[t >> 6][t & 63] = (uint16_t)st.ov;
  }
  {
    const int r = t >> 2, kc = (t & 3) * 16;
    *reinterpret_cast<u32x4*>(As + r * W8_LDS + kc) = st.a0;
    *reinterpret_cast<u32x4*>(As + r * W8_LDS + kc + 8) = st.a1;
  }
  if constexpr (!ND) {
    const int c = t >> 2, kc = (t & 3) * 16;
    u32x4 lo, hi;
    if constexpr (B4) convert_n16<ACT>(st.b.x, st.b.y, lo, hi);
    else convert_k16<ACT>(st.b, lo, hi);
    *reinterpret_cast<u32x4*>(Bs + c * W8_LDS + kc) = lo;
    *reinterpret_cast<u32x4*>(Bs + c * W8_LDS + kc + 8) = hi;
  } else {
    const int rg = t >> 4, c4 = (t & 15) * 4;
    const uint32_t r[4] = {st.b[0], st.b[1], st.b[2], st.b[3]};
    u32x2 out[4];
    if constexpr (B4) convert_rows4_n<ACT>(r, out);
    else convert_rows4<ACT>(r, out);
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x2*>(Bs + (c4 + j) * W8_LDS + 4 * rg) = out[j];
  }
}

struct W8Acc {
  f32x4 acc[2][2], part[2][2], rs[2];
};

// The two 32-deep halves of one K step from LDS (past the end of K they
// hold zeros); a half that closes a group folds it:
// acc += s * sum x q + o * sum x.
template <int ACT>
__device__ __forceinline__ void compute_stage(const W8Args& a, const uint16_t* As, const uint16_t* Bs,
                                              const W8Scales& ss, int kend, int k0, FoldPos& fp, W8Acc& z) {
  const int t = threadIdx.x & 255, lane = t & 63, wave = t >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const uint32_t one2 = pack2<ACT>(1.f, 1.f);
  const u32x4 ones = {one2, one2, one2, one2};
  const bool off = a.offset != nullptr;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kq = 32 * h + 8 * (lane >> 4);
    u32x4 af[2], bf[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      af[i] = *reinterpret_cast<const u32x4*>(As + (wr * 32 + 16 * i + (lane & 15)) * W8_LDS + kq);
      bf[i] = *reinterpret_cast<const u32x4*>(Bs + (wc * 32 + 16 * i + (lane & 15)) * W8_LDS + kq);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j) z.part[i][j] = mfma16<ACT>(af[i], bf[j], z.part[i][j]);
      if (off) z.rs[i] = mfma16<ACT>(af[i], ones, z.rs[i]);
    }
    const bool fold = closes_group(a, kend, k0 + 32 * h, fp);
    fp = fp.next(a.upg);
    if (__builtin_expect(fold, 0)) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = wc * 32 + 16 * j + (lane & 15);
        const float s = to_f32<ACT>(ss.s[h][c]);
        const float o = off ? to_f32<ACT>(ss.o[h][c]) : 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            z.acc[i][j][e] = fmaf(s, z.part[i][j][e], z.acc[i][j][e]);
            if (off) z.acc[i][j][e] = fmaf(o, z.rs[i][e], z.acc[i][j][e]);
            z.part[i][j][e] = 0.f;
          }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) z.rs[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  }
}

template <int ACT, bool ND, bool B4>
__global__ __launch_bounds__(256 * W8_KS) void gemm_w8(W8Args a) {
  // per slice: x1 and weight tiles, double-buffered, and the fold scales;
  // after the K loop the tiles hold the slices' sums
  __shared__ __attribute__((aligned(16))) uint16_t As[W8_KS][2][W8_BM * W8_LDS];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[W8_KS][2][W8_BN * W8_LDS];
  __shared__ W8Scales Ss[W8_KS][2];
  const int q = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 8));   // K slice
  const int t = threadIdx.x & 255, lane = t & 63, wave = t >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * W8_BM;
  const int64_t n0 = (int64_t)blockIdx.x * W8_BN;

  // Buffer resources start at the workgroup's rows / columns, so every
  // offset stays below 2^31 (x1: 64 rows; the transposed weight: 64
  // columns; the row-major weight is below 2 GiB as a whole).
  W8Lane ln;
  ln.rows = (int)(a.m - m0 < W8_BM ? a.m - m0 : W8_BM);
  ln.cols = (int)(a.n - n0 < W8_BN ? a.n - n0 : W8_BN);
  ln.x = buf_rsrc(a.x1 + m0 * a.k, (uint32_t)(ln.rows * a.k * 2));
  if constexpr (B4 && ND) ln.w = buf_rsrc(a.x2 + n0 / 2, (uint32_t)((a.k - 1) * (a.n / 2) + ln.cols / 2));
  else if constexpr (B4)
    ln.w = a.np ? buf_rsrc(a.x2 + n0 * 64, (uint32_t)(((a.k + 127) / 128 * a.np - n0) * 64))
                : buf_rsrc(a.x2 + n0 * (a.k / 2), (uint32_t)(ln.cols * (a.k / 2)));
  else if constexpr (ND) ln.w = buf_rsrc(a.x2 + n0, (uint32_t)((a.k - 1) * a.n + ln.cols));
  else ln.w = buf_rsrc(a.x2 + n0 * a.k, (uint32_t)(ln.cols * a.k));
  ln.s = buf_rsrc(a.scale, a.s_bytes);
  ln.o = buf_rsrc(a.offset ? a.offset : a.scale, a.s_bytes);

  W8Acc z;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    z.rs[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      z.acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
      z.part[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  }

  // Slice q: steps [q * sps, (q + 1) * sps), K values below kend. Steps s + 1
  // and s + 2 in flight while step s is multiplied: stage sa holds even
  // steps, sb odd ones; LDS buffer s % 2 holds step s. Every slice runs the
  // same even number of steps with every load unconditional (a step past its
  // slice reads zeros through out-of-range offsets and multiplies nothing),
  // so the barriers match and the waits see one straight sequence of loads.
  const int kz0 = (int)(blockIdx.z * a.kz);
  const int kz1 = kz0 + a.kz < a.k ? kz0 + (int)a.kz : (int)a.k;
  const int steps = (kz1 - kz0 + W8_BK - 1) / W8_BK;
  const int sps = (steps + W8_KS - 1) / W8_KS;
  const int kb = kz0 + q * sps * W8_BK;
  const int kend = kb + sps * W8_BK < kz1 ? kb + sps * W8_BK : kz1;
  uint16_t* A0 = As[q][0];
  uint16_t* A1 = As[q][1];
  uint16_t* B0 = Bs[q][0];
  uint16_t* B1 = Bs[q][1];
  // unit positions of the loads (two steps ahead) and of the MFMAs
  const int u0 = kb >> 5;
  FoldPos fl = {u0 % a.upg, u0 / a.upg};
  FoldPos fc = fl;
  W8Stage sa, sb;
  load_stage<ND, B4>(a, ln, n0, kend, kb, fl, sa);
  load_stage<ND, B4>(a, ln, n0, kend, kb + W8_BK, fl, sb);
  store_stage<ACT, ND, B4>(sa, A0, B0, Ss[q][0]);
  __syncthreads();
  for (int s = 0; s < sps; s += 2) {
    const int k0 = kb + s * W8_BK;
    load_stage<ND, B4>(a, ln, n0, kend, k0 + 2 * W8_BK, fl, sa);
    compute_stage<ACT>(a, A0, B0, Ss[q][0], kend, k0, fc, z);
    store_stage<ACT, ND, B4>(sb, A1, B1, Ss[q][1]);
    __syncthreads();
    load_stage<ND, B4>(a, ln, n0, kend, k0 + 3 * W8_BK, fl, sb);
    compute_stage<ACT>(a, A1, B1, Ss[q][1], kend, k0 + W8_BK, fc, z);
    store_stage<ACT, ND, B4>(sa, A0, B0, Ss[q][0]);
    __syncthreads();
  }

  // ---- the slices' sums: each slice's 64 x 64 tile to its LDS (rows of 68
  // floats: the 16 columns of a row and the four rows one MFMA lane group
  // apart land in distinct banks), then every thread adds four adjacent
  // outputs over the slices in slice order ----
  // (every slice's LDS reads are complete: the loop ended with a barrier)
  constexpr int CS = W8_BN + 4;
  static_assert(W8_BM * CS * 4 <= 2 * W8_BM * W8_LDS * 2, "a slice's sums fit its tiles");
  {
    float* cq = reinterpret_cast<float*>(As[q][0]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          cq[(wr * 32 + 16 * i + 4 * (lane >> 4) + e) * CS + wc * 32 + 16 * j + (lane & 15)] = z.acc[i][j][e];
  }
  __syncthreads();

  // ---- epilogue: thread T takes row T / 16, columns 4 (T % 16) .. + 3:
  // y = sum + bias + residual, and the sum of y^2 over each 32-column tile
  // (eight threads) ----
  const int T = threadIdx.x, er = T >> 4, ec = (T & 15) * 4;
  f32x4 v = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(As[0][0]) + er * CS + ec);
#pragma unroll
  for (int p = 1; p < W8_KS; ++p) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(As[p][0]) + er * CS + ec);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] += w[e];
  }
  const int64_t row = m0 + er, col = n0 + ec;
  if (a.ypart) {
    // K split: this workgroup's sums only (bias, residual and the norm are
    // the split finish's)
    if (row < a.m) {
      float* pz = a.ypart + blockIdx.z * a.m * a.n + row * a.n + col;
      if ((a.n & 3) == 0 && col + 3 < a.n) {
        *reinterpret_cast<f32x4*>(pz) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < a.n) pz[e] = v[e];
      }
    }
    return;
  }
  float ss = 0.f;
  if (row < a.m) {
    const int64_t idx = row * a.n + col;
    if ((a.n & 3) == 0 && col + 3 < a.n) {
      // 8-byte accesses: rows start 8-byte aligned when n % 4 == 0
      const u32x2 bb = a.bias ? *reinterpret_cast<const u32x2*>(a.bias + col) : (u32x2){0u, 0u};
      const u32x2 rr = a.residual ? *reinterpret_cast<const u32x2*>(a.residual + idx) : (u32x2){0u, 0u};
      float y[4];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        y[2 * e] = v[2 * e] + lo_f32<ACT>(bb[e]) + lo_f32<ACT>(rr[e]);
        y[2 * e + 1] = v[2 * e + 1] + hi_f32<ACT>(bb[e]) + hi_f32<ACT>(rr[e]);
      }
      *reinterpret_cast<u32x2*>(a.y + idx) = (u32x2){pack2<ACT>(y[0], y[1]), pack2<ACT>(y[2], y[3])};
      ss = (y[0] * y[0] + y[1] * y[1]) + (y[2] * y[2] + y[3] * y[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (col + e < a.n) {
          const float y = v[e] + (a.bias ? to_f32<ACT>(a.bias[col + e]) : 0.f) +
                          (a.residual ? to_f32<ACT>(a.residual[idx + e]) : 0.f);
          a.y[idx + e] = from_f32<ACT>(y);
          ss += y * y;
        }
    }
  }
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  ss += __shfl_xor(ss, 4);
  if ((T & 7) == 0 && row < a.m && col < a.n) a.partial[row * ((a.n + 31) / 32) + col / 32] = ss;
}

// The finish of a K split (S splits): one workgroup per row. y = (sum of the
// splits' sums, in split order) + bias + residual, stored rounded, the row's
// sum of y^2 taken in float32 before rounding (as the tile's epilogue takes
// it); then, with a norm output, normOut = y * rstd * gamma from the stored
// (rounded) y.
// A split grid has at most 256 tiles over S splits, so a row holds at most
// 64 * 256 / S columns (W8_SPLIT_MAX_N at S = 2) and S * n <= 16384. With
// n % 4 == 0 each thread takes four adjacent columns per pass of 1024, at
// most 16 / S passes: every load of the row (the splits' sums, bias,
// residual, gamma) is issued before the first store, through buffer
// resources that read zeros past their ends (y may be the residual's
// memory, so no load may follow a store), and the stored y stays in
// registers across the row's reduction.
constexpr int W8_SPLIT_MAX_N = 8192;

template <int ACT, int S>
__global__ __launch_bounds__(256) void w8_split_finish(const float* __restrict__ ypart,
                                                       const uint16_t* bias, const uint16_t* residual,
                                                       const uint16_t* __restrict__ gamma, uint16_t* y,
                                                       uint16_t* __restrict__ out, int64_t m, int64_t n,
                                                       float eps) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x, mn = m * n;
  const int t = threadIdx.x;
  float ss = 0.f;
  constexpr int J = 16 / S;
  u32x2 ys[J], gs[J];
  const bool vec = (n & 3) == 0;
  if (vec) {
    const __amdgpu_buffer_rsrc_t rp = buf_rsrc(ypart + row * n, (uint32_t)((S - 1) * mn * 4 + n * 4));
    const __amdgpu_buffer_rsrc_t rb = buf_rsrc(bias ? (const void*)bias : ypart, bias ? (uint32_t)(n * 2) : 0u);
    const __amdgpu_buffer_rsrc_t rr = buf_rsrc(residual ? (const void*)(residual + row * n) : ypart,
                                               residual ? (uint32_t)(n * 2) : 0u);
    const __amdgpu_buffer_rsrc_t rg = buf_rsrc(out ? (const void*)gamma : ypart, out ? (uint32_t)(n * 2) : 0u);
    f32x4 pv[S][J];
    u32x2 bv[J], rv[J];
    // passes past the row's end are skipped whole (a workgroup-uniform
    // branch); in the last one, lanes past n read zeros
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (1024 * j >= n) break;
      const int64_t c = 4 * t + 1024 * j;
      const bool ok = c < n;
      const uint32_t o2 = ok ? (uint32_t)(c * 2) : BUF_OOB;
#pragma unroll
      for (int z = 0; z < S; ++z)
        pv[z][j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rp, ok ? (uint32_t)((z * mn + c) * 4) : BUF_OOB, 0, 0));
      bv[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rb, o2, 0, 0));
      rv[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rr, o2, 0, 0));
      gs[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, o2, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (1024 * j >= n) break;
      const int64_t c = 4 * t + 1024 * j;
      f32x4 v = pv[0][j];
#pragma unroll
      for (int z = 1; z < S; ++z)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += pv[z][j][e];
      float yv[4];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        yv[2 * e] = v[2 * e] + lo_f32<ACT>(bv[j][e]) + lo_f32<ACT>(rv[j][e]);
        yv[2 * e + 1] = v[2 * e + 1] + hi_f32<ACT>(bv[j][e]) + hi_f32<ACT>(rv[j][e]);
      }
      ys[j] = (u32x2){pack2<ACT>(yv[0], yv[1]), pack2<ACT>(yv[2], yv[3])};
      if (c < n) {
        *reinterpret_cast<u32x2*>(y + row * n + c) = ys[j];
        ss += (yv[0] * yv[0] + yv[1] * yv[1]) + (yv[2] * yv[2] + yv[3] * yv[3]);
      }
    }
  } else {
    for (int64_t c = t; c < n; c += 256) {
      const int64_t idx = row * n + c;
      float v = ypart[idx];
#pragma unroll
      for (int z = 1; z < S; ++z) v += ypart[z * mn + idx];
      const float yv = v + (bias ? to_f32<ACT>(bias[c]) : 0.f) + (residual ? to_f32<ACT>(residual[idx]) : 0.f);
      y[idx] = from_f32<ACT>(yv);
      ss += yv * yv;
    }
  }
  if (!out) return;   // the standalone matmul
  ss = wave_sum(ss);
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  ss = (red[0] + red[1]) + (red[2] + red[3]);
  const float rstd = 1.0f / sqrtf(ss / (float)n + eps);
  if (vec) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (1024 * j >= n) break;
      const int64_t c = 4 * t + 1024 * j;
      if (c < n) {
        u32x2 o;
#pragma unroll
        for (int e = 0; e < 2; ++e)
          o[e] = pack2<ACT>(lo_f32<ACT>(ys[j][e]) * rstd * lo_f32<ACT>(gs[j][e]),
                            hi_f32<ACT>(ys[j][e]) * rstd * hi_f32<ACT>(gs[j][e]));
        *reinterpret_cast<u32x2*>(out + row * n + c) = o;
      }
    }
  } else {
    // every thread reads back only the y values it stored
    for (int64_t c = t; c < n; c += 256) {
      const int64_t idx = row * n + c;
      out[idx] = from_f32<ACT>(to_f32<ACT>(y[idx]) * rstd * to_f32<ACT>(gamma[c]));
    }
  }
}

// K splits for an (m, k, n) problem on this tile: the largest of 1, 2, 4
// whose grid stays within one workgroup per CU (256) while every slice keeps
// at least two K steps. A small grid over a long K is a chain of load
// latencies per slice; splitting it shortens the chain.
int w8_split_count(int64_t m, int64_t k, int64_t n) {
  const int64_t tiles = ((m + W8_BM - 1) / W8_BM) * ((n + W8_BN - 1) / W8_BN);
  const int64_t steps = (k + W8_BK - 1) / W8_BK;
  int s = 1;
  while (s < 4 && tiles * 2 * s <= 256 && steps >= 2 * W8_KS * 2 * s) s *= 2;
  // (the grid bound implies what the finish relies on: s * n <= 16384)
  return s * n <= 2 * W8_SPLIT_MAX_N ? s : 1;
}

template <int ACT>
hipError_t launch_w8_t(const WqProblem& p, float* partial, hipStream_t s, bool& finished) {
  W8Args a;
  a.x1 = static_cast<const uint16_t*>(p.x1);
  a.x2 = static_cast<const uint8_t*>(p.x2);
  a.scale = static_cast<const uint16_t*>(p.scale);
  a.offset = static_cast<const uint16_t*>(p.offset);
  a.bias = static_cast<const uint16_t*>(p.bias);
  a.residual = static_cast<const uint16_t*>(p.residual);
  a.y = static_cast<uint16_t*>(p.y);
  a.partial = partial;
  a.m = p.m;
  a.k = p.k;
  a.n = p.n;
  a.np = p.layout == WQ_LAYOUT_GFX950_B ? 16 * ((p.n + 15) / 16) : 0;
  const int64_t group = p.group >= p.k ? p.k : p.group;
  a.upg = p.group >= p.k ? INT32_MAX : (int)(group / 32);
  a.s_row = p.s_row;
  a.s_col = p.s_col;
  const int64_t groups = (p.k + group - 1) / group;
  a.s_bytes = (uint32_t)(((groups - 1) * p.s_row + (p.n - 1) * p.s_col + 1) * 2);
  // K split: the splits' sums go to the workspace, whose size covers them
  // (w8_split_bytes); the split finish then forms y and normOut
  const int splits = w8_split_count(p.m, p.k, p.n);
  const bool split = splits > 1 && (size_t)splits * p.m * p.n * sizeof(float) <= p.workspace_size;
  const int64_t steps = (p.k + W8_BK - 1) / W8_BK;
  a.ypart = split ? partial : nullptr;
  a.kz = split ? (steps + splits - 1) / splits * W8_BK : p.k;
  const dim3 grid((unsigned)((p.n + W8_BN - 1) / W8_BN), (unsigned)((p.m + W8_BM - 1) / W8_BM),
                  split ? (unsigned)splits : 1u);
  prof_begin(s);
  if (p.w_bits == 4 && p.layout == WQ_LAYOUT_ND && !p.transpose_x2) gemm_w8<ACT, true, true><<<grid, 256 * W8_KS, 0, s>>>(a);
  else if (p.w_bits == 4) gemm_w8<ACT, false, true><<<grid, 256 * W8_KS, 0, s>>>(a);
  else if (p.transpose_x2) gemm_w8<ACT, false, false><<<grid, 256 * W8_KS, 0, s>>>(a);
  else gemm_w8<ACT, true, false><<<grid, 256 * W8_KS, 0, s>>>(a);
  prof_end(s);
  finished = split;
  if (!split) return hipGetLastError();
  const uint16_t* gamma = static_cast<const uint16_t*>(p.gamma);
  uint16_t* norm_out = static_cast<uint16_t*>(p.norm_out);
  if (splits == 2)
    w8_split_finish<ACT, 2><<<dim3((unsigned)p.m), 256, 0, s>>>(partial, a.bias, a.residual, gamma, a.y,
                                                                norm_out, p.m, p.n, p.eps);
  else
    w8_split_finish<ACT, 4><<<dim3((unsigned)p.m), 256, 0, s>>>(partial, a.bias, a.residual, gamma, a.y,
                                                                norm_out, p.m, p.n, p.eps);
  return hipGetLastError();
}

}  // namespace

// INT8 weights, k a multiple of 16 (16-byte loads never straddle a row of
// x1 or of the transposed weight); row-major weights with n a multiple of 4
// (4-byte column groups) and below 2 GiB (one buffer resource).
// INT4 GFX950_B weights (the shapes the prefill tile does not take: groups
// of 32, 64 or any multiple of 32 not dividing 128, or k not a multiple of
// 128) and ND INT4 weights (transposed, or row-major with n a multiple of
// 4): k a multiple of 16, the packed weight below 2 GiB.
bool w8_ok(const WqProblem& p) {
  if (p.w_bits == 4) {
    if (p.k % 16 != 0) return false;
    if (p.layout == WQ_LAYOUT_GFX950_B) return (p.k + 127) / 128 * (16 * ((p.n + 15) / 16)) * 64 < (int64_t(1) << 31);
    if (p.transpose_x2) return p.n * (p.k / 2) < (int64_t(1) << 31);
    return p.n % 4 == 0 && p.k * (p.n / 2) < (int64_t(1) << 31);
  }
  if (p.w_bits != 8 || p.k % 16 != 0) return false;
  if (p.transpose_x2) return true;
  return p.n % 4 == 0 && p.k * p.n < (int64_t(1) << 31);
}

hipError_t launch_w8(const WqProblem& p, float* partial, hipStream_t s, bool& finished) {
  return p.bf16 ? launch_w8_t<ACT_BF16>(p, partial, s, finished)
                : launch_w8_t<ACT_F16>(p, partial, s, finished);
}

size_t w8_split_bytes(int64_t m, int64_t k, int64_t n) {
  const int splits = w8_split_count(m, k, n);
  return splits > 1 ? (size_t)splits * m * n * sizeof(float) : 0;
}

}  // namespace wq
