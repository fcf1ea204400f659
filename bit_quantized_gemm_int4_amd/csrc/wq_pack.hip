// INT4 weight pack (aclnnConvertWeightToINT4Pack page, operator description):
// one 4-bit value per int32 in, tightly packed nibbles out, in the ND layout
// or the gfx950 MFMA-operand layout GFX950_B (byte formula in wq.h). The
// same page packs FLOAT weights into FLOAT4_E2M1 on the newer chips: with FP4
// each 32-bit input is a float, encoded to its E2M1 code (nearest, ties to
// even, saturating at +-6) instead of taking its low nibble.
//
// GFX950_B is built in registers (each word's eight codes come from eight
// coalesced loads or one 32-byte run) and leaves as one contiguous run per
// workgroup. ND stages a 128 (K) x 64 (N) tile of codes in LDS as bytes, so
// global reads are coalesced for either input orientation, then writes
// 16-byte runs of packed rows. The op is HBM-bound: 4 bytes read per 0.5
// byte written.
#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int TK = 128;        // tile depth (K)
constexpr int TN = 64;         // tile width (N)
constexpr int LROW = TK + 4;   // LDS row (one column's codes), padded

// The 4-bit code of one 32-bit input word.
template <bool FP4>
__device__ __forceinline__ uint32_t code_of(uint32_t v) {
  return FP4 ? e2m1(__uint_as_float(v)) : (v & 0xFu);
}

template <bool TRANSPOSED, bool FP4>
__device__ __forceinline__ void stage_tile(const int32_t* __restrict__ w, int64_t K, int64_t N,
                                           int64_t k0, int64_t n0, uint8_t (*tile)[LROW]) {
  const int t = threadIdx.x;
  if constexpr (!TRANSPOSED) {
    // weight stored (K, N): 64 consecutive threads read one 256-byte row piece
    const int nn = t & 63;
    const int64_t n = n0 + nn;
#pragma unroll 4
    for (int kk = t >> 6; kk < TK; kk += 4) {
      const int64_t k = k0 + kk;
      const int v = (k < K && n < N) ? w[k * N + n] : 0;
      tile[nn][kk] = (uint8_t)code_of<FP4>((uint32_t)v);
    }
  } else {
    // weight stored (N, K): 128 consecutive threads read one 512-byte row piece
    const int kk = t & 127;
    const int64_t k = k0 + kk;
#pragma unroll 4
    for (int nn = t >> 7; nn < TN; nn += 2) {
      const int64_t n = n0 + nn;
      const int v = (k < K && n < N) ? w[n * K + k] : 0;
      tile[nn][kk] = (uint8_t)code_of<FP4>((uint32_t)v);
    }
  }
}

// ---- GFX950_B ------------------------------------------------------------
// In GFX950_B a column's 128-deep K block is one 64-byte record of sixteen
// words, word w holding K rows 8w..8w+7 (row 8w+j in nibble j), and the
// records of consecutive columns are consecutive. One workgroup of 16 waves
// packs one K block of PB_N columns: wave w builds word w of every column
// straight from registers, the words meet in LDS, and the workgroup's output
// (PB_N records, one contiguous 16 KiB run) leaves as 16-byte stores.
constexpr int PB_N = 256;

// LDS slot of word w of tile column c: records stay 64 bytes apart, but the
// word order inside a record is XOR-swizzled by c/4 so that both ways of
// building the words write without bank conflicts, and a 16-byte read-back of
// a record quarter still hits one aligned quarter (with its words permuted).
__device__ __forceinline__ int pb_slot(int c, int w) { return c * 16 + (w ^ ((c >> 2) & 15)); }

// Eight input words -> one word of their codes, the first code lowest.
template <bool FP4>
__device__ __forceinline__ uint32_t nibbles_of(const uint32_t (&v)[8]) {
  if constexpr (FP4) {
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = __uint_as_float(v[j]);
    return e2m1x8(f);
  } else {
    uint32_t word = code_of<FP4>(v[0]);
#pragma unroll
    for (int j = 1; j < 8; ++j) word |= code_of<FP4>(v[j]) << (4 * j);
    return word;
  }
}

template <bool TRANSPOSED, bool FP4>
__global__ __launch_bounds__(1024) void pack_gfx950b_kernel(const int32_t* __restrict__ w,
                                                            int64_t K, int64_t N, int64_t Np,
                                                            uint8_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint32_t rec[PB_N * 16];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int64_t k0 = (int64_t)blockIdx.y * 128;
  const int64_t n0 = (int64_t)blockIdx.x * PB_N;
  if constexpr (!TRANSPOSED) {
    // weight (K, N): wave `wave` reads rows k0+8*wave.. +7; lane takes tile
    // columns lane + 64c, so every load instruction reads 256 contiguous bytes.
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(w + k0 * N + n0, 0x7FFFFFFFu);
    const int kr = 8 * wave;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = lane + 64 * c;
      const bool nok = n0 + col < N;
      uint32_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool ok = nok && k0 + kr + j < K;
        v[j] = __builtin_amdgcn_raw_buffer_load_b32(
            rs, ok ? (uint32_t)(((kr + j) * N + col) * 4) : BUF_OOB, 0, 0);
      }
      rec[pb_slot(col, wave)] = nibbles_of<FP4>(v);
    }
  } else {
    // weight (N, K): a column's 8 codes of one word are 32 contiguous bytes;
    // 16 lanes cover one column's K block, 4 columns per wave per pass.
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(w + n0 * K + k0, 0x7FFFFFFFu);
    const int wd = lane & 15;
    const bool kfull = (K & 7) == 0;   // then a word is wholly in or out of range
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = 4 * wave + (lane >> 4) + 64 * c;
      const bool nok = n0 + col < N;
      const uint32_t off = (uint32_t)((col * K + 8 * wd) * 4);
      uint32_t v[8];
      if (kfull) {
        const uint32_t o = nok && k0 + 8 * wd < K ? off : BUF_OOB;
        const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0));
        const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 16, 0));
        v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
        v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool ok = nok && k0 + 8 * wd + j < K;
          v[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? off + 4 * j : BUF_OOB, 0, 0);
        }
      }
      rec[pb_slot(col, wd)] = nibbles_of<FP4>(v);
    }
  }
  __syncthreads();
  // thread t stores bytes 16t..16t+15 of the run: quarter q of column t/4
  const int col = t >> 2, q = t & 3;
  if (n0 + col >= Np) return;
  const int sw = (col >> 2) & 15;
  const u32x4 r = *reinterpret_cast<const u32x4*>(&rec[col * 16 + 4 * (q ^ (sw >> 2))]);
  // word j of the quarter sits at element j ^ (sw & 3)
  u32x4 v = r;
  if (sw & 1) v = u32x4{v.y, v.x, v.w, v.z};
  if (sw & 2) v = u32x4{v.z, v.w, v.x, v.y};
  *reinterpret_cast<u32x4*>(out + ((k0 / 128) * Np + n0) * 64 + 16 * t) = v;
}

template <bool TRANSPOSED, bool FP4>
__global__ __launch_bounds__(256) void pack_nd_kernel(const int32_t* __restrict__ w, int64_t K,
                                                      int64_t N, uint8_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[TN][LROW];
  const int64_t k0 = (int64_t)blockIdx.y * TK;
  const int64_t n0 = (int64_t)blockIdx.x * TN;
  stage_tile<TRANSPOSED, FP4>(w, K, N, k0, n0, tile);
  __syncthreads();
  // thread -> packed row kk, 16 output bytes = columns n0 + half*32 .. +32
  const int t = threadIdx.x;
  const int kk = t >> 1, half = t & 1;
  const int64_t k = k0 + kk;
  if (k >= K) return;
  const int64_t row_bytes = N / 2;
  const int64_t b0 = (n0 + half * 32) / 2;   // first output byte in the row
  if (b0 >= row_bytes) return;
  uint8_t bytes[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int c = half * 32 + 2 * j;
    bytes[j] = (uint8_t)(tile[c][kk] | (tile[c + 1][kk] << 4));
  }
  uint8_t* dst = out + k * row_bytes + b0;
  if (b0 + 16 <= row_bytes && (((uintptr_t)dst) & 15) == 0) {
    u32x4 v;
    v.x = bytes[0] | (bytes[1] << 8) | (bytes[2] << 16) | ((uint32_t)bytes[3] << 24);
    v.y = bytes[4] | (bytes[5] << 8) | (bytes[6] << 16) | ((uint32_t)bytes[7] << 24);
    v.z = bytes[8] | (bytes[9] << 8) | (bytes[10] << 16) | ((uint32_t)bytes[11] << 24);
    v.w = bytes[12] | (bytes[13] << 8) | (bytes[14] << 16) | ((uint32_t)bytes[15] << 24);
    *reinterpret_cast<u32x4*>(dst) = v;
  } else {
    for (int j = 0; j < 16 && b0 + j < row_bytes; ++j) dst[j] = bytes[j];
  }
}

}  // namespace

hipError_t launch_pack_int4(const int32_t* w, int64_t k, int64_t n, bool transpose,
                            wq_layout layout, uint8_t* out, hipStream_t s, bool fp4) {
  if (layout == WQ_LAYOUT_GFX950_B) {
    const int64_t Kp = 128 * ((k + 127) / 128);
    const int64_t Np = 16 * ((n + 15) / 16);
    // tile-relative byte offsets stay below 2^31 (the buffer bound)
    if ((transpose ? (PB_N * k) : (128 * n)) >= (int64_t(1) << 29)) return hipErrorInvalidValue;
    dim3 grid((unsigned)((Np + PB_N - 1) / PB_N), (unsigned)(Kp / 128));
    if (fp4) {
      if (transpose) pack_gfx950b_kernel<true, true><<<grid, 1024, 0, s>>>(w, k, n, Np, out);
      else pack_gfx950b_kernel<false, true><<<grid, 1024, 0, s>>>(w, k, n, Np, out);
    } else {
      if (transpose) pack_gfx950b_kernel<true, false><<<grid, 1024, 0, s>>>(w, k, n, Np, out);
      else pack_gfx950b_kernel<false, false><<<grid, 1024, 0, s>>>(w, k, n, Np, out);
    }
  } else {
    dim3 grid((unsigned)((n + TN - 1) / TN), (unsigned)((k + TK - 1) / TK));
    if (fp4) {
      if (transpose) pack_nd_kernel<true, true><<<grid, 256, 0, s>>>(w, k, n, out);
      else pack_nd_kernel<false, true><<<grid, 256, 0, s>>>(w, k, n, out);
    } else {
      if (transpose) pack_nd_kernel<true, false><<<grid, 256, 0, s>>>(w, k, n, out);
      else pack_nd_kernel<false, false><<<grid, 256, 0, s>>>(w, k, n, out);
    }
  }
  return hipGetLastError();
}

}  // namespace wq
