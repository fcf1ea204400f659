// INT4 weight pack (aclnnConvertWeightToINT4Pack page, operator description):
// one 4-bit value per int32 in, tightly packed nibbles out, in the ND layout
// or the gfx950 MFMA-operand layout GFX950_B (byte formula in wq.h).
//
// One workgroup packs a 128 (K) x 64 (N) tile. The tile's codes are staged in
// LDS as bytes [n][k], loaded so that global reads are coalesced for either
// input orientation, then written out in the target layout: GFX950_B as one
// 16-byte chunk per thread (a column's 32-deep K block), ND as 16-byte runs
// of a packed row. The op is HBM-bound: 4 bytes read per 0.5 byte written.
#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int TK = 128;        // tile depth (K)
constexpr int TN = 64;         // tile width (N)
constexpr int LROW = TK + 4;   // LDS row (one column's codes), padded

template <bool TRANSPOSED>
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
      tile[nn][kk] = (uint8_t)(v & 0xF);
    }
  } else {
    // weight stored (N, K): 128 consecutive threads read one 512-byte row piece
    const int kk = t & 127;
    const int64_t k = k0 + kk;
#pragma unroll 4
    for (int nn = t >> 7; nn < TN; nn += 2) {
      const int64_t n = n0 + nn;
      const int v = (k < K && n < N) ? w[n * K + k] : 0;
      tile[nn][kk] = (uint8_t)(v & 0xF);
    }
  }
}

// Eight byte-sized codes (two dwords read from LDS) -> one word of nibbles,
// the first code in the lowest nibble.
__device__ __forceinline__ uint32_t nibbles8(uint32_t d0, uint32_t d1) {
  auto pack4 = [](uint32_t d) {
    return (d & 0xFu) | ((d >> 4) & 0xF0u) | ((d >> 8) & 0xF00u) | ((d >> 12) & 0xF000u);
  };
  return pack4(d0) | (pack4(d1) << 16);
}

template <bool TRANSPOSED>
__global__ __launch_bounds__(256) void pack_gfx950b_kernel(const int32_t* __restrict__ w,
                                                           int64_t K, int64_t N, int64_t Np,
                                                           uint8_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[TN][LROW];
  const int64_t k0 = (int64_t)blockIdx.y * TK;
  const int64_t n0 = (int64_t)blockIdx.x * TN;
  stage_tile<TRANSPOSED>(w, K, N, k0, n0, tile);
  __syncthreads();
  const int t = threadIdx.x;
  const int nn = t >> 2, blk = t & 3;
  const int64_t n = n0 + nn;
  if (n >= Np) return;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(&tile[nn][blk * 32]);
  u32x4 v;
  v.x = nibbles8(src[0], src[1]);
  v.y = nibbles8(src[2], src[3]);
  v.z = nibbles8(src[4], src[5]);
  v.w = nibbles8(src[6], src[7]);
  *reinterpret_cast<u32x4*>(out + ((k0 / TK) * Np + n) * 64 + blk * 16) = v;
}

template <bool TRANSPOSED>
__global__ __launch_bounds__(256) void pack_nd_kernel(const int32_t* __restrict__ w, int64_t K,
                                                      int64_t N, uint8_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[TN][LROW];
  const int64_t k0 = (int64_t)blockIdx.y * TK;
  const int64_t n0 = (int64_t)blockIdx.x * TN;
  stage_tile<TRANSPOSED>(w, K, N, k0, n0, tile);
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
                            wq_layout layout, uint8_t* out, hipStream_t s) {
  if (layout == WQ_LAYOUT_GFX950_B) {
    const int64_t Kp = 128 * ((k + 127) / 128);
    const int64_t Np = 16 * ((n + 15) / 16);
    dim3 grid((unsigned)((Np + TN - 1) / TN), (unsigned)(Kp / TK));
    if (transpose)
      pack_gfx950b_kernel<true><<<grid, 256, 0, s>>>(w, k, n, Np, out);
    else
      pack_gfx950b_kernel<false><<<grid, 256, 0, s>>>(w, k, n, Np, out);
  } else {
    dim3 grid((unsigned)((n + TN - 1) / TN), (unsigned)((k + TK - 1) / TK));
    if (transpose)
      pack_nd_kernel<true><<<grid, 256, 0, s>>>(w, k, n, out);
    else
      pack_nd_kernel<false><<<grid, 256, 0, s>>>(w, k, n, out);
  }
  return hipGetLastError();
}

}  // namespace wq
