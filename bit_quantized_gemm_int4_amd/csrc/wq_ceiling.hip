// Achievable-ceiling microkernels: measurement aids, not operators of any
// page. The measurement reports a kernel's rate against MI355X's published
// peaks; these two kernels give, beside them, what this GPU reaches on the
// same resource with nothing else in the way:
//   - stream read: every 16-byte chunk of a buffer loaded once (one buffer
//     load of 16 bytes per lane, four per thread issued before any use, the
//     words XOR-folded so that no load is dead), one 32-bit word per wave out;
//   - MFMA loop: eight independent v_mfma_f32_16x16x32_bf16 per round on
//     register operands (random bf16 values that change from one MFMA to
//     the next), the bf16 instruction the prefill tile issues.
#include "wq_device.h"
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int SR_THREADS = 256;
constexpr int SR_PER_THREAD = 4;                                   // 16-byte loads per thread
constexpr int64_t SR_WG_BYTES = (int64_t)SR_THREADS * SR_PER_THREAD * 16;   // 16 KiB per workgroup

__global__ __launch_bounds__(SR_THREADS) void stream_read_kernel(const uint8_t* __restrict__ src, int64_t bytes,
                                                                 uint32_t* __restrict__ out) {
  const int t = threadIdx.x, lane = t & 63;
  const int64_t base = (int64_t)blockIdx.x * SR_WG_BYTES;
  const int64_t left = bytes - base;
  // this workgroup's 16 KiB (or the tail): offsets past it read zeros
  const __amdgpu_buffer_rsrc_t r = buf_rsrc(src + base, (uint32_t)(left < SR_WG_BYTES ? left : SR_WG_BYTES));
  u32x4 v[SR_PER_THREAD];
#pragma unroll
  for (int i = 0; i < SR_PER_THREAD; ++i)
    v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         r, (uint32_t)((i * SR_THREADS + t) * 16), 0, 0));
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < SR_PER_THREAD; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x ^= (uint32_t)__shfl_xor((int)x, s);
  if (lane == 0) out[blockIdx.x * (SR_THREADS / 64) + (t >> 6)] = x;
}

constexpr int ML_THREADS = 256;

// One operand dword (two bf16) of lane l, operand set `set` (A: 0..3,
// B: 4..7), dword d: a 32-bit integer hash of the three indices, each half
// turned into a value of magnitude in [0.5, 2) with random sign and
// mantissa (bits: sign | 0x3F00 | low exponent bit | 7 mantissa bits).
// Random operands that change from one MFMA to the next switch as many bits
// as a GEMM on real data does, so the loop draws the power such a GEMM
// draws.
__device__ __forceinline__ uint32_t ml_dword(uint32_t l, uint32_t set, uint32_t d) {
  uint32_t x = l * 0x9E3779B1u + set * 0x85EBCA77u + d * 0xC2B2AE3Du + 0x27D4EB2Fu;
  x ^= x >> 15;
  x *= 0x2C1B3C6Du;
  x ^= x >> 12;
  x *= 0x297A2D39u;
  x ^= x >> 15;
  return (x & 0x80FF80FFu) | 0x3F003F00u;
}

__global__ __launch_bounds__(ML_THREADS) void mfma_loop_kernel(int iters, float* __restrict__ out) {
  const uint32_t l = threadIdx.x & 63;
  u32x4 a[4], b[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    a[s] = (u32x4){ml_dword(l, s, 0), ml_dword(l, s, 1), ml_dword(l, s, 2), ml_dword(l, s, 3)};
    b[s] = (u32x4){ml_dword(l, s + 4, 0), ml_dword(l, s + 4, 1), ml_dword(l, s + 4, 2), ml_dword(l, s + 4, 3)};
  }
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // accumulator j: A set j % 4, B set j / 2
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = mfma16<ACT_BF16>(a[j & 3], b[j >> 1], acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
  out[(int64_t)blockIdx.x * ML_THREADS + threadIdx.x] = s;
}

}  // namespace
}  // namespace wq

extern "C" size_t wq_ceiling_stream_read_words(size_t bytes) {
  if (bytes == 0 || bytes % 16 != 0 || bytes >= ((size_t)1 << 40)) return 0;
  return (size_t)((bytes + wq::SR_WG_BYTES - 1) / wq::SR_WG_BYTES) * (wq::SR_THREADS / 64);
}

extern "C" wq_status wq_ceiling_stream_read(const void* src, size_t bytes, uint32_t* out, hipStream_t stream) {
  if (!src || !out) return WQ_ERR_NULLPTR;
  const size_t words = wq_ceiling_stream_read_words(bytes);
  if (words == 0 || (reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(out) & 3) != 0)
    return WQ_ERR_SHAPE;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), o0 = reinterpret_cast<uintptr_t>(out);
  if (o0 < s0 + bytes && s0 < o0 + words * 4) return WQ_ERR_ALIAS;
  const size_t grid = words / (wq::SR_THREADS / 64);
  if (grid > 0xFFFFFFFFull) return WQ_ERR_SHAPE;
  wq::stream_read_kernel<<<dim3((unsigned)grid), wq::SR_THREADS, 0, stream>>>(
      static_cast<const uint8_t*>(src), (int64_t)bytes, out);
  return hipGetLastError() == hipSuccess ? WQ_OK : WQ_ERR_LAUNCH;
}

extern "C" wq_status wq_ceiling_mfma_loop(int64_t workgroups, int32_t iters, float* out, hipStream_t stream) {
  if (!out) return WQ_ERR_NULLPTR;
  if (workgroups < 1 || workgroups > (int64_t(1) << 20) || iters < 1 || iters > 16384 ||
      (reinterpret_cast<uintptr_t>(out) & 3) != 0)
    return WQ_ERR_SHAPE;
  wq::mfma_loop_kernel<<<dim3((unsigned)workgroups), wq::ML_THREADS, 0, stream>>>(iters, out);
  return hipGetLastError() == hipSuccess ? WQ_OK : WQ_ERR_LAUNCH;
}
