// The four-stage buffer->LDS ring of the 8-bit integer tiles (i8_gemm.hip,
// a8w4_gemm.hip): the x1 operand's DMA addressing, its LDS swizzle and the
// barrier that leaves later stages' DMA in flight. x1 is (M, K) int8
// row-major; a step moves 64 K bytes of 256 rows (16 KiB).
#pragma once

#include "wq_device.h"

namespace wq {

constexpr int I8_BK = 64;                 // K bytes per step
constexpr int I8_STAGE = 256 * I8_BK;   // one 256-row operand stage: 16 KiB

// LDS rows are 64 bytes (one step of one row / column), four 16-byte chunks.
// Chunk c of row r sits at position c ^ ((r >> 1) & 3). Of the swizzles
// timed on this LDS for 16-byte reads of 16 rows (one chunk each), this one
// runs as fast as a conflict-free read; c ^ ((r >> 2) & 3) ran about 20%
// slower, as slow as no swizzle.
__device__ __forceinline__ int i8_pos(int r, int c) { return c ^ ((r >> 1) & 3); }

// Per-lane DMA addressing of one operand: 256 rows x 64 K bytes per stage by
// 16 DMA instructions of 1 KiB (16 rows); wave w issues 2w + j, lane l fills
// row 16 (2w + j) + l / 4 at position l % 4, fetching logical chunk
// (l % 4) ^ ((row >> 1) & 3). `base` is the byte offset of that chunk at K 0
// (BUF_OOB for rows past the operand), `klim` the step origins k0 < klim for
// which the chunk lies inside K; outside, the lane reads zeros.
struct I8Dma {
  uint32_t base[2];
  int klim[2];
};

__device__ __forceinline__ I8Dma i8_dma_setup(int rows, int64_t k) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  I8Dma d;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 16 * (2 * wave + j) + (lane >> 2);
    const int c = i8_pos(row, lane & 3);
    d.base[j] = row < rows ? (uint32_t)(row * k + 16 * c) : BUF_OOB;
    d.klim[j] = (int)k - 16 * c;
  }
  return d;
}

// DMA instruction j (0 or 1) of this wave for one operand stage starting at
// K offset k0.
__device__ __forceinline__ void i8_dma(__amdgpu_buffer_rsrc_t rs, const I8Dma& d, int j, int k0, uint8_t* buf) {
  const uint32_t off = k0 < d.klim[j] ? d.base[j] + (uint32_t)k0 : BUF_OOB;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(buf + (2 * wave_id() + j) * 1024), 16, off, 0, 0, 0);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// A workgroup barrier that orders LDS accesses only: the caller has already
// waited for what must be complete (its own DMA and LDS reads), so the
// buffer->LDS DMA of later stages stays in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace wq
