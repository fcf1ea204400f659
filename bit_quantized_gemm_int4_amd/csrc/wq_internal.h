// Host-side launchers shared between the kernel files and the C ABI layer.
// Arguments here are already validated; launchers only pick a kernel and a
// grid and enqueue it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/wq.h"

namespace wq {

// Rows per launch for kernels whose grid runs over rows: every row-parallel
// operator splits taller inputs into independent chunks of this many rows, so
// that no grid passes 2^32 threads in a dimension (the pages allow up to
// 2^31 - 1 rows).
constexpr int64_t kRowChunk = int64_t(1) << 20;

// fp4: the 32-bit inputs are floats, encoded to E2M1 codes (else int4 values)
hipError_t launch_pack_int4(const int32_t* w, int64_t k, int64_t n, bool transpose,
                            wq_layout layout, uint8_t* out, hipStream_t s, bool fp4);

hipError_t launch_quant_per_token(const void* x, bool bf16, int64_t rows, int64_t cols,
                                  const void* smooth, wq_dtype y_dtype, void* y,
                                  float* scale, hipStream_t s);

hipError_t launch_quant_mx(const void* x, bool bf16, int64_t rows, int64_t cols,
                           const void* smooth, wq_dtype y_dtype, bool transpose_y,
                           uint8_t* y, uint8_t* scale, hipStream_t s);

// Weight-quantized matmul + AddRmsNorm problem after validation.
struct WqProblem {
  const void* x1;
  const void* x2;
  const void* scale;
  const void* offset;   // may be null
  const void* bias;     // may be null
  const void* residual;  // null: zero (the standalone matmul)
  const void* gamma;
  void* y;
  void* norm_out;       // null: no norm pass (the standalone matmul)
  void* workspace;
  size_t workspace_size;
  int64_t m, k, n;
  bool bf16;
  int w_bits;           // 4 or 8
  wq_layout layout;
  bool transpose_x2;    // int8 only
  // dequant indexing: scale index of (k, n) = (k / group) * s_row + n * s_col
  int64_t group;        // k-group length (>= k for per-channel / per-tensor)
  int64_t s_row;
  int64_t s_col;
  float eps;
};

size_t wq_workspace_bytes(int64_t m, int64_t k, int64_t n);

// AddRmsNorm on (rows, d) act-dtype rows: y = x + residual, normOut =
// y * rstd * gamma (add_rmsnorm.hip).
hipError_t launch_add_rmsnorm(const void* x, const void* residual, const void* gamma, int64_t rows,
                              int64_t d, bool bf16, float eps, void* y, void* norm_out, hipStream_t s);
hipError_t launch_wq_matmul_add_rmsnorm(const WqProblem& p, hipStream_t s);

// Fast GFX950_B INT4 path (group a multiple of 128, or per channel/tensor).
bool fast_path_ok(const WqProblem& p);
size_t fast_rowsum_bytes(int64_t m, int64_t k);
size_t fast_corr_bytes(int64_t n, int64_t k);
hipError_t launch_prefill(const WqProblem& p, float* partial, uint16_t* rs, uint16_t* corr,
                          hipStream_t s);

// Weight-streaming kernel for m <= 32 (INT4, GFX950_B, k a multiple of 128,
// any group); writes one sum of y^2 per (row, workgroup) at
// partial[row * decode_grid(p) + workgroup]; decode_partial_bytes(n) bounds
// that array over every group size.
bool decode_ok(const WqProblem& p);
int64_t decode_grid(const WqProblem& p);
size_t decode_partial_bytes(int64_t n);
hipError_t launch_decode(const WqProblem& p, float* partial, hipStream_t s);

// INT8-weight tile (any m; k a multiple of 16; row-major weights with n a
// multiple of 4 below 2 GiB, or transposed); partials as gemm_generic's:
// [row][ceil(n / 32)].
bool w8_ok(const WqProblem& p);
// `finished`: set when the call also formed y and normOut (a K split with
// its own finish), so that no norm pass follows.
hipError_t launch_w8(const WqProblem& p, float* partial, hipStream_t s, bool& finished);
// Workspace bytes of the INT8 tile's K split for an (m, k, n) row chunk (0:
// no split).
size_t w8_split_bytes(int64_t m, int64_t k, int64_t n);

struct MxProblem {
  const uint8_t* x1;     // (k, m) e4m3
  const uint8_t* x2;     // GFX950_B e2m1
  const uint8_t* s1;     // (m, kb)
  const uint8_t* s2;     // (kb, n)
  float* y;
  int64_t m, k, n;
  uint8_t* x1pad;        // null, or mx_x1pad_bytes(m, k, n) bytes for x1 with rows padded to 16
};

// Workspace the MX GEMM can use when m is not a multiple of 16: x1 copied to
// (k, 16 ceil(m / 16)) so that the 256 x 256 tile can take the shape; 0 when
// the shape needs none (or cannot take the tile anyway).
size_t mx_x1pad_bytes(int64_t m, int64_t k, int64_t n);
hipError_t launch_mx_matmul(const MxProblem& p, hipStream_t s);

struct I8Problem {
  const int8_t* x1;      // (m, k)
  const int8_t* x2t;     // (n, k)
  const float* s1;       // (m)
  const float* s2;       // (n)
  float* y;              // (m, n)
  int64_t m, k, n;
};

hipError_t launch_i8_matmul(const I8Problem& p, hipStream_t s);

// INT8 (or INT4) x INT4 (GFX950_B) quantized matmul with in-place add
// (a8w4_gemm.hip).
struct A8W4Problem {
  const uint8_t* x1;     // int8 (m, k), or INT4 codes (m, k/2) bytes when x1_int4
  const uint8_t* x2;     // INT4 codes, logical (k, n), GFX950_B
  const float* s1;       // (m)
  const float* s2;       // (n)
  float* y;              // (m, n)
  int64_t m, k, n;
  bool x1_int4;
};

hipError_t launch_a8w4_matmul(const A8W4Problem& p, hipStream_t s);

// MXFP4 x MXFP4 with in-place add (mx4_gemm.hip). The workspace holds the
// scales rearranged for the lanes (mx4_workspace_bytes).
struct Mx4Problem {
  const uint8_t* x1;     // E2M1 (m, k), two per byte along k
  const uint8_t* x2;     // E2M1 in GFX950_B
  const uint8_t* s1;     // E8M0 (m, ceil(k/32))
  const uint8_t* s2;     // E8M0 (ceil(k/32), n)
  float* y;              // (m, n)
  int64_t m, k, n;
  void* workspace;
};

size_t mx4_workspace_bytes(int64_t m, int64_t k, int64_t n);
hipError_t launch_mx4_matmul(const Mx4Problem& p, hipStream_t s);

// Profiling hook (wq_profile.cpp): event pair around a contraction kernel.
void prof_begin(hipStream_t s);
void prof_end(hipStream_t s);

}  // namespace wq
