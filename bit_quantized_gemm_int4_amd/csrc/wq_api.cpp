// C ABI of libwq: argument validation (host only, before any launch) and
// dispatch to the kernel launchers. Every rule cited here comes from the
// operator pages named in wq.h; the status codes are this library's own.
#include <cmath>
#include <cstdint>

#include "wq_internal.h"

namespace {

constexpr int kAbiVersion = 1;
constexpr int64_t kMaxKN = 65535;            // k, n range (AddRmsNorm page, Constraints)
constexpr int64_t kMaxRows = 2147483647LL;   // b*s range (same)

bool is_act(wq_dtype d) { return d == WQ_F16 || d == WQ_BF16; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// [a, a+na) and [b, b+nb) overlap (both non-empty).
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

wq_status from_hip(hipError_t e) { return e == hipSuccess ? WQ_OK : WQ_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* wq_status_string(wq_status status) {
  switch (status) {
    case WQ_OK: return "WQ_OK";
    case WQ_ERR_NULLPTR: return "WQ_ERR_NULLPTR: a required pointer is null";
    case WQ_ERR_SHAPE: return "WQ_ERR_SHAPE: size out of range, shapes disagree or pointer misaligned";
    case WQ_ERR_DTYPE: return "WQ_ERR_DTYPE: unsupported dtype";
    case WQ_ERR_GROUP: return "WQ_ERR_GROUP: group size / scale shape rule broken";
    case WQ_ERR_WORKSPACE: return "WQ_ERR_WORKSPACE: workspace missing or too small";
    case WQ_ERR_UNSUPPORTED: return "WQ_ERR_UNSUPPORTED: option not offered by this library";
    case WQ_ERR_LAUNCH: return "WQ_ERR_LAUNCH: the HIP runtime refused a launch";
    case WQ_ERR_ALIAS: return "WQ_ERR_ALIAS: an output overlaps an input it may not alias";
  }
  return "unknown wq_status";
}

int wq_abi_version(void) { return kAbiVersion; }

// ---------------------------------------------------------------------------
size_t wq_pack_int4_bytes(int64_t k, int64_t n, wq_layout layout) {
  if (k < 0 || n < 0) return 0;
  if (layout == WQ_LAYOUT_ND) return (n % 2) ? 0 : (size_t)(k * (n / 2));
  if (layout == WQ_LAYOUT_GFX950_B) {
    const int64_t kp = 128 * ((k + 127) / 128), np = 16 * ((n + 15) / 16);
    return (size_t)(kp * np / 2);
  }
  return 0;
}

namespace {

// Both packs: the same sizes, limits and layouts (32-bit inputs either way).
wq_status pack_checked(const void* weight, int64_t k, int64_t n, int transpose, wq_layout layout,
                       void* out, hipStream_t stream, bool fp4) {
  if (layout != WQ_LAYOUT_ND && layout != WQ_LAYOUT_GFX950_B) return WQ_ERR_UNSUPPORTED;
  if (k < 0 || n < 0) return WQ_ERR_SHAPE;
  if (layout == WQ_LAYOUT_ND && (n % 2)) return WQ_ERR_SHAPE;
  if ((k + 127) / 128 > 65535 || (n + 63) / 64 > 2147483647LL) return WQ_ERR_SHAPE;
  // GFX950_B kernels address one 128 x 256 tile with 32-bit byte offsets
  if (layout == WQ_LAYOUT_GFX950_B && (transpose ? 256 * k : 128 * n) >= (int64_t(1) << 29))
    return WQ_ERR_SHAPE;
  if (k == 0 || n == 0) return WQ_OK;
  if (!weight || !out) return WQ_ERR_NULLPTR;
  if (!aligned16(out)) return WQ_ERR_SHAPE;
  if (overlap(weight, (size_t)(k * n) * 4, out, wq_pack_int4_bytes(k, n, layout))) return WQ_ERR_ALIAS;
  return from_hip(wq::launch_pack_int4(static_cast<const int32_t*>(weight), k, n, transpose != 0,
                                       layout, static_cast<uint8_t*>(out), stream, fp4));
}

}  // namespace

wq_status wq_pack_int4(const int32_t* weight, int64_t k, int64_t n, int transpose,
                       wq_layout layout, void* out, hipStream_t stream) {
  return pack_checked(weight, k, n, transpose, layout, out, stream, false);
}

wq_status wq_pack_fp4(const float* weight, int64_t k, int64_t n, int transpose, wq_layout layout,
                      void* out, hipStream_t stream) {
  return pack_checked(weight, k, n, transpose, layout, out, stream, true);
}

// ---------------------------------------------------------------------------
wq_status wq_dynamic_quant(const void* x, wq_dtype x_dtype, int64_t rows, int64_t cols,
                           const void* smooth, wq_dtype y_dtype, int64_t block_k,
                           int transpose_y, void* y, void* scale, hipStream_t stream) {
  if (!is_act(x_dtype)) return WQ_ERR_DTYPE;
  if (rows < 0 || cols < 0 || rows > kMaxRows) return WQ_ERR_SHAPE;
  const bool bf16 = x_dtype == WQ_BF16;
  if (block_k == 0) {
    if (y_dtype != WQ_INT8 && y_dtype != WQ_INT4 && y_dtype != WQ_INT32) return WQ_ERR_DTYPE;
    if (transpose_y) return WQ_ERR_UNSUPPORTED;
    // Constraints: INT4 needs an even last dim, INT32 one divisible by 8.
    if (y_dtype == WQ_INT4 && (cols % 2)) return WQ_ERR_SHAPE;
    if (y_dtype == WQ_INT32 && (cols % 8)) return WQ_ERR_SHAPE;
    if (cols >= (int64_t(1) << 30)) return WQ_ERR_SHAPE;   // row byte offsets are 32-bit
    if (rows == 0 || cols == 0) return WQ_OK;
    if (!x || !y || !scale) return WQ_ERR_NULLPTR;
    if (!aligned16(x) || (smooth && !aligned16(smooth)) || !aligned16(y)) return WQ_ERR_SHAPE;
    return from_hip(wq::launch_quant_per_token(x, bf16, rows, cols, smooth, y_dtype, y,
                                               static_cast<float*>(scale), stream));
  }
  if (block_k != 32) return WQ_ERR_UNSUPPORTED;
  if (y_dtype != WQ_FP8_E4M3 && y_dtype != WQ_FP4_E2M1) return WQ_ERR_DTYPE;
  if (transpose_y && y_dtype != WQ_FP8_E4M3) return WQ_ERR_UNSUPPORTED;
  if (y_dtype == WQ_FP4_E2M1 && (cols % 2)) return WQ_ERR_SHAPE;
  if ((cols + 63) / 64 > 65535) return WQ_ERR_SHAPE;
  if (rows == 0 || cols == 0) return WQ_OK;
  if (!x || !y || !scale) return WQ_ERR_NULLPTR;
  if (!aligned16(x) || (smooth && !aligned16(smooth)) || !aligned16(y)) return WQ_ERR_SHAPE;
  return from_hip(wq::launch_quant_mx(x, bf16, rows, cols, smooth, y_dtype, transpose_y != 0,
                                      static_cast<uint8_t*>(y), static_cast<uint8_t*>(scale),
                                      stream));
}

// ---------------------------------------------------------------------------
size_t wq_matmul_add_rmsnorm_workspace_size(int64_t m, int64_t k, int64_t n) {
  if (m < 0 || k < 0 || n < 0) return 0;
  return wq::wq_workspace_bytes(m, k, n);
}

namespace {

// Checks shared by the fused operator and the standalone matmul (the pages'
// Constraints): dtypes, layouts, sizes and the scale granularity. Fills the
// problem's dequant indexing.
wq_status check_wq_common(int64_t m, int64_t k, wq_dtype act_dtype, int64_t n, wq_dtype w_dtype,
                          wq_layout x2_layout, int transpose_x2, int64_t scale_rows,
                          int64_t scale_cols, int64_t antiquant_group_size, wq::WqProblem& p) {
  // dtypes: x2 int8 or int4; every other input shares one dtype (Constraints)
  if (!is_act(act_dtype)) return WQ_ERR_DTYPE;
  if (w_dtype != WQ_INT4 && w_dtype != WQ_INT8) return WQ_ERR_DTYPE;
  if (x2_layout != WQ_LAYOUT_ND && x2_layout != WQ_LAYOUT_GFX950_B) return WQ_ERR_UNSUPPORTED;
  // a transposed GFX950_B weight is the same layout: the pack takes the transpose
  if (w_dtype == WQ_INT4 && transpose_x2 && x2_layout != WQ_LAYOUT_ND) return WQ_ERR_UNSUPPORTED;
  if (w_dtype == WQ_INT8 && x2_layout != WQ_LAYOUT_ND) return WQ_ERR_UNSUPPORTED;
  // shapes: b*s in [0, 2^31-1] (0 = empty); k in [1, 65535]; n in [0, 65535]
  if (m < 0 || m > kMaxRows) return WQ_ERR_SHAPE;
  if (k < 1 || k > kMaxKN) return WQ_ERR_SHAPE;
  if (n < 0 || n > kMaxKN) return WQ_ERR_SHAPE;
  // INT4 ND packs the last stored dimension: n, or k when transposed (n, k)
  if (w_dtype == WQ_INT4 && x2_layout == WQ_LAYOUT_ND && ((transpose_x2 ? k : n) % 2))
    return WQ_ERR_SHAPE;
  // quantization granularity (Constraints): per tensor (1), per channel
  // (1, n) / (n), per group (ceil(k/G), n) with G in [32, k-1], G % 32 == 0.
  const int64_t G = antiquant_group_size;
  if (G != 0) {
    if (G < 32 || G % 32 != 0 || G > k - 1) return WQ_ERR_GROUP;
    if (scale_rows != (k + G - 1) / G || scale_cols != n) return WQ_ERR_GROUP;
    p.group = G;
    p.s_row = n;
    p.s_col = 1;
  } else if (scale_rows == 1 && scale_cols == 1) {
    p.group = k;
    p.s_row = 0;
    p.s_col = 0;
  } else if (scale_rows == 1 && scale_cols == n) {
    p.group = k;
    p.s_row = 0;
    p.s_col = 1;
  } else {
    return WQ_ERR_GROUP;
  }
  p.m = m;
  p.k = k;
  p.n = n;
  p.bf16 = act_dtype == WQ_BF16;
  p.w_bits = w_dtype == WQ_INT4 ? 4 : 8;
  p.layout = x2_layout;
  p.transpose_x2 = transpose_x2 != 0;
  return WQ_OK;
}

}  // namespace

wq_status wq_matmul_add_rmsnorm(const void* x1, int64_t m, int64_t k, wq_dtype act_dtype,
                                const void* x2, int64_t n, wq_dtype w_dtype, wq_layout x2_layout,
                                int transpose_x2, const void* antiquant_scale, int64_t scale_rows,
                                int64_t scale_cols, const void* antiquant_offset,
                                int64_t antiquant_group_size, const void* bias,
                                const void* residual, const void* gamma, double epsilon, void* y,
                                void* norm_out, void* workspace, size_t workspace_size,
                                hipStream_t stream) {
  wq::WqProblem p{};
  const wq_status st = check_wq_common(m, k, act_dtype, n, w_dtype, x2_layout, transpose_x2,
                                       scale_rows, scale_cols, antiquant_group_size, p);
  if (st != WQ_OK) return st;
  if (!std::isfinite(epsilon) || epsilon < 0) return WQ_ERR_SHAPE;
  if (m == 0 || n == 0) return WQ_OK;                  // empty tensors (Constraints)
  if (!x1 || !x2 || !antiquant_scale || !residual || !gamma || !y || !norm_out)
    return WQ_ERR_NULLPTR;
  const size_t need = wq::wq_workspace_bytes(m, k, n);
  if (!workspace || workspace_size < need) return WQ_ERR_WORKSPACE;
  const void* ptrs[] = {x1, x2, antiquant_scale, antiquant_offset, bias, residual, gamma,
                        y, norm_out, workspace};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return WQ_ERR_SHAPE;
  // aliasing: y may be residual (inplace); norm_out may overlap nothing
  const size_t mn2 = (size_t)(m * n) * 2;
  const size_t wbytes = w_dtype == WQ_INT8 ? (size_t)(k * n)
                                            : wq_pack_int4_bytes(k, n, x2_layout);
  const size_t sbytes = (size_t)(scale_rows * scale_cols) * 2;
  if (overlap(norm_out, mn2, x1, (size_t)(m * k) * 2) || overlap(norm_out, mn2, x2, wbytes) ||
      overlap(norm_out, mn2, antiquant_scale, sbytes) ||
      overlap(norm_out, mn2, antiquant_offset, sbytes) ||
      overlap(norm_out, mn2, bias, (size_t)n * 2) || overlap(norm_out, mn2, residual, mn2) ||
      overlap(norm_out, mn2, gamma, (size_t)n * 2) || overlap(norm_out, mn2, y, mn2) ||
      overlap(norm_out, mn2, workspace, need))
    return WQ_ERR_ALIAS;
  if (y != residual && overlap(y, mn2, residual, mn2)) return WQ_ERR_ALIAS;
  if (overlap(y, mn2, x1, (size_t)(m * k) * 2) || overlap(y, mn2, x2, wbytes) ||
      overlap(y, mn2, workspace, need))
    return WQ_ERR_ALIAS;
  // the pre-pass writes the workspace before the GEMM reads its inputs
  if (overlap(workspace, need, x1, (size_t)(m * k) * 2) || overlap(workspace, need, x2, wbytes) ||
      overlap(workspace, need, antiquant_scale, sbytes) ||
      overlap(workspace, need, antiquant_offset, sbytes) ||
      overlap(workspace, need, bias, (size_t)n * 2) || overlap(workspace, need, residual, mn2) ||
      overlap(workspace, need, gamma, (size_t)n * 2))
    return WQ_ERR_ALIAS;

  p.x1 = x1;
  p.x2 = x2;
  p.scale = antiquant_scale;
  p.offset = antiquant_offset;
  p.bias = bias;
  p.residual = residual;
  p.gamma = gamma;
  p.y = y;
  p.norm_out = norm_out;
  p.workspace = workspace;
  p.workspace_size = workspace_size;
  p.eps = (float)epsilon;
  return from_hip(wq::launch_wq_matmul_add_rmsnorm(p, stream));
}

// ---------------------------------------------------------------------------
size_t wq_weight_quant_matmul_workspace_size(int64_t m, int64_t k, int64_t n) {
  if (m < 0 || k < 0 || n < 0) return 0;
  return wq::wq_workspace_bytes(m, k, n);
}

wq_status wq_weight_quant_matmul(const void* x1, int64_t m, int64_t k, wq_dtype act_dtype,
                                 const void* x2, int64_t n, wq_dtype w_dtype, wq_layout x2_layout,
                                 int transpose_x2, const void* antiquant_scale, int64_t scale_rows,
                                 int64_t scale_cols, const void* antiquant_offset,
                                 int64_t antiquant_group_size, const void* bias, void* out,
                                 void* workspace, size_t workspace_size, hipStream_t stream) {
  wq::WqProblem p{};
  const wq_status st = check_wq_common(m, k, act_dtype, n, w_dtype, x2_layout, transpose_x2,
                                       scale_rows, scale_cols, antiquant_group_size, p);
  if (st != WQ_OK) return st;
  if (m == 0 || n == 0) return WQ_OK;
  if (!x1 || !x2 || !antiquant_scale || !out) return WQ_ERR_NULLPTR;
  const size_t need = wq::wq_workspace_bytes(m, k, n);
  if (!workspace || workspace_size < need) return WQ_ERR_WORKSPACE;
  const void* ptrs[] = {x1, x2, antiquant_scale, antiquant_offset, bias, out, workspace};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return WQ_ERR_SHAPE;
  const size_t mn2 = (size_t)(m * n) * 2;
  const size_t wbytes = w_dtype == WQ_INT8 ? (size_t)(k * n)
                                            : wq_pack_int4_bytes(k, n, x2_layout);
  const size_t sbytes = (size_t)(scale_rows * scale_cols) * 2;
  if (overlap(out, mn2, x1, (size_t)(m * k) * 2) || overlap(out, mn2, x2, wbytes) ||
      overlap(out, mn2, antiquant_scale, sbytes) || overlap(out, mn2, antiquant_offset, sbytes) ||
      overlap(out, mn2, bias, (size_t)n * 2) || overlap(out, mn2, workspace, need))
    return WQ_ERR_ALIAS;
  if (overlap(workspace, need, x1, (size_t)(m * k) * 2) || overlap(workspace, need, x2, wbytes) ||
      overlap(workspace, need, antiquant_scale, sbytes) ||
      overlap(workspace, need, antiquant_offset, sbytes) || overlap(workspace, need, bias, (size_t)n * 2))
    return WQ_ERR_ALIAS;
  p.x1 = x1;
  p.x2 = x2;
  p.scale = antiquant_scale;
  p.offset = antiquant_offset;
  p.bias = bias;
  p.residual = nullptr;             // read as zeros by every path
  p.gamma = nullptr;
  p.y = out;
  p.norm_out = nullptr;             // no norm pass
  p.workspace = workspace;
  p.workspace_size = workspace_size;
  p.eps = 0.f;
  return from_hip(wq::launch_wq_matmul_add_rmsnorm(p, stream));
}

// ---------------------------------------------------------------------------
wq_status wq_add_rms_norm(const void* x, const void* residual, const void* gamma, int64_t rows,
                          int64_t cols, wq_dtype dtype, double epsilon, void* y, void* norm_out,
                          hipStream_t stream) {
  if (!is_act(dtype)) return WQ_ERR_DTYPE;
  if (rows < 0 || rows > kMaxRows || cols < 1 || cols > kMaxKN) return WQ_ERR_SHAPE;
  if (!std::isfinite(epsilon) || epsilon < 0) return WQ_ERR_SHAPE;
  if (rows == 0) return WQ_OK;
  if (!x || !residual || !gamma || !y || !norm_out) return WQ_ERR_NULLPTR;
  const void* ptrs[] = {x, residual, gamma, y, norm_out};
  for (const void* q : ptrs)
    if (!aligned16(q)) return WQ_ERR_SHAPE;
  const size_t b = (size_t)(rows * cols) * 2, gb = (size_t)cols * 2;
  // y: exactly x or residual (in place), or apart from both; norm_out apart
  // from everything
  if ((y != x && overlap(y, b, x, b)) || (y != residual && overlap(y, b, residual, b)) ||
      overlap(y, b, gamma, gb))
    return WQ_ERR_ALIAS;
  if (overlap(norm_out, b, x, b) || overlap(norm_out, b, residual, b) ||
      overlap(norm_out, b, gamma, gb) || overlap(norm_out, b, y, b))
    return WQ_ERR_ALIAS;
  return from_hip(wq::launch_add_rmsnorm(x, residual, gamma, rows, cols, dtype == WQ_BF16,
                                         (float)epsilon, y, norm_out, stream));
}

// ---------------------------------------------------------------------------
size_t mx_quant_matmul_inplace_add_workspace_size(int64_t m, int64_t k, int64_t n) {
  return wq::mx_x1pad_bytes(m, k, n);
}

wq_status mx_quant_matmul_inplace_add(const void* x1, const void* x2, wq_layout x2_layout,
                                      const uint8_t* x1_scale, const uint8_t* x2_scale,
                                      int64_t m, int64_t k, int64_t n, int transpose_x1,
                                      int transpose_x2, int64_t group_size, float* y,
                                      void* workspace, size_t workspace_size,
                                      hipStream_t stream) {
  // Constraints: only transposeX1 = true, transposeX2 = false.
  if (transpose_x1 != 1 || transpose_x2 != 0) return WQ_ERR_UNSUPPORTED;
  if (x2_layout != WQ_LAYOUT_GFX950_B) return WQ_ERR_UNSUPPORTED;
  if (m < 0 || k < 0 || n < 0 || m > kMaxRows || k > kMaxRows || n > kMaxRows) return WQ_ERR_SHAPE;
  // the small-tile kernel's grid: m / 64 blocks in y, n / 64 of 256 threads in x
  if ((m + 63) / 64 > 65535 || n >= (int64_t(1) << 30)) return WQ_ERR_SHAPE;
  // groupSize = K | N << 16 | M << 32; zero fields inferred from the shapes:
  // scale1 is (m, ceil(k/32)) and scale2 (ceil(k/32), n), so M and N infer to
  // 1 by exact division and K to 32.
  if (group_size < 0 || (group_size >> 48) != 0) return WQ_ERR_GROUP;
  const int64_t gk = group_size & 0xFFFF, gn = (group_size >> 16) & 0xFFFF,
                gm = (group_size >> 32) & 0xFFFF;
  if ((gk != 0 && gk != 32) || (gn != 0 && gn != 1) || (gm != 0 && gm != 1)) return WQ_ERR_GROUP;
  if (m == 0 || n == 0 || k == 0) return WQ_OK;
  if (!x1 || !x2 || !x1_scale || !x2_scale || !y) return WQ_ERR_NULLPTR;
  // the tiled kernel copies x1 in 16-byte and the scales in 4-byte pieces
  if (!aligned16(x1) || !aligned16(x2) || !aligned16(y) || !aligned4(x1_scale) || !aligned4(x2_scale))
    return WQ_ERR_SHAPE;
  const size_t ybytes = (size_t)(m * n) * 4;
  const int64_t kb = (k + 31) / 32;
  if (overlap(y, ybytes, x1, (size_t)(k * m)) ||
      overlap(y, ybytes, x2, wq_pack_int4_bytes(k, n, WQ_LAYOUT_GFX950_B)) ||
      overlap(y, ybytes, x1_scale, (size_t)(m * kb)) || overlap(y, ybytes, x2_scale, (size_t)(kb * n)))
    return WQ_ERR_ALIAS;
  // the workspace is optional: with one of the queried size, shapes whose m
  // is not a multiple of 16 run on the large tile over a padded copy of x1
  const size_t need = wq::mx_x1pad_bytes(m, k, n);
  uint8_t* pad = nullptr;
  if (need > 0 && workspace && workspace_size >= need) {
    if (!aligned16(workspace)) return WQ_ERR_SHAPE;
    if (overlap(workspace, need, y, ybytes) || overlap(workspace, need, x1, (size_t)(k * m)) ||
        overlap(workspace, need, x2, wq_pack_int4_bytes(k, n, WQ_LAYOUT_GFX950_B)) ||
        overlap(workspace, need, x1_scale, (size_t)(m * kb)) ||
        overlap(workspace, need, x2_scale, (size_t)(kb * n)))
      return WQ_ERR_ALIAS;
    pad = static_cast<uint8_t*>(workspace);
  }
  wq::MxProblem p{static_cast<const uint8_t*>(x1), static_cast<const uint8_t*>(x2), x1_scale,
                  x2_scale, y, m, k, n, pad};
  return from_hip(wq::launch_mx_matmul(p, stream));
}

// ---------------------------------------------------------------------------
wq_status wq_quant_matmul_inplace_add(const void* x1, const void* x2, const float* x1_scale,
                                      const float* x2_scale, int64_t m, int64_t k, int64_t n,
                                      float* y, hipStream_t stream) {
  if (m < 0 || n < 0 || m > kMaxRows || n > kMaxKN) return WQ_ERR_SHAPE;
  // k rows of 16-byte chunks; sums of |x| <= 128 products stay inside int32
  if (k < 1 || k > kMaxKN || (k % 16)) return WQ_ERR_SHAPE;
  if (m == 0 || n == 0) return WQ_OK;
  if (!x1 || !x2 || !x1_scale || !x2_scale || !y) return WQ_ERR_NULLPTR;
  if (!aligned16(x1) || !aligned16(x2) || (reinterpret_cast<uintptr_t>(y) & 3) ||
      (reinterpret_cast<uintptr_t>(x1_scale) & 3) || (reinterpret_cast<uintptr_t>(x2_scale) & 3))
    return WQ_ERR_SHAPE;
  const size_t ybytes = (size_t)(m * n) * 4;
  if (overlap(y, ybytes, x1, (size_t)(m * k)) || overlap(y, ybytes, x2, (size_t)(n * k)) ||
      overlap(y, ybytes, x1_scale, (size_t)m * 4) || overlap(y, ybytes, x2_scale, (size_t)n * 4))
    return WQ_ERR_ALIAS;
  if ((m + 255) / 256 * ((n + 255) / 256) > 2147483647LL) return WQ_ERR_SHAPE;
  wq::I8Problem p{static_cast<const int8_t*>(x1), static_cast<const int8_t*>(x2), x1_scale, x2_scale,
                  y, m, k, n};
  return from_hip(wq::launch_i8_matmul(p, stream));
}

wq_status wq_quant_matmul_inplace_add_w4(const void* x1, wq_dtype x1_dtype, const void* x2,
                                         wq_layout x2_layout, const float* x1_scale,
                                         const float* x2_scale, int64_t m, int64_t k, int64_t n,
                                         float* y, hipStream_t stream) {
  if (x1_dtype != WQ_INT8 && x1_dtype != WQ_INT4) return WQ_ERR_DTYPE;
  if (x2_layout != WQ_LAYOUT_GFX950_B) return WQ_ERR_UNSUPPORTED;
  if (m < 0 || n < 0 || m > kMaxRows || n > kMaxKN) return WQ_ERR_SHAPE;
  // x1 rows of 16-byte chunks (INT8: k bytes, INT4: k / 2); the scaled sums
  // (16 or 256 times the sum) stay inside int32 for k < 2^16
  const bool a4 = x1_dtype == WQ_INT4;
  if (k < 1 || k > kMaxKN || (k % (a4 ? 32 : 16))) return WQ_ERR_SHAPE;
  if (m == 0 || n == 0) return WQ_OK;
  if (!x1 || !x2 || !x1_scale || !x2_scale || !y) return WQ_ERR_NULLPTR;
  if (!aligned16(x1) || !aligned16(x2) || (reinterpret_cast<uintptr_t>(y) & 3) ||
      (reinterpret_cast<uintptr_t>(x1_scale) & 3) || (reinterpret_cast<uintptr_t>(x2_scale) & 3))
    return WQ_ERR_SHAPE;
  const size_t wbytes = wq_pack_int4_bytes(k, n, WQ_LAYOUT_GFX950_B);
  if (wbytes >= (size_t(1) << 31)) return WQ_ERR_SHAPE;     // 32-bit buffer offsets
  const size_t ybytes = (size_t)(m * n) * 4;
  if (overlap(y, ybytes, x1, (size_t)(m * (a4 ? k / 2 : k))) || overlap(y, ybytes, x2, wbytes) ||
      overlap(y, ybytes, x1_scale, (size_t)m * 4) || overlap(y, ybytes, x2_scale, (size_t)n * 4))
    return WQ_ERR_ALIAS;
  if ((m + 255) / 256 * ((n + 255) / 256) > 2147483647LL) return WQ_ERR_SHAPE;
  wq::A8W4Problem p{static_cast<const uint8_t*>(x1), static_cast<const uint8_t*>(x2), x1_scale,
                    x2_scale, y, m, k, n, a4};
  return from_hip(wq::launch_a8w4_matmul(p, stream));
}

// ---------------------------------------------------------------------------
size_t mx_fp4_quant_matmul_inplace_add_workspace_size(int64_t m, int64_t k, int64_t n) {
  if (m < 0 || k < 0 || n < 0) return 0;
  return wq::mx4_workspace_bytes(m, k, n);
}

wq_status mx_fp4_quant_matmul_inplace_add(const void* x1, const void* x2, wq_layout x2_layout,
                                          const uint8_t* x1_scale, const uint8_t* x2_scale,
                                          int64_t m, int64_t k, int64_t n, int64_t group_size,
                                          float* y, void* workspace, size_t workspace_size,
                                          hipStream_t stream) {
  if (x2_layout != WQ_LAYOUT_GFX950_B) return WQ_ERR_UNSUPPORTED;
  if (m < 0 || n < 0 || m > kMaxRows || n > kMaxKN) return WQ_ERR_SHAPE;
  // whole 32-slices, so every x1 row is whole 16-byte chunks
  if (k < 1 || k > kMaxKN || (k % 32)) return WQ_ERR_SHAPE;
  // groupSize as for the mx mode: only (K, N, M) = (32, 1, 1), zero fields inferred
  if (group_size < 0 || (group_size >> 48) != 0) return WQ_ERR_GROUP;
  const int64_t gk = group_size & 0xFFFF, gn = (group_size >> 16) & 0xFFFF,
                gm = (group_size >> 32) & 0xFFFF;
  if ((gk != 0 && gk != 32) || (gn != 0 && gn != 1) || (gm != 0 && gm != 1)) return WQ_ERR_GROUP;
  if (m == 0 || n == 0) return WQ_OK;
  if (!x1 || !x2 || !x1_scale || !x2_scale || !y) return WQ_ERR_NULLPTR;
  const size_t need = wq::mx4_workspace_bytes(m, k, n);
  if (!workspace || workspace_size < need) return WQ_ERR_WORKSPACE;
  if (!aligned16(x1) || !aligned16(x2) || !aligned16(y) || !aligned16(workspace)) return WQ_ERR_SHAPE;
  // the weight and its per-step offsets stay below the 2 GiB buffer bound
  const size_t wbytes = wq_pack_int4_bytes(k, n, WQ_LAYOUT_GFX950_B);
  if (wbytes >= ((size_t)1 << 31)) return WQ_ERR_SHAPE;
  if ((m + 255) / 256 * ((n + 255) / 256) > 2147483647LL) return WQ_ERR_SHAPE;
  const size_t ybytes = (size_t)(m * n) * 4, x1bytes = (size_t)(m * (k / 2));
  const int64_t kb = k / 32;
  if (overlap(y, ybytes, x1, x1bytes) || overlap(y, ybytes, x2, wbytes) ||
      overlap(y, ybytes, x1_scale, (size_t)(m * kb)) || overlap(y, ybytes, x2_scale, (size_t)(kb * n)) ||
      overlap(y, ybytes, workspace, need) || overlap(workspace, need, x1, x1bytes) ||
      overlap(workspace, need, x2, wbytes) || overlap(workspace, need, x1_scale, (size_t)(m * kb)) ||
      overlap(workspace, need, x2_scale, (size_t)(kb * n)))
    return WQ_ERR_ALIAS;
  wq::Mx4Problem p{static_cast<const uint8_t*>(x1), static_cast<const uint8_t*>(x2), x1_scale, x2_scale,
                   y, m, k, n, workspace};
  return from_hip(wq::launch_mx4_matmul(p, stream));
}

}  // extern "C"
