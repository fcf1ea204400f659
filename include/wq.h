/*
 * wq.h - C ABI of libwq: weight-quantized matmul + AddRmsNorm and its
 * companions, written for AMD Instinct MI355X (gfx950).
 *
 * The operators, each following one operator page:
 *   wq_pack_int4                  aclnnConvertWeightToINT4Pack
 *   wq_dynamic_quant              aclnnDynamicQuant (plus an MX block-32 mode)
 *   wq_matmul_add_rmsnorm         aclnnWeightQuantMatmulAllReduceAddRmsNorm
 *                                 (single device: the AllReduce is the identity)
 *   mx_quant_matmul_inplace_add   aclnnQuantBatchMatmulInplaceAdd (mx)
 *   mx_fp4_quant_matmul_inplace_add  the same, both operands MXFP4
 *   wq_quant_matmul_inplace_add      the same Formula, INT8 x INT8 (A8W8)
 *   wq_quant_matmul_inplace_add_w4   the same Formula, INT8 / INT4 x packed INT4
 *   wq_pack_fp4                   aclnnConvertWeightToINT4Pack (FLOAT -> E2M1)
 *   wq_weight_quant_matmul        \ the unfused chain that the fused operator's
 *   wq_add_rms_norm               / page names as its replacement
 *
 * Conventions shared by every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller, row-major
 *     ("ND") unless stated otherwise. Sizes are element counts.
 *   - The library never allocates, frees or synchronizes. Work is enqueued on
 *     `stream` (0 = the null stream) and the call returns at once; errors
 *     raised by the kernels themselves surface at the caller's next sync.
 *   - Arguments are validated on the host before anything is launched. On an
 *     error the call returns a non-zero wq_status, launches nothing and
 *     writes nothing.
 *   - Two-phase pattern of the pages (GetWorkspaceSize, then execute) becomes
 *     `*_workspace_size()` (pure host arithmetic) plus the execute call.
 *   - Results are deterministic: every reduction has a fixed order.
 *   - Calls that share a workspace must be ordered (same stream).
 */
#ifndef WQ_H_
#define WQ_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wq_status {
  WQ_OK = 0,
  WQ_ERR_NULLPTR = 1,      /* a required pointer is null */
  WQ_ERR_SHAPE = 2,        /* a size is out of range or shapes disagree */
  WQ_ERR_DTYPE = 3,        /* unsupported dtype or dtype combination */
  WQ_ERR_GROUP = 4,        /* group size / scale shape rule broken */
  WQ_ERR_WORKSPACE = 5,    /* workspace missing or too small */
  WQ_ERR_UNSUPPORTED = 6,  /* valid on the pages but not offered here */
  WQ_ERR_LAUNCH = 7,       /* the HIP runtime refused a launch */
  WQ_ERR_ALIAS = 8         /* an output overlaps an input it may not alias */
} wq_status;

typedef enum wq_dtype {
  WQ_F16 = 1,
  WQ_BF16 = 2,
  WQ_F32 = 3,
  WQ_INT8 = 4,
  WQ_INT4 = 5,             /* two per byte, even index in the low nibble */
  WQ_INT32 = 6,            /* as a quant output: eight INT4 per word, lowest nibble first */
  WQ_FP8_E4M3 = 7,         /* OCP E4M3 (FN): bias 7, max 448, NaN = S.1111.111 */
  WQ_FP4_E2M1 = 8,         /* OCP E2M1, two per byte like WQ_INT4 */
  WQ_E8M0 = 9              /* one byte, value 2^(c-127) */
} wq_dtype;

typedef enum wq_layout {
  /* (K, N) 4-bit codes packed along N: byte [k][n/2], even n in the low
   * nibble. N must be even. */
  WQ_LAYOUT_ND = 0,
  /* gfx950 MFMA-operand order for a logical (K, N) matrix of 4-bit codes.
   * Kp = 128*ceil(K/128), Np = 16*ceil(N/16), Kp*Np/2 bytes; the padding
   * holds code 0. Code (k, n) sits in
   *     byte   ((k/128)*Np + n)*64 + ((k/32)%4)*16 + (k%32)/2
   *     nibble k%2  (0 = bits 0..3)
   * so the 32 codes of one column in one 32-deep K block are 16 contiguous
   * bytes (one dwordx4 per lane) and the 16 columns x 128 K read by one
   * wavefront are 1 KiB contiguous. */
  WQ_LAYOUT_GFX950_B = 1
} wq_layout;

/* Text of a status code (static storage). */
const char* wq_status_string(wq_status status);

/* Incremented when an entry point changes its arguments. */
int wq_abi_version(void);

/* ------------------------------------------------------------------------
 * INT4 weight pack. aclnnConvertWeightToINT4Pack page, operator description:
 * INT32 weights holding one 4-bit value each become tightly packed nibbles
 * (the pages' FRACTAL_NZ output is replaced by WQ_LAYOUT_GFX950_B).
 *
 * weight     device int32, logical (k, n); stored (k, n) row-major, or
 *            (n, k) row-major when transpose != 0.
 * out        device, wq_pack_int4_bytes(k, n, layout) bytes.
 * Stores v & 0xF for each value v (two's complement of an int4 in [-8, 7],
 * or an FP4 E2M1 code 0..15). Values outside [-8, 15] are outside the
 * contract: their low nibble is stored.
 * Errors: WQ_ERR_NULLPTR; WQ_ERR_SHAPE if k < 0, n < 0, layout ND with n
 * odd, or layout GFX950_B with n >= 2^22 (k >= 2^21 when transposed);
 * WQ_ERR_UNSUPPORTED for an unknown layout. k == 0 or n == 0 is a no-op.
 * ---------------------------------------------------------------------- */
size_t wq_pack_int4_bytes(int64_t k, int64_t n, wq_layout layout);
wq_status wq_pack_int4(const int32_t* weight, int64_t k, int64_t n,
                       int transpose, wq_layout layout, void* out,
                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * FLOAT -> FLOAT4_E2M1 pack. aclnnConvertWeightToINT4Pack page, operator
 * description: on the newer chips the pack also turns FLOAT weights into
 * tightly packed FLOAT4_E2M1 data.
 *
 * weight     device float32, logical (k, n); stored as for wq_pack_int4.
 * out        device, wq_pack_int4_bytes(k, n, layout) bytes: the E2M1 codes
 *            in the INT4 code layout (WQ_LAYOUT_GFX950_B is the MX GEMMs' x2).
 * Each value goes to its nearest E2M1 value, ties to even; magnitudes beyond
 * 6 saturate to +-6; the sign of zero is kept (-0.0 -> code 8). NaN is
 * outside the contract. Limits and errors as wq_pack_int4.
 * ---------------------------------------------------------------------- */
wq_status wq_pack_fp4(const float* weight, int64_t k, int64_t n, int transpose,
                      wq_layout layout, void* out, hipStream_t stream);


/* ------------------------------------------------------------------------
 * Dynamic quantization. aclnnDynamicQuant page, Formula: with optional
 * smooth scales, input = x * smooth; scale = row_max(|input|) / dtypeMax;
 * y = round(input / scale). Constraints section: an INT4 output needs an even
 * last dimension and an INT32 output one divisible by 8.
 *
 * x          device (rows, cols), x_dtype WQ_F16 or WQ_BF16 (leading
 *            dimensions flattened into rows).
 * smooth     device (cols) of x_dtype, or NULL.
 * block_k == 0  per-token mode. y_dtype WQ_INT8 (y int8 (rows, cols)),
 *            WQ_INT4 (y uint8 (rows, cols/2)) or WQ_INT32 (y int32
 *            (rows, cols/8)); dtypeMax 127 for INT8 and 7 otherwise.
 *            scale: device float32 (rows). The scale is the correctly rounded
 *            float32 quotient row_max / dtypeMax, the code the float32
 *            quotient input / scale rounded half to even, clamped to
 *            [-dtypeMax, dtypeMax]; an all-zero row gives scale 0, codes 0.
 * block_k == 32 MX mode (the 32-long K blocks of the
 *            aclnnQuantBatchMatmulInplaceAdd page). y_dtype WQ_FP8_E4M3
 *            (one byte per element) or WQ_FP4_E2M1 (two per byte).
 *            scale: device uint8 E8M0 codes (rows, ceil(cols/32)), code
 *            e + 127 with e the smallest integer such that
 *            dtypeMax * 2^e >= block max (dtypeMax 448 / 6), clamped to
 *            [-127, 127]; an all-zero block gets 127. Codes are
 *            input * 2^-e rounded to nearest even, keeping the sign of zero.
 *            transpose_y != 0 (WQ_FP8_E4M3 only) stores y as (cols, rows):
 *            the transposeX1 layout of the MX matmul.
 * Products x * smooth must be exact in float32 (always true for fp16).
 * Errors: WQ_ERR_NULLPTR; WQ_ERR_SHAPE (negative sizes, odd cols for INT4 or
 * FP4, cols % 8 for INT32, cols >= 2^30 per token, more than 65535 column
 * tiles of 64 for MX); WQ_ERR_DTYPE; WQ_ERR_UNSUPPORTED (other block_k,
 * transpose with a non-FP8 output). rows == 0 or cols == 0 is a no-op.
 * ---------------------------------------------------------------------- */
wq_status wq_dynamic_quant(const void* x, wq_dtype x_dtype, int64_t rows,
                           int64_t cols, const void* smooth, wq_dtype y_dtype,
                           int64_t block_k, int transpose_y, void* y,
                           void* scale, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Weight-quantized matmul + residual add + RMSNorm.
 * aclnnWeightQuantMatmulAllReduceAddRmsNorm page, Formula:
 *     mm      = x1 @ (x2 * antiquantScale + antiquantOffset) + bias
 *     y       = mm + residual
 *     normOut = y / RMS(y) * gamma,  RMS(y) = sqrt(mean_n(y^2) + epsilon)
 * (the page's AllReduce is the identity on one device). Constraints section:
 * x1 (b, s, k) or (s, k), m = b*s in [0, 2^31-1]; x2 (k, n) with k in
 * [1, 65535], n in [0, 65535]; bias (n); residual (b, s, n); gamma (n);
 * per-tensor scale (1), per-channel (1, n) or (n), per-group (ceil(k/G), n)
 * with G in [32, k-1] a multiple of 32; the offset has the scale's shape;
 * m == 0 or n == 0 is an empty no-op, k == 0 an error; the inplace variant
 * writes y into residual's memory.
 *
 * x1          device (m, k) of act_dtype (WQ_F16 or WQ_BF16), row-major.
 * x2          device weight. w_dtype WQ_INT4: packed by wq_pack_int4 in
 *             x2_layout. ND: (k, n/2) bytes (n even), or, when transpose_x2
 *             != 0, the transpose stored (n, k/2) bytes (k even), even k in
 *             the low nibble (the Constraints section lets x2 be
 *             transposed). GFX950_B: transpose_x2 must be 0 (the pack takes
 *             the transpose and writes the same layout). w_dtype WQ_INT8:
 *             layout ND, (k, n) row-major, or (n, k) row-major when
 *             transpose_x2 != 0.
 * antiquant_scale   device act_dtype, (scale_rows, scale_cols):
 *             (1, 1) per tensor, (1, n) per channel, (ceil(k/G), n) per group.
 * antiquant_offset  device, same shape and dtype, or NULL (zero).
 * antiquant_group_size  G for per-group scales, else 0.
 * bias        device (n) act_dtype, or NULL (zero).
 * residual    device (m, n) act_dtype.
 * gamma       device (n) act_dtype.
 * y           device (m, n) act_dtype; may equal residual (inplace).
 * norm_out    device (m, n) act_dtype; may not overlap any other argument.
 * workspace   device, >= wq_matmul_add_rmsnorm_workspace_size(m, k, n)
 *             bytes, no initial contents needed.
 * Numerics: the integer codes enter the MFMA exactly (as act_dtype values)
 * and each group's scale and offset are applied to that group's float32
 * partial sums: mm = sum_g (s_g * sum_{k in g} x1*q + o_g * sum_{k in g} x1),
 * which equals the Formula's x1 @ (q*s + o) without rounding the dequantized
 * weight. Accumulation is float32; y is rounded to act_dtype once; RMS uses
 * the float32 y; normOut = y * rstd * gamma rounded once.
 * Errors: WQ_ERR_NULLPTR, WQ_ERR_SHAPE, WQ_ERR_DTYPE, WQ_ERR_GROUP,
 * WQ_ERR_WORKSPACE, WQ_ERR_UNSUPPORTED, WQ_ERR_ALIAS (norm_out overlapping).
 * ---------------------------------------------------------------------- */
size_t wq_matmul_add_rmsnorm_workspace_size(int64_t m, int64_t k, int64_t n);
wq_status wq_matmul_add_rmsnorm(
    const void* x1, int64_t m, int64_t k, wq_dtype act_dtype,
    const void* x2, int64_t n, wq_dtype w_dtype, wq_layout x2_layout,
    int transpose_x2,
    const void* antiquant_scale, int64_t scale_rows, int64_t scale_cols,
    const void* antiquant_offset, int64_t antiquant_group_size,
    const void* bias, const void* residual, const void* gamma,
    double epsilon, void* y, void* norm_out,
    void* workspace, size_t workspace_size, hipStream_t stream);

/* ------------------------------------------------------------------------
 * The same operator for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops and harnesses that forbid
 * allocation. Arguments and results are those of wq_matmul_add_rmsnorm
 * without the workspace: the kernels use a library-owned device array of
 * WQ_NOALLOC_MAX_WORKSPACE bytes instead (one per GPU, held until the process
 * ends; its address is looked up once per device, with the calling thread's
 * current device). The call allocates and frees nothing.
 * A problem whose wq_matmul_add_rmsnorm_workspace_size(m, k, n) exceeds
 * WQ_NOALLOC_MAX_WORKSPACE returns WQ_ERR_WORKSPACE before any other check;
 * so does any non-empty problem when the array cannot be located. Every
 * other rule and error is wq_matmul_add_rmsnorm's.
 * Every call on one GPU shares that GPU's array (the kernels need no initial
 * contents): calls that can overlap on one GPU (different streams without
 * ordering) race on it and must not be issued.
 * ---------------------------------------------------------------------- */
#define WQ_NOALLOC_MAX_WORKSPACE ((size_t)32 << 20)
wq_status wq_matmul_add_rmsnorm_noalloc(
    const void* x1, int64_t m, int64_t k, wq_dtype act_dtype,
    const void* x2, int64_t n, wq_dtype w_dtype, wq_layout x2_layout,
    int transpose_x2,
    const void* antiquant_scale, int64_t scale_rows, int64_t scale_cols,
    const void* antiquant_offset, int64_t antiquant_group_size,
    const void* bias, const void* residual, const void* gamma,
    double epsilon, void* y, void* norm_out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * MXFP4 x MXFP4 quantized matmul with in-place add.
 * aclnnQuantBatchMatmulInplaceAdd page, Formula (mx quantization), read with
 * both operands FLOAT4_E2M1:
 *     y[m,n] += sum_j (sum_{k in slice j} x1[m,k] * x2[k,n])
 *                     * scale1[m,j] * scale2[j,n]
 * with 32-long K slices, j < k/32. The scaled MFMA runs at the FP4 rate.
 *
 * x1          device E2M1 codes (m, k) row-major, two per byte along k, even
 *             k in the low nibble (wq_dynamic_quant's block-32 E2M1 output;
 *             transposeX1 = false).
 * x2          device E2M1 codes, logical (k, n), in WQ_LAYOUT_GFX950_B
 *             (wq_pack_fp4 or wq_pack_int4 of the codes); ND is
 *             WQ_ERR_UNSUPPORTED.
 * x1_scale    device E8M0 (m, k/32) = scale1[m][j].
 * x2_scale    device E8M0 (k/32, n) = scale2[j][n].
 * m in [0, 2^31 - 1], n in [0, 65535] (0: nothing to do); k in [32, 65535]
 * and a multiple of 32 (else WQ_ERR_SHAPE).
 * group_size  0 or 32 | 1 << 16 | 1 << 32, as for mx_quant_matmul_inplace_add.
 * y           device float32 (m, n), read and written.
 * workspace   device, >= mx_fp4_quant_matmul_inplace_add_workspace_size(m, k,
 *             n) bytes (the scales rearranged for the matrix cores), no
 *             initial contents needed.
 * x1, x2, y and the workspace 16-byte aligned. Accumulation is float32 and
 * starts from y; every slice sum is exact.
 * Errors: WQ_ERR_NULLPTR, WQ_ERR_SHAPE, WQ_ERR_GROUP, WQ_ERR_WORKSPACE,
 * WQ_ERR_UNSUPPORTED, WQ_ERR_ALIAS (y or the workspace overlapping an input).
 * ---------------------------------------------------------------------- */
size_t mx_fp4_quant_matmul_inplace_add_workspace_size(int64_t m, int64_t k, int64_t n);
wq_status mx_fp4_quant_matmul_inplace_add(const void* x1, const void* x2, wq_layout x2_layout,
                                          const uint8_t* x1_scale, const uint8_t* x2_scale,
                                          int64_t m, int64_t k, int64_t n, int64_t group_size,
                                          float* y, void* workspace, size_t workspace_size,
                                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * Weight-quantized matmul alone (the first half of the unfused chain).
 * aclnnWeightQuantMatmulAllReduceAddRmsNorm page: the deprecation note names
 * a weight-quantized matmul (with AllReduce) followed by AddRmsNorm as the
 * replacement; this is the Formula's first line on one device:
 *     out = x1 @ (x2 * antiquantScale + antiquantOffset) + bias
 * Every argument but the outputs means what it means for
 * wq_matmul_add_rmsnorm (dtypes, layouts, scale shapes and group rules,
 * limits, alignment); residual, gamma, epsilon and norm_out are absent.
 *
 * out         device (m, n) act_dtype, rounded once from the float32 sum; may
 *             not overlap x1, x2, the scales, bias or the workspace.
 * workspace   device, >= wq_weight_quant_matmul_workspace_size(m, k, n)
 *             bytes, no initial contents needed.
 * Errors: as wq_matmul_add_rmsnorm (WQ_ERR_ALIAS for an overlapping out).
 * ---------------------------------------------------------------------- */
size_t wq_weight_quant_matmul_workspace_size(int64_t m, int64_t k, int64_t n);
wq_status wq_weight_quant_matmul(
    const void* x1, int64_t m, int64_t k, wq_dtype act_dtype,
    const void* x2, int64_t n, wq_dtype w_dtype, wq_layout x2_layout,
    int transpose_x2,
    const void* antiquant_scale, int64_t scale_rows, int64_t scale_cols,
    const void* antiquant_offset, int64_t antiquant_group_size,
    const void* bias, void* out,
    void* workspace, size_t workspace_size, hipStream_t stream);

/* ------------------------------------------------------------------------
 * AddRmsNorm (the second half of the unfused chain).
 * aclnnWeightQuantMatmulAllReduceAddRmsNorm page, Formula, last two lines:
 *     y = x + residual
 *     normOut = y / RMS(y) * gamma,  RMS(y) = sqrt(mean over the row of y^2 + epsilon)
 *
 * x, residual device (rows, cols) dtype (WQ_F16 or WQ_BF16); rows in
 *             [0, 2^31 - 1] (0: nothing to do), cols in [1, 65535].
 * gamma       device (cols) dtype.
 * epsilon     finite, >= 0.
 * y           device (rows, cols) dtype; may equal x or residual (in place)
 *             but not overlap them otherwise.
 * norm_out    device (rows, cols) dtype; may not overlap any other argument.
 * Every pointer 16-byte aligned. The sum of squares uses the float32 y (one
 * float32 addition of the two inputs); y is rounded to dtype once and
 * normOut = y_rounded * rstd * gamma is rounded once, as in the fused
 * operator.
 * Errors: WQ_ERR_NULLPTR, WQ_ERR_SHAPE, WQ_ERR_DTYPE, WQ_ERR_ALIAS.
 * ---------------------------------------------------------------------- */
wq_status wq_add_rms_norm(const void* x, const void* residual, const void* gamma,
                          int64_t rows, int64_t cols, wq_dtype dtype, double epsilon,
                          void* y, void* norm_out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * MX block-32 quantized matmul with in-place add.
 * aclnnQuantBatchMatmulInplaceAdd page, Formula (mx quantization):
 *     y[m,n] += sum_j (sum_{k in slice j} x1[m,k] * x2[k,n])
 *                     * scale1[m,j] * scale2[j,n]
 * with 32-long K slices, j < ceil(K/32), the last slice possibly shorter.
 * Constraints section: only transposeX1 = true and transposeX2 = false;
 * groupSize = groupSizeK | groupSizeN << 16 | groupSizeM << 32, a zero field
 * inferred from the shapes.
 *
 * x1          device E4M3 codes stored (k, m) (transposeX1).
 * x2          device E2M1 codes, logical (k, n), packed by wq_pack_int4 in
 *             WQ_LAYOUT_GFX950_B (ND is rejected: WQ_ERR_UNSUPPORTED).
 * x1_scale    device E8M0 (m, ceil(k/32)) = scale1[m][j].
 * x2_scale    device E8M0 (ceil(k/32), n) = scale2[j][n].
 * transpose_x1 must be 1, transpose_x2 must be 0 (else WQ_ERR_UNSUPPORTED).
 * group_size  0 or 32 | 1 << 16 | 1 << 32 (= 4295032864); zero fields are
 *             inferred (M and N by exact division, K as 32 when ceil(k/32)
 *             slices match); anything else is WQ_ERR_GROUP.
 * y           device float32 (m, n), read and written.
 * workspace   optional, device, 16-byte aligned, owned by the caller, no
 *             initial contents needed, overlapping no argument. The query
 *             returns nonzero only when m is not a multiple of 16 (x1's
 *             rows are then not 16-byte aligned): with a workspace of that
 *             size the call copies x1 into it with padded rows and runs the
 *             large tile; with NULL (or a smaller one) it runs the small
 *             tile, correct but much slower.
 * Pointers: x1, x2, y and the workspace 16-byte aligned, the scales 4-byte
 * aligned (else WQ_ERR_SHAPE); y and a used workspace may not overlap an
 * input or each other (WQ_ERR_ALIAS).
 * Accumulation is float32 inside the scaled MFMA: products are added in
 * groups of 8 K values aligned to the group's largest exponent sum and
 * truncated 13 bits below it, group sums and y aligned to 2^-24 of the
 * largest, the result rounded to float32; the order is fixed. Empty m or n
 * is a no-op; k == 0 leaves y unchanged.
 * ---------------------------------------------------------------------- */
size_t mx_quant_matmul_inplace_add_workspace_size(int64_t m, int64_t k, int64_t n);
wq_status mx_quant_matmul_inplace_add(
    const void* x1, const void* x2, wq_layout x2_layout,
    const uint8_t* x1_scale, const uint8_t* x2_scale,
    int64_t m, int64_t k, int64_t n, int transpose_x1, int transpose_x2,
    int64_t group_size, float* y, void* workspace, size_t workspace_size,
    hipStream_t stream);

/* ------------------------------------------------------------------------
 * INT8 quantized matmul with in-place add (aclnnQuantBatchMatmulInplaceAdd
 * page, Formula, read for INT8 operands with one K group, i.e. groupSizeK =
 * K, a per-token scale for x1 and a per-channel scale for x2):
 *
 *   y[m,n] = (sum_k x1[m,k] * x2[n,k]) * (x1_scale[m] * x2_scale[n]) + y[m,n]
 *
 * x1: int8 (m, k) row-major (the per-token output of wq_dynamic_quant with
 *     y_dtype INT8); x1_scale: float32 (m) (its scale output).
 * x2: int8 stored (n, k) row-major (transposed: each output column's k
 *     values contiguous); x2_scale: float32 (n).
 * y:  float32 (m, n) row-major, read and written in place.
 * The sum over k is exact (int32); then, in float32 with round-to-nearest-
 * even at each step: s = x1_scale[m] * x2_scale[n], t = float(sum) * s,
 * y = y + t. All pointers are device memory owned by the caller; x1 and x2
 * 16-byte aligned, the scales and y 4-byte aligned; y must not overlap an
 * input. No workspace. m == 0 or n == 0 is an empty no-op.
 * Errors: WQ_ERR_NULLPTR; WQ_ERR_SHAPE (m < 0, n outside [0, 65535], k
 * outside [1, 65535] or not a multiple of 16, misaligned pointers);
 * WQ_ERR_ALIAS (y overlapping an input).
 * ---------------------------------------------------------------------- */
wq_status wq_quant_matmul_inplace_add(const void* x1, const void* x2, const float* x1_scale,
                                      const float* x2_scale, int64_t m, int64_t k, int64_t n,
                                      float* y, hipStream_t stream);

/* ------------------------------------------------------------------------
 * INT8 / INT4 x INT4 quantized matmul with in-place add (A8W4, A4W4): the
 * same Formula and roundings as wq_quant_matmul_inplace_add, with x2 given
 * as INT4 codes packed by wq_pack_int4 (aclnnConvertWeightToINT4Pack page)
 * and x1 as either output of wq_dynamic_quant's per-token mode
 * (aclnnDynamicQuant page: INT8, or INT4 codes two per byte):
 *
 *   y[m,n] = (sum_k x1[m,k] * q[k,n]) * (x1_scale[m] * x2_scale[n]) + y[m,n]
 *
 * x1: x1_dtype WQ_INT8: int8 (m, k) row-major; WQ_INT4: codes in [-8, 7]
 *     stored (m, k/2) bytes, even k in the low nibble. Other dtypes:
 *     WQ_ERR_DTYPE. x1_scale: float32 (m).
 * x2: the codes q in [-8, 7], logical (k, n), in WQ_LAYOUT_GFX950_B
 *     (wq_pack_int4_bytes(k, n, layout) bytes, under 2^31); ND is
 *     WQ_ERR_UNSUPPORTED. x2_scale: float32 (n).
 * y:  float32 (m, n) row-major, read and written in place.
 * The sum over k is exact (int32); then s = x1_scale[m] * x2_scale[n],
 * t = float(sum) * s, y = y + t, each rounded to nearest even in float32.
 * Device pointers owned by the caller; x1 and x2 16-byte aligned, the scales
 * and y 4-byte aligned; y must not overlap an input. No workspace. m == 0 or
 * n == 0 is an empty no-op.
 * Errors: WQ_ERR_NULLPTR; WQ_ERR_DTYPE; WQ_ERR_SHAPE (m < 0, n outside
 * [0, 65535], k outside [1, 65535] or not a multiple of 16 (32 for an INT4
 * x1), misaligned pointers, a weight of 2^31 bytes or more);
 * WQ_ERR_UNSUPPORTED (x2_layout not GFX950_B); WQ_ERR_ALIAS (y overlapping
 * an input).
 * ---------------------------------------------------------------------- */
wq_status wq_quant_matmul_inplace_add_w4(const void* x1, wq_dtype x1_dtype,
                                         const void* x2, wq_layout x2_layout,
                                         const float* x1_scale, const float* x2_scale,
                                         int64_t m, int64_t k, int64_t n, float* y,
                                         hipStream_t stream);

/* ------------------------------------------------------------------------
 * Profiling of the contraction kernels (a measurement aid, not part of any
 * operator): while enabled, each wq_matmul_add_rmsnorm and
 * mx_quant_matmul_inplace_add call records a pair of HIP events on its
 * stream around its contraction kernel (the MFMA tile, the decode weight
 * stream or the generic tile; not the pre-passes or the RMSNorm finish).
 *
 * wq_profile_enable(1) creates the events on first use and clears the
 * record; (0) stops recording. wq_profile_read waits for the recorded
 * events, stores *launches = the number of timed launches since the last
 * enable / read (at most 4096; later ones are not timed), writes the first
 * min(capacity, *launches) kernel times in milliseconds, in launch order, to
 * times_ms (host memory, caller-owned; may be null when capacity is 0), and
 * clears the record. The record is process-wide; calls on several threads
 * interleave in it.
 * Errors: WQ_ERR_NULLPTR; WQ_ERR_LAUNCH if the runtime refuses an event.
 * ---------------------------------------------------------------------- */
wq_status wq_profile_enable(int enable);
wq_status wq_profile_read(float* times_ms, int64_t capacity, int64_t* launches);

/* ------------------------------------------------------------------------
 * Achievable ceilings (measurement aids, not operators of any page): two
 * microkernels that the measurement times next to the published MI355X
 * peaks, so that a kernel's fraction of peak can be read against what this
 * GPU reaches on the same resource with nothing else in the way.
 *
 * wq_ceiling_stream_read loads each 16-byte chunk of `bytes` bytes at src
 * once (one 16-byte load per lane, four per thread issued before any use)
 * and writes, per wave, the XOR of the 32-bit words it read:
 * wq_ceiling_stream_read_words(bytes) words to out. The XOR of all of them
 * is the XOR of every word of the input. src: device memory, 16-byte
 * aligned, bytes a positive multiple of 16 below 2^40 (otherwise
 * wq_ceiling_stream_read_words returns 0); out: device memory,
 * caller-owned, 4-byte aligned.
 *
 * wq_ceiling_mfma_loop runs `workgroups` workgroups of four waves; each
 * wave issues `iters` rounds of eight independent v_mfma_f32_16x16x32_bf16
 * on register operands, i.e. 2 * 16 * 16 * 32 * 8 * 4 * iters * workgroups
 * flops in all. The operands are random bf16 values of magnitude in
 * [0.5, 2), four A and four B fragments per lane (accumulator j multiplies
 * A set j % 4 by B set j / 2), fixed functions of the lane index; each lane
 * writes the sum of its accumulators to out[workgroups * 256] (device
 * memory, caller-owned, floats), the same for every workgroup.
 *
 * Errors: WQ_ERR_NULLPTR; WQ_ERR_SHAPE (sizes or alignment as above;
 * workgroups outside [1, 2^20], iters outside [1, 16384]); WQ_ERR_ALIAS
 * (the stream read's out overlapping src); WQ_ERR_LAUNCH.
 * ---------------------------------------------------------------------- */
size_t wq_ceiling_stream_read_words(size_t bytes);
wq_status wq_ceiling_stream_read(const void* src, size_t bytes, uint32_t* out, hipStream_t stream);
wq_status wq_ceiling_mfma_loop(int64_t workgroups, int32_t iters, float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H_ */
