/*
 * qaff -- grouped affine dequantization and quantized matmul for AMD Instinct MI355X (gfx950).
 *
 * Storage format (MLX layout):
 *   packed  uint32 [rows, cols*bits/32]. Each row is one little-endian bit stream: code j occupies
 *           stream bits [j*bits, (j+1)*bits), least significant bit first; stream bit p is bit
 *           p%32 of word p/32, so 3-, 5- and 6-bit codes may straddle two words.
 *           (nuvec_core quantized.rs, module documentation; rlx-moshi mlx_dequant.rs, doc comment of
 *           dequantize_affine. For 8 bits this is spark_runtime weights/mlx_int8.rs, module
 *           documentation: byte c%4 of word c/4 is column c, low byte first.)
 *   scales  bf16 bit patterns (uint16) [rows, cols/group_size]
 *   biases  bf16 bit patterns (uint16) [rows, cols/group_size]
 *   A weight is w[r,c] = scale[r,c/G] * code[r,c] + bias[r,c/G], computed in float32 (the product
 *   first, then the bias) -- rlx-moshi dequantize_affine; spark_runtime module formula.
 *
 * Common rules for every entry point below:
 *   - All array pointers are DEVICE pointers to row-major, contiguous buffers. The caller owns every
 *     buffer; the library never allocates, frees or retains them (spark_runtime MlxInt8Weight: the
 *     consumer owns the device pointers).
 *   - bits must be 1, 2, 3, 4, 5, 6 or 8 (else QAFF_ERR_UNSUPPORTED); group_size 32, 64 or 128
 *     (nuvec_core check_params); cols (k) must be a multiple of group_size.
 *   - A weight has at most 2^32 - 1 rows, and a row's code stream, cols * bits bits, stays below
 *     2^32 bits (the kernels address within a row in 32 bits); larger is QAFF_ERR_UNSUPPORTED.
 *   - Alignment: packed 4 bytes, scales/biases their element size (2 bytes; 4 for float32), indices
 *     4 bytes; x, y, out, w, gate, up and resid their element size (4 bytes for float32, 2 for bf16
 *     and float16). 16-byte aligned x, y and out take the vector kernels; others (a row slice, an
 *     odd offset into a buffer) are loaded and stored element by element: dequantize, dequant_rows
 *     and quantize give the same bits, the products the same float32 arithmetic in another
 *     summation order (within the same bounds). The MFMA paths, when forced (QAFF_PATH_GEMM,
 *     QAFF_PATH_GEMV_MFMA), need 16-byte aligned x and y and are UNSUPPORTED otherwise.
 *   - Every argument is checked on the host before any launch, so a rejected call writes nothing.
 *   - Calls are asynchronous on `stream` (NULL = the null stream): they return once the kernel is
 *     enqueued and never synchronize (unless the environment sets QAFF_DEBUG_SYNC=1).
 *   - A size of zero in any output dimension is a successful no-op.
 *   - On failure the call returns a non-zero status and qaff_last_error() describes it. A launch
 *     failure maps to QAFF_ERR_DEVICE; a fault inside a kernel surfaces asynchronously, on a later
 *     synchronization of the stream.
 *   - Calls are re-entrant; the only global state is the calling thread's error text.
 */
#ifndef QAFF_H
#define QAFF_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QAFF_ABI_VERSION 1

typedef enum {
    QAFF_OK = 0,
    QAFF_ERR_INVALID_ARGUMENT = 1,
    QAFF_ERR_UNSUPPORTED = 2,
    QAFF_ERR_DEVICE = 3
} qaff_status;

typedef enum { QAFF_F32 = 0, QAFF_BF16 = 1, QAFF_F16 = 2 } qaff_dtype;

/* Kernel choice for qaff_qmm_ex. AUTO: float32 x -> the VALU kernel at any m; bf16 x with
 * m <= qaff_gemv_max_m() -> the decode path: the VALU GEMV for m below qaff_gemv_mfma_min_m()
 * (below 2 where K exceeds 4096), the matrix-core decode kernel (GEMV_MFMA) from there on where it
 * applies (K a multiple of 512 and at most 32768, 4-byte aligned scales and biases), the VALU GEMV
 * otherwise; bf16 x with a larger m -> the bf16-MFMA GEMM, except that up to 128 rows with no K
 * split (no workspace, or one qaff_qmm_ws does not use) run as 16-row slices, each as the decode
 * path would run it alone, where the matrix-core decode kernel takes K and 4-byte aligned scales
 * (up to 48 rows at any n, 96 where n <= 8192, 128 where n <= 4096: a GEMM with that few tiles
 * leaves most of the chip idle). GEMV_MFMA forced on a shape it does not take is UNSUPPORTED. */
typedef enum { QAFF_PATH_AUTO = 0, QAFF_PATH_GEMV = 1, QAFF_PATH_GEMM = 2, QAFF_PATH_GEMV_MFMA = 3 } qaff_path;

/*
 * Dense dequantization (rlx-moshi dequantize_affine; spark_runtime dequantize_to; maya2_mlx QW.dense).
 *   out [rows, cols] in out_dtype: float32 holds w exactly as defined above; bf16 holds w rounded
 *   to nearest, ties to even.
 * Errors: INVALID_ARGUMENT for negative sizes, a bad group size, cols % group_size != 0, a bad
 * dtype, a null or misaligned pointer where the size is non-zero; UNSUPPORTED for a bit width
 * outside {1,2,3,4,5,6,8}.
 */
qaff_status qaff_dequantize(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                            int64_t rows, int64_t cols, int32_t group_size, int32_t bits,
                            void* out, qaff_dtype out_dtype, hipStream_t stream);

/*
 * Other float types (nuvec_core quantized.rs: quantized_matmul and dequantize promote x, scales and
 * biases to one float type; scales keep the weight's dtype). QAFF_F16 is accepted only by the
 * *_typed entry points and as qaff_quantize's w; every other entry point takes float32 or bf16 x
 * and bf16 scales.
 *
 * qaff_promote_dtype: the common type of two dtypes, as y's dtype: equal types stay, anything
 * else (float32 with anything, bf16 with float16) is float32.
 */
qaff_dtype qaff_promote_dtype(qaff_dtype a, qaff_dtype b);

/*
 * Dense dequantization with scales and biases of sb_dtype (float32, bf16 or float16):
 * w = s * c, then + b, in float32 (two roundings as written: with float32 scales the product is not
 * always exact), stored in out_dtype (float32, bf16 or float16, round to nearest even).
 *   scales and biases [rows, cols/group_size] of sb_dtype; out [rows, cols] of out_dtype.
 * bf16 scales with a float32 or bf16 output take qaff_dequantize's kernel (the same values).
 * Errors: as qaff_dequantize, plus INVALID_ARGUMENT for an unknown dtype or scales and biases not
 * aligned to their element size.
 */
qaff_status qaff_dequantize_typed(const uint32_t* packed, const void* scales, const void* biases,
                                  qaff_dtype sb_dtype, int64_t rows, int64_t cols, int32_t group_size,
                                  int32_t bits, void* out, qaff_dtype out_dtype, hipStream_t stream);

/*
 * y = x . dequantize(W)^T with x of x_dtype and scales and biases of sb_dtype (each float32, bf16 or
 * float16); y [m, n] of qaff_promote_dtype(x_dtype, sb_dtype); float32 sums.
 * bf16 scales with a float32 or bf16 x take qaff_qmm's kernels (QAFF_PATH_AUTO); float16 x with
 * float16 scales and biases take their float16 forms under the same rules, without the K split:
 * below the matrix-core rows the GEMV in float16 (codes as the exact values 1024 + c,
 * v_dot2_f32_f16), then the matrix-core decode kernel (exact 4-bit codes 1024 + c where they apply,
 * else weights rounded to float16; float16 MFMA), past 16 rows the GEMM (weights rounded to
 * float16, float16 MFMA) or, for up to 128 rows, the 16-row slices of QAFF_PATH_AUTO; float32 sums,
 * y rounded to nearest even. Every other combination runs on
 * a VALU GEMV that reads the types as given (any m, any k).
 * Errors: as qaff_qmm, plus INVALID_ARGUMENT for an unknown dtype or misaligned scales.
 */
qaff_status qaff_qmm_typed(const void* x, qaff_dtype x_dtype, int64_t m, const uint32_t* packed,
                           const void* scales, const void* biases, qaff_dtype sb_dtype, int64_t n,
                           int64_t k, int32_t group_size, int32_t bits, void* y, hipStream_t stream);

/*
 * Quantization of a dense weight into this format (nuvec_core quantized.rs: module documentation
 * and quantize; rlx-moshi mlx_dequant.rs: the bias is the group minimum). Per group of group_size
 * values of a row:
 *   bias  = the group minimum; scale = (max - min) / (2^bits - 1); both stored as bf16 (round to
 *           nearest even), the scales' type every kernel here consumes (qaff_quantize_typed stores
 *           them in another type);
 *   code  = round((w - bias) / scale) with the stored bias and scale, half away from zero, clamped
 *           to [0, 2^bits - 1]; a stored scale of 0 (all values of the group equal) gives code 0,
 *           so such a group dequantizes to its value exactly.
 * The minimum, maximum, max - min and its quotient by 2^bits - 1 are float32 (w widened exactly)
 * before the rounding to the stored type. The code is the rounding of the exact value of
 * (w - bias) / scale: neither the difference nor the quotient is rounded first. NaN or infinite
 * inputs, or a stored scale or bias that is not finite (past the stored type's range), give
 * unspecified (but in-range) codes.
 *   w [rows, cols] in w_dtype (float32, bf16 or float16); packed uint32 [rows, cols*bits/32];
 *   scales and biases bf16 [rows, cols/group_size]. All caller-owned device buffers.
 * Errors: as qaff_dequantize (the outputs are checked as a weight), plus INVALID_ARGUMENT for a
 * null w, or one not aligned to its element size, where the size is non-zero.
 */
qaff_status qaff_quantize(const void* w, qaff_dtype w_dtype, int64_t rows, int64_t cols,
                          int32_t group_size, int32_t bits, uint32_t* packed, uint16_t* scales,
                          uint16_t* biases, hipStream_t stream);

/*
 * qaff_quantize with the scales and biases stored as sb_dtype (float32 as is, bf16 or float16
 * rounded to nearest even): nuvec_core quantized.rs, quantize, returns them in w's own dtype
 * (sb_dtype = w_dtype). The codes follow the same rule with the values so stored.
 *   scales and biases [rows, cols/group_size] of sb_dtype, aligned to its element size.
 * Errors: as qaff_quantize, plus INVALID_ARGUMENT for an unknown dtype.
 */
qaff_status qaff_quantize_typed(const void* w, qaff_dtype w_dtype, int64_t rows, int64_t cols,
                                int32_t group_size, int32_t bits, uint32_t* packed, void* scales,
                                void* biases, qaff_dtype sb_dtype, hipStream_t stream);

/*
 * Quantized matmul y = x . dequantize(W)^T without materialising W (nuvec_core quantized_matmul with
 * transpose, for weights stored [out, in]; maya2_mlx mm).
 *   x [m, k] in x_dtype (float32 or bf16); W is packed/scales/biases of shape [n, k];
 *   y [m, n] in the same dtype as x (x, scales and biases promote to x's type: bf16 scales never
 *   widen a float32 x, and a bf16 x stays bf16). Sums accumulate in float32; a bf16 y is the float32
 *   sum rounded to nearest even.
 * Kernel choice follows QAFF_PATH_AUTO. k == 0 writes zeros.
 * Errors: as qaff_dequantize, plus INVALID_ARGUMENT for negative m, n or k.
 */
qaff_status qaff_qmm(const void* x, qaff_dtype x_dtype, int64_t m,
                     const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                     int64_t n, int64_t k, int32_t group_size, int32_t bits,
                     void* y, hipStream_t stream);

/* qaff_qmm with the kernel forced, for tests and benchmarks. QAFF_PATH_GEMM or
 * QAFF_PATH_GEMV_MFMA with a float32 x is UNSUPPORTED (the MFMA paths would round x to bf16), and
 * so is QAFF_PATH_GEMV_MFMA with m > 16 or a shape it does not take; an unknown path is
 * INVALID_ARGUMENT. */
qaff_status qaff_qmm_ex(const void* x, qaff_dtype x_dtype, int64_t m,
                        const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                        int64_t n, int64_t k, int32_t group_size, int32_t bits,
                        void* y, hipStream_t stream, qaff_path path);

/*
 * qaff_qmm (QAFF_PATH_AUTO) with a workspace that lets the bf16 GEMM path split K (nuvec_core
 * quantized_matmul with transpose, as qaff_qmm). Where the GEMM's tiles (64 x 256 up to 128 rows
 * of x, 128 x 256 above) are fewer than the compute units (m up to about 1024 at n = 4096, K a
 * multiple of 1024; and 8 <= m <= 16 with K above 32768, which the decode kernels would otherwise
 * take on the VALU), K is split into ranges of whole 1024-code chunks: each range's float32
 * partial sums go to `workspace`, and a second kernel adds the ranges in a fixed order (results
 * are deterministic) and rounds y to bf16.
 *   Arguments as qaff_qmm, plus workspace: a caller-owned device buffer of at least
 *   qaff_qmm_workspace_size(m, n, k, group_size, bits) bytes, 16-byte aligned, which the call
 *   overwrites; it may be NULL when that size is 0. Calls that share a workspace must not overlap.
 * Errors: as qaff_qmm, plus INVALID_ARGUMENT for a missing, short or misaligned workspace where
 * one is needed.
 */
qaff_status qaff_qmm_ws(const void* x, qaff_dtype x_dtype, int64_t m, const uint32_t* packed,
                        const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                        int32_t group_size, int32_t bits, void* workspace, size_t workspace_bytes, void* y,
                        hipStream_t stream);

/* Bytes of workspace qaff_qmm_ws can use for these sizes with a bf16 x (0 where it would not split
 * K: enough tiles, K not a multiple of 1024, m <= 16 inside the decode kernels' range, or up to 32
 * rows of a weight with n and k at most 4096, whose 16-row slices of the decode path beat the
 * split). From 8 rows on, K above 32768 codes (past the matrix-core decode kernel) also takes the
 * split GEMM. */
size_t qaff_qmm_workspace_size(int64_t m, int64_t n, int64_t k, int32_t group_size, int32_t bits);

/*
 * The product without the transpose (nuvec_core quantized.rs quantized_matmul with transpose =
 * false): y = x . dequantize(W) for a weight stored [k, n], i.e. y[m, n] = sum_k x[m, k] w[k, n],
 * without materialising W.
 *   x [m, k] in x_dtype (float32 or bf16); packed uint32 [k, n*bits/32], scales and biases bf16
 *   [k, n/group_size] (groups run along n); y [m, n] in x's dtype; float32 sums.
 *   K is split over thread blocks: float32 partial sums go to `workspace`, a caller-owned device
 *   buffer of at least qaff_qmm_nt_workspace_size(m, k, n, bits) bytes (16-byte aligned), which the
 *   call overwrites; a second kernel adds the chunks in a fixed order, so results are
 *   deterministic. Calls that share a workspace must be ordered (the same stream).
 * k == 0 writes zeros. Errors: as qaff_qmm (the weight checked as [k, n]), plus INVALID_ARGUMENT
 * for a missing, short or misaligned workspace; UNSUPPORTED for m*n >= 2^31.
 */
qaff_status qaff_qmm_nt(const void* x, qaff_dtype x_dtype, int64_t m, const uint32_t* packed,
                        const uint16_t* scales, const uint16_t* biases, int64_t k, int64_t n,
                        int32_t group_size, int32_t bits, void* workspace, size_t workspace_bytes,
                        void* y, hipStream_t stream);

/*
 * qaff_qmm_nt with x of x_dtype and scales and biases of sb_dtype (each float32, bf16 or float16;
 * nuvec_core quantized.rs: quantized_matmul promotes x, scales and biases to one float type):
 * y [m, n] of qaff_promote_dtype(x_dtype, sb_dtype), float32 sums, the same kernels and K split
 * (every operand widened to float32 exactly as it is loaded; y rounded to nearest even). The
 * workspace is qaff_qmm_nt's: qaff_qmm_nt_workspace_size(m, k, n, bits) bytes.
 * bf16 scales with a float32 or bf16 x give qaff_qmm_nt's results, bit for bit.
 * Errors: as qaff_qmm_nt, plus INVALID_ARGUMENT for an unknown dtype, float32 scales and biases not
 * 4-byte aligned, or x or y not aligned to their element size.
 */
qaff_status qaff_qmm_nt_typed(const void* x, qaff_dtype x_dtype, int64_t m, const uint32_t* packed,
                              const void* scales, const void* biases, qaff_dtype sb_dtype, int64_t k,
                              int64_t n, int32_t group_size, int32_t bits, void* workspace,
                              size_t workspace_bytes, void* y, hipStream_t stream);

/* Bytes of workspace qaff_qmm_nt and qaff_qmm_nt_typed need for these sizes and bit width (0 when
 * there is nothing to compute). */
size_t qaff_qmm_nt_workspace_size(int64_t m, int64_t k, int64_t n, int32_t bits);

/*
 * qaff_qmm_nt for callers that cannot allocate device memory (code under graph capture, serving
 * loops, harnesses that forbid hipMalloc): the same kernels and the same results, bit for bit, with
 * the float32 partial sums in a scratch array that the library holds in every device's memory
 * (qaff_qmm_nt_static_max_bytes() bytes per device, from the library's load until the process
 * ends) instead of a caller workspace. The call allocates and frees nothing.
 *   Arguments as qaff_qmm_nt without the workspace. The scratch is resolved for the device current
 *   at the call (once per device).
 *   Every call on a device shares that device's scratch and leaves its last contents there (no
 *   state is carried: every partial sum a call reads, it wrote first). Calls that overlap on one
 *   device race: order them (the same stream, or events between streams).
 * Errors: as qaff_qmm_nt, plus UNSUPPORTED where the sizes need more partial sums than the scratch
 * holds (qaff_qmm_nt_workspace_size(m, k, n, bits) > qaff_qmm_nt_static_max_bytes()).
 */
qaff_status qaff_qmm_nt_static(const void* x, qaff_dtype x_dtype, int64_t m, const uint32_t* packed,
                               const uint16_t* scales, const uint16_t* biases, int64_t k, int64_t n,
                               int32_t group_size, int32_t bits, void* y, hipStream_t stream);

/* Bytes of the per-device scratch array behind qaff_qmm_nt_static. */
size_t qaff_qmm_nt_static_max_bytes(void);

/*
 * Dual decode product (spark_runtime weights/mlx_int8.rs gemv_gate_up): gate_y = x . dequantize(G)^T
 * and up_y = x . dequantize(U)^T in one launch, x read once. Both weights share n, k, group_size
 * and bits. x bf16 [m, k] with 1 <= m <= 16; gate_y, up_y bf16 [m, n]; sums in float32, each output
 * rounded to nearest even. k == 0 writes zeros.
 * Errors: as qaff_qmm for each weight; UNSUPPORTED for m > 16; INVALID_ARGUMENT for a null or
 * misaligned (2-byte) x or output.
 */
qaff_status qaff_gemv_gate_up(const void* x, int64_t m, const uint32_t* gate_packed,
                              const uint16_t* gate_scales, const uint16_t* gate_biases,
                              const uint32_t* up_packed, const uint16_t* up_scales,
                              const uint16_t* up_biases, int64_t n, int64_t k, int32_t group_size,
                              int32_t bits, void* gate_y, void* up_y, hipStream_t stream);

/*
 * Fused activation and decode product (spark_runtime weights/mlx_int8.rs gemv_silu_gate and
 * gemv_silu_gate_resid): y = h . dequantize(W)^T (+ resid), where h = silu(gate) * up,
 * silu(v) = v / (1 + exp(-v)). h is formed in float32 and rounded to bf16 (the element type of
 * gate and up, as the staging buffer that the fusion removes would hold it); the sum is float32;
 * a residual is added in float32 before y is rounded to nearest even.
 *   gate, up bf16 [m, k] with 1 <= m <= 16; resid bf16 [m, n] or NULL; y bf16 [m, n].
 * k == 0 writes resid (or zeros).
 * Errors: as qaff_qmm for the weight; UNSUPPORTED for m > 16; INVALID_ARGUMENT for a null or
 * misaligned (2-byte) gate, up or y, or a resid that is not 2-byte aligned.
 */
qaff_status qaff_gemv_silu_gate(const void* gate, const void* up, int64_t m, const uint32_t* packed,
                                const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                                int32_t group_size, int32_t bits, const void* resid, void* y,
                                hipStream_t stream);

/*
 * Quantized products of gathered batches (nuvec_core quantized.rs gather_qmm with the transpose;
 * its mixture-of-experts use: one weight batch per expert). Output batch b is
 *     y[b] = x[lhs_indices[b]] . dequantize(W[rhs_indices[b]])^T.
 *   x [x_batches, m, k] in x_dtype (float32 or bf16); the weight is w_batches matrices [n, k] stacked:
 *   packed [w_batches, n, k*bits/32], scales and biases [w_batches, n, k/group_size];
 *   lhs_indices, rhs_indices: uint32 device arrays of `batch` entries (nuvec_core gather_indices
 *   casts integer indices to U32), or NULL for 0 .. batch-1 (then batch must not exceed that
 *   operand's batches). Broadcasting index arrays against each other is left to the caller, who
 *   passes them expanded to `batch` entries. y [batch, m, n] in x's dtype; sums in float32.
 *   An index at or past its operand's batches cannot be checked on the host without a
 *   synchronization: that output batch is filled with quiet NaNs.
 *   sorted_indices != 0 promises that rhs_indices is non-decreasing (rows grouped by expert). With
 *   m == 1, lhs_indices NULL and a bf16 x, the matrix-core kernel then walks each expert once over
 *   all of its rows (rows [#(rhs < e), #(rhs < e + 1)) of expert e). A broken promise leaves rows
 *   unwritten or computed with another expert. Without the conditions the flag changes nothing.
 * Kernels (QAFF_PATH_AUTO): with the sorted promise kept as above, once the experts average 32 rows
 * or more (batch >= 32 * w_batches), k a multiple of 1024 and every weight batch's scales and biases
 * 16-byte aligned, a bf16-MFMA GEMM over each expert's rows (each expert's weights dequantized once
 * per 128 rows); otherwise the matrix-core decode kernel where it applies (bf16 x, k a multiple of
 * 512 up to 4096, 4-byte aligned scales and biases) when grouped, or when m >= qaff_gemv_mfma_min_m();
 * the VALU GEMV otherwise (any m). x or y not 16-byte aligned: the element-by-element GEMV.
 * Errors: as qaff_qmm, plus INVALID_ARGUMENT for negative batch counts, a NULL index array with
 * batch above its operand's batches, or misaligned (4-byte) indices.
 */
qaff_status qaff_gather_qmm(const void* x, qaff_dtype x_dtype, int64_t x_batches, int64_t m,
                            const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                            int64_t w_batches, int64_t n, int64_t k, int32_t group_size, int32_t bits,
                            const uint32_t* lhs_indices, const uint32_t* rhs_indices, int64_t batch,
                            int32_t sorted_indices, void* y, hipStream_t stream);

/*
 * qaff_gather_qmm with x and the scales and biases of any of the three types (nuvec_core
 * quantized.rs, gather_qmm: x, scales and biases promote to one float type): y [batch, m, n] of
 * qaff_promote_dtype(x_dtype, sb_dtype); float32 sums.
 *   scales and biases [w_batches, n, k/group_size] of sb_dtype (float32 4-byte aligned); the other
 *   arguments as qaff_gather_qmm. bf16 scales with a float32 or bf16 x take qaff_gather_qmm itself
 *   (the same kernels and results); float16 x, scales and biases take the float16 forms of its
 *   matrix-core kernels under its rules (the grouped GEMM, the grouped or batched decode kernel;
 *   x and y 16-byte aligned) and otherwise the typed GEMV below; every other combination runs on
 *   the typed VALU GEMV with grid z
 *   over the output batches (x 16-byte aligned; otherwise element by element), or, with the sorted
 *   promise, one x row per batch, no lhs and at least 16 rows per weight batch on average, over the
 *   experts, each walking its rows [#(rhs < e), #(rhs < e + 1)) and reading its weights once (as
 *   with qaff_gather_qmm, unsorted rhs under the promise leaves results undefined).
 * Errors: as qaff_gather_qmm, plus INVALID_ARGUMENT for an unknown dtype or misaligned scales.
 */
qaff_status qaff_gather_qmm_typed(const void* x, qaff_dtype x_dtype, int64_t x_batches, int64_t m,
                                  const uint32_t* packed, const void* scales, const void* biases,
                                  qaff_dtype sb_dtype, int64_t w_batches, int64_t n, int64_t k,
                                  int32_t group_size, int32_t bits, const uint32_t* lhs_indices,
                                  const uint32_t* rhs_indices, int64_t batch, int32_t sorted_indices,
                                  void* y, hipStream_t stream);

/* qaff_gather_qmm with the kernel forced: QAFF_PATH_GEMV (the VALU GEMV; the sorted promise is not
 * used), QAFF_PATH_GEMV_MFMA (UNSUPPORTED where that kernel does not apply) or QAFF_PATH_GEMM (the
 * GEMM over each expert's rows; UNSUPPORTED unless the sorted promise holds with m == 1, no lhs and
 * a bf16 x, k is a multiple of 1024 and scales and biases are 16-byte aligned per weight batch). */
qaff_status qaff_gather_qmm_ex(const void* x, qaff_dtype x_dtype, int64_t x_batches, int64_t m,
                               const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                               int64_t w_batches, int64_t n, int64_t k, int32_t group_size, int32_t bits,
                               const uint32_t* lhs_indices, const uint32_t* rhs_indices, int64_t batch,
                               int32_t sorted_indices, void* y, hipStream_t stream, qaff_path path);

/*
 * Gathered-row dequantization: out[i, :] = dequantize(table)[indices[i], :] (maya2_mlx rows: an
 * embedding lookup that dequantizes only the gathered rows). Indices are uint32 (nuvec_core
 * gather_indices casts integer indices to U32); duplicates are allowed. An index >= table_rows
 * cannot be checked on the host without a synchronization: its output row is filled with quiet
 * NaNs (0x7FC00000 in float32, 0x7FC0 in bf16).
 *   packed/scales/biases: the table [table_rows, cols]; out [n_indices, cols] in out_dtype.
 * Errors: as qaff_dequantize, plus INVALID_ARGUMENT for negative table_rows or n_indices, or a
 * null/misaligned indices pointer when n_indices > 0.
 */
qaff_status qaff_dequant_rows(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                              int64_t table_rows, int64_t cols, int32_t group_size, int32_t bits,
                              const uint32_t* indices, int64_t n_indices,
                              void* out, qaff_dtype out_dtype, hipStream_t stream);

/* Text for the last non-OK status returned on the calling thread ("" if none). The pointer stays
 * valid until the thread's next qaff call. */
const char* qaff_last_error(void);

/* A constant name for a status code. */
const char* qaff_status_string(qaff_status status);

/* QAFF_ABI_VERSION of the loaded library. */
int qaff_abi_version(void);

/* Largest m that QAFF_PATH_AUTO sends to the decode path for a bf16 x. */
int qaff_gemv_max_m(void);

/* Smallest m that QAFF_PATH_AUTO sends to the matrix-core decode kernel (where it applies) for K
 * up to 4096; above 4096 it is 2. */
int qaff_gemv_mfma_min_m(void);

#ifdef __cplusplus
}
#endif

#endif /* QAFF_H */
