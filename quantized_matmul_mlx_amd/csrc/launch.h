// Internal launchers behind the C ABI. Arguments are already validated by api.cpp; every launcher
// only enqueues work on `stream` and returns hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qaff {

// out[i, :] = dequantize(row src(i)) for i < out_rows, where src(i) = indices[i] when indices is
// non-null (an index >= table_rows gives a NaN row) and i otherwise.
hipError_t launch_dequant(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                          const uint32_t* indices, int64_t table_rows, int64_t out_rows,
                          int64_t cols, int group_size, int bits, void* out, bool out_bf16,
                          hipStream_t stream);

// y[m, n] = x . dequantize(W)^T on the VALU: float32 sums, x float32 or bf16, y in x's dtype.
hipError_t launch_gemv(const void* x, bool x_f32, int64_t m, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                       int group_size, int bits, void* y, hipStream_t stream);

// Fused decode products on the bf16 GEMV (spark_runtime gemv_gate_up, gemv_silu_gate,
// gemv_silu_gate_resid). Null members are unused.
struct GemvFused {
    const uint16_t* up;       // x is the gate; the product's input is bf16(silu(x) * up)
    const uint16_t* resid;    // y = bf16(sum + resid[m, n])
    const uint32_t* packed2;  // a second weight of the same shape (n, k, group, bits) ...
    const uint16_t* scales2;
    const uint16_t* biases2;
    uint16_t* y2;             // ... whose product with the same x goes to y2
};
hipError_t launch_gemv_fused(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                             const uint16_t* biases, int64_t n, int64_t k, int group_size, int bits,
                             uint16_t* y, const GemvFused& f, hipStream_t stream);

// The same GEMV with float16 x, scales and biases and a float16 y: codes as the exact float16 values
// 1024 + c, v_dot2_f32_f16, float32 sums.
hipError_t launch_gemv_f16(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                           const uint16_t* biases, int64_t n, int64_t k, int group_size, int bits, uint16_t* y,
                           hipStream_t stream);

// A gathered product (nuvec_core quantized.rs, `gather_qmm`): output batch b is
// x[lhs[b]] . dequantize(W[rhs[b]])^T. Launches index the batch through the grid; `b0` is the
// first batch (or expert) of a launch, since one grid dimension holds at most 65535 blocks.
struct Gather {
    const uint32_t* lhs;  // x batch of output batch b; null: b
    const uint32_t* rhs;  // weight batch of output batch b; null: b
    uint32_t x_count;     // batches of x and of the weight; an index at or past its count
    uint32_t w_count;     // gives a NaN output batch
    uint32_t batch;       // output batches
    uint32_t b0;
    int grouped;          // matrix-core kernel only: rhs is sorted, m == 1 and lhs is null; the grid
                          // walks experts 0 .. w_count (the last one: rows past every expert)
    uint64_t x_stride;    // x elements per batch (m * k)
    uint64_t w_stride;    // packed words per weight batch
    uint64_t sb_stride;   // scales (biases) per weight batch
    uint64_t y_stride;    // y elements per batch (m * n)
};

// The VALU GEMV over gathered batches (any m, x float32 or bf16, y in x's dtype).
hipError_t launch_gemv_gather(const void* x, bool x_f32, int64_t m, const uint32_t* packed,
                              const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                              int group_size, int bits, void* y, const Gather& g, hipStream_t stream);

// The decode product on the matrix cores: y[m, n] (bf16) = x (bf16) . dequantize(W)^T for
// 1 <= m <= 16, with each code dequantized to bf16 in registers. Only for shapes where
// gemv_mfma_supported(m, k) holds (k a multiple of 512 up to 32768), and scales/biases 4-byte
// aligned.
bool gemv_mfma_supported(int64_t m, int64_t k);
hipError_t launch_gemv_mfma(const uint16_t* x, int64_t m, const uint32_t* packed,
                            const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                            int group_size, int bits, uint16_t* y, hipStream_t stream);

// The matrix-core decode kernel over gathered batches (any m, in tiles of up to 16 rows; bf16), or
// with g.grouped over the rows of each expert, reading each expert's weights once. Only where
// gemv_mfma_gather_supported(k) holds (k a multiple of 512 up to 4096) and scales/biases are
// 4-byte aligned.
bool gemv_mfma_gather_supported(int64_t k);
hipError_t launch_gemv_mfma_gather(const uint16_t* x, int64_t m, const uint32_t* packed,
                                   const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                                   int group_size, int bits, uint16_t* y, const Gather& g,
                                   hipStream_t stream);

// The same two in float16 (x, scales, biases and y float16), for the same shapes.
hipError_t launch_gemv_mfma_f16(const uint16_t* x, int64_t m, const uint32_t* packed,
                                const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                                int group_size, int bits, uint16_t* y, hipStream_t stream);
hipError_t launch_gemv_mfma_gather_f16(const uint16_t* x, int64_t m, const uint32_t* packed,
                                       const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                                       int group_size, int bits, uint16_t* y, const Gather& g,
                                       hipStream_t stream);

// y[m, n] (bf16) = x (bf16) . dequantize(W)^T with W dequantized to bf16 and bf16 MFMA, float32
// accumulation. With a workspace of at least gemm_workspace_bytes(m, n, k) bytes (16-byte
// aligned), few tiles split K: float32 partial sums go to the workspace and a second kernel adds
// them in order.
hipError_t launch_gemm(const uint16_t* x, int64_t m, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                       int group_size, int bits, uint16_t* y, hipStream_t stream, void* workspace = nullptr,
                       size_t workspace_bytes = 0);
size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);

// The GEMM above over gathered batches grouped by expert: output row r (one x row per batch, no lhs)
// is x[r] . dequantize(W[rhs[r]])^T with rhs sorted (non-decreasing); each expert's rows form a plain
// GEMM against its weight batch. Rows whose index is at or past w_count get NaN. Supported where
// gemm_grouped_supported holds (K a multiple of 1024, 16-byte aligned scales and biases of every
// weight batch).
bool gemm_grouped_supported(int64_t k, const uint16_t* scales, const uint16_t* biases, uint64_t sb_stride);
hipError_t launch_gemm_grouped(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                               const uint16_t* biases, int64_t n, int64_t k, int group_size, int bits, uint16_t* y,
                               const uint32_t* rhs, int64_t batch, int64_t w_count, uint64_t w_stride,
                               uint64_t sb_stride, hipStream_t stream);

// The same two in float16 (x, scales, biases and y float16, W rounded to float16), without the
// K split, for the same shapes.
hipError_t launch_gemm_f16(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                           const uint16_t* biases, int64_t n, int64_t k, int group_size, int bits, uint16_t* y,
                           hipStream_t stream);
hipError_t launch_gemm_grouped_f16(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                                   const uint16_t* biases, int64_t n, int64_t k, int group_size, int bits,
                                   uint16_t* y, const uint32_t* rhs, int64_t batch, int64_t w_count,
                                   uint64_t w_stride, uint64_t sb_stride, hipStream_t stream);

// packed/scales/biases of a dense [rows, cols] weight of dtype code w_dtype (0 float32, 1 bf16,
// 2 float16): bias = group min, scale = (max - min) / (2^bits - 1), both stored as sb_dtype; code =
// round((w - bias) / scale), clamped. w 16-byte aligned: 16-byte loads; otherwise element by element.
hipError_t launch_quantize(const void* w, int w_dtype, int64_t rows, int64_t cols, int group_size, int bits,
                           uint32_t* packed, void* scales, void* biases, int sb_dtype, hipStream_t stream);

// y[m, n] = x[m, k] . dequantize(W) for W stored [k, n] (groups along n); float32 partial sums
// of K chunks go to `workspace` (qmm_nt_workspace_bytes(m, k, n) bytes), then a second kernel
// adds them in order. Dtype codes 0 float32, 1 bf16, 2 float16 for x, the scales and biases, and y.
void qmm_nt_plan(int64_t k, int64_t n, int bits, int64_t* kchunk, int64_t* chunks);
size_t qmm_nt_workspace_bytes(int64_t m, int64_t k, int64_t n, int bits);
hipError_t launch_qmm_nt(const void* x, int x_dtype, int64_t m, const uint32_t* packed, const void* scales,
                         const void* biases, int sb_dtype, int64_t k, int64_t n, int group_size, int bits,
                         void* workspace, void* y, int y_dtype, hipStream_t stream);

// The device address of the static scratch array that stands in for qmm_nt's workspace
// (kQmmNtStaticScratchBytes on every device), resolved once per device with it current.
constexpr size_t kQmmNtStaticScratchBytes = (size_t)8 << 20;
hipError_t qmm_nt_static_scratch(void** ptr);

// Other float types (dtype codes 0 float32, 1 bf16, 2 float16) for scales, biases, x and outputs.
// The dequantization stores element by element (out needs only its element size of alignment); with
// `indices`, output row r is table row indices[r] (an index >= table_rows gives a NaN row).
hipError_t launch_dequant_typed(const uint32_t* packed, const void* scales, const void* biases, int sb_dtype,
                                int64_t rows, int64_t cols, int group_size, int bits, void* out, int out_dtype,
                                hipStream_t stream, const uint32_t* indices = nullptr, int64_t table_rows = 0);
// With `gather`, the product over its output batches (x batch lhs[b] against weight batch rhs[b],
// strides in elements of each operand's own type; NaN batches past either operand).
hipError_t launch_gemv_typed(const void* x, int x_dtype, int64_t m, const uint32_t* packed, const void* scales,
                             const void* biases, int sb_dtype, int64_t n, int64_t k, int group_size, int bits, void* y,
                             int y_dtype, hipStream_t stream, const Gather* gather = nullptr);

// The element-by-element GEMV behind operands that are not 16-byte aligned: y = x . dequantize(W)^T
// with x, scales, biases and y of the given dtype codes, each loaded and stored one element at a time
// (every operand needs only its element size of alignment), float32 sums. Options:
//  * up: x is the gate and the product's input is bf16(silu(x) * up) (bf16 x and up);
//  * resid: y = bf16(sum + resid) (bf16 y);
//  * gather: output batch b is x[lhs[b]] . dequantize(W[rhs[b]])^T (NaN batch for an index out of
//    range).
struct ScalarGemv {
    const uint16_t* up = nullptr;
    const uint16_t* resid = nullptr;
    bool gather = false;
    Gather g{};
};
hipError_t launch_gemv_scalar(const void* x, int x_dtype, int64_t m, const uint32_t* packed, const void* scales,
                              const void* biases, int sb_dtype, int64_t n, int64_t k, int group_size, int bits,
                              void* y, int y_dtype, const ScalarGemv& opt, hipStream_t stream);

// Writes `bytes` zero bytes (bytes % 2 == 0, p 2-byte aligned) with a kernel, so that the call
// also behaves under stream capture.
hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t stream);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace qaff
