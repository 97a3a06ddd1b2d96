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

// The decode product on the matrix cores: y[m, n] (bf16) = x (bf16) . dequantize(W)^T for
// 1 <= m <= 16, with each code dequantized to bf16 in registers. Only for shapes where
// gemv_mfma_supported(m, k) holds, and scales/biases 4-byte aligned.
bool gemv_mfma_supported(int64_t m, int64_t k);
hipError_t launch_gemv_mfma(const uint16_t* x, int64_t m, const uint32_t* packed,
                            const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                            int group_size, int bits, uint16_t* y, hipStream_t stream);

// y[m, n] (bf16) = x (bf16) . dequantize(W)^T with W tiles dequantized to bf16 and bf16 MFMA,
// float32 accumulation.
hipError_t launch_gemm(const uint16_t* x, int64_t m, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                       int group_size, int bits, uint16_t* y, hipStream_t stream);

// Writes `bytes` zero bytes (bytes % 2 == 0, p 2-byte aligned) with a kernel, so that the call
// also behaves under stream capture.
hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t stream);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace qaff
