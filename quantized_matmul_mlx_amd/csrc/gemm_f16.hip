// The prefill GEMM kernels (gemm_impl.h) in float16: x, scales, biases and y float16, W dequantized
// and rounded to float16 for v_mfma_f32_32x32x16_f16.
#include "gemm_impl.h"

namespace qaff {

hipError_t launch_gemm_grouped_f16(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                                   const uint16_t* biases, int64_t n, int64_t k, int group_size, int bits,
                                   uint16_t* y, const uint32_t* rhs, int64_t batch, int64_t w_count,
                                   uint64_t w_stride, uint64_t sb_stride, hipStream_t stream) {
    return grouped_run<true>(x, packed, scales, biases, n, k, group_size, bits, y, rhs, batch, w_count, w_stride,
                             sb_stride, stream);
}

hipError_t launch_gemm_f16(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                           const uint16_t* biases, int64_t n, int64_t k, int group_size, int bits, uint16_t* y,
                           hipStream_t stream) {
    return gemm_run<true>(x, m, packed, scales, biases, n, k, group_size, bits, y, stream, nullptr, 0);
}

}  // namespace qaff
