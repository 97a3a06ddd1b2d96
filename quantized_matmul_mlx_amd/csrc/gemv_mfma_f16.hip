// The matrix-core decode kernels (gemv_mfma_impl.h) in float16: x, scales, biases and y float16,
// the weights entering v_mfma_f32_16x16x32_f16 as exact codes 1024 + c or rounded to float16.
#include "gemv_mfma_impl.h"

namespace qaff {

hipError_t launch_gemv_mfma_f16(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                                const uint16_t* biases, int64_t n, int64_t k, int group_size, int bits,
                                uint16_t* y, hipStream_t stream) {
    return mfma_decode<true>(x, m, packed, scales, biases, n, k, group_size, bits, y, stream);
}

hipError_t launch_gemv_mfma_gather_f16(const uint16_t* x, int64_t m, const uint32_t* packed,
                                       const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                                       int group_size, int bits, uint16_t* y, const Gather& g,
                                       hipStream_t stream) {
    return mfma_gather<true>(x, m, packed, scales, biases, n, k, group_size, bits, y, g, stream);
}

}  // namespace qaff
