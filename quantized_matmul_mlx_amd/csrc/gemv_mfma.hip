// The matrix-core decode kernels (gemv_mfma_impl.h) in bf16: x, scales, biases and y bf16. Their
// float16 form is gemv_mfma_f16.hip, a translation unit of its own so that both build in parallel.
#include "gemv_mfma_impl.h"

namespace qaff {

hipError_t launch_gemv_mfma(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                            const uint16_t* biases, int64_t n, int64_t k, int group_size, int bits,
                            uint16_t* y, hipStream_t stream) {
    return mfma_decode<false>(x, m, packed, scales, biases, n, k, group_size, bits, y, stream);
}

hipError_t launch_gemv_mfma_gather(const uint16_t* x, int64_t m, const uint32_t* packed,
                                   const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                                   int group_size, int bits, uint16_t* y, const Gather& g,
                                   hipStream_t stream) {
    return mfma_gather<false>(x, m, packed, scales, biases, n, k, group_size, bits, y, g, stream);
}

bool gemv_mfma_supported(int64_t m, int64_t k) {
    return m >= 1 && m <= 16 && k % kSlice == 0 && k > 0 && k <= kMaxK;
}

// the gathered kernel: one slice per wave, at most 8 waves
bool gemv_mfma_gather_supported(int64_t k) { return k % kSlice == 0 && k > 0 && k <= 8 * kSlice; }

}  // namespace qaff
