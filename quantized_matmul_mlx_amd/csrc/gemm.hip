// The prefill GEMM kernels (gemm_impl.h) in bf16: x, scales, biases and y bf16. Their float16 form
// is gemm_f16.hip, a translation unit of its own so that both build in parallel.
#include "gemm_impl.h"

namespace qaff {

bool gemm_grouped_supported(int64_t k, const uint16_t* scales, const uint16_t* biases, uint64_t sb_stride) {
    auto a16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
    return k > 0 && k % (64 * kDirectBody) == 0 && a16(scales) && a16(biases) && (sb_stride * 2) % 16 == 0;
}

hipError_t launch_gemm_grouped(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                               const uint16_t* biases, int64_t n, int64_t k, int group_size, int bits, uint16_t* y,
                               const uint32_t* rhs, int64_t batch, int64_t w_count, uint64_t w_stride,
                               uint64_t sb_stride, hipStream_t stream) {
    return grouped_run<false>(x, packed, scales, biases, n, k, group_size, bits, y, rhs, batch, w_count, w_stride,
                              sb_stride, stream);
}

size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    const int64_t s = direct_splits(m, n, k);
    return s > 1 ? (size_t)s * (size_t)m * (size_t)n * sizeof(float) : 0;
}

hipError_t launch_gemm(const uint16_t* x, int64_t m, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                       int group_size, int bits, uint16_t* y, hipStream_t stream, void* workspace,
                       size_t workspace_bytes) {
    return gemm_run<false>(x, m, packed, scales, biases, n, k, group_size, bits, y, stream, workspace,
                           workspace_bytes);
}

}  // namespace qaff
