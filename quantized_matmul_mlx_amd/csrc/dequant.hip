// Dense and gathered-row dequantization, w = scale * code + bias (rlx-moshi mlx_dequant.rs,
// dequantize_affine; spark_runtime weights/mlx_int8.rs, module formula and dequantize_to;
// maya2_mlx quant.py, rows).
//
// HBM-bound and write-dominated: a 4-bit weight reads 0.5 B of codes and writes 4 B (float32) or
// 2 B (bf16). One thread owns one 32-code block: it loads the block's `bits` words in one or two
// vector loads, reads the block's single scale and bias, and writes 32 outputs as 16-byte stores.
#include "launch.h"
#include "qaff_device.h"

#include <hip/hip_runtime.h>

namespace qaff {
namespace {

constexpr int kThreads = 256;

template <int BITS, bool OUT_BF16, bool GATHER>
__global__ __launch_bounds__(kThreads) void dequant_kernel(
    const uint32_t* __restrict__ packed, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const uint32_t* __restrict__ indices, uint32_t table_rows,
    uint32_t out_rows, uint32_t kb, uint32_t gshift, void* __restrict__ out) {
#pragma clang fp contract(off)
    const uint32_t total = out_rows * kb;  // the host guarantees this fits in 32 bits
    const uint32_t gpr = kb >> gshift;     // groups per row
    for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < total; b += gridDim.x * kThreads) {
        const uint32_t r = b / kb;
        const uint32_t j = b - r * kb;
        uint32_t src = r;
        if constexpr (GATHER) src = indices[r];
        float v[32];
        if (GATHER && src >= table_rows) {
#pragma unroll
            for (int c = 0; c < 32; ++c) v[c] = __uint_as_float(0x7fc00000u);
        } else {
            uint32_t w[BITS];
            load_block<BITS>(packed + (size_t)src * kb * BITS + (size_t)j * BITS, w);
            const size_t gi = (size_t)src * gpr + (j >> gshift);
            const float s = bf16_to_f32(scales[gi]);
            const float bias = bf16_to_f32(biases[gi]);
#pragma unroll
            for (int c = 0; c < 32; ++c) {
                const float p = s * (float)code_at<BITS>(w, c);
                v[c] = p + bias;
            }
        }
        if constexpr (OUT_BF16) {
            u32x4a* o = reinterpret_cast<u32x4a*>(static_cast<uint16_t*>(out) + ((size_t)r * kb + j) * 32);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                u32x4a d;
                d.x = pack_bf16x2(v[8 * q + 0], v[8 * q + 1]);
                d.y = pack_bf16x2(v[8 * q + 2], v[8 * q + 3]);
                d.z = pack_bf16x2(v[8 * q + 4], v[8 * q + 5]);
                d.w = pack_bf16x2(v[8 * q + 6], v[8 * q + 7]);
                o[q] = d;
            }
        } else {
            f32x4* o = reinterpret_cast<f32x4*>(static_cast<float*>(out) + ((size_t)r * kb + j) * 32);
#pragma unroll
            for (int q = 0; q < 8; ++q) o[q] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
        }
    }
}

template <int BITS, bool OUT_BF16, bool GATHER>
hipError_t launch_one(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                      const uint32_t* indices, int64_t table_rows, int64_t out_rows, int64_t kb,
                      uint32_t gshift, void* out, hipStream_t stream) {
    const int64_t total = out_rows * kb;
    int64_t grid = (total + kThreads - 1) / kThreads;
    const int64_t cap = (int64_t)device_cu_count() * 16;
    if (grid > cap) grid = cap;
    dequant_kernel<BITS, OUT_BF16, GATHER><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
        packed, scales, biases, indices, (uint32_t)table_rows,
        (uint32_t)out_rows, (uint32_t)kb, gshift, out);
    return hipGetLastError();
}

template <int BITS>
hipError_t dispatch_out(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                        const uint32_t* indices, int64_t table_rows, int64_t out_rows, int64_t kb,
                        uint32_t gshift, void* out, bool out_bf16, hipStream_t stream) {
    if (indices) {
        return out_bf16 ? launch_one<BITS, true, true>(packed, scales, biases, indices, table_rows, out_rows, kb, gshift, out, stream)
                        : launch_one<BITS, false, true>(packed, scales, biases, indices, table_rows, out_rows, kb, gshift, out, stream);
    }
    return out_bf16 ? launch_one<BITS, true, false>(packed, scales, biases, nullptr, table_rows, out_rows, kb, gshift, out, stream)
                    : launch_one<BITS, false, false>(packed, scales, biases, nullptr, table_rows, out_rows, kb, gshift, out, stream);
}

__global__ void fill_zero_kernel(uint16_t* __restrict__ p, uint64_t halves) {
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < halves;
         i += (uint64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

}  // namespace

hipError_t launch_dequant(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                          const uint32_t* indices, int64_t table_rows, int64_t out_rows,
                          int64_t cols, int group_size, int bits, void* out, bool out_bf16,
                          hipStream_t stream) {
    const int64_t kb = cols / 32;
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    switch (bits) {
        case 2: return dispatch_out<2>(packed, scales, biases, indices, table_rows, out_rows, kb, gshift, out, out_bf16, stream);
        case 3: return dispatch_out<3>(packed, scales, biases, indices, table_rows, out_rows, kb, gshift, out, out_bf16, stream);
        case 4: return dispatch_out<4>(packed, scales, biases, indices, table_rows, out_rows, kb, gshift, out, out_bf16, stream);
        case 5: return dispatch_out<5>(packed, scales, biases, indices, table_rows, out_rows, kb, gshift, out, out_bf16, stream);
        case 6: return dispatch_out<6>(packed, scales, biases, indices, table_rows, out_rows, kb, gshift, out, out_bf16, stream);
        case 8: return dispatch_out<8>(packed, scales, biases, indices, table_rows, out_rows, kb, gshift, out, out_bf16, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t stream) {
    const uint64_t halves = (uint64_t)bytes / 2;
    if (halves == 0) return hipSuccess;
    uint64_t grid = (halves + 255) / 256;
    if (grid > 4096) grid = 4096;
    fill_zero_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(static_cast<uint16_t*>(p), halves);
    return hipGetLastError();
}

}  // namespace qaff
