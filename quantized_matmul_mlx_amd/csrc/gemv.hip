// Quantized GEMV on the VALU: y[m, n] = sum_k x[m, k] * w[n, k] for a few rows of x (the decode
// path of spark_runtime weights/mlx_int8.rs, `gemv`; the product itself is nuvec_core
// quantized.rs, `quantized_matmul` with transpose). W is never materialised.
//
// HBM-bound: every packed word is read exactly once per launch for up to MB rows of x. One wave
// owns RW rows of W; its 64 lanes split the row's 32-code blocks (lane l takes blocks l, l+64, ...),
// so each wave-wide load of a block reads contiguous words. Per block the scale and bias are
// applied once, using the group identity
//     sum_{k in block} x_k * (s*c_k + b) = s * sum x_k c_k + b * sum x_k,
// so the inner loop is one multiply-add per code and x-row. The float32 partial sums are reduced
// across the wave at the end.
#include "launch.h"
#include "qaff_device.h"

#include <hip/hip_runtime.h>

namespace qaff {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// The 32 x values of block j of x row `row`, as float32.
template <bool XF32>
__device__ __forceinline__ void load_x_block(const void* __restrict__ x, uint32_t row, uint32_t k,
                                             uint32_t j, float (&xv)[32]) {
    if constexpr (XF32) {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + (size_t)row * k + (size_t)j * 32);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const f32x4 v = p[q];
            xv[4 * q] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
        }
    } else {
        const u32x4a* p = reinterpret_cast<const u32x4a*>(static_cast<const uint16_t*>(x) + (size_t)row * k + (size_t)j * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4a v = p[q];
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xv[8 * q + 2 * e] = __uint_as_float(d[e] << 16);
                xv[8 * q + 2 * e + 1] = __uint_as_float(d[e] & 0xffff0000u);
            }
        }
    }
}

template <int BITS, bool XF32, int MB, int RW>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    const void* __restrict__ x, uint32_t m, const uint32_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases, uint32_t n,
    uint32_t kb, uint32_t gshift, void* __restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint32_t n0 = (blockIdx.x * kWaves + wave) * RW;
    if (n0 >= n) return;  // wave-uniform; this kernel has no block-level barrier
    const uint32_t m0 = blockIdx.y * MB;
    const uint32_t k = kb * 32;
    const uint32_t gpr = kb >> gshift;

    float acc[RW][MB];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int i = 0; i < MB; ++i) acc[r][i] = 0.f;

    for (uint32_t j = lane; j < kb; j += 64) {
        float xv[MB][32];
        float xs[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            if (m0 + i < m) {
                load_x_block<XF32>(x, m0 + i, k, j, xv[i]);
            } else {
#pragma unroll
                for (int c = 0; c < 32; ++c) xv[i][c] = 0.f;
            }
            float t = 0.f;
#pragma unroll
            for (int c = 0; c < 32; ++c) t += xv[i][c];
            xs[i] = t;
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const uint32_t row = n0 + r;
            if (row >= n) break;
            uint32_t w[BITS];
            load_block<BITS>(packed + (size_t)row * kb * BITS + (size_t)j * BITS, w);
            const size_t gi = (size_t)row * gpr + (j >> gshift);
            const float s = bf16_to_f32(scales[gi]);
            const float b = bf16_to_f32(biases[gi]);
            float cf[32];
#pragma unroll
            for (int c = 0; c < 32; ++c) cf[c] = (float)code_at<BITS>(w, c);
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                float d = 0.f;
#pragma unroll
                for (int c = 0; c < 32; ++c) d += xv[i][c] * cf[c];
                acc[r][i] += s * d + b * xs[i];
            }
        }
    }

#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const uint32_t row = n0 + r;
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const float v = wave_sum(acc[r][i]);
            if (lane == 0 && row < n && m0 + i < m) {
                const size_t o = (size_t)(m0 + i) * n + row;
                if constexpr (XF32) static_cast<float*>(y)[o] = v;
                else static_cast<uint16_t*>(y)[o] = to_bf16_bits(v);
            }
        }
    }
}

constexpr int kRowsPerWave = 2;

template <int BITS, bool XF32, int MB>
hipError_t launch_mb(const void* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                     const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, void* y,
                     hipStream_t stream) {
    const int64_t rows_per_block = (int64_t)kWaves * kRowsPerWave;
    const unsigned gx = (unsigned)((n + rows_per_block - 1) / rows_per_block);
    const size_t xsize = XF32 ? 4 : 2;
    // grid.y is limited to 65535 blocks: long x goes in slices of at most 65535 * MB rows.
    const int64_t max_rows = (int64_t)65535 * MB;
    for (int64_t m_off = 0; m_off < m; m_off += max_rows) {
        const int64_t mm = (m - m_off < max_rows) ? (m - m_off) : max_rows;
        const unsigned gy = (unsigned)((mm + MB - 1) / MB);
        gemv_kernel<BITS, XF32, MB, kRowsPerWave><<<dim3(gx, gy), dim3(kThreads), 0, stream>>>(
            static_cast<const char*>(x) + (size_t)m_off * kb * 32 * xsize, (uint32_t)mm, packed,
            scales, biases, (uint32_t)n, (uint32_t)kb, gshift,
            static_cast<char*>(y) + (size_t)m_off * n * xsize);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int BITS, bool XF32>
hipError_t launch_bits(const void* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                       const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, void* y,
                       hipStream_t stream) {
    if (m == 1) return launch_mb<BITS, XF32, 1>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
    if (m == 2) return launch_mb<BITS, XF32, 2>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
    return launch_mb<BITS, XF32, 4>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
}

template <bool XF32>
hipError_t launch_x(const void* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                    const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, int bits,
                    void* y, hipStream_t stream) {
    switch (bits) {
        case 2: return launch_bits<2, XF32>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 3: return launch_bits<3, XF32>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 4: return launch_bits<4, XF32>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 5: return launch_bits<5, XF32>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 6: return launch_bits<6, XF32>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 8: return launch_bits<8, XF32>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemv(const void* x, bool x_f32, int64_t m, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                       int group_size, int bits, void* y, hipStream_t stream) {
    const int64_t kb = k / 32;
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    return x_f32 ? launch_x<true>(x, m, packed, scales, biases, n, kb, gshift, bits, y, stream)
                 : launch_x<false>(x, m, packed, scales, biases, n, kb, gshift, bits, y, stream);
}

}  // namespace qaff
