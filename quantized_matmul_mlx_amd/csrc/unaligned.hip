// The element-by-element GEMV behind operands that are not 16-byte aligned (a row slice of a
// larger tensor, an odd offset into a buffer): every operand is loaded and stored one element at a
// time, so each needs only its element size of alignment. It serves the products whose fast
// kernels move x and y in 16-byte units: qmm (nuvec_core quantized.rs, `quantized_matmul` with
// transpose; maya2_mlx `mm`), the fused decode products (spark_runtime weights/mlx_int8.rs,
// `gemv_gate_up`, `gemv_silu_gate`, `gemv_silu_gate_resid`), the gathered products (nuvec_core
// `gather_qmm`) and the other float types. The same float32 arithmetic as the fast kernels, in
// another summation order: per 32-code block, s * sum(x c) + b * sum(x).
//  * A block of 4 waves owns 8 rows of W (2 per wave); lanes take the row's 32-code blocks
//    l, l + 64, ...; grid y walks x in tiles of MB rows, grid z the gathered batches.
//  * With `up`, x is the gate and the input is h = bf16(silu(gate) * up), formed in float32.
//  * With `resid`, y = bf16(sum + resid).
#include "launch.h"
#include "qaff_device.h"

#include <hip/hip_runtime.h>

namespace qaff {
namespace {

constexpr int kScalarThreads = 256;
constexpr int kScalarRows = 2;  // W rows per wave

template <int BITS, int MB>
__global__ __launch_bounds__(kScalarThreads) void gemv_scalar_kernel(
    const void* x, int xt, uint32_t m, const uint32_t* packed, const void* scales, const void* biases, int st,
    uint32_t n, uint32_t kb, uint32_t gshift, void* y, int yt, const uint16_t* up, const uint16_t* resid,
    Gather ga, int gather) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint32_t n0 = (blockIdx.x * (kScalarThreads / 64) + wave) * kScalarRows;
    const uint32_t m0 = blockIdx.y * MB;
    const uint32_t k = kb * 32;
    const uint32_t gpr = kb >> gshift;
    const size_t xsz = xt == 0 ? 4 : 2, ysz = yt == 0 ? 4 : 2;
    if (gather) {  // block-uniform
        const uint32_t b = ga.b0 + blockIdx.z;
        const uint32_t li = ga.lhs ? ga.lhs[b] : b;
        const uint32_t ri = ga.rhs ? ga.rhs[b] : b;
        y = static_cast<uint8_t*>(y) + (size_t)b * ga.y_stride * ysz;
        if (li >= ga.x_count || ri >= ga.w_count) {
            if (lane < kScalarRows * MB) {
                const uint32_t row = n0 + lane % kScalarRows, i = m0 + lane / kScalarRows;
                if (row < n && i < m) store_from_f32(y, (size_t)i * n + row, yt, __uint_as_float(0x7fc00000u));
            }
            return;
        }
        x = static_cast<const uint8_t*>(x) + (size_t)li * ga.x_stride * xsz;
        packed += (size_t)ri * ga.w_stride;
        scales = static_cast<const uint8_t*>(scales) + (size_t)ri * ga.sb_stride * (st == 0 ? 4 : 2);
        biases = static_cast<const uint8_t*>(biases) + (size_t)ri * ga.sb_stride * (st == 0 ? 4 : 2);
    }
    if (n0 >= n) return;  // wave-uniform; no barrier follows

    float acc[kScalarRows][MB];
#pragma unroll
    for (int r = 0; r < kScalarRows; ++r)
#pragma unroll
        for (int i = 0; i < MB; ++i) acc[r][i] = 0.f;

    for (uint32_t j = lane; j < kb; j += 64) {
        float xv[MB][32];
        float xs[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const uint32_t xr = min(m0 + i, m - 1);
            const size_t o = (size_t)xr * k + (size_t)j * 32;
            float t = 0.f;
#pragma unroll
            for (int c = 0; c < 32; ++c) {
                float v = load_as_f32(x, o + c, xt);
                if (up) v = bf16_to_f32(to_bf16_bits(silu_f32(v) * bf16_to_f32(up[o + c])));
                xv[i][c] = m0 + i < m ? v : 0.f;
                t += xv[i][c];
            }
            xs[i] = t;
        }
#pragma unroll
        for (int r = 0; r < kScalarRows; ++r) {
            const uint32_t row = n0 + r;
            if (row >= n) break;
            uint32_t w[BITS];
            load_block<BITS>(packed + ((size_t)row * kb + j) * BITS, w);
            const size_t gi = (size_t)row * gpr + (j >> gshift);
            const float s = load_as_f32(scales, gi, st);
            const float b = load_as_f32(biases, gi, st);
            float cf[32];
#pragma unroll
            for (int c = 0; c < 32; ++c) cf[c] = (float)code_at<BITS>(w, c);
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                float d = 0.f;
#pragma unroll
                for (int c = 0; c < 32; ++c) d = __builtin_fmaf(xv[i][c], cf[c], d);
                acc[r][i] = __builtin_fmaf(s, d, __builtin_fmaf(b, xs[i], acc[r][i]));
            }
        }
    }

#pragma unroll
    for (int r = 0; r < kScalarRows; ++r) {
        const uint32_t row = n0 + r;
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            float v = wave_sum(acc[r][i]);
            if (lane == 0 && row < n && m0 + i < m) {
                const size_t o = (size_t)(m0 + i) * n + row;
                if (resid) v += bf16_to_f32(resid[o]);
                store_from_f32(y, o, yt, v);
            }
        }
    }
}

template <int BITS, int MB>
hipError_t launch_mb(const void* x, int xt, int64_t m, const uint32_t* packed, const void* scales,
                     const void* biases, int st, int64_t n, int64_t kb, uint32_t gshift, void* y, int yt,
                     const ScalarGemv& opt, hipStream_t stream) {
    const unsigned gx = (unsigned)((n + (kScalarThreads / 64) * kScalarRows - 1) / ((kScalarThreads / 64) * kScalarRows));
    const size_t xsz = xt == 0 ? 4 : 2, ysz = yt == 0 ? 4 : 2;
    const int64_t batches = opt.gather ? (int64_t)opt.g.batch : 1;
    const int64_t max_rows = (int64_t)65535 * MB;
    for (int64_t b0 = 0; b0 < batches; b0 += 65535) {
        const int64_t nb = batches - b0 < 65535 ? batches - b0 : 65535;
        Gather g = opt.g;
        g.b0 = (uint32_t)b0;
        for (int64_t m0 = 0; m0 < m; m0 += max_rows) {
            const int64_t mm = m - m0 < max_rows ? m - m0 : max_rows;
            const unsigned gy = (unsigned)((mm + MB - 1) / MB);
            // a slice of x rows: the gathered batches keep their strides, their row offset moves
            const uint8_t* xs = static_cast<const uint8_t*>(x) + (size_t)m0 * kb * 32 * xsz;
            uint8_t* ys = static_cast<uint8_t*>(y) + (size_t)m0 * n * ysz;
            gemv_scalar_kernel<BITS, MB><<<dim3(gx, gy, (unsigned)nb), kScalarThreads, 0, stream>>>(
                xs, xt, (uint32_t)mm, packed, scales, biases, st, (uint32_t)n, (uint32_t)kb, gshift, ys, yt,
                opt.up ? opt.up + (size_t)m0 * kb * 32 : nullptr, opt.resid ? opt.resid + (size_t)m0 * n : nullptr, g,
                opt.gather ? 1 : 0);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

template <int BITS>
hipError_t launch_bits(const void* x, int xt, int64_t m, const uint32_t* packed, const void* scales,
                       const void* biases, int st, int64_t n, int64_t kb, uint32_t gshift, void* y, int yt,
                       const ScalarGemv& opt, hipStream_t stream) {
    if (m == 1) return launch_mb<BITS, 1>(x, xt, m, packed, scales, biases, st, n, kb, gshift, y, yt, opt, stream);
    return launch_mb<BITS, 4>(x, xt, m, packed, scales, biases, st, n, kb, gshift, y, yt, opt, stream);
}

}  // namespace

hipError_t launch_gemv_scalar(const void* x, int x_dtype, int64_t m, const uint32_t* packed, const void* scales,
                              const void* biases, int sb_dtype, int64_t n, int64_t k, int group_size, int bits,
                              void* y, int y_dtype, const ScalarGemv& opt, hipStream_t stream) {
    const int64_t kb = k / 32;
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    switch (bits) {
        case 1: return launch_bits<1>(x, x_dtype, m, packed, scales, biases, sb_dtype, n, kb, gshift, y, y_dtype, opt, stream);
        case 2: return launch_bits<2>(x, x_dtype, m, packed, scales, biases, sb_dtype, n, kb, gshift, y, y_dtype, opt, stream);
        case 3: return launch_bits<3>(x, x_dtype, m, packed, scales, biases, sb_dtype, n, kb, gshift, y, y_dtype, opt, stream);
        case 4: return launch_bits<4>(x, x_dtype, m, packed, scales, biases, sb_dtype, n, kb, gshift, y, y_dtype, opt, stream);
        case 5: return launch_bits<5>(x, x_dtype, m, packed, scales, biases, sb_dtype, n, kb, gshift, y, y_dtype, opt, stream);
        case 6: return launch_bits<6>(x, x_dtype, m, packed, scales, biases, sb_dtype, n, kb, gshift, y, y_dtype, opt, stream);
        case 8: return launch_bits<8>(x, x_dtype, m, packed, scales, biases, sb_dtype, n, kb, gshift, y, y_dtype, opt, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qaff
