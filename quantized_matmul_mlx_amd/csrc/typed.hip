// Other float types for x, scales and biases (nuvec_core quantized.rs: `quantized_matmul` and
// `dequantize` promote x, scales and biases to one float type; scales keep the weight's dtype,
// float16, bfloat16 or float32). The bf16-scale paths have their own kernels; these take every
// other combination, with the types as run-time (block-uniform) switches:
//  * dequant_typed_kernel: w = s * c, then + b, in float32 with two roundings as written (with
//    float32 scales the product is not always exact, so no fused multiply-add), stored as
//    float32, bf16 or float16 (round to nearest even).
//  * gemv_typed_kernel: y = x . dequantize(W)^T on the VALU, float32 sums, x of any of the three
//    types, y in the promoted type. Per block of 32 codes: s * sum(x c) + b * sum(x). Gathered
//    (nuvec_core quantized.rs, `gather_qmm`): grid z is the output batch, x batch lhs[z] against
//    weight batch rhs[z]; an index past its operand gives a NaN batch. Grouped (sorted rhs, one
//    row per batch, no lhs): grid z is the expert e, whose rows [#(rhs < e), #(rhs < e + 1)) the
//    block walks in tiles of MB, reading e's weights once for all of them; expert w_count takes
//    the rows past every expert (NaN).
#include "launch.h"
#include "qaff_device.h"

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

namespace qaff {
namespace {

constexpr int kTypedThreads = 256;

// One thread per 32-code block of the output, stored element by element (so `out` needs only its
// element size of alignment). With `indices`, output row r is table row indices[r], and an index
// at or past table_rows gives a row of quiet NaNs.
template <int BITS>
__global__ __launch_bounds__(kTypedThreads) void dequant_typed_kernel(
    const uint32_t* packed, const void* scales, const void* biases, int st, uint64_t blocks, uint32_t kb,
    uint32_t gshift, void* out, int ot, const uint32_t* indices, uint32_t table_rows) {
    // two roundings, product then sum: the compiler must not fuse them (device code contracts by
    // default, and __fmul_rn / __fadd_rn are plain operators)
#pragma clang fp contract(off)
    const uint64_t idx = (uint64_t)blockIdx.x * kTypedThreads + threadIdx.x;
    if (idx >= blocks) return;
    const uint64_t orow = idx / kb;
    const uint32_t j = (uint32_t)(idx - orow * kb);
    const uint64_t row = indices ? (uint64_t)indices[orow] : orow;
    if (indices && row >= table_rows) {
#pragma unroll
        for (int c = 0; c < 32; ++c) store_from_f32(out, idx * 32 + c, ot, __uint_as_float(0x7fc00000u));
        return;
    }
    uint32_t w[BITS];
    load_block<BITS>(packed + (row * kb + j) * BITS, w);
    const size_t gi = row * (kb >> gshift) + (j >> gshift);
    const float s = load_as_f32(scales, gi, st);
    const float b = load_as_f32(biases, gi, st);
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        const float prod = s * (float)code_at<BITS>(w, c);
        store_from_f32(out, idx * 32 + c, ot, prod + b);
    }
}

// A wave owns kTypedRows rows of W; lanes take the row's 32-code blocks l, l + 64, ... (x needs
// 16-byte alignment: the ABI checks it, and a block of 32 values keeps it)
constexpr int kTypedRows = 2;

template <int BITS, int MB>
__global__ __launch_bounds__(kTypedThreads) void gemv_typed_kernel(
    const void* x, int xt, uint32_t m, const uint32_t* packed, const void* scales, const void* biases, int st,
    uint32_t n, uint32_t kb, uint32_t gshift, void* y, int yt, Gather ga, int gathered) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint32_t n0 = (blockIdx.x * (kTypedThreads / 64) + wave) * kTypedRows;
    if (n0 >= n) return;  // wave-uniform; no block-level barrier
    const uint32_t k = kb * 32;
    const uint32_t gpr = kb >> gshift;
    // x rows [t0, t1) in tiles of MB from t0, rows below m: one tile (grid y), or an expert's rows
    uint32_t t0 = blockIdx.y * MB, t1 = t0 + 1;
    if (gathered && ga.grouped) {
        const uint32_t e = ga.b0 + blockIdx.z;
        uint32_t r0, r1;
        count_below2(ga.rhs, ga.batch, e, e + 1, lane, r0, r1);
        if (e >= ga.w_count) {  // rows past every expert
            for (uint32_t o = lane; o < (ga.batch - r0) * kTypedRows; o += 64) {
                const uint32_t row = n0 + o % kTypedRows, i = r0 + o / kTypedRows;
                if (row < n) store_from_f32(y, (size_t)i * n + row, yt, __builtin_nanf(""));
            }
            return;
        }
        if (r0 >= r1) return;
        packed += (size_t)e * ga.w_stride;
        const size_t sb = (size_t)e * ga.sb_stride * (st == 0 ? 4 : 2);
        scales = static_cast<const uint8_t*>(scales) + sb;
        biases = static_cast<const uint8_t*>(biases) + sb;
        t0 = r0;
        t1 = r1;
        m = r1;  // the expert's last row bounds the tiles
    } else if (gathered) {
        const uint32_t m0 = t0;
        // this output batch's x, weight and y (element sizes: 4 for float32, else 2)
        const uint32_t z = ga.b0 + blockIdx.z;
        const uint32_t li = ga.lhs ? ga.lhs[z] : z;
        const uint32_t ri = ga.rhs ? ga.rhs[z] : z;
        y = static_cast<uint8_t*>(y) + (size_t)z * ga.y_stride * (yt == 0 ? 4 : 2);
        if (li >= ga.x_count || ri >= ga.w_count) {
            if (lane < kTypedRows * MB) {
                const uint32_t row = n0 + (uint32_t)lane / MB, i = m0 + (uint32_t)lane % MB;
                if (row < n && i < m) store_from_f32(y, (size_t)i * n + row, yt, __builtin_nanf(""));
            }
            return;
        }
        x = static_cast<const uint8_t*>(x) + (size_t)li * ga.x_stride * (xt == 0 ? 4 : 2);
        packed += (size_t)ri * ga.w_stride;
        const size_t sb = (size_t)ri * ga.sb_stride * (st == 0 ? 4 : 2);
        scales = static_cast<const uint8_t*>(scales) + sb;
        biases = static_cast<const uint8_t*>(biases) + sb;
    }

    for (uint32_t m0 = t0; m0 < t1; m0 += MB) {
    float acc[kTypedRows][MB];
#pragma unroll
    for (int r = 0; r < kTypedRows; ++r)
#pragma unroll
        for (int i = 0; i < MB; ++i) acc[r][i] = 0.f;

    for (uint32_t j = lane; j < kb; j += 64) {
        float xv[MB][32];
        float xs[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const uint32_t xr = min(m0 + i, m - 1);
            const size_t o = (size_t)xr * k + (size_t)j * 32;  // the block's 32 x values, 16-byte loads
            if (xt == 0) {
                const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + o);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const f32x4 v = p[q];
                    xv[i][4 * q] = v.x; xv[i][4 * q + 1] = v.y; xv[i][4 * q + 2] = v.z; xv[i][4 * q + 3] = v.w;
                }
            } else {
                const u32x4a* p = reinterpret_cast<const u32x4a*>(static_cast<const uint16_t*>(x) + o);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x4a v = p[q];
                    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (xt == 1) {
                            xv[i][8 * q + 2 * e] = __uint_as_float(u[e] << 16);
                            xv[i][8 * q + 2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
                        } else {
                            xv[i][8 * q + 2 * e] = __half2float(__ushort_as_half((uint16_t)(u[e] & 0xffffu)));
                            xv[i][8 * q + 2 * e + 1] = __half2float(__ushort_as_half((uint16_t)(u[e] >> 16)));
                        }
                    }
                }
            }
            float t = 0.f;
#pragma unroll
            for (int c = 0; c < 32; ++c) {
                if (m0 + i >= m) xv[i][c] = 0.f;
                t += xv[i][c];
            }
            xs[i] = t;
        }
#pragma unroll
        for (int r = 0; r < kTypedRows; ++r) {
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
    for (int r = 0; r < kTypedRows; ++r) {
        const uint32_t row = n0 + r;
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const float v = wave_sum(acc[r][i]);
            if (lane == 0 && row < n && m0 + i < m) store_from_f32(y, (size_t)(m0 + i) * n + row, yt, v);
        }
    }
    }
}

template <int BITS>
hipError_t launch_dequant_bits(const uint32_t* packed, const void* scales, const void* biases, int st, int64_t rows,
                               int64_t kb, uint32_t gshift, void* out, int ot, const uint32_t* indices,
                               int64_t table_rows, hipStream_t stream) {
    const uint64_t blocks = (uint64_t)rows * (uint64_t)kb;
    const unsigned grid = (unsigned)((blocks + kTypedThreads - 1) / kTypedThreads);
    dequant_typed_kernel<BITS><<<grid, kTypedThreads, 0, stream>>>(packed, scales, biases, st, blocks, (uint32_t)kb,
                                                                   gshift, out, ot, indices, (uint32_t)table_rows);
    return hipGetLastError();
}

// Grid: x = row groups of W, y = x rows in tiles of MB (at most 65535 per launch), z = output
// batches when gathered (at most 65535 per launch).
template <int BITS, int MB>
hipError_t launch_gemv_mb(const void* x, int xt, int64_t m, const uint32_t* packed, const void* scales,
                          const void* biases, int st, int64_t n, int64_t kb, uint32_t gshift, void* y, int yt,
                          const Gather* ga, hipStream_t stream) {
    const unsigned gx = (unsigned)((n + (kTypedThreads / 64) * kTypedRows - 1) / ((kTypedThreads / 64) * kTypedRows));
    const size_t xsize = xt == 0 ? 4 : 2, ysize = yt == 0 ? 4 : 2;
    const int64_t max_rows = (int64_t)65535 * MB;
    // grid z: output batches, or experts 0 .. w_count when grouped (then one grid row walks all x rows)
    const int64_t batches = ga ? (ga->grouped ? (int64_t)ga->w_count + 1 : ga->batch) : 1;
    if (ga && ga->grouped) m = 1;
    for (int64_t b0 = 0; b0 < batches; b0 += 65535) {
        Gather g = ga ? *ga : Gather{};
        g.b0 = (uint32_t)b0;
        const unsigned gz = (unsigned)(batches - b0 < 65535 ? batches - b0 : 65535);
        for (int64_t m0 = 0; m0 < m; m0 += max_rows) {
            const int64_t mm = m - m0 < max_rows ? m - m0 : max_rows;
            const unsigned gy = (unsigned)((mm + MB - 1) / MB);
            gemv_typed_kernel<BITS, MB><<<dim3(gx, gy, gz), kTypedThreads, 0, stream>>>(
                static_cast<const uint8_t*>(x) + (size_t)m0 * kb * 32 * xsize, xt, (uint32_t)mm, packed, scales, biases,
                st, (uint32_t)n, (uint32_t)kb, gshift, static_cast<uint8_t*>(y) + (size_t)m0 * n * ysize, yt, g,
                ga ? 1 : 0);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

// x rows per block: 1 for a single row, else 4 (also for the grouped walk over an expert's rows)
template <int BITS>
hipError_t launch_gemv_bits(const void* x, int xt, int64_t m, const uint32_t* packed, const void* scales,
                            const void* biases, int st, int64_t n, int64_t kb, uint32_t gshift, void* y, int yt,
                            const Gather* ga, hipStream_t stream) {
    if (m == 1 && !(ga && ga->grouped)) return launch_gemv_mb<BITS, 1>(x, xt, m, packed, scales, biases, st, n, kb, gshift, y, yt, ga, stream);
    return launch_gemv_mb<BITS, 4>(x, xt, m, packed, scales, biases, st, n, kb, gshift, y, yt, ga, stream);
}

}  // namespace

hipError_t launch_dequant_typed(const uint32_t* packed, const void* scales, const void* biases, int sb_dtype,
                                int64_t rows, int64_t cols, int group_size, int bits, void* out, int out_dtype,
                                hipStream_t stream, const uint32_t* indices, int64_t table_rows) {
    const int64_t kb = cols / 32;
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    switch (bits) {
        case 1: return launch_dequant_bits<1>(packed, scales, biases, sb_dtype, rows, kb, gshift, out, out_dtype, indices, table_rows, stream);
        case 2: return launch_dequant_bits<2>(packed, scales, biases, sb_dtype, rows, kb, gshift, out, out_dtype, indices, table_rows, stream);
        case 3: return launch_dequant_bits<3>(packed, scales, biases, sb_dtype, rows, kb, gshift, out, out_dtype, indices, table_rows, stream);
        case 4: return launch_dequant_bits<4>(packed, scales, biases, sb_dtype, rows, kb, gshift, out, out_dtype, indices, table_rows, stream);
        case 5: return launch_dequant_bits<5>(packed, scales, biases, sb_dtype, rows, kb, gshift, out, out_dtype, indices, table_rows, stream);
        case 6: return launch_dequant_bits<6>(packed, scales, biases, sb_dtype, rows, kb, gshift, out, out_dtype, indices, table_rows, stream);
        case 8: return launch_dequant_bits<8>(packed, scales, biases, sb_dtype, rows, kb, gshift, out, out_dtype, indices, table_rows, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_typed(const void* x, int x_dtype, int64_t m, const uint32_t* packed, const void* scales,
                             const void* biases, int sb_dtype, int64_t n, int64_t k, int group_size, int bits, void* y,
                             int y_dtype, hipStream_t stream, const Gather* gather) {
    const int64_t kb = k / 32;
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    switch (bits) {
        case 1: return launch_gemv_bits<1>(x, x_dtype, m, packed, scales, biases, sb_dtype, n, kb, gshift, y, y_dtype, gather, stream);
        case 2: return launch_gemv_bits<2>(x, x_dtype, m, packed, scales, biases, sb_dtype, n, kb, gshift, y, y_dtype, gather, stream);
        case 3: return launch_gemv_bits<3>(x, x_dtype, m, packed, scales, biases, sb_dtype, n, kb, gshift, y, y_dtype, gather, stream);
        case 4: return launch_gemv_bits<4>(x, x_dtype, m, packed, scales, biases, sb_dtype, n, kb, gshift, y, y_dtype, gather, stream);
        case 5: return launch_gemv_bits<5>(x, x_dtype, m, packed, scales, biases, sb_dtype, n, kb, gshift, y, y_dtype, gather, stream);
        case 6: return launch_gemv_bits<6>(x, x_dtype, m, packed, scales, biases, sb_dtype, n, kb, gshift, y, y_dtype, gather, stream);
        case 8: return launch_gemv_bits<8>(x, x_dtype, m, packed, scales, biases, sb_dtype, n, kb, gshift, y, y_dtype, gather, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qaff
