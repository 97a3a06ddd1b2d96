// Dense and gathered-row dequantization, w = scale * code + bias (rlx-moshi mlx_dequant.rs,
// dequantize_affine; spark_runtime weights/mlx_int8.rs, module formula and dequantize_to;
// maya2_mlx quant.py, rows).
//
// HBM-bound and write-dominated: a 4-bit weight reads 0.5 B of codes and writes 4 B (float32) or
// 2 B (bf16), so the stores decide the speed. Each lane produces 16 bytes of consecutive outputs
// at a time (a "unit": 4 float32, or 8 bf16 for codes up to 4 bits, else 4), and the lanes of a
// wave take consecutive units, so that every store instruction writes one contiguous run. A
// unit's codes are consecutive bits of the row: one funnel shift of the two words they lie in. Its
// scale and bias are those of its group; the lanes of a group read the same two values.
// Blocks map to (row segment, row), so a lane finds its row and column without a division;
// one block covers 256 * kUnits units of one row. The gathered form reads the source row index
// once per block (a scalar load) and writes quiet NaNs for an index past the table.
#include "launch.h"
#include "qaff_device.h"

#include <hip/hip_runtime.h>

namespace qaff {
namespace {

constexpr int kThreads = 256;
constexpr int kUnits = 4;  // units per lane: all their loads are issued before any store

// Codes per unit: 4 (16 bytes of float32), or 8 for bf16 outputs of codes up to 4 bits (16 bytes
// of bf16, still one funnel shift of two words).
template <int BITS, bool OUT_BF16>
constexpr int kUnitCodes = (OUT_BF16 && BITS <= 4) ? 8 : 4;

// The pointers are deliberately not __restrict__: with it, the compiler moves each unit's loads
// down to its store, one unit at a time, past the empty asm that keeps them together.
template <int BITS, bool OUT_BF16, bool GATHER>
__global__ __launch_bounds__(kThreads) void dequant_kernel(
    const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
    const uint32_t* indices, uint32_t table_rows, uint32_t kb, uint32_t gshift, void* out) {
    constexpr int UC = kUnitCodes<BITS, OUT_BF16>;
    constexpr int LUC = UC == 8 ? 3 : 2;
    const uint32_t r = blockIdx.y;
    const uint32_t upr = kb * (32 / UC);  // units per row
    const uint32_t wpr = kb * BITS;    // packed words per row
    const uint32_t gpr = kb >> gshift;  // groups per row
    uint32_t src = r;
    bool ok = true;
    if constexpr (GATHER) {
        src = indices[r];  // uniform: a scalar load
        ok = src < table_rows;
        if (!ok) src = 0;  // read a valid row; the outputs are NaN
    }
    const uint32_t* prow = packed + (size_t)src * wpr;
    const uint16_t* srow = scales + (size_t)src * gpr;
    const uint16_t* brow = biases + (size_t)src * gpr;
    const uint32_t u0 = blockIdx.x * (kThreads * kUnits) + threadIdx.x;

    uint32_t w0[kUnits], w1[kUnits], sh[kUnits];
    uint16_t sv[kUnits], bv[kUnits];
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
        const uint32_t p = min(u0 + i * kThreads, upr - 1);  // clamped: loads stay in the row
        const uint32_t bit = p * UC * BITS;
        const uint32_t wi = bit >> 5;
        sh[i] = bit & 31;
        w0[i] = prow[wi];
        w1[i] = prow[min(wi + 1, wpr - 1)];  // only read when the unit straddles two words
        const uint32_t g = p >> (5 + gshift - LUC);
        sv[i] = srow[g];
        bv[i] = brow[g];
    }
    asm volatile("" ::: "memory");  // every load of the lane before its first store
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
        const uint32_t p = u0 + i * kThreads;
        const uint32_t v = __builtin_amdgcn_alignbit(w1[i], w0[i], sh[i]);
        const float s = bf16_to_f32(sv[i]);
        const float b = bf16_to_f32(bv[i]);
        float o[UC];
#pragma unroll
        for (int c = 0; c < UC; ++c) {
            // s * code is exact in float32, so the fused form rounds once, like s * c then + b
            o[c] = ok ? __builtin_fmaf(s, (float)((v >> (c * BITS)) & ((1u << BITS) - 1u)), b)
                      : __uint_as_float(0x7fc00000u);
        }
        const size_t e = (size_t)r * upr * UC + (size_t)p * UC;
        // non-temporal stores: the output streams past the caches (measured at [4096, 4096] 4-bit:
        // float32 17.3 -> 12.3 us, bf16 10.3 -> 7.3 us)
        if (p < upr) {
            if constexpr (OUT_BF16 && UC == 8) {
                __builtin_nontemporal_store(u32x4a{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])},
                                            reinterpret_cast<u32x4a*>(static_cast<uint16_t*>(out) + e));
            } else if constexpr (OUT_BF16) {
                __builtin_nontemporal_store(u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])},
                                            reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + e));
            } else {
                __builtin_nontemporal_store(f32x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<f32x4*>(static_cast<float*>(out) + e));
            }
        }
    }
}

template <int BITS, bool OUT_BF16, bool GATHER>
hipError_t launch_one(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                      const uint32_t* indices, int64_t table_rows, int64_t out_rows, int64_t kb,
                      uint32_t gshift, void* out, hipStream_t stream) {
    const int64_t upr = kb * (32 / kUnitCodes<BITS, OUT_BF16>);
    const unsigned gx = (unsigned)((upr + kThreads * kUnits - 1) / (kThreads * kUnits));
    const size_t osize = OUT_BF16 ? 2 : 4;
    // grid.y is limited to 65535 rows per launch
    for (int64_t r0 = 0; r0 < out_rows; r0 += 65535) {
        const int64_t rows = out_rows - r0 < 65535 ? out_rows - r0 : 65535;
        const uint32_t* pk = GATHER ? packed : packed + (size_t)r0 * kb * BITS;
        const uint16_t* sc = GATHER ? scales : scales + (size_t)r0 * (kb >> gshift);
        const uint16_t* bi = GATHER ? biases : biases + (size_t)r0 * (kb >> gshift);
        const uint32_t* ix = GATHER ? indices + r0 : nullptr;
        void* o = static_cast<char*>(out) + (size_t)r0 * kb * 32 * osize;
        dequant_kernel<BITS, OUT_BF16, GATHER><<<dim3(gx, (unsigned)rows), dim3(kThreads), 0, stream>>>(
            pk, sc, bi, ix, (uint32_t)table_rows, (uint32_t)kb, gshift, o);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
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
        case 1: return dispatch_out<1>(packed, scales, biases, indices, table_rows, out_rows, kb, gshift, out, out_bf16, stream);
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
