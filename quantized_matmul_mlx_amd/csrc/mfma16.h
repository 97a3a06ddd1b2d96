// The two 16-bit formats of the matrix-core kernels: bf16 (F16 = false) and float16 (F16 = true).
// x, the scales and biases and y are all in the format (nuvec_core quantized.rs promotes x, scales
// and biases to one float type); each weight enters the multiply as a 16-bit operand of the same
// format, either dequantized and rounded to it or as an exact code. Products and sums are float32
// in both formats, and both have a 16x16x32 and a 32x32x16 matrix instruction on gfx950.
#pragma once

#include "qaff_device.h"

namespace qaff {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <bool F16> struct Op8 { typedef bf16x8 type; };
template <> struct Op8<true> { typedef f16x8 type; };
// Eight 16-bit operand values (one lane's share of an MFMA operand).
template <bool F16> using op8 = typename Op8<F16>::type;

// The 16-bit value in the low half of h, widened to float32 (exactly).
template <bool F16>
__device__ __forceinline__ float half_to_f32(uint32_t h) {
    if constexpr (F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    else return __uint_as_float(h << 16);
}

// float32 -> the format's bits, round to nearest even.
template <bool F16>
__device__ __forceinline__ uint16_t f32_to_half_bits(float v) {
    if constexpr (F16) return __builtin_bit_cast(uint16_t, (_Float16)v);
    else return to_bf16_bits(v);
}

// Two float32 -> two 16-bit values in one dword (lo in bits 0..15), round to nearest even: one
// v_cvt_pk_bf16_f32 or v_cvt_pk_f16_f32.
template <bool F16>
__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
    if constexpr (F16) return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
    else return pack_bf16x2(lo, hi);
}

template <bool F16>
__device__ __forceinline__ f32x4 mfma16x16x32(op8<F16> a, op8<F16> b, f32x4 c) {
    if constexpr (F16) return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <bool F16>
__device__ __forceinline__ f32x16 mfma32x32x16(op8<F16> a, op8<F16> b, f32x16 c) {
    if constexpr (F16) return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Codes 8 j .. 8 j + 7 of a 32-code block as MFMA operands of the format: dequant8m's values (its
// float32 arithmetic, see there) rounded to bf16 or to float16.
template <bool F16, int BITS>
__device__ __forceinline__ op8<F16> dequant_op(const uint32_t (&w)[BITS], int j, const Dq& p) {
    if constexpr (!F16) {
        return dequant8m<BITS>(w, j, p);
    } else if constexpr (BITS == 4) {
        constexpr uint32_t kOne = 0x64006400u;  // float16 1024.0 in both halves
        const uint32_t v = w[j];
        const uint32_t v8 = v >> 8;
        const f16x2 h0 = __builtin_bit_cast(f16x2, and_or(v, 0x000F000Fu, kOne));   // codes 0, 4
        const f16x2 h1 = __builtin_bit_cast(f16x2, and_or(v, 0x00F000F0u, kOne));   // 16 x codes 1, 5
        const f16x2 h2 = __builtin_bit_cast(f16x2, and_or(v8, 0x000F000Fu, kOne));  // codes 2, 6
        const f16x2 h3 = __builtin_bit_cast(f16x2, and_or(v8, 0x00F000F0u, kOne));  // 16 x codes 3, 7
        const float c0 = __builtin_fmaf(p.s, (float)h0.x, p.b1024), c4 = __builtin_fmaf(p.s, (float)h0.y, p.b1024);
        const float c1 = __builtin_fmaf(p.s16, (float)h1.x, p.b64), c5 = __builtin_fmaf(p.s16, (float)h1.y, p.b64);
        const float c2 = __builtin_fmaf(p.s, (float)h2.x, p.b1024), c6 = __builtin_fmaf(p.s, (float)h2.y, p.b1024);
        const float c3 = __builtin_fmaf(p.s16, (float)h3.x, p.b64), c7 = __builtin_fmaf(p.s16, (float)h3.y, p.b64);
        return __builtin_bit_cast(f16x8, u32x4a{pack_half2<true>(c0, c1), pack_half2<true>(c2, c3),
                                                pack_half2<true>(c4, c5), pack_half2<true>(c6, c7)});
    } else if constexpr (BITS == 8) {
        constexpr uint32_t kOne = 0x64006400u;
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t v = w[2 * j + q];
            const f16x2 ha = __builtin_bit_cast(f16x2, and_or(v, 0x00FF00FFu, kOne));       // bytes 0, 2
            const f16x2 hb = __builtin_bit_cast(f16x2, and_or(v >> 8, 0x00FF00FFu, kOne));  // bytes 1, 3
            o[2 * q] = pack_half2<true>(__builtin_fmaf(p.s, (float)ha.x, p.b1024), __builtin_fmaf(p.s, (float)hb.x, p.b1024));
            o[2 * q + 1] = pack_half2<true>(__builtin_fmaf(p.s, (float)ha.y, p.b1024), __builtin_fmaf(p.s, (float)hb.y, p.b1024));
        }
        return __builtin_bit_cast(f16x8, u32x4a{o[0], o[1], o[2], o[3]});
    } else {
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = pack_half2<true>(__builtin_fmaf(p.s, (float)code_at<BITS>(w, 8 * j + 2 * e), p.b),
                                    __builtin_fmaf(p.s, (float)code_at<BITS>(w, 8 * j + 2 * e + 1), p.b));
        return __builtin_bit_cast(f16x8, u32x4a{o[0], o[1], o[2], o[3]});
    }
}

}  // namespace qaff
