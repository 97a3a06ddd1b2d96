// Device helpers for the qaff kernels (gfx950 only): bf16 conversions, whole-block loads of packed
// words, and code extraction from a row's little-endian bit stream.
//
// A "block" is 32 consecutive codes of one row. At any bit width b, 32 codes are exactly b words,
// so a block always starts on a word boundary and never shares a word with another block. Every
// group size (32, 64, 128) is a whole number of blocks, so a block has exactly one scale and one
// bias. The kernels all work block by block.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qaff {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4a __attribute__((ext_vector_type(4)));        // 16-byte aligned
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// bf16 bit pattern -> float32: the upper half of the float32 pattern (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two float32 -> two bf16 in one dword (lo in bits 0..15), round to nearest even: one
// v_cvt_pk_bf16_f32 (two scalar conversions would each be a separate instruction plus a merge).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ __forceinline__ uint16_t to_bf16_bits(float v) {
    const __bf16 a = (__bf16)v;
    return __builtin_bit_cast(uint16_t, a);
}

// Loads the BITS words of one block. The pointer only needs 4-byte alignment: gfx950 global loads
// of 2-4 dwords accept any dword-aligned address.
template <int BITS>
__device__ __forceinline__ void load_block(const uint32_t* __restrict__ p, uint32_t (&w)[BITS]) {
    if constexpr (BITS == 1) {
        w[0] = p[0];
    } else if constexpr (BITS == 2) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(p);
        w[0] = v.x; w[1] = v.y;
    } else if constexpr (BITS == 3) {
        const u32x3 v = *reinterpret_cast<const u32x3*>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z;
    } else if constexpr (BITS == 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (BITS == 5) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w; w[4] = p[4];
    } else if constexpr (BITS == 6) {
        const u32x3 v = *reinterpret_cast<const u32x3*>(p);
        const u32x3 u = *reinterpret_cast<const u32x3*>(p + 3);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = u.x; w[4] = u.y; w[5] = u.z;
    } else {
        static_assert(BITS == 8, "bit width");
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
        const u32x4 u = *reinterpret_cast<const u32x4*>(p + 4);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        w[4] = u.x; w[5] = u.y; w[6] = u.z; w[7] = u.w;
    }
}

// Code j (0..31) of a block. j is a compile-time constant after unrolling, so this folds to one
// bit-field extract, or for a code that straddles words j*BITS/32 and the next, one funnel shift
// (v_alignbit_b32) and a mask.
template <int BITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[BITS], int j) {
    const int bit = j * BITS;
    const int wi = bit >> 5;
    const int sh = bit & 31;
    const uint32_t mask = (1u << BITS) - 1u;
    if (sh + BITS <= 32) return (w[wi] >> sh) & mask;
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & mask;
}

// Codes 8 j .. 8 j + 7 of a 32-code block, dequantized and rounded to bf16, in k order.
template <int BITS>
__device__ __forceinline__ bf16x8 dequant8(const uint32_t (&w)[BITS], int j, float s, float b) {
    uint32_t o[4];
    if constexpr (BITS == 4) {
        // even codes in the bytes of lo, odd codes in those of hi (the empty asm keeps the byte
        // converts from being turned into one bit-field extract per code)
        uint32_t lo = w[j] & 0x0f0f0f0fu;
        uint32_t hi = (w[j] >> 4) & 0x0f0f0f0fu;
        asm("" : "+v"(lo), "+v"(hi));
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = pack_bf16x2(__builtin_fmaf(s, (float)((lo >> (8 * e)) & 0xffu), b),
                               __builtin_fmaf(s, (float)((hi >> (8 * e)) & 0xffu), b));
    } else if constexpr (BITS == 8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t v = w[2 * j + h];
            o[2 * h] = pack_bf16x2(__builtin_fmaf(s, (float)(v & 0xffu), b), __builtin_fmaf(s, (float)((v >> 8) & 0xffu), b));
            o[2 * h + 1] = pack_bf16x2(__builtin_fmaf(s, (float)((v >> 16) & 0xffu), b), __builtin_fmaf(s, (float)(v >> 24), b));
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = pack_bf16x2(__builtin_fmaf(s, (float)code_at<BITS>(w, 8 * j + 2 * e), b),
                               __builtin_fmaf(s, (float)code_at<BITS>(w, 8 * j + 2 * e + 1), b));
    }
    return __builtin_bit_cast(bf16x8, u32x4a{o[0], o[1], o[2], o[3]});
}

// (a & mask) | orv in one v_and_or_b32 (the compiler otherwise emits an AND and an OR).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t orv) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(orv));
    return r;
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Per-group constants of dequant8m: the scale, the scale / 16, and the bias less 1024 and 64 scales.
struct Dq {
    float s, s16, b, b1024, b64;
};
__device__ __forceinline__ Dq make_dq(float s, float b) {
    return Dq{s, s * 0.0625f, b, __builtin_fmaf(-1024.0f, s, b), __builtin_fmaf(-64.0f, s, b)};
}

// Codes 8 j .. 8 j + 7 of a 32-code block as bf16 MFMA operands, like dequant8, for the GEMM and
// the matrix-core decode kernel. For 4- and 8-bit codes each code becomes a float16 value without a
// conversion: one AND-OR puts two codes (or two codes times 16) into the mantissas of
// 1024.0 (0x6400), and a mixed-precision fused multiply-add (v_fma_mix_f32, which widens the
// float16 half exactly) forms s (1024 + c) + (b - 1024 s) = s c + b, or (s / 16)(1024 + 16 c) +
// (b - 64 s). Wherever b - 1024 s (b - 64 s) is exact in float32 -- a scale and a bias within 2^15
// of each other in magnitude -- that is s c + b rounded once, exactly dequant8's value; otherwise it
// differs from it by at most one float32 rounding before the bf16 one. 4-bit: 17 instructions per
// 8 codes against 23.
template <int BITS>
__device__ __forceinline__ bf16x8 dequant8m(const uint32_t (&w)[BITS], int j, const Dq& p) {
    if constexpr (BITS == 4) {
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
        return __builtin_bit_cast(bf16x8, u32x4a{pack_bf16x2(c0, c1), pack_bf16x2(c2, c3), pack_bf16x2(c4, c5),
                                                 pack_bf16x2(c6, c7)});
    } else if constexpr (BITS == 8) {
        constexpr uint32_t kOne = 0x64006400u;
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t v = w[2 * j + q];
            const f16x2 ha = __builtin_bit_cast(f16x2, and_or(v, 0x00FF00FFu, kOne));       // bytes 0, 2
            const f16x2 hb = __builtin_bit_cast(f16x2, and_or(v >> 8, 0x00FF00FFu, kOne));  // bytes 1, 3
            o[2 * q] = pack_bf16x2(__builtin_fmaf(p.s, (float)ha.x, p.b1024), __builtin_fmaf(p.s, (float)hb.x, p.b1024));
            o[2 * q + 1] = pack_bf16x2(__builtin_fmaf(p.s, (float)ha.y, p.b1024), __builtin_fmaf(p.s, (float)hb.y, p.b1024));
        }
        return __builtin_bit_cast(bf16x8, u32x4a{o[0], o[1], o[2], o[3]});
    } else {
        return dequant8<BITS>(w, j, p.s, p.b);
    }
}

// Element i of an array of dtype code `dtype` (0 float32, 1 bf16, 2 float16), widened to float32
// (exactly), and the store of a float32 into such an array (round to nearest even). One element
// per access: the array needs only its element size of alignment.
__device__ __forceinline__ float load_as_f32(const void* p, size_t i, int dtype) {
    if (dtype == 1) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    if (dtype == 2) return __half2float(__ushort_as_half(static_cast<const uint16_t*>(p)[i]));
    return static_cast<const float*>(p)[i];
}

__device__ __forceinline__ void store_from_f32(void* p, size_t i, int dtype, float v) {
    if (dtype == 1) static_cast<uint16_t*>(p)[i] = to_bf16_bits(v);
    else if (dtype == 2) static_cast<uint16_t*>(p)[i] = __half_as_ushort(__float2half_rn(v));
    else static_cast<float*>(p)[i] = v;
}

// silu(v) = v / (1 + e^-v) from the hardware exp2 and reciprocal (a few ulp in float32).
__device__ __forceinline__ float silu_f32(float v) {
    const float e = __builtin_amdgcn_exp2f(-v * 1.4426950408889634f);  // exp(-v)
    return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// Full-wave sum of a float (64 lanes), result in every lane.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// #(idx[i] < v1) and #(idx[i] < v2) over a sorted idx[0 .. len), len >= 1.
//  * len <= 1024: every lane counts 16 consecutive entries (four 16-byte loads, one round trip);
//    the wave total of a count below 32 is the sum over its bits of the ballot popcounts.
//  * longer: a 64-ary search per bound, both in lockstep so that their loads go out together.
//    Each step probes lo + lane * step; the probes below v are a prefix (the array is sorted), and
//    the bound lies after the last one and no later than the next.
constexpr uint32_t kCountMax = 1024;

__device__ __forceinline__ uint32_t wave_total(uint32_t c) {  // 0 <= c < 32 in every lane
    uint32_t t = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b)
        t += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64((c >> b) & 1u)) << b;
    return t;
}

__device__ __forceinline__ void count_below2(const uint32_t* idx, uint32_t len, uint32_t v1, uint32_t v2,
                                             int lane, uint32_t& c1, uint32_t& c2) {
    if (len <= kCountMax) {
        uint32_t a[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t i0 = min((uint32_t)lane * 16 + 4 * q, len - 1);
            if (i0 + 4 <= len) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(idx + i0);
                a[4 * q] = v.x; a[4 * q + 1] = v.y; a[4 * q + 2] = v.z; a[4 * q + 3] = v.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) a[4 * q + e] = idx[min(i0 + e, len - 1)];
            }
        }
        uint32_t n1 = 0, n2 = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const bool in = (uint32_t)lane * 16 + e < len;
            n1 += (in && a[e] < v1) ? 1u : 0u;
            n2 += (in && a[e] < v2) ? 1u : 0u;
        }
        c1 = wave_total(n1);
        c2 = wave_total(n2);
        return;
    }
    uint32_t lo1 = 0, hi1 = len, lo2 = 0, hi2 = len;
    while (lo1 < hi1 || lo2 < hi2) {
        const uint32_t st1 = (hi1 - lo1 + 63) >> 6, st2 = (hi2 - lo2 + 63) >> 6;
        const uint32_t i1 = lo1 + (uint32_t)lane * st1, i2 = lo2 + (uint32_t)lane * st2;
        const uint32_t a1 = idx[min(i1, len - 1)];
        const uint32_t a2 = idx[min(i2, len - 1)];
        const uint32_t n1 = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(i1 < hi1 && a1 < v1));
        const uint32_t n2 = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(i2 < hi2 && a2 < v2));
        if (lo1 < hi1) {
            if (n1 == 0) {
                hi1 = lo1;
            } else {
                hi1 = min(lo1 + n1 * st1, hi1);
                lo1 += (n1 - 1) * st1 + 1;
            }
        }
        if (lo2 < hi2) {
            if (n2 == 0) {
                hi2 = lo2;
            } else {
                hi2 = min(lo2 + n2 * st2, hi2);
                lo2 += (n2 - 1) * st2 + 1;
            }
        }
    }
    c1 = lo1;
    c2 = lo2;
}

}  // namespace qaff
