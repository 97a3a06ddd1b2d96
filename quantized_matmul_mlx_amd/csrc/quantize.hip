// Quantization of a dense [rows, cols] weight into the packed form (nuvec_core quantized.rs:
// module documentation and `quantize`: float16, bfloat16 or float32 w, scales and biases in w's
// dtype; the bias is the group minimum, as rlx-moshi's mlx_dequant.rs doc comment says). Per group
// of G values of a row:
//   bias  = the group minimum, scale = (max - min) / (2^bits - 1), both stored in the scales' type
//           (float32 as is, bf16 or float16 rounded to nearest even);
//   code  = round((w - bias) / scale), half away from zero, with the stored bias and scale,
//           clamped to [0, 2^bits - 1]; a stored scale of 0 (a constant group) gives code 0.
// The code is the rounded value of the formula itself: neither w - bias nor the quotient is rounded
// before the decision.
//
// One lane per 32-value block: it loads its block, the G/32 lanes of a group (adjacent, since a
// row holds a whole number of groups) combine their minima and maxima, and each lane writes its
// block's `bits` words of the bit stream; the group's first lane writes the scale and bias.
// HBM-bound work: a 2-byte weight reads 64 bytes and writes 4 * bits bytes per lane.
#include "launch.h"
#include "qaff_device.h"

#include <hip/hip_runtime.h>

namespace qaff {
namespace {

constexpr int kQuantThreads = 256;

// The running minimum and maximum of the group, combined in block order: the value from the
// later block wins only if it is strictly smaller (larger), which keeps the first of equal
// values (as a sequential scan does, e.g. between -0 and +0).
template <int LANES>
__device__ __forceinline__ void group_min_max(float& lo, float& hi, int lane) {
#pragma unroll
    for (int d = 1; d < LANES; d <<= 1) {
        const float olo = __shfl_xor(lo, d, 64);
        const float ohi = __shfl_xor(hi, d, 64);
        const bool later = (lane & d) == 0;  // the other lane holds the later blocks
        if (later) {
            lo = olo < lo ? olo : lo;
            hi = ohi > hi ? ohi : hi;
        } else {
            lo = lo < olo ? lo : olo;
            hi = hi > ohi ? hi : ohi;
        }
    }
}

// The sign (-1, 0, 1) of (v - bias) - p for float32 v and bias and a double p, exactly (no
// overflow): v - bias is x + ex exactly in double (Knuth's two-sum), and x - p is r + er exactly (a
// second two-sum), so the value is r + (er + ex). Where r is 0 or x and p are within a factor of 2
// of each other, er is 0 and the rounded sum r + ex keeps the sign of the exact one (round to
// nearest gives 0 only for an exact 0); otherwise |r| >= |x| / 2 outweighs |er + ex| (at most about
// an ulp of x).
__device__ __forceinline__ int residual_sign(float v, float bias, double p) {
    const double a = (double)v, b = -(double)bias;
    const double x = a + b;
    const double bx = x - a;
    const double ex = (a - (x - bx)) + (b - bx);
    const double r = x - p;
    const double pr = x - r;
    const double er = (x - (r + pr)) + (pr - p);
    const double t = r + (er + ex);
    return (t > 0.0) - (t < 0.0);
}

// VEC: w is 16-byte aligned and read in 16-byte loads; otherwise one element at a time.
// IN: w's type (0 float32, 1 bf16, 2 float16); st: the scales' and biases' type (block-uniform).
template <int BITS, int GSHIFT, int IN, bool VEC>
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(const void* w, uint64_t blocks,
                                                                 uint32_t* packed, void* scales,
                                                                 void* biases, int st) {
    constexpr int kLanes = 1 << GSHIFT;  // lanes (32-value blocks) per group
    constexpr float kTop = (float)((1 << BITS) - 1);
    const uint64_t idx = (uint64_t)blockIdx.x * kQuantThreads + threadIdx.x;
    const int lane = threadIdx.x & 63;
    const bool live = idx < blocks;  // whole groups are live or not: blocks is a multiple of kLanes
    const uint64_t src = live ? idx : 0;

    float v[32];
    if constexpr (!VEC) {
#pragma unroll
        for (int j = 0; j < 32; ++j) v[j] = load_as_f32(w, src * 32 + j, IN);
    } else if constexpr (IN != 0) {
        const u32x4a* p = reinterpret_cast<const u32x4a*>(static_cast<const uint16_t*>(w) + src * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4a a = p[q];
            const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (IN == 1) {
                    v[8 * q + 2 * e] = __uint_as_float(u[e] << 16);
                    v[8 * q + 2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
                } else {
                    v[8 * q + 2 * e] = __half2float(__ushort_as_half((uint16_t)(u[e] & 0xffffu)));
                    v[8 * q + 2 * e + 1] = __half2float(__ushort_as_half((uint16_t)(u[e] >> 16)));
                }
            }
        }
    } else {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(w) + src * 32);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const f32x4 a = p[q];
            v[4 * q] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
        }
    }

    float lo = v[0], hi = v[0];
#pragma unroll
    for (int j = 1; j < 32; ++j) {
        lo = v[j] < lo ? v[j] : lo;
        hi = v[j] > hi ? v[j] : hi;
    }
    group_min_max<kLanes>(lo, hi, lane);

    // the scale and bias as stored (sbits, bbits: float32 bits or a 16-bit pattern) and their values
    const float q = (hi - lo) / kTop;
    uint32_t sbits, bbits;
    float sc, bi;
    if (st == 1) {
        sbits = to_bf16_bits(q);
        bbits = to_bf16_bits(lo);
        sc = bf16_to_f32((uint16_t)sbits);
        bi = bf16_to_f32((uint16_t)bbits);
    } else if (st == 2) {
        sbits = __half_as_ushort(__float2half_rn(q));
        bbits = __half_as_ushort(__float2half_rn(lo));
        sc = __half2float(__ushort_as_half((uint16_t)sbits));
        bi = __half2float(__ushort_as_half((uint16_t)bbits));
    } else {
        sbits = __float_as_uint(q);
        bbits = __float_as_uint(lo);
        sc = q;
        bi = lo;
    }

    uint32_t words[BITS];
#pragma unroll
    for (int i = 0; i < BITS; ++i) words[i] = 0u;
    // code = round((w - bias) / scale), half away from zero, decided exactly. A candidate c0 from
    // the reciprocal is off by at most one; the signs of (w - bias) - (c0 -+ 1/2) s settle it.
    // bf16 and float16 scales: d = fl(w - bias) and its rounding error e (Two-Sum: d + e = w - bias
    // exactly). Each (c0 -+ 1/2) s has at most 9 + 11 significant bits, exact in float32, so the
    // fused form rounds only d - p and keeps its sign. Where d != p, |d - p| is at least one ulp of d
    // (d is on a grid of that ulp, p on one at least as coarse unless it is far smaller than d),
    // which |e| (half an ulp at most) cannot overturn; where d == p, the sign is e's.
    // float32 scales: (c0 -+ 1/2) s has up to 9 + 24 bits, exact only in double, and the sign comes
    // from residual_sign.
    // Most values need none of that: t = fma(d, 1/s, 1/2) lies within 3u|q| + u/2 (u = 2^-24) of
    // q + 1/2, q the exact quotient, so for |q| <= 2^9 (every code not settled by the clamps) t is
    // off by less than 2^-14, and where t's fraction is at least 2^-12 from an integer, floor(t) is
    // already the decision. Only the other values (about one in two thousand) take the exact test,
    // in a branch the wave skips when none of its lanes needs it (an empty exec mask). Past |q| = 2^9 the clamp gives
    // the same code either way.
    // A scale of 0 (a constant group) gives code 0 everywhere: the loop runs with a reciprocal of
    // 0 (t = 1/2, or NaN for a non-finite d, which takes the exact test) and its words are
    // cleared after it, instead of a branch per value.
    const float rcp = sc != 0.0f ? 1.0f / sc : 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const float d = v[j] - bi;
        const float t = __builtin_fmaf(d, rcp, 0.5f);
        const float c0 = __builtin_floorf(t);
        // near a tie: t's fraction within 2^-12 of 0 or 1, or NaN (the comparison is then false)
        const bool near = !(__builtin_fabsf((t - c0) - 0.5f) < 0.5f - 0x1p-12f);
        float adj = 0.0f;  // the exact test's correction of c0: +1, 0 or -1
        if (near) {
            bool up, down;
            if (st != 0) {
                const float dv = d - v[j];
                const float e = (v[j] - (d - dv)) + (-bi - dv);
                const float rh = __builtin_fmaf(-(c0 + 0.5f), sc, d);
                const float rl = __builtin_fmaf(-(c0 - 0.5f), sc, d);
                up = rh > 0.0f || (rh == 0.0f && e >= 0.0f);    // w - bias >= (c0 + 1/2) s
                down = rl < 0.0f || (rl == 0.0f && e < 0.0f);   // w - bias <  (c0 - 1/2) s
            } else {
                up = residual_sign(v[j], bi, ((double)c0 + 0.5) * (double)sc) >= 0;
                down = residual_sign(v[j], bi, ((double)c0 - 0.5) * (double)sc) < 0;
            }
            adj = (up ? 1.0f : 0.0f) - (down ? 1.0f : 0.0f);
        }
        float c = c0 + adj;
        c = __builtin_fminf(__builtin_fmaxf(c, 0.0f), kTop);  // a NaN quotient gives 0
        const uint32_t code = (uint32_t)c;
        const int p = j * BITS;  // bit position in the block's stream (compile-time after unrolling)
        words[p >> 5] |= code << (p & 31);
        if ((p & 31) + BITS > 32) words[(p >> 5) + 1] |= code >> (32 - (p & 31));
    }
    if (sc == 0.0f) {
#pragma unroll
        for (int i = 0; i < BITS; ++i) words[i] = 0u;
    }

    if (!live) return;
    uint32_t* out = packed + idx * BITS;
    if constexpr (BITS == 4) {
        *reinterpret_cast<u32x4*>(out) = u32x4{words[0], words[1], words[2], words[3]};
    } else if constexpr (BITS == 8) {
        *reinterpret_cast<u32x4*>(out) = u32x4{words[0], words[1], words[2], words[3]};
        *reinterpret_cast<u32x4*>(out + 4) = u32x4{words[4], words[5], words[6], words[7]};
    } else if constexpr (BITS == 2) {
        *reinterpret_cast<u32x2*>(out) = u32x2{words[0], words[1]};
    } else {
#pragma unroll
        for (int i = 0; i < BITS; ++i) out[i] = words[i];
    }
    if ((idx & (kLanes - 1)) == 0) {
        if (st == 0) {
            static_cast<uint32_t*>(scales)[idx >> GSHIFT] = sbits;
            static_cast<uint32_t*>(biases)[idx >> GSHIFT] = bbits;
        } else {
            static_cast<uint16_t*>(scales)[idx >> GSHIFT] = (uint16_t)sbits;
            static_cast<uint16_t*>(biases)[idx >> GSHIFT] = (uint16_t)bbits;
        }
    }
}

template <int BITS, int GSHIFT, bool VEC>
hipError_t launch_v(const void* w, int in, uint64_t blocks, uint32_t* packed, void* scales, void* biases, int st,
                    hipStream_t stream) {
    const unsigned grid = (unsigned)((blocks + kQuantThreads - 1) / kQuantThreads);
    if (in == 1)
        quantize_kernel<BITS, GSHIFT, 1, VEC><<<grid, kQuantThreads, 0, stream>>>(w, blocks, packed, scales, biases, st);
    else if (in == 2)
        quantize_kernel<BITS, GSHIFT, 2, VEC><<<grid, kQuantThreads, 0, stream>>>(w, blocks, packed, scales, biases, st);
    else
        quantize_kernel<BITS, GSHIFT, 0, VEC><<<grid, kQuantThreads, 0, stream>>>(w, blocks, packed, scales, biases, st);
    return hipGetLastError();
}

template <int BITS, int GSHIFT>
hipError_t launch_g(const void* w, int in, uint64_t blocks, uint32_t* packed, void* scales, void* biases, int st,
                    hipStream_t stream) {
    if (reinterpret_cast<uintptr_t>(w) % 16 == 0)
        return launch_v<BITS, GSHIFT, true>(w, in, blocks, packed, scales, biases, st, stream);
    return launch_v<BITS, GSHIFT, false>(w, in, blocks, packed, scales, biases, st, stream);
}

template <int BITS>
hipError_t launch_bits(const void* w, int in, uint64_t blocks, uint32_t gshift, uint32_t* packed, void* scales,
                       void* biases, int st, hipStream_t stream) {
    if (gshift == 0) return launch_g<BITS, 0>(w, in, blocks, packed, scales, biases, st, stream);
    if (gshift == 1) return launch_g<BITS, 1>(w, in, blocks, packed, scales, biases, st, stream);
    return launch_g<BITS, 2>(w, in, blocks, packed, scales, biases, st, stream);
}

}  // namespace

hipError_t launch_quantize(const void* w, int w_dtype, int64_t rows, int64_t cols, int group_size, int bits,
                           uint32_t* packed, void* scales, void* biases, int sb_dtype, hipStream_t stream) {
    const uint64_t blocks = (uint64_t)rows * (uint64_t)(cols / 32);
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    switch (bits) {
        case 1: return launch_bits<1>(w, w_dtype, blocks, gshift, packed, scales, biases, sb_dtype, stream);
        case 2: return launch_bits<2>(w, w_dtype, blocks, gshift, packed, scales, biases, sb_dtype, stream);
        case 3: return launch_bits<3>(w, w_dtype, blocks, gshift, packed, scales, biases, sb_dtype, stream);
        case 4: return launch_bits<4>(w, w_dtype, blocks, gshift, packed, scales, biases, sb_dtype, stream);
        case 5: return launch_bits<5>(w, w_dtype, blocks, gshift, packed, scales, biases, sb_dtype, stream);
        case 6: return launch_bits<6>(w, w_dtype, blocks, gshift, packed, scales, biases, sb_dtype, stream);
        case 8: return launch_bits<8>(w, w_dtype, blocks, gshift, packed, scales, biases, sb_dtype, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qaff
