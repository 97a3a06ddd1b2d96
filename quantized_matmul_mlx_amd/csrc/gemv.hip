// Quantized GEMV on the VALU: y[m, n] = sum_k x[m, k] * w[n, k] for a few rows of x (the decode
// path of spark_runtime weights/mlx_int8.rs, `gemv`; the product itself is nuvec_core
// quantized.rs, `quantized_matmul` with transpose). W is never materialised.
//
// HBM-bound: every packed word is read once per launch for up to MB rows of x, so the design goal
// is to have all of a launch's weight bytes in flight as early as possible and to spend few VALU
// operations per code.
//
// bf16 x (the decode path):
//   * A 256-thread block owns 4 * RPW rows of W (RPW per wave). Lane l of a wave takes the 32-code
//     blocks l, l + 64, ... of each of its rows, so a wave-wide load of one block per lane reads
//     contiguous words. Before touching x, each lane issues the loads of every block it needs in
//     the current pass (RPW rows x P blocks), plus their scales and biases.
//   * x is staged once per block of threads in LDS, already permuted into the pairing order in
//     which the codes are unpacked, as bf16 pairs.
//   * Codes become exact bf16 values with one AND-OR per pair of codes: for codes below 128,
//     OR-ing the code into the mantissa of bf16 128.0 (0x4300) gives exactly 128 + c. The 4-bit
//     pairs (c_i, c_{i+4}) of a word are (w >> 4i) & 0x000F000F | 0x43004300; 2-bit pairs
//     (c_i, c_{i+8}) likewise. 3-bit pairs (c_i, c_{i+8}) and 6-bit pairs (c_i, c_{i+4}) sit 24
//     bits apart: one funnel shift, one byte permute and one AND-OR per pair. 5-bit codes are
//     extracted one by one (a bit-field extract, or a funnel shift for codes that straddle words)
//     and paired in column order. 8-bit codes go through the byte-to-float converts, exact in bf16
//     since c <= 255 has 8 bits.
//   * v_dot2_f32_bf16 multiplies two code pairs by two x pairs and accumulates in float32. Per
//     block, with d = sum x_k (o + c_k) and xs = sum x_k (o = 128, or 0 for 8-bit codes),
//         sum_k x_k (s c_k + b) = s * d + (b - o s) * xs,
//     so the scale, the bias and the offset cost two multiply-adds per block.
//   * The float32 partial sums are reduced across the wave; lane 0 writes y.
//
// float32 x: the straightforward form of the same loop in float32 (codes converted to float, one
// multiply-add per code and x row), used for float32 inputs at any m.
#include "launch.h"
#include "qaff_device.h"

#include <hip/hip_runtime.h>

namespace qaff {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The 16-bit format F of x, scales, biases and y: 0 bf16, 1 float16. Codes become exact values
// o + c of that format (o = 128 in bf16, whose 8 significant bits hold 128 + c for c < 128; o =
// 1024 in float16, whose 11 hold 1024 + c for every code up to 8 bits), and v_dot2 of the format
// multiplies two of them by two x values exactly and adds in float32.
template <int F> constexpr uint32_t kMagicF = F ? 0x64006400u : 0x43004300u;  // o in both halves
template <int F> constexpr float kOffsetF = F ? 1024.f : 128.f;

template <int F>
__device__ __forceinline__ float dot2f(uint32_t a, uint32_t b, float c) {
    if constexpr (F == 1)
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
    else
        return dot2(a, b, c);
}

template <int F>
__device__ __forceinline__ float widen16(uint32_t h) {  // exact
    if constexpr (F == 1)
        return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    else
        return bf16_to_f32(h);
}

template <int F>
__device__ __forceinline__ uint16_t narrow16(float v) {  // round to nearest even
    if constexpr (F == 1)
        return __builtin_bit_cast(uint16_t, (_Float16)v);
    else
        return to_bf16_bits(v);
}

// ---- per-bit-width unpacking into 16 bf16 pairs per 32-code block ---------------------------

template <int BITS, int F = 0> struct Codes;

// 4-bit: pair 4q + p of block = (c_{8q+p}, c_{8q+p+4}), values o + c.
template <int F> struct Codes<4, F> {
    static constexpr float kOffset = kOffsetF<F>;
    __device__ __forceinline__ static void unpack(const uint32_t (&w)[4], uint32_t (&pr)[16]) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int p = 0; p < 4; ++p) pr[4 * q + p] = and_or(w[q] >> (4 * p), 0x000F000Fu, kMagicF<F>);
    }
    // x pairs in the same order, from the block's 32 x values as 16 natural-order dwords.
    __device__ __forceinline__ static void pair_x(const uint32_t (&xn)[16], uint32_t (&xp)[16]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t d0 = xn[4 * q], d1 = xn[4 * q + 1], d2 = xn[4 * q + 2], d3 = xn[4 * q + 3];
            // x_{8q+0..7} = lo(d0) hi(d0) lo(d1) hi(d1) lo(d2) hi(d2) lo(d3) hi(d3)
            xp[4 * q + 0] = __builtin_amdgcn_perm(d2, d0, 0x05040100u);  // (lo d0, lo d2)
            xp[4 * q + 1] = __builtin_amdgcn_perm(d2, d0, 0x07060302u);  // (hi d0, hi d2)
            xp[4 * q + 2] = __builtin_amdgcn_perm(d3, d1, 0x05040100u);  // (lo d1, lo d3)
            xp[4 * q + 3] = __builtin_amdgcn_perm(d3, d1, 0x07060302u);  // (hi d1, hi d3)
        }
    }
};

// 2-bit: pair 8q + p = (c_{16q+p}, c_{16q+p+8}), values o + c.
template <int F> struct Codes<2, F> {
    static constexpr float kOffset = kOffsetF<F>;
    __device__ __forceinline__ static void unpack(const uint32_t (&w)[2], uint32_t (&pr)[16]) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int p = 0; p < 8; ++p) pr[8 * q + p] = and_or(w[q] >> (2 * p), 0x00030003u, kMagicF<F>);
    }
    __device__ __forceinline__ static void pair_x(const uint32_t (&xn)[16], uint32_t (&xp)[16]) {
        // x_{16q+j}: dword 8q + j/2, half j%2. Pair p takes x_{16q+p} and x_{16q+p+8}.
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const uint32_t a = xn[8 * q + p / 2], b = xn[8 * q + 4 + p / 2];
                xp[8 * q + p] = (p & 1) ? __builtin_amdgcn_perm(b, a, 0x07060302u)
                                        : __builtin_amdgcn_perm(b, a, 0x05040100u);
            }
    }
};

// 1-bit: pair 8q + p = (c_{16q+p}, c_{16q+p+8}), values o + c. x is staged in halves of 16, so
// a pair must stay within a half: swapping the word's middle bytes puts c_{8..15} at bits 16..23
// and c_{16..23} at bits 8..15, after which bits i and i + 16 are such a pair.
template <int F> struct Codes<1, F> {
    static constexpr float kOffset = kOffsetF<F>;
    __device__ __forceinline__ static void unpack(const uint32_t (&w)[1], uint32_t (&pr)[16]) {
        const uint32_t v = __builtin_amdgcn_perm(w[0], w[0], 0x03010200u);  // bytes b0 b2 b1 b3
#pragma unroll
        for (int i = 0; i < 16; ++i) pr[i] = and_or(v >> i, 0x00010001u, kMagicF<F>);
    }
    // the 2-bit pairing of x: pair 8q + p takes x_{16q+p} and x_{16q+p+8}
    __device__ __forceinline__ static void pair_x(const uint32_t (&xn)[16], uint32_t (&xp)[16]) {
        Codes<2, F>::pair_x(xn, xp);
    }
};

// 8-bit: pair 2q + h = (c_{4q+2h}, c_{4q+2h+1}), exact values c (offset 0).
template <> struct Codes<8, 0> {
    static constexpr float kOffset = 0.f;
    __device__ __forceinline__ static void unpack(const uint32_t (&w)[8], uint32_t (&pr)[16]) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t f0 = __float_as_uint((float)(w[q] & 0xffu));
            const uint32_t f1 = __float_as_uint((float)((w[q] >> 8) & 0xffu));
            const uint32_t f2 = __float_as_uint((float)((w[q] >> 16) & 0xffu));
            const uint32_t f3 = __float_as_uint((float)(w[q] >> 24));
            // the upper halves of the float32 patterns are the exact bf16 values
            pr[2 * q] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
            pr[2 * q + 1] = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
        }
    }
    __device__ __forceinline__ static void pair_x(const uint32_t (&xn)[16], uint32_t (&xp)[16]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) xp[i] = xn[i];
    }
};

// 8-bit, float16: pair 2q + h = (c_{4q+2h}, c_{4q+2h+1}), values 1024 + c: one byte permute
// puts two codes under the exponent bytes of 1024.0.
template <> struct Codes<8, 1> {
    static constexpr float kOffset = 1024.f;
    __device__ __forceinline__ static void unpack(const uint32_t (&w)[8], uint32_t (&pr)[16]) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            pr[2 * q] = __builtin_amdgcn_perm(0x64646464u, w[q], 0x04010400u);      // c0, c1
            pr[2 * q + 1] = __builtin_amdgcn_perm(0x64646464u, w[q], 0x04030402u);  // c2, c3
        }
    }
    __device__ __forceinline__ static void pair_x(const uint32_t (&xn)[16], uint32_t (&xp)[16]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) xp[i] = xn[i];
    }
};

// 32 bits of a block's stream from bit `bit` on (compile-time after unrolling): one funnel shift,
// or a plain shift in the last word (the bits above the block are not used).
template <int NW>
__device__ __forceinline__ uint32_t stream_window(const uint32_t (&w)[NW], int bit) {
    const int wi = bit >> 5, sh = bit & 31;
    if (wi + 1 < NW) return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh);
    return w[wi] >> sh;
}

// 3-bit: pair 8q + p = (c_{16q+p}, c_{16q+p+8}), values o + c. With the stream shifted so that
// c_i starts at bit 0, c_{i+8} starts at bit 24; one byte permute (bytes 0, 1, 3, 3) moves it to
// bit 16, and one AND-OR forms the pair. x pairs as for 2-bit codes.
template <int F> struct Codes<3, F> {
    static constexpr float kOffset = kOffsetF<F>;
    __device__ __forceinline__ static void unpack(const uint32_t (&w)[3], uint32_t (&pr)[16]) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const uint32_t v = stream_window<3>(w, 3 * (16 * q + p));
                pr[8 * q + p] = and_or(__builtin_amdgcn_perm(v, v, 0x03030100u), 0x00070007u, kMagicF<F>);
            }
    }
    __device__ __forceinline__ static void pair_x(const uint32_t (&xn)[16], uint32_t (&xp)[16]) {
        Codes<2, F>::pair_x(xn, xp);
    }
};

// 6-bit: pair 4q + p = (c_{8q+p}, c_{8q+p+4}), values o + c: c_{i+4} starts 24 bits after c_i, so
// the same permute forms the pair. x pairs as for 4-bit codes.
template <int F> struct Codes<6, F> {
    static constexpr float kOffset = kOffsetF<F>;
    __device__ __forceinline__ static void unpack(const uint32_t (&w)[6], uint32_t (&pr)[16]) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t v = stream_window<6>(w, 6 * (8 * q + p));
                pr[4 * q + p] = and_or(__builtin_amdgcn_perm(v, v, 0x03030100u), 0x003F003Fu, kMagicF<F>);
            }
    }
    __device__ __forceinline__ static void pair_x(const uint32_t (&xn)[16], uint32_t (&xp)[16]) {
        Codes<4, F>::pair_x(xn, xp);
    }
};

// 5-bit: pair i = (c_{2i}, c_{2i+1}) in column order, values o + c (no pair of 5-bit codes sits
// 16 or 24 bits apart within 32).
template <int BITS, int F> struct Codes {
    static_assert(BITS == 5, "bit width");
    static constexpr float kOffset = kOffsetF<F>;
    __device__ __forceinline__ static void unpack(const uint32_t (&w)[BITS], uint32_t (&pr)[16]) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            pr[i] = (code_at<BITS>(w, 2 * i) | (code_at<BITS>(w, 2 * i + 1) << 16)) | kMagicF<F>;
    }
    __device__ __forceinline__ static void pair_x(const uint32_t (&xn)[16], uint32_t (&xp)[16]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) xp[i] = xn[i];
    }
};

// ---- bf16 x kernel -----------------------------------------------------------------------------

// Sum over the 64 lanes of a wave with DPP row operations; every lane gets the total.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
    const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false);
    return v + __int_as_float(moved);
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
    v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]: quad sums
    v = dpp_add<0x141, 0xF>(v);  // row_half_mirror: half-row sums
    v = dpp_add<0x140, 0xF>(v);  // row_mirror: row sums
    v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3: lane 63 holds the total
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// silu (silu_f32 in qaff_device.h: float32 from the hardware exp2 and reciprocal, each within a few
// ulp): h is rounded to bf16 right after, which an error of that size moves only in rare ties.
// Every block of the GEMV recomputes the activation for its x, so its cost counts.

// FUSED adds the decode fusions of `GemvFused` (uniform flags read at run time): the x transform,
// the residual, and a second weight whose rows follow the first's (rows n .. 2n - 1).
// The x batch and weight batch of a gathered product's block (grid z = output batch). Returns
// false, after writing NaN over the block's outputs, when an index is out of range.
template <int RPW, int MB, typename XP, typename PP, typename SP, typename YP>
__device__ __forceinline__ bool gather_batch(const Gather& ga, uint32_t row0, uint32_t m0, uint32_t m, uint32_t n,
                                             int lane, XP& x, PP& packed, SP& scales, SP& biases, YP& y) {
    const uint32_t b = ga.b0 + blockIdx.z;
    const uint32_t li = ga.lhs ? ga.lhs[b] : b;
    const uint32_t ri = ga.rhs ? ga.rhs[b] : b;
    y += (size_t)b * ga.y_stride;
    if (li >= ga.x_count || ri >= ga.w_count) {
        if (lane == 0)
#pragma unroll
            for (int r = 0; r < RPW; ++r)
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    if (row0 + r < n && m0 + i < m) {
                        if constexpr (sizeof(*y) == 2) y[(size_t)(m0 + i) * n + row0 + r] = 0x7FC0u;
                        else y[(size_t)(m0 + i) * n + row0 + r] = __builtin_nanf("");
                    }
        return false;
    }
    x += (size_t)li * ga.x_stride;
    packed += (size_t)ri * ga.w_stride;
    scales += (size_t)ri * ga.sb_stride;
    biases += (size_t)ri * ga.sb_stride;
    return true;
}

// STAGE_SB (long rows, an even number of groups per row): the pass's scales and biases of each of
// the wave's rows come in one 16-byte load per lane and row, through a wave-private LDS area,
// instead of one 2-byte load per lane, block and row.
template <int BITS, int MB, int RPW, int WAVES, int P, bool FUSED, bool GATHER = false, bool STAGE_SB = false, int F = 0>
__global__ __launch_bounds__(WAVES * 64) void gemv_bf16_kernel(
    const uint16_t* __restrict__ x, uint32_t m, const uint32_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases, uint32_t n,
    uint32_t kb, uint32_t gshift, uint16_t* __restrict__ y, GemvFused fz, Gather ga) {
    static_assert(F == 0 || (!FUSED && !GATHER), "float16 operands: the plain product only");
    constexpr int kBlockThreads = WAVES * 64;
    constexpr int kPassBlocks = 64 * P;  // 32-code blocks per row per pass
    // x of the pass as bf16 pairs in unpack order: [x row][quarter of a block][block] of 16 bytes,
    // so that lane l reading quarter t of its block reads the 16 bytes after lane l-1's.
    __shared__ u32x4a xl[MB][4][kPassBlocks];
    __shared__ float xsl[MB][kPassBlocks][2];  // float32 sums of each half of each block of x
    __shared__ uint16_t sbl[STAGE_SB ? WAVES : 1][RPW][2][STAGE_SB ? kPassBlocks : 1];  // [wave][row][s, b][group]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const uint32_t row0 = (blockIdx.x * WAVES + wave) * RPW;
    const uint32_t m0 = blockIdx.y * MB;
    const uint32_t gpr = kb >> gshift;
    if constexpr (GATHER) {  // block-uniform: the whole block returns
        if (!gather_batch<RPW, MB>(ga, row0, m0, m, n, lane, x, packed, scales, biases, y)) return;
    }
    // rows of the launch: n, or 2n with a second weight (its rows after the first's)
    const uint32_t nrows = (FUSED && fz.packed2) ? 2 * n : n;
    const bool silu = FUSED && fz.up != nullptr;
    const uint16_t* __restrict__ upx = silu ? fz.up : x;  // read either way: no branch around loads

    float acc[RPW][MB];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int i = 0; i < MB; ++i) acc[r][i] = 0.f;

    for (uint32_t pass0 = 0; pass0 < kb; pass0 += kPassBlocks) {
        // 1. Load the pass's x first (one unit = 16 values of one x row), so that it arrives
        //    ahead of the weights: the wait for it before staging then leaves the weight loads
        //    in flight, and each block's multiply waits only for its own weight load.
        constexpr int kUnitsTotal = MB * 2 * kPassBlocks;
        constexpr int kUnits = (kUnitsTotal + kBlockThreads - 1) / kBlockThreads;
        u32x4a xg[kUnits][2];
        u32x4a ug[FUSED ? kUnits : 1][2];
        bool xvalid[kUnits];
#pragma unroll
        for (int t = 0; t < kUnits; ++t) {
            // clamped so that every load is in bounds and none sits in a branch; values that are
            // not part of x are zeroed when staged
            const int u = min(tid + kBlockThreads * t, kUnitsTotal - 1);
            const int mi = u / (2 * kPassBlocks);
            const int rem = u - mi * 2 * kPassBlocks;
            const int h = rem / kPassBlocks;      // which half of the block
            const int b = rem - h * kPassBlocks;  // block within the pass
            const uint32_t j = pass0 + b;
            xvalid[t] = m0 + mi < m && j < kb;
            const uint32_t xr = min(m0 + mi, m - 1);
            const uint32_t jc = min(j, kb - 1);
            const size_t xo = (size_t)xr * kb * 32 + (size_t)jc * 32 + h * 16;
            const u32x4a* src = reinterpret_cast<const u32x4a*>(x + xo);
            xg[t][0] = src[0];
            xg[t][1] = src[1];
            if constexpr (FUSED) {
                const u32x4a* usrc = reinterpret_cast<const u32x4a*>(upx + xo);
                ug[t][0] = usrc[0];
                ug[t][1] = usrc[1];
            }
        }

        // 2. Issue every weight load of the pass. Rows are wave-uniform, so each row's base
        //    address is scalar and a lane only adds its own 32-bit offset. Indices are clamped
        //    into the weight instead of branching around the loads (a branch per load makes the
        //    compiler wait for each one): a lane past the row's end reads a valid block that it
        //    never uses, and rows past n are computed but not stored. Scales and biases stay raw
        //    until use, so no conversion waits on a load here.
        uint32_t wq[RPW][P][BITS];
        uint32_t sraw[RPW][P], braw[RPW][P];
        u32x4 sbw[STAGE_SB ? RPW : 1][2];   // STAGE_SB: 8 scales and 8 biases from group gl
        const uint32_t g0 = pass0 >> gshift;
        const uint32_t gl = min(g0 + 8 * (uint32_t)lane, gpr - 8);  // clamped into the row
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            uint32_t row = min(row0 + r, nrows - 1);
            const uint32_t* pk = packed;
            const uint16_t* sc = scales;
            const uint16_t* bi = biases;
            if (FUSED && row >= n) {  // wave-uniform: the second weight
                row -= n;
                pk = fz.packed2;
                sc = fz.scales2;
                bi = fz.biases2;
            }
            const uint32_t* prow = pk + (size_t)row * kb * BITS;
            const uint16_t* srow = sc + (size_t)row * gpr;
            const uint16_t* brow = bi + (size_t)row * gpr;
            if constexpr (STAGE_SB) {  // 4-byte aligned: gpr and g0 are even
                sbw[r][0] = *reinterpret_cast<const u32x4*>(srow + gl);
                sbw[r][1] = *reinterpret_cast<const u32x4*>(brow + gl);
            }
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const uint32_t j = min(pass0 + p * 64 + lane, kb - 1);
                if constexpr (BITS == 4) {
                    // non-temporal: each weight is read once (measured: 4-bit decode 3.81 -> 3.73 us,
                    // gate_up 15.4 -> 14.4 us; the 8-bit GEMV lost 12% with them, so only here)
                    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(prow + j * BITS));
                    wq[r][p][0] = v.x; wq[r][p][1] = v.y; wq[r][p][2] = v.z; wq[r][p][3] = v.w;
                } else {
                    load_block<BITS>(prow + j * BITS, wq[r][p]);
                }
                if constexpr (!STAGE_SB) {
                    sraw[r][p] = srow[j >> gshift];
                    braw[r][p] = brow[j >> gshift];
                }
            }
        }

        // 3. Stage x in LDS, paired in unpack order, with the float32 sum of each 16 values.
        //    Every pairing only mixes values within 16 (2-bit codes) or 8 (the other widths), so
        //    a unit is paired on its own: it is placed at its position in a block of 32 and the
        //    block is paired.
        if (pass0 > 0) __syncthreads();  // the previous pass has finished reading xl and xsl
#pragma unroll
        for (int t = 0; t < kUnits; ++t) {
            const int u = tid + kBlockThreads * t;
            if (u >= kUnitsTotal) break;
            const int mi = u / (2 * kPassBlocks);
            const int rem = u - mi * 2 * kPassBlocks;
            const int h = rem / kPassBlocks;
            const int b = rem - h * kPassBlocks;
            uint32_t xn[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) xn[q] = 0u;
            uint32_t v[8] = {xg[t][0].x, xg[t][0].y, xg[t][0].z, xg[t][0].w,
                             xg[t][1].x, xg[t][1].y, xg[t][1].z, xg[t][1].w};
            if constexpr (FUSED) {
                if (silu) {
                    // h = silu(gate) * up in float32, rounded to bf16: the GEMV's input
                    const uint32_t uv[8] = {ug[t][0].x, ug[t][0].y, ug[t][0].z, ug[t][0].w,
                                            ug[t][1].x, ug[t][1].y, ug[t][1].z, ug[t][1].w};
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const float g0 = __uint_as_float(v[q] << 16), g1 = __uint_as_float(v[q] & 0xffff0000u);
                        const float u0 = __uint_as_float(uv[q] << 16), u1 = __uint_as_float(uv[q] & 0xffff0000u);
                        v[q] = pack_bf16x2(silu_f32(g0) * u0, silu_f32(g1) * u1);
                    }
                }
            }
            if (!xvalid[t]) {
#pragma unroll
                for (int q = 0; q < 8; ++q) v[q] = 0u;
            }
            float hs = 0.f;
#pragma unroll
            for (int q = 0; q < 8; ++q) hs = dot2f<F>(v[q], F ? 0x3C003C00u : 0x3F803F80u, hs);  // pairs of 1.0
            xsl[mi][b][h] = hs;
            uint32_t xp[16];
            if (h == 0) {
#pragma unroll
                for (int q = 0; q < 8; ++q) xn[q] = v[q];
                Codes<BITS, F>::pair_x(xn, xp);
                xl[mi][0][b] = u32x4a{xp[0], xp[1], xp[2], xp[3]};
                xl[mi][1][b] = u32x4a{xp[4], xp[5], xp[6], xp[7]};
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) xn[8 + q] = v[q];
                Codes<BITS, F>::pair_x(xn, xp);
                xl[mi][2][b] = u32x4a{xp[8], xp[9], xp[10], xp[11]};
                xl[mi][3][b] = u32x4a{xp[12], xp[13], xp[14], xp[15]};
            }
        }
        __syncthreads();

        // STAGE_SB: each lane stores its chunk's group pairs that fall in the pass at their own
        // positions (a chunk clamped at the row's end can start before the pass, and overlaps its
        // neighbour with the same values), then reads its blocks' groups.
        if constexpr (STAGE_SB) {
            const uint32_t ng = kPassBlocks >> gshift;  // groups of the pass
#pragma unroll
            for (int r = 0; r < RPW; ++r)
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    const u32x4 v = sbw[r][a];
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint32_t gd = gl + 2 * d;  // the pair's first group
                        if (8 * (uint32_t)lane < ng && gd >= g0 && gd - g0 < ng)
                            *reinterpret_cast<uint32_t*>(&sbl[wave][r][a][gd - g0]) = w4[d];
                    }
                }
#pragma unroll
            for (int r = 0; r < RPW; ++r)
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    const uint32_t q = min((uint32_t)(p * 64 + lane) >> gshift, ng - 1);
                    sraw[r][p] = sbl[wave][r][0][q];
                    braw[r][p] = sbl[wave][r][1][q];
                }
        }

        // 4. Multiply.
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const uint32_t j = pass0 + p * 64 + lane;
            if (j >= kb) break;
            uint32_t xp[MB][16];
            float xs[MB];
#pragma unroll
            for (int i = 0; i < MB; ++i) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const u32x4a v = xl[i][t][p * 64 + lane];
                    xp[i][4 * t] = v.x; xp[i][4 * t + 1] = v.y; xp[i][4 * t + 2] = v.z; xp[i][4 * t + 3] = v.w;
                }
                xs[i] = xsl[i][p * 64 + lane][0] + xsl[i][p * 64 + lane][1];
            }
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                uint32_t pr[16];
                Codes<BITS, F>::unpack(wq[r][p], pr);
                const float sc = widen16<F>(sraw[r][p]);
                const float boff = widen16<F>(braw[r][p]) - Codes<BITS, F>::kOffset * sc;
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    float d = 0.f;
#pragma unroll
                    for (int t = 0; t < 16; ++t) d = dot2f<F>(pr[t], xp[i][t], d);
                    // written as two fused multiply-adds so that every instantiation rounds
                    // the same way (left to the compiler, the contraction varies with the code)
                    acc[r][i] = __builtin_fmaf(sc, d, __builtin_fmaf(boff, xs[i], acc[r][i]));
                }
            }
        }
    }

#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        uint32_t row = row0 + r;
        uint16_t* yo = y;
        if (FUSED && row >= n) {
            row -= n;
            yo = fz.y2;
        }
        const bool in_range = row0 + r < nrows;
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            float v = wave_sum_dpp(acc[r][i]);
            if (lane == 0 && in_range && m0 + i < m) {
                const size_t o = (size_t)(m0 + i) * n + row;
                if (FUSED && fz.resid) v += bf16_to_f32(fz.resid[o]);
                yo[o] = narrow16<F>(v);
            }
        }
    }
}

// ---- float32 x kernel ----------------------------------------------------------------------------

template <int MB>
__device__ __forceinline__ void load_x_f32_block(const float* __restrict__ x, uint32_t row, uint32_t k,
                                                 uint32_t j, float (&xv)[32]) {
    const f32x4* p = reinterpret_cast<const f32x4*>(x + (size_t)row * k + (size_t)j * 32);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const f32x4 v = p[q];
        xv[4 * q] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
    }
}

template <int BITS, int MB, int RW, bool GATHER = false>
__global__ __launch_bounds__(kThreads) void gemv_f32_kernel(
    const float* __restrict__ x, uint32_t m, const uint32_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases, uint32_t n,
    uint32_t kb, uint32_t gshift, float* __restrict__ y, Gather ga) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint32_t n0 = (blockIdx.x * kWaves + wave) * RW;
    if (n0 >= n) return;  // wave-uniform; this kernel has no block-level barrier
    const uint32_t m0 = blockIdx.y * MB;
    if constexpr (GATHER) {
        if (!gather_batch<RW, MB>(ga, n0, m0, m, n, lane, x, packed, scales, biases, y)) return;
    }
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
                load_x_f32_block<MB>(x, m0 + i, k, j, xv[i]);
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
            if (lane == 0 && row < n && m0 + i < m) y[(size_t)(m0 + i) * n + row] = v;
        }
    }
}

// ---- launchers -----------------------------------------------------------------------------------

// grid.y is limited to 65535 blocks: long x goes in slices of at most 65535 * MB rows.
template <typename Launch>
hipError_t over_m_slices(int64_t m, int mb, Launch&& launch) {
    const int64_t max_rows = (int64_t)65535 * mb;
    for (int64_t m_off = 0; m_off < m; m_off += max_rows) {
        const int64_t mm = (m - m_off < max_rows) ? (m - m_off) : max_rows;
        launch(m_off, mm, (unsigned)((mm + mb - 1) / mb));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Rows per wave and waves per block of the bf16 GEMV, per number of x rows handled by one block.
constexpr int kRpw1 = 1, kWaves1 = 8;  // M = 1
constexpr int kRpwN = 2, kWavesN = 4;  // M >= 2

// Blocks per lane and pass: 2 (128 blocks, 4096 codes: one pass at the decode shape). Each pass
// waits for its own loads, so long rows at small MB take wider passes: 8 (MB = 1) or 4 (MB = 2)
// blocks per lane, one pass up to 16384 (8192) codes, within the registers and LDS they need.
template <int MB>
constexpr int kLongPass = MB == 1 ? 8 : MB == 2 ? 4 : 2;

template <int BITS, int MB, int RPW, int WAVES, bool FUSED, int P, bool STAGE_SB = false, int F = 0>
hipError_t launch_bf16_p(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                         const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, uint16_t* y,
                         const GemvFused& fz, hipStream_t stream) {
    const int64_t rows_per_block = (int64_t)WAVES * RPW;
    const int64_t nrows = (FUSED && fz.packed2) ? 2 * n : n;
    const unsigned gx = (unsigned)((nrows + rows_per_block - 1) / rows_per_block);
    return over_m_slices(m, MB, [&](int64_t m_off, int64_t mm, unsigned gy) {
        GemvFused f = fz;
        if (FUSED) {
            if (f.up) f.up += (size_t)m_off * kb * 32;
            if (f.resid) f.resid += (size_t)m_off * n;
            if (f.y2) f.y2 += (size_t)m_off * n;
        }
        gemv_bf16_kernel<BITS, MB, RPW, WAVES, P, FUSED, false, STAGE_SB, F><<<dim3(gx, gy), dim3(WAVES * 64), 0, stream>>>(
            x + (size_t)m_off * kb * 32, (uint32_t)mm, packed, scales, biases, (uint32_t)n,
            (uint32_t)kb, gshift, y + (size_t)m_off * n, f, Gather{});
    });
}

template <int BITS, int MB, int RPW, int WAVES, bool FUSED, int F = 0>
hipError_t launch_bf16(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                       const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, uint16_t* y,
                       const GemvFused& fz, hipStream_t stream) {
    // long rows: the wider pass, and scales and biases through LDS when a row has an even number
    // of groups and the arrays are 4-byte aligned (their 16-byte loads need 4-byte aligned words)
    if (kLongPass<MB> > 2 && kb > 128) {
        const bool sb4 = reinterpret_cast<uintptr_t>(scales) % 4 == 0 && reinterpret_cast<uintptr_t>(biases) % 4 == 0;
        if (((kb >> gshift) & 1) == 0 && sb4)
            return launch_bf16_p<BITS, MB, RPW, WAVES, FUSED, kLongPass<MB>, true, F>(x, m, packed, scales, biases, n,
                                                                                   kb, gshift, y, fz, stream);
        return launch_bf16_p<BITS, MB, RPW, WAVES, FUSED, kLongPass<MB>, false, F>(x, m, packed, scales, biases, n, kb,
                                                                                   gshift, y, fz, stream);
    }
    return launch_bf16_p<BITS, MB, RPW, WAVES, FUSED, 2, false, F>(x, m, packed, scales, biases, n, kb, gshift, y, fz, stream);
}

template <int BITS, bool FUSED, int F = 0>
hipError_t launch_bf16_m(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                         const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, uint16_t* y,
                         const GemvFused& f, hipStream_t stream) {
    // The fused products recompute their x transform per block: 16 rows per block at M = 1 halve
    // that work against the plain GEMV's 8.
    if (m == 1 && FUSED)
        return launch_bf16<BITS, 1, 2, 8, FUSED>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
    // Per width at M = 1 (measured, 500 calls over rotated copies): 4-bit rows of one pass take 16
    // waves of one row (decode [4096, 4096]: 3.73 -> 3.66 us), 3-bit rows 8 waves of two rows
    // ([11008, 4096]: 8.15 -> 7.34 us); the 6- and 8-bit rows were fastest as the default.
    if (m == 1 && BITS == 4 && kb <= 128)
        return launch_bf16<BITS, 1, 1, 16, FUSED, F>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
    if (m == 1 && BITS == 3)
        return launch_bf16<BITS, 1, 2, 8, FUSED, F>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
    if (m == 1)
        return launch_bf16<BITS, 1, kRpw1, kWaves1, FUSED, F>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
    if (m == 2)
        return launch_bf16<BITS, 2, kRpwN, kWavesN, FUSED, F>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
    if (m <= 4)
        return launch_bf16<BITS, 4, kRpwN, kWavesN, FUSED, F>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
    return launch_bf16<BITS, 8, kRpwN, kWavesN, FUSED, F>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
}

template <int BITS, int MB>
hipError_t launch_f32(const float* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                      const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, float* y,
                      hipStream_t stream) {
    constexpr int RW = 2;
    const int64_t rows_per_block = (int64_t)kWaves * RW;
    const unsigned gx = (unsigned)((n + rows_per_block - 1) / rows_per_block);
    return over_m_slices(m, MB, [&](int64_t m_off, int64_t mm, unsigned gy) {
        gemv_f32_kernel<BITS, MB, RW><<<dim3(gx, gy), dim3(kThreads), 0, stream>>>(
            x + (size_t)m_off * kb * 32, (uint32_t)mm, packed, scales, biases, (uint32_t)n,
            (uint32_t)kb, gshift, y + (size_t)m_off * n, Gather{});
    });
}

template <int BITS>
hipError_t launch_f32_m(const float* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                        const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, float* y,
                        hipStream_t stream) {
    if (m == 1) return launch_f32<BITS, 1>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
    if (m == 2) return launch_f32<BITS, 2>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
    return launch_f32<BITS, 4>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
}

template <int BITS>
hipError_t launch_bits(const void* x, bool x_f32, int64_t m, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t kb,
                       uint32_t gshift, void* y, hipStream_t stream) {
    if (x_f32)
        return launch_f32_m<BITS>(static_cast<const float*>(x), m, packed, scales, biases, n, kb, gshift,
                                  static_cast<float*>(y), stream);
    return launch_bf16_m<BITS, false>(static_cast<const uint16_t*>(x), m, packed, scales, biases, n, kb, gshift,
                                      static_cast<uint16_t*>(y), GemvFused{}, stream);
}

// ---- gathered batches: grid z = output batch, in launches of at most 65535 batches ----------------

template <typename Launch>
hipError_t over_batches(const Gather& ga, Launch&& launch) {
    for (uint64_t b0 = 0; b0 < ga.batch; b0 += 65535) {
        Gather g = ga;
        g.b0 = (uint32_t)b0;
        const unsigned gz = (unsigned)(ga.batch - b0 < 65535 ? ga.batch - b0 : 65535);
        const hipError_t e = launch(g, gz);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int BITS, int MB, int RPW, int WAVES, int P>
hipError_t launch_bf16_gather_p(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                                const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, uint16_t* y,
                                const Gather& ga, hipStream_t stream) {
    const unsigned gx = (unsigned)((n + WAVES * RPW - 1) / (WAVES * RPW));
    return over_batches(ga, [&](const Gather& g, unsigned gz) {
        return over_m_slices(m, MB, [&](int64_t m_off, int64_t mm, unsigned gy) {
            gemv_bf16_kernel<BITS, MB, RPW, WAVES, P, false, true><<<dim3(gx, gy, gz), dim3(WAVES * 64), 0, stream>>>(
                x + (size_t)m_off * kb * 32, (uint32_t)mm, packed, scales, biases, (uint32_t)n,
                (uint32_t)kb, gshift, y + (size_t)m_off * n, GemvFused{}, g);
        });
    });
}

template <int BITS, int MB, int RPW, int WAVES>
hipError_t launch_bf16_gather(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                              const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, uint16_t* y,
                              const Gather& ga, hipStream_t stream) {
    if (kLongPass<MB> > 2 && kb > 128)
        return launch_bf16_gather_p<BITS, MB, RPW, WAVES, kLongPass<MB>>(x, m, packed, scales, biases, n, kb,
                                                                        gshift, y, ga, stream);
    return launch_bf16_gather_p<BITS, MB, RPW, WAVES, 2>(x, m, packed, scales, biases, n, kb, gshift, y, ga, stream);
}

template <int BITS, int MB>
hipError_t launch_f32_gather(const float* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                             const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, float* y,
                             const Gather& ga, hipStream_t stream) {
    constexpr int RW = 2;
    const unsigned gx = (unsigned)((n + kWaves * RW - 1) / (kWaves * RW));
    return over_batches(ga, [&](const Gather& g, unsigned gz) {
        return over_m_slices(m, MB, [&](int64_t m_off, int64_t mm, unsigned gy) {
            gemv_f32_kernel<BITS, MB, RW, true><<<dim3(gx, gy, gz), dim3(kThreads), 0, stream>>>(
                x + (size_t)m_off * kb * 32, (uint32_t)mm, packed, scales, biases, (uint32_t)n,
                (uint32_t)kb, gshift, y + (size_t)m_off * n, g);
        });
    });
}

template <int BITS>
hipError_t launch_gather_bits(const void* x, bool x_f32, int64_t m, const uint32_t* packed,
                              const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t kb,
                              uint32_t gshift, void* y, const Gather& g, hipStream_t stream) {
    if (x_f32) {
        const float* xf = static_cast<const float*>(x);
        float* yf = static_cast<float*>(y);
        if (m == 1) return launch_f32_gather<BITS, 1>(xf, m, packed, scales, biases, n, kb, gshift, yf, g, stream);
        if (m == 2) return launch_f32_gather<BITS, 2>(xf, m, packed, scales, biases, n, kb, gshift, yf, g, stream);
        return launch_f32_gather<BITS, 4>(xf, m, packed, scales, biases, n, kb, gshift, yf, g, stream);
    }
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    uint16_t* yb = static_cast<uint16_t*>(y);
    if (m == 1)
        return launch_bf16_gather<BITS, 1, kRpw1, kWaves1>(xb, m, packed, scales, biases, n, kb, gshift, yb, g, stream);
    if (m == 2)
        return launch_bf16_gather<BITS, 2, kRpwN, kWavesN>(xb, m, packed, scales, biases, n, kb, gshift, yb, g, stream);
    if (m <= 4)
        return launch_bf16_gather<BITS, 4, kRpwN, kWavesN>(xb, m, packed, scales, biases, n, kb, gshift, yb, g, stream);
    return launch_bf16_gather<BITS, 8, kRpwN, kWavesN>(xb, m, packed, scales, biases, n, kb, gshift, yb, g, stream);
}

}  // namespace

hipError_t launch_gemv_gather(const void* x, bool x_f32, int64_t m, const uint32_t* packed,
                              const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                              int group_size, int bits, void* y, const Gather& g, hipStream_t stream) {
    const int64_t kb = k / 32;
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    switch (bits) {
        case 1: return launch_gather_bits<1>(x, x_f32, m, packed, scales, biases, n, kb, gshift, y, g, stream);
        case 2: return launch_gather_bits<2>(x, x_f32, m, packed, scales, biases, n, kb, gshift, y, g, stream);
        case 3: return launch_gather_bits<3>(x, x_f32, m, packed, scales, biases, n, kb, gshift, y, g, stream);
        case 4: return launch_gather_bits<4>(x, x_f32, m, packed, scales, biases, n, kb, gshift, y, g, stream);
        case 5: return launch_gather_bits<5>(x, x_f32, m, packed, scales, biases, n, kb, gshift, y, g, stream);
        case 6: return launch_gather_bits<6>(x, x_f32, m, packed, scales, biases, n, kb, gshift, y, g, stream);
        case 8: return launch_gather_bits<8>(x, x_f32, m, packed, scales, biases, n, kb, gshift, y, g, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv(const void* x, bool x_f32, int64_t m, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                       int group_size, int bits, void* y, hipStream_t stream) {
    const int64_t kb = k / 32;
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    switch (bits) {
        case 1: return launch_bits<1>(x, x_f32, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 2: return launch_bits<2>(x, x_f32, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 3: return launch_bits<3>(x, x_f32, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 4: return launch_bits<4>(x, x_f32, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 5: return launch_bits<5>(x, x_f32, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 6: return launch_bits<6>(x, x_f32, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 8: return launch_bits<8>(x, x_f32, m, packed, scales, biases, n, kb, gshift, y, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_f16(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                           const uint16_t* biases, int64_t n, int64_t k, int group_size, int bits, uint16_t* y,
                           hipStream_t stream) {
    const int64_t kb = k / 32;
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    const GemvFused f{};
    switch (bits) {
        case 1: return launch_bf16_m<1, false, 1>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
        case 2: return launch_bf16_m<2, false, 1>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
        case 3: return launch_bf16_m<3, false, 1>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
        case 4: return launch_bf16_m<4, false, 1>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
        case 5: return launch_bf16_m<5, false, 1>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
        case 6: return launch_bf16_m<6, false, 1>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
        case 8: return launch_bf16_m<8, false, 1>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_fused(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                             const uint16_t* biases, int64_t n, int64_t k, int group_size, int bits,
                             uint16_t* y, const GemvFused& f, hipStream_t stream) {
    const int64_t kb = k / 32;
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    switch (bits) {
        case 1: return launch_bf16_m<1, true>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
        case 2: return launch_bf16_m<2, true>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
        case 3: return launch_bf16_m<3, true>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
        case 4: return launch_bf16_m<4, true>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
        case 5: return launch_bf16_m<5, true>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
        case 6: return launch_bf16_m<6, true>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
        case 8: return launch_bf16_m<8, true>(x, m, packed, scales, biases, n, kb, gshift, y, f, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qaff
