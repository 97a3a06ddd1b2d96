// Quantized decode matmul on the matrix cores: y[m, n] = sum_k x[m, k] * w[n, k] for a few rows
// of a bf16 x (the decode path of spark_runtime weights/mlx_int8.rs, `gemv`, at m > 1; the
// product itself is nuvec_core quantized.rs, `quantized_matmul` with transpose). W is never
// materialised: each code is dequantized once, in registers, straight into an MFMA operand.
//
// On the VALU the work per code grows with m (one multiply per code and x row, and the x values
// through LDS), so from a few rows on the VALU, not HBM, sets the time. Here
// v_mfma_f32_16x16x32_bf16 takes all (up to 16) x rows at once, and the VALU work per code is
// the dequantization alone: w = s c + b rounded to bf16, as in the prefill GEMM (dequant8m: 4- and
// 8-bit codes enter a mixed-precision multiply-add as float16 mantissas).
//
// Layout of the work:
//  * A block of `kb / 16` waves owns 16 * NT rows of W (NT tiles of 16 rows) and all of K; wave w
//    takes the K slice [512 w, 512 w + 512): four chunks of 128 codes.
//  * In chunk c, lane (r, g) = (l % 16, l / 16) of tile t holds the whole 32-code block 4 c + g of
//    row 16 t + r (BITS words, one load). MFMA j of the chunk takes codes 8 j .. 8 j + 7 of every
//    lane's block, i.e. K is visited in the order (chunk, j, g, e). The x operand follows the same
//    order: lane (r, g) supplies x[r][128 c + 32 g + 8 j + e]. The 16x16x32 operand layout: lane l
//    supplies row l % 16 of A (x) and of W, the 8 values at k-slot l / 16; result value v of lane l
//    is D[4 (l / 16) + v][l % 16].
//  * Each wave loads its slice of the x rows (m rounded up to 4, 8 or 16: a compile-time count
//    keeps the loaded rows in fixed registers) with one contiguous 1 KB load per row and stores
//    it into its own LDS region, from which the lanes read their operands; no barrier is needed
//    before the multiply. (LDS-direct copies would skip the registers, but the compiler can only
//    wait for every outstanding load before reading LDS they wrote.)
//  * Scales and biases of a tile row come as one window over the slice (16, 8 or 4 groups),
//    not one load per block: small scattered loads were a third of the time.
//  * The slices' float32 partial tiles are summed through LDS at the end.
//  * Exact 4-bit codes (x rows rounded to 4 with any group size, to 8 with groups of 64 or 128,
//    to 16 with groups of 128): a chunk's 4 >> log2(G / 32) groups each get a band of MB of the 16
//    operand rows, in which only the lanes whose k-slot lies in that group read x (the others read
//    a zeroed LDS area). Each result lane then holds the sums of a single group, so the codes can
//    enter unscaled, as bf16 128 + c (one AND-OR per pair of codes), and the group's scale and bias
//    are applied to the sums: s D + (b / 128 - s) X, with X = sum x 128 from one more MFMA per
//    step against a constant 128 (shared by the tiles). The bands are added in the final sum.
//    The weights are then not rounded to bf16: the result is the float32 product of the oracle.
//  * Past 4096 codes, each wave takes several slices in turn (gemv_mfma_long_kernel).
//  * The 16-bit format (bf16 or float16, mfma16.h) is a template parameter: x, scales, biases and y
//    in it, and the operands of v_mfma_f32_16x16x32_bf16 or _f16.
// Requirements (checked by the caller): K a multiple of 512 and at most 32768 (4096 for the gathered
// kernel).
#pragma once

#include "launch.h"
#include "mfma16.h"

#include <hip/hip_runtime.h>

namespace qaff {
namespace {

constexpr int kSlice = 512;                // codes of K per wave (per slice past 4096 codes)
constexpr int64_t kMaxK = 64 * kSlice;       // longest K taken: 8 waves of 8 slices (the narrow blocks)

// v_cndmask_b32 with a lane mask: `if_set` in the lanes of `mask`, `if_clear` elsewhere.
__device__ __forceinline__ uint32_t lane_select(uint64_t mask, uint32_t if_set, uint32_t if_clear) {
    uint32_t r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(if_clear), "v"(if_set), "s"(mask));
    return r;
}

constexpr int kXPitch = 2 * kSlice + 16;  // bytes per x row in a wave's LDS region (banks: see below)

// A row's scales (biases) over one slice: 16, 8 or 4 groups, loaded whole (32, 16 or 8 bytes).
template <int GSHIFT, bool F16>
struct SbWindow {
    static constexpr int kWords = 8 >> GSHIFT;
    uint32_t w[kWords];
    __device__ __forceinline__ void load(const uint16_t* p) {
        if constexpr (kWords == 8) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(p);
            const u32x4 b = *reinterpret_cast<const u32x4*>(p + 8);
            w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
        } else if constexpr (kWords == 4) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(p);
            w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        } else {
            const u32x2 a = *reinterpret_cast<const u32x2*>(p);
            w[0] = a.x; w[1] = a.y;
        }
    }
    // float32 value of the group of block 4 c + g (c compile-time, g = lane / 16)
    __device__ __forceinline__ float get(int c, int g, uint64_t g_hi) const {
        uint32_t word, sh;
        if constexpr (GSHIFT == 0) {         // group 4 c + g: word 2 c + g / 2, half g % 2
            word = lane_select(g_hi, w[2 * c + 1], w[2 * c]);
            sh = 16u * (uint32_t)(g & 1);
        } else if constexpr (GSHIFT == 1) {  // group 2 c + g / 2: word c, half g / 2
            word = w[c];
            sh = 16u * (uint32_t)(g >> 1);
        } else {                             // group c: word c / 2, half c % 2
            word = w[c >> 1];
            sh = 16u * (uint32_t)(c & 1);
        }
        return half_to_f32<F16>(word >> sh);
    }
};

// ---- exact 4-bit codes ---------------------------------------------------------------------------

// Whether the codes enter exactly: every group of a chunk (4 >> GSHIFT of them) needs a band of MB
// of the 16 operand rows.
template <int BITS, int GSHIFT, int MB>
constexpr bool kExactCodes = BITS == 4 && (4 >> GSHIFT) * MB <= 16;

// The exact codes enter as B + c: B = 128 in bf16 (7 mantissa bits, so c < 128 is exact), 1024 in
// float16 (10 mantissa bits). kExactBase is B in both halves of a word, kExactInv 1 / B.
template <bool F16> constexpr uint32_t kExactBase = F16 ? 0x64006400u : 0x43004300u;
template <bool F16> constexpr float kExactInv = F16 ? 1.0f / 1024.0f : 1.0f / 128.0f;

// The constants of the exact operands: the code mask in a scalar register and B (both halves) in a
// vector register, for one v_and_or_b32 per pair of codes, and the all-B operand.
template <bool F16>
struct ExactConsts {
    uint32_t mask, base;
    op8<F16> kbase;
};
template <bool F16>
__device__ __forceinline__ ExactConsts<F16> make_exact_consts() {
    uint32_t base = kExactBase<F16>;
    asm volatile("" : "+v"(base));  // kept in a register: the AND-OR takes it as its third operand
    constexpr uint32_t b = kExactBase<F16>;
    return ExactConsts<F16>{(uint32_t)__builtin_amdgcn_readfirstlane(0x000F000F), base,
                            __builtin_bit_cast(op8<F16>, u32x4a{b, b, b, b})};
}

// The eight 4-bit codes of a word as exact values B + c in the pair order (c0, c4), (c1, c5),
// (c2, c6), (c3, c7): the codes go into the mantissas of B. Plain C on purpose: this value is
// an MFMA operand, and the compiler keeps the wait states that a matrix instruction needs after a
// VALU write of its operand only behind instructions it emitted itself, not behind inline asm (a
// v_xor_b32 in asm got one wait state before the MFMA reading its result, the same instruction
// compiled from C two).
template <bool F16>
__device__ __forceinline__ op8<F16> codes4_exact(uint32_t w, const ExactConsts<F16>& e) {
    return __builtin_bit_cast(op8<F16>, u32x4a{(w & e.mask) | e.base, ((w >> 4) & e.mask) | e.base,
                                             ((w >> 8) & e.mask) | e.base, ((w >> 12) & e.mask) | e.base});
}

// Eight bf16 values x0..x7 (four words, natural order) in that pair order: x0 x4 x1 x5 x2 x6 x3 x7.
__device__ __forceinline__ u32x4a pair_order4(u32x4a v) {
    return u32x4a{__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                  __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u)};
}

// Lane (r, g)'s x operand: row min(r, MB - 1) of its wave's LDS region at k-slot g; with exact
// codes, row r % MB of band r / MB, which reads x only where the band is the group of the lane's
// k-slot (g >> GSHIFT) and the zeroed area elsewhere.
template <int GSHIFT, int MB, bool EXACT>
__device__ __forceinline__ const uint8_t* x_operand(const uint8_t* xl, const uint8_t* zero, int lr16, int lg) {
    if constexpr (!EXACT) {
        return xl + min(lr16, MB - 1) * kXPitch + lg * 64;
    } else {
        const int band = lr16 / MB, r = lr16 % MB;
        return band == (lg >> GSHIFT) ? xl + r * kXPitch + lg * 64 : zero + lg * 64;
    }
}

// The window selector of the group whose scale and bias a result lane takes: the lane's own block
// (lane / 16) for dequantized codes; with exact codes, the band of its result rows 4 (lane / 16) ..
// + 3, as a block index of that group (bands past the chunk's groups hold zeros: any group will do).
template <int GSHIFT, int MB, bool EXACT>
__device__ __forceinline__ int fold_selector(int lg) {
    if constexpr (!EXACT) return lg;
    const int band = (4 * lg) / MB;
    return (band & ((4 >> GSHIFT) - 1)) << GSHIFT;
}

// Chunk c of the multiply: acc[t] += x_chunk . w_chunk(tile t)^T, from the codes wq[t][c] of each
// tile, its scale and bias windows and the x operand at xa (see x_operand), dequantized (scale and
// bias per lane) or exact (scale and bias per band, on the MFMA sums).
template <int BITS, int NT, int GSHIFT, int MB, bool F16>
__device__ __forceinline__ void chunk_product(int c, const uint32_t (&wq)[NT][4][BITS],
                                              const SbWindow<GSHIFT, F16> (&sw)[NT], const SbWindow<GSHIFT, F16> (&bw)[NT],
                                              const uint8_t* xa, int sel, uint64_t sel_hi, const ExactConsts<F16>& ec,
                                              f32x4 (&acc)[NT]) {
    if constexpr (kExactCodes<BITS, GSHIFT, MB>) {
        f32x4 d[NT];
        f32x4 dx = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NT; ++t) d[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const op8<F16> a = *reinterpret_cast<const op8<F16>*>(xa + 256 * c + 16 * j);
#pragma unroll
            for (int t = 0; t < NT; ++t) d[t] = mfma16x16x32<F16>(a, codes4_exact<F16>(wq[t][c][j], ec), d[t]);
            dx = mfma16x16x32<F16>(a, ec.kbase, dx);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            // sum x (s c + b) = s sum x (B + c) + (b / B - s) sum x B
            const float s = sw[t].get(c, sel, sel_hi);
            const float beta = __builtin_fmaf(bw[t].get(c, sel, sel_hi), kExactInv<F16>, -s);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[t][v] = __builtin_fmaf(s, d[t][v], __builtin_fmaf(beta, dx[v], acc[t][v]));
        }
    } else {
        op8<F16> wb[NT][4];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const Dq dq = make_dq(sw[t].get(c, sel, sel_hi), bw[t].get(c, sel, sel_hi));
#pragma unroll
            for (int j = 0; j < 4; ++j) wb[t][j] = dequant_op<F16, BITS>(wq[t][c], j, dq);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const op8<F16> a = *reinterpret_cast<const op8<F16>*>(xa + 256 * c + 16 * j);
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = mfma16x16x32<F16>(a, wb[t][j], acc[t]);
        }
    }
}

// Extra LDS of the exact-code kernels: the zeroed x area (1 KB: k-slot offsets up to 64 * 3 plus
// a chunk's 1 KB of steps).
template <int BITS, int GSHIFT, int MB>
constexpr size_t kZeroBytes = kExactCodes<BITS, GSHIFT, MB> ? 1024 : 0;

template <int BITS, int NT, int GSHIFT, int MB, bool F16>
__global__ __launch_bounds__(512) void gemv_mfma_kernel(
    const uint16_t* x, uint32_t m, const uint32_t* packed, const uint16_t* scales,
    const uint16_t* biases, uint32_t n, uint32_t kb, uint16_t* y, uint32_t red_off) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int waves = (int)(kb >> 4);
    const uint32_t n0 = blockIdx.x * (16 * NT);
    const uint32_t k = kb * 32;
    const uint32_t gpr = kb >> GSHIFT;  // groups per row
    const int lr16 = lane & 15;
    const int lg = lane >> 4;

    // 1. Loads, oldest first: this wave's slice of every x row (one contiguous 1 KB load per row),
    //    then per tile the scale and bias windows and, chunk by chunk, the W blocks, so that each
    //    chunk waits only for what it uses.
    // MB = m rounded up to 4, 8 or 16; rows past m repeat row m - 1 (their results are not stored)
    u32x4a xg[MB];
    const uint16_t* xs = x + (size_t)wave * kSlice + lane * 8;
#pragma unroll
    for (int r = 0; r < MB; ++r) xg[r] = *reinterpret_cast<const u32x4a*>(xs + (size_t)min((uint32_t)r, m - 1) * k);
    SbWindow<GSHIFT, F16> sw[NT], bw[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const uint32_t row = min(n0 + 16 * t + lr16, n - 1);
        const size_t e = (size_t)row * gpr + (size_t)wave * (16 >> GSHIFT);
        sw[t].load(scales + e);
        bw[t].load(biases + e);
    }
    uint32_t wq[NT][4][BITS];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t row = min(n0 + 16 * t + lr16, n - 1);
            const uint32_t jb = (uint32_t)wave * 16 + 4 * c + lg;
            const uint32_t* src = packed + (size_t)row * kb * BITS + (size_t)jb * BITS;
            if constexpr (BITS == 4) {
                // non-temporal (each weight is read once): decode M = 4 5.15 -> 4.83 us; the 3-
                // and 6-bit rows were slower with them, so only here
                const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
                wq[t][c][0] = v.x; wq[t][c][1] = v.y; wq[t][c][2] = v.z; wq[t][c][3] = v.w;
            } else {
                load_block<BITS>(src, wq[t][c]);
            }
        }
        asm volatile("" ::: "memory");  // chunk by chunk, in issue order
    }

    // 2. x into this wave's LDS region: row r at r * 1040 bytes, so the 16 rows that the operand
    //    read touches at one offset fall on distinct banks (1040 / 4 = 4 mod 64). Exact codes: each
    //    8-value unit in the codes' pair order, and the zeroed area after the regions (every wave
    //    writes the same zeros there before reading it).
    constexpr bool kExact = kExactCodes<BITS, GSHIFT, MB>;
    uint8_t* xl = smem + (size_t)wave * (MB * kXPitch);
    uint8_t* zero = smem + (size_t)waves * (MB * kXPitch);
#pragma unroll
    for (int r = 0; r < MB; ++r)
        *reinterpret_cast<u32x4a*>(xl + r * kXPitch + lane * 16) = kExact ? pair_order4(xg[r]) : xg[r];
    if constexpr (kExact) *reinterpret_cast<u32x4a*>(zero + lane * 16) = u32x4a{0u, 0u, 0u, 0u};
    const uint8_t* xa = x_operand<GSHIFT, MB, kExact>(xl, zero, lr16, lg);
    const int sel = fold_selector<GSHIFT, MB, kExact>(lg);
    const uint64_t sel_hi = __builtin_amdgcn_ballot_w64(sel >= 2);
    const ExactConsts<F16> ec = make_exact_consts<F16>();

    // 3. Multiply, chunk by chunk. Lane (r, g) of chunk c holds block 4 c + g of its row; MFMA j
    //    takes codes 8 j .. 8 j + 7 of each lane's block, and x in the same order.
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        // The empty asm makes chunk c's arithmetic start here, after every load is issued and
        // after chunk c - 1's multiply (its input): the compiler would otherwise hoist the cheap
        // scale selection of every chunk into the loads and wait for all of them there.
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < BITS; ++i) asm volatile("" : "+v"(wq[t][c][i]) : "v"(acc[0]));
        chunk_product<BITS, NT, GSHIFT, MB, F16>(c, wq, sw, bw, xa, sel, sel_hi, ec, acc);
    }

    // 4. Sum the slices' partial tiles (and the bands of exact codes) through LDS:
    //    [wave][tile][v][lane] float32, at byte red_off: past the x regions where the launcher gave
    //    the block that much LDS (no wave then waits for the others to finish with x before writing
    //    its tile), else over them (red_off = 0).
    constexpr int kBands = kExact ? (4 >> GSHIFT) : 1;
    if (red_off == 0) __syncthreads();  // every wave is done with its x rows
    float* red = reinterpret_cast<float*>(smem + red_off);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[((wave * NT + t) * 4 + v) * 64 + lane] = acc[t][v];
    __syncthreads();
    for (int o = tid; o < 16 * MB * NT; o += (int)blockDim.x) {
        const int t = o / (16 * MB), rem = o % (16 * MB);
        const int mm = rem >> 4, nn = rem & 15;
        float sum = 0.f;
#pragma unroll
        for (int p = 0; p < kBands; ++p) {
            const int rr = p * MB + mm;
            const int l = ((rr >> 2) << 4) | nn, v = rr & 3;
            for (int w = 0; w < waves; ++w) sum += red[((w * NT + t) * 4 + v) * 64 + l];
        }
        const uint32_t row = n0 + 16 * t + nn;
        if ((uint32_t)mm < m && row < n) y[(size_t)mm * n + row] = f32_to_half_bits<F16>(sum);
    }
}

// Blocks of `bytes` of LDS that fit on a compute unit (at most 4: the kernels' launches assume no
// more).
inline int64_t blocks_per_cu(size_t bytes) {
    const int64_t b = (int64_t)(160 * 1024) / (int64_t)bytes;
    return b < 1 ? 1 : (b > 4 ? 4 : b);
}

// LDS of a block and the offset of its reduction area: past the x regions when the sum fits a
// block's LDS and keeps as many blocks on a compute unit, else over them (offset 0).
inline size_t reduction_layout(size_t regions, size_t red, uint32_t* red_off) {
    if (regions + red <= (size_t)(160 * 1024) && blocks_per_cu(regions + red) >= blocks_per_cu(regions)) {
        *red_off = (uint32_t)regions;
        return regions + red;
    }
    *red_off = 0;
    return regions > red ? regions : red;
}

template <int BITS, int NT, int GSHIFT, int MB, bool F16>
hipError_t launch_nt(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                     const uint16_t* biases, int64_t n, int64_t kb, uint16_t* y, hipStream_t stream) {
    const int waves = (int)(kb / 16);
    uint32_t red_off;
    const size_t lds = reduction_layout((size_t)waves * MB * kXPitch + kZeroBytes<BITS, GSHIFT, MB>,
                                        (size_t)waves * NT * 4 * 64 * sizeof(float), &red_off);
    const unsigned blocks = (unsigned)((n + 16 * NT - 1) / (16 * NT));
    gemv_mfma_kernel<BITS, NT, GSHIFT, MB, F16><<<dim3(blocks), dim3(waves * 64), lds, stream>>>(
        x, (uint32_t)m, packed, scales, biases, (uint32_t)n, (uint32_t)kb, y, red_off);
    return hipGetLastError();
}

// ---- K past 4096 ---------------------------------------------------------------------------------
//
// The same tiles and slices over a longer K (the down projection's 14336 codes): a block of up to 16
// waves owns 16 * NT rows (NT = 1 is launched), and wave w takes the slices [w S, min(w S + S,
// K / 512)) one after another. While it multiplies one slice, the loads of the next (x rows, scale
// and bias windows, codes) are in flight, in a second set of registers: the loop is unrolled by two
// so that the two sets swap roles without copies. Each slice's x rows go through the wave's LDS region as in the
// kernel above (LDS operations of one wave complete in order, so the next slice's stores follow
// the reads of the last one without a wait).

template <int BITS, int NT, int GSHIFT, int MB, bool F16>
struct SliceLoads {
    u32x4a xg[MB];
    SbWindow<GSHIFT, F16> sw[NT], bw[NT];
    uint32_t wq[NT][4][BITS];
};

// Issue the loads of slice s, oldest first: the x rows (rows past m repeat row m - 1), the scale
// and bias windows of each tile, then the codes chunk by chunk. A slice that is not `real` (past
// the wave's last) issues the same loads at harmless addresses whose results go unused: x rows of
// slice s_last, codes and windows from the start of x (32 bytes per lane; x holds more than 8 KB
// here). The loop below then has the same loads outstanding on every path.
template <int BITS, int NT, int GSHIFT, int MB, bool F16>
__device__ __forceinline__ void load_slice(SliceLoads<BITS, NT, GSHIFT, MB, F16>& L, const uint16_t* x, uint32_t m,
                                           const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                                           uint32_t n, uint32_t n0, uint32_t kb, int s, int s_last, int lane) {
    const bool real = s <= s_last;
    const uint32_t k = kb * 32, gpr = kb >> GSHIFT;
    const int lr16 = lane & 15, lg = lane >> 4;
    const uint16_t* xs = x + (size_t)(real ? s : s_last) * kSlice + lane * 8;
#pragma unroll
    for (int r = 0; r < MB; ++r) L.xg[r] = *reinterpret_cast<const u32x4a*>(xs + (size_t)min((uint32_t)r, m - 1) * k);
    const uint16_t* dummy = x + lane * 16;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const uint32_t row = min(n0 + 16 * t + lr16, n - 1);
        const size_t e = (size_t)row * gpr + (size_t)s * (16 >> GSHIFT);
        L.sw[t].load(real ? scales + e : dummy);
        L.bw[t].load(real ? biases + e : dummy);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t row = min(n0 + 16 * t + lr16, n - 1);
            const uint32_t jb = (uint32_t)s * 16 + 4 * c + lg;
            const uint32_t* src = real ? packed + (size_t)row * kb * BITS + (size_t)jb * BITS
                                       : reinterpret_cast<const uint32_t*>(dummy);
            if constexpr (BITS == 4) {
                const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
                L.wq[t][c][0] = v.x; L.wq[t][c][1] = v.y; L.wq[t][c][2] = v.z; L.wq[t][c][3] = v.w;
            } else {
                load_block<BITS>(src, L.wq[t][c]);
            }
        }
        asm volatile("" ::: "memory");
    }
}

// The multiply of one loaded slice: its x rows into the wave's LDS region (exact codes: in the
// codes' pair order), then the four chunks.
template <int BITS, int NT, int GSHIFT, int MB, bool F16>
__device__ __forceinline__ void slice_product(SliceLoads<BITS, NT, GSHIFT, MB, F16>& L, uint8_t* xl, const uint8_t* xa,
                                              int sel, uint64_t sel_hi, const ExactConsts<F16>& ec, f32x4 (&acc)[NT],
                                              int lane) {
    constexpr bool kExact = kExactCodes<BITS, GSHIFT, MB>;
#pragma unroll
    for (int r = 0; r < MB; ++r)
        *reinterpret_cast<u32x4a*>(xl + r * kXPitch + lane * 16) = kExact ? pair_order4(L.xg[r]) : L.xg[r];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        // chunk c's arithmetic starts after chunk c - 1's multiply (see the kernel above)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < BITS; ++i) asm volatile("" : "+v"(L.wq[t][c][i]) : "v"(acc[0]));
        chunk_product<BITS, NT, GSHIFT, MB, F16>(c, L.wq, L.sw, L.bw, xa, sel, sel_hi, ec, acc);
    }
}

// Whether a block may take 16 waves (1024 threads, hence at most 128 registers per lane): where the
// two register sets fit in them without spills (from the compiler's register reports). Twice the
// waves keep twice the loads in flight on a compute unit; the others take 8.
template <int BITS, int GSHIFT, int MB>
constexpr bool kWideBlock = MB == 4   ? !(BITS == 8 && GSHIFT == 0)
                            : MB == 8 ? (BITS <= 2 || ((BITS == 3 || BITS == 4) && GSHIFT >= 1))
                                      : false;

template <int BITS, int NT, int GSHIFT, int MB, int S, bool F16>
__global__ __launch_bounds__((kWideBlock<BITS, GSHIFT, MB> ? 1024 : 512)) void gemv_mfma_long_kernel(
    const uint16_t* x, uint32_t m, const uint32_t* packed, const uint16_t* scales,
    const uint16_t* biases, uint32_t n, uint32_t kb, uint16_t* y, uint32_t red_off) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int waves = (int)(blockDim.x >> 6);
    const uint32_t n0 = blockIdx.x * (16 * NT);
    const int lr16 = lane & 15;
    const int lg = lane >> 4;
    // every wave has at least one slice: the launcher takes waves = ceil(slices / S)
    const int s0 = wave * S;
    const int s1 = min(s0 + S, (int)(kb >> 4));

    constexpr bool kExact = kExactCodes<BITS, GSHIFT, MB>;
    uint8_t* xl = smem + (size_t)wave * (MB * kXPitch);
    uint8_t* zero = smem + (size_t)waves * (MB * kXPitch);
    if constexpr (kExact) *reinterpret_cast<u32x4a*>(zero + lane * 16) = u32x4a{0u, 0u, 0u, 0u};
    const uint8_t* xa = x_operand<GSHIFT, MB, kExact>(xl, zero, lr16, lg);
    const int sel = fold_selector<GSHIFT, MB, kExact>(lg);
    const uint64_t sel_hi = __builtin_amdgcn_ballot_w64(sel >= 2);
    const ExactConsts<F16> ec = make_exact_consts<F16>();

    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Two register sets in turn: while one slice is multiplied, the next one's loads are in flight
    // (past the wave's last slice, loads that go unused: see load_slice). Unrolled in full: the
    // compiler's waits before each multiply then cover that slice's loads alone (around a loop
    // back-edge it also waited for the other set's).
    SliceLoads<BITS, NT, GSHIFT, MB, F16> a, b;
    const int last = s1 - 1;
    load_slice(a, x, m, packed, scales, biases, n, n0, kb, s0, last, lane);
#pragma unroll
    for (int i = 0; i < S; i += 2) {
        if (i + 1 < S) load_slice(b, x, m, packed, scales, biases, n, n0, kb, s0 + i + 1, last, lane);
        if (s0 + i <= last) slice_product(a, xl, xa, sel, sel_hi, ec, acc, lane);
        if (i + 1 < S) {
            if (i + 2 < S) load_slice(a, x, m, packed, scales, biases, n, n0, kb, s0 + i + 2, last, lane);
            if (s0 + i + 1 <= last) slice_product(b, xl, xa, sel, sel_hi, ec, acc, lane);
        }
    }

    // the waves' partial tiles (and the bands of exact codes) summed through LDS, as above
    constexpr int kBands = kExact ? (4 >> GSHIFT) : 1;
    if (red_off == 0) __syncthreads();  // every wave is done with its x rows
    float* red = reinterpret_cast<float*>(smem + red_off);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[((wave * NT + t) * 4 + v) * 64 + lane] = acc[t][v];
    __syncthreads();
    for (int o = tid; o < 16 * MB * NT; o += (int)blockDim.x) {
        const int t = o / (16 * MB), rem = o % (16 * MB);
        const int mm = rem >> 4, nn = rem & 15;
        float sum = 0.f;
#pragma unroll
        for (int p = 0; p < kBands; ++p) {
            const int rr = p * MB + mm;
            const int l = ((rr >> 2) << 4) | nn, v = rr & 3;
            for (int w = 0; w < waves; ++w) sum += red[((w * NT + t) * 4 + v) * 64 + l];
        }
        const uint32_t row = n0 + 16 * t + nn;
        if ((uint32_t)mm < m && row < n) y[(size_t)mm * n + row] = f32_to_half_bits<F16>(sum);
    }
}

template <int BITS, int GSHIFT, int MB, int S, bool F16>
hipError_t launch_long_s(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                         const uint16_t* biases, int64_t n, int64_t kb, uint16_t* y, hipStream_t stream) {
    const int64_t waves = (kb / 16 + S - 1) / S;
    uint32_t red_off;
    const size_t lds = reduction_layout((size_t)waves * MB * kXPitch + kZeroBytes<BITS, GSHIFT, MB>,
                                        (size_t)waves * 4 * 64 * sizeof(float), &red_off);
    gemv_mfma_long_kernel<BITS, 1, GSHIFT, MB, S, F16><<<dim3((unsigned)((n + 15) / 16)), dim3((unsigned)waves * 64), lds,
                                                    stream>>>(x, (uint32_t)m, packed, scales, biases, (uint32_t)n,
                                                              (uint32_t)kb, y, red_off);
    return hipGetLastError();
}

template <int BITS, int GSHIFT, int MB, bool F16>
hipError_t launch_long(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                       const uint16_t* biases, int64_t n, int64_t kb, uint16_t* y, hipStream_t stream) {
    // S slices per wave (2, 4 or 8), as few as the block's waves (16 or 8) allow, then as few waves
    // as S needs. One row tile per block: with two, the two register sets no longer fit without
    // spills, and n = 4096 already gives one block per compute unit.
    constexpr int64_t kWaves = kWideBlock<BITS, GSHIFT, MB> ? 16 : 8;
    const int64_t slices = kb / 16;
    if (slices <= 2 * kWaves) return launch_long_s<BITS, GSHIFT, MB, 2, F16>(x, m, packed, scales, biases, n, kb, y, stream);
    if (slices <= 4 * kWaves) return launch_long_s<BITS, GSHIFT, MB, 4, F16>(x, m, packed, scales, biases, n, kb, y, stream);
    return launch_long_s<BITS, GSHIFT, MB, 8, F16>(x, m, packed, scales, biases, n, kb, y, stream);
}

template <int BITS, int GSHIFT, int MB, bool F16>
hipError_t launch_g(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                    const uint16_t* biases, int64_t n, int64_t kb, uint16_t* y, hipStream_t stream) {
    if (kb > 8 * (kSlice / 32)) return launch_long<BITS, GSHIFT, MB, F16>(x, m, packed, scales, biases, n, kb, y, stream);
    // The kernel is latency-bound: all blocks should be resident at once. A block's LDS (its x
    // slices: MB x 1040 bytes per wave) sets how many fit on a compute unit; each block takes as
    // many 16-row tiles (1 to 4) as needed to cover n in one round of the compute units.
    const int64_t waves = kb / 16;
    int64_t per_cu = (int64_t)(160 * 1024) / (waves * MB * kXPitch + (int64_t)kZeroBytes<BITS, GSHIFT, MB>);
    if (per_cu < 1) per_cu = 1;
    if (per_cu > 4) per_cu = 4;
    const int64_t cus = device_cu_count();
    const int64_t slots = cus * per_cu;
    int64_t nt = (n + 16 * slots - 1) / (16 * slots);
    // 8-bit codes: more than two tiles of W (64 registers each) crowd out the waves that hide the
    // latency (measured: 8-bit M = 16 on [14336, 4096] 20 us at two tiles, 25 us at three)
    constexpr int kMaxNt = BITS == 8 ? 2 : 4;
    if (nt > kMaxNt) nt = kMaxNt;
    // The dequantization keeps the VALU busy, so the compute unit with the most rows sets the
    // time: among the tile counts that still fit one round, take the one that gives it the fewest
    // (3-bit [11008, 4096] at m = 8: three tiles, 48 rows per unit, where two tiles put 64 rows on
    // some units).
    auto busiest = [&](int64_t t) {
        const int64_t blocks = (n + 16 * t - 1) / (16 * t);
        const int64_t per = (blocks + cus - 1) / cus;
        return per > per_cu ? INT64_MAX : per * 16 * t;
    };
    for (int64_t t = 1; t <= kMaxNt; ++t)
        if (busiest(t) < busiest(nt)) nt = t;
    if (nt <= 1) return launch_nt<BITS, 1, GSHIFT, MB, F16>(x, m, packed, scales, biases, n, kb, y, stream);
    if (nt == 2) return launch_nt<BITS, 2, GSHIFT, MB, F16>(x, m, packed, scales, biases, n, kb, y, stream);
    if (nt == 3 || kMaxNt == 3) return launch_nt<BITS, 3, GSHIFT, MB, F16>(x, m, packed, scales, biases, n, kb, y, stream);
    return launch_nt<BITS, kMaxNt, GSHIFT, MB, F16>(x, m, packed, scales, biases, n, kb, y, stream);
}

template <int BITS, int GSHIFT, bool F16>
hipError_t launch_mb(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                     const uint16_t* biases, int64_t n, int64_t kb, uint16_t* y, hipStream_t stream) {
    if (m <= 4) return launch_g<BITS, GSHIFT, 4, F16>(x, m, packed, scales, biases, n, kb, y, stream);
    if (m <= 8) return launch_g<BITS, GSHIFT, 8, F16>(x, m, packed, scales, biases, n, kb, y, stream);
    return launch_g<BITS, GSHIFT, 16, F16>(x, m, packed, scales, biases, n, kb, y, stream);
}

template <int BITS, bool F16>
hipError_t launch_bits(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                       const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, uint16_t* y,
                       hipStream_t stream) {
    if (gshift == 0) return launch_mb<BITS, 0, F16>(x, m, packed, scales, biases, n, kb, y, stream);
    if (gshift == 1) return launch_mb<BITS, 1, F16>(x, m, packed, scales, biases, n, kb, y, stream);
    return launch_mb<BITS, 2, F16>(x, m, packed, scales, biases, n, kb, y, stream);
}

// ---- gathered batches ---------------------------------------------------------------------------
//
// The decode kernel's layout over gathered batches: a block owns 16 * NT rows of one weight batch
// and walks every x row that uses it, in tiles of MB rows; the codes stay in registers across the
// tiles (each tile dequantizes them again, chunk by chunk, as the decode kernel does).
//  * Batched: grid y = output batch b; x rows 0 .. m - 1 of batch lhs[b] against weight rhs[b].
//  * Grouped (rhs sorted, m == 1, no lhs): grid y = expert e; the rows of e are
//    [#(rhs < e), #(rhs < e + 1)), so each expert's weights are read once however many rows use
//    it. Expert w_count takes the rows past every expert (NaN).
// An out-of-range index gives a NaN output batch.

template <int BITS, int NT, int GSHIFT, int MB, bool F16>
__global__ __launch_bounds__(512) void gemv_mfma_gather_kernel(
    const uint16_t* x, uint32_t m, const uint32_t* packed, const uint16_t* scales,
    const uint16_t* biases, uint32_t n, uint32_t kb, uint16_t* y, Gather ga) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int waves = (int)(kb >> 4);
    const uint32_t n0 = blockIdx.x * (16 * NT);
    const uint32_t k = kb * 32;
    const uint32_t gpr = kb >> GSHIFT;
    const int lr16 = lane & 15;
    const int lg = lane >> 4;
    const uint32_t z = ga.b0 + blockIdx.y;

    // 1. This block's x rows [r0, r1) (row r at xb + r k, its output at yb + r n) and weight batch.
    uint32_t r0, r1, wi;
    const uint16_t* xb = x;
    uint16_t* yb = y;
    bool nan_rows;
    if (ga.grouped) {
        uint32_t s, t;
        count_below2(ga.rhs, ga.batch, z, z + 1, lane, s, t);
        r0 = s;
        r1 = z >= ga.w_count ? ga.batch : t;
        wi = z;
        nan_rows = z >= ga.w_count;
    } else {
        const uint32_t li = ga.lhs ? ga.lhs[z] : z;
        const uint32_t ri = ga.rhs ? ga.rhs[z] : z;
        r0 = 0;
        r1 = m;
        wi = ri;
        yb = y + (size_t)z * ga.y_stride;
        nan_rows = li >= ga.x_count || ri >= ga.w_count;
        if (!nan_rows) xb = x + (size_t)li * ga.x_stride;
    }
    if (r0 >= r1) return;  // the same in every wave: the whole block returns
    if (nan_rows) {
        for (uint32_t o = tid; o < (r1 - r0) * 16 * NT; o += blockDim.x) {
            const uint32_t col = n0 + o % (16 * NT);
            if (col < n) yb[(size_t)(r0 + o / (16 * NT)) * n + col] = F16 ? 0x7E00u : 0x7FC0u;  // quiet NaN
        }
        return;
    }
    const uint32_t* pw = packed + (size_t)wi * ga.w_stride;
    const uint16_t* sp = scales + (size_t)wi * ga.sb_stride;
    const uint16_t* bp = biases + (size_t)wi * ga.sb_stride;

    // 2. Loads, oldest first: the first x tile, the scale and bias windows, then the codes chunk
    //    by chunk (as in the decode kernel).
    u32x4a xg[MB];
    const uint16_t* xs = xb + (size_t)wave * kSlice + lane * 8;
#pragma unroll
    for (int r = 0; r < MB; ++r) xg[r] = *reinterpret_cast<const u32x4a*>(xs + (size_t)min(r0 + r, r1 - 1) * k);
    SbWindow<GSHIFT, F16> sw[NT], bw[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const uint32_t row = min(n0 + 16 * t + lr16, n - 1);
        const size_t e = (size_t)row * gpr + (size_t)wave * (16 >> GSHIFT);
        sw[t].load(sp + e);
        bw[t].load(bp + e);
    }
    uint32_t wq[NT][4][BITS];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t row = min(n0 + 16 * t + lr16, n - 1);
            const uint32_t jb = (uint32_t)wave * 16 + 4 * c + lg;
            load_block<BITS>(pw + (size_t)row * kb * BITS + (size_t)jb * BITS, wq[t][c]);
        }
        asm volatile("" ::: "memory");
    }

    // 3. Walk the x rows in tiles of MB: x through this wave's LDS region, the multiply chunk by
    //    chunk, and the slices' partial tiles (and the bands of exact codes) summed through a
    //    separate LDS area. Exact codes: x in the codes' pair order, and the zeroed area after the
    //    x regions (see the decode kernel).
    constexpr bool kExact = kExactCodes<BITS, GSHIFT, MB>;
    constexpr int kBands = kExact ? (4 >> GSHIFT) : 1;
    uint8_t* xl = smem + (size_t)wave * (MB * kXPitch);
    uint8_t* zero = smem + (size_t)waves * (MB * kXPitch);
    float* red = reinterpret_cast<float*>(zero + kZeroBytes<BITS, GSHIFT, MB>);
    if constexpr (kExact) *reinterpret_cast<u32x4a*>(zero + lane * 16) = u32x4a{0u, 0u, 0u, 0u};
    const uint8_t* xa = x_operand<GSHIFT, MB, kExact>(xl, zero, lr16, lg);
    const int sel = fold_selector<GSHIFT, MB, kExact>(lg);
    const uint64_t sel_hi = __builtin_amdgcn_ballot_w64(sel >= 2);
    const ExactConsts<F16> ec = make_exact_consts<F16>();
    for (uint32_t t0 = r0; t0 < r1; t0 += MB) {
        if (t0 != r0) {
#pragma unroll
            for (int r = 0; r < MB; ++r) xg[r] = *reinterpret_cast<const u32x4a*>(xs + (size_t)min(t0 + r, r1 - 1) * k);
        }
#pragma unroll
        for (int r = 0; r < MB; ++r)
            *reinterpret_cast<u32x4a*>(xl + r * kXPitch + lane * 16) = kExact ? pair_order4(xg[r]) : xg[r];
        f32x4 acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            // chunk c's arithmetic starts after chunk c - 1's multiply (see the decode kernel)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int i = 0; i < BITS; ++i) asm volatile("" : "+v"(wq[t][c][i]) : "v"(acc[0]));
            chunk_product<BITS, NT, GSHIFT, MB, F16>(c, wq, sw, bw, xa, sel, sel_hi, ec, acc);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[((wave * NT + t) * 4 + v) * 64 + lane] = acc[t][v];
        __syncthreads();
        // result rows past MB repeat row MB - 1: only the first MB are stored
        for (int o = tid; o < 16 * MB * NT; o += (int)blockDim.x) {
            const int t = o / (16 * MB), rem = o % (16 * MB);
            const int mm = rem >> 4, nn = rem & 15;
            float sum = 0.f;
#pragma unroll
            for (int p = 0; p < kBands; ++p) {
                const int rr = p * MB + mm;
                const int l = ((rr >> 2) << 4) | nn, v = rr & 3;
                for (int w = 0; w < waves; ++w) sum += red[((w * NT + t) * 4 + v) * 64 + l];
            }
            const uint32_t r = t0 + (uint32_t)mm, col = n0 + 16 * t + (uint32_t)nn;
            if (r < r1 && col < n) yb[(size_t)r * n + col] = f32_to_half_bits<F16>(sum);
        }
        __syncthreads();  // red is written again by the next tile
    }
}

template <int BITS, int NT, int GSHIFT, int MB, bool F16>
hipError_t launch_gather_nt(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                            const uint16_t* biases, int64_t n, int64_t kb, uint16_t* y, const Gather& ga,
                            hipStream_t stream) {
    const int waves = (int)(kb / 16);
    const size_t lds = (size_t)waves * MB * kXPitch + kZeroBytes<BITS, GSHIFT, MB> +
                       (size_t)waves * NT * 4 * 64 * sizeof(float);
    const unsigned gx = (unsigned)((n + 16 * NT - 1) / (16 * NT));
    // grid y: output batches, or experts 0 .. w_count when grouped
    const uint64_t count = ga.grouped ? (uint64_t)ga.w_count + 1 : ga.batch;
    for (uint64_t b0 = 0; b0 < count; b0 += 65535) {
        Gather g = ga;
        g.b0 = (uint32_t)b0;
        const unsigned gy = (unsigned)(count - b0 < 65535 ? count - b0 : 65535);
        gemv_mfma_gather_kernel<BITS, NT, GSHIFT, MB, F16><<<dim3(gx, gy), dim3(waves * 64), lds, stream>>>(
            x, (uint32_t)m, packed, scales, biases, (uint32_t)n, (uint32_t)kb, y, g);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int BITS, int GSHIFT, int MB, bool F16>
hipError_t launch_gather_mb(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                            const uint16_t* biases, int64_t n, int64_t kb, uint16_t* y, const Gather& ga,
                            hipStream_t stream) {
    // Row tiles per block as in the decode kernel: enough that the blocks with work fit in one
    // round of the compute units (a block's x regions set how many fit on one).
    const int64_t waves = kb / 16;
    int64_t per_cu = (int64_t)(160 * 1024) / (waves * MB * kXPitch + (int64_t)kZeroBytes<BITS, GSHIFT, MB> + waves * 4 * 1024);
    if (per_cu < 1) per_cu = 1;
    if (per_cu > 4) per_cu = 4;
    const int64_t slots = (int64_t)device_cu_count() * per_cu;
    const int64_t batches = ga.grouped ? (ga.batch < ga.w_count ? ga.batch : ga.w_count) : ga.batch;
    const int64_t tiles = ((n + 15) / 16) * (batches > 0 ? batches : 1);
    const int64_t nt = (tiles + slots - 1) / slots;
    // at most two tiles (measured on 128 experts of [768, 2048] 4-bit, 512 and 4096 sorted rows:
    // two tiles 40 and 86 us, four 43 and 116 us, one 42 and 114 us)
    if (nt <= 1) return launch_gather_nt<BITS, 1, GSHIFT, MB, F16>(x, m, packed, scales, biases, n, kb, y, ga, stream);
    return launch_gather_nt<BITS, 2, GSHIFT, MB, F16>(x, m, packed, scales, biases, n, kb, y, ga, stream);
}

template <int BITS, int GSHIFT, bool F16>
hipError_t launch_gather_g(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                           const uint16_t* biases, int64_t n, int64_t kb, uint16_t* y, const Gather& ga,
                           hipStream_t stream) {
    // rows per tile: m, or twice the mean number of rows per expert when grouped, so that most
    // experts take one tile (each tile dequantizes the weights again). Measured at 512 rows over
    // 128 experts (mean 4): 4 rows per tile 40 us, 8 rows 37 us, 16 rows 48 us.
    const int64_t rows = ga.grouped ? (2 * (int64_t)ga.batch + ga.w_count - 1) / (ga.w_count ? ga.w_count : 1) : m;
    if (rows <= 4) return launch_gather_mb<BITS, GSHIFT, 4, F16>(x, m, packed, scales, biases, n, kb, y, ga, stream);
    if (rows <= 8) return launch_gather_mb<BITS, GSHIFT, 8, F16>(x, m, packed, scales, biases, n, kb, y, ga, stream);
    return launch_gather_mb<BITS, GSHIFT, 16, F16>(x, m, packed, scales, biases, n, kb, y, ga, stream);
}

template <int BITS, bool F16>
hipError_t launch_gather_bits(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                              const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, uint16_t* y,
                              const Gather& ga, hipStream_t stream) {
    if (gshift == 0) return launch_gather_g<BITS, 0, F16>(x, m, packed, scales, biases, n, kb, y, ga, stream);
    if (gshift == 1) return launch_gather_g<BITS, 1, F16>(x, m, packed, scales, biases, n, kb, y, ga, stream);
    return launch_gather_g<BITS, 2, F16>(x, m, packed, scales, biases, n, kb, y, ga, stream);
}

// The entry points' dispatch on bits and group size (one format per translation unit).
template <bool F16>
hipError_t mfma_decode(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                       const uint16_t* biases, int64_t n, int64_t k, int group_size, int bits, uint16_t* y,
                       hipStream_t stream) {
    const int64_t kb = k / 32;
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    switch (bits) {
        case 1: return launch_bits<1, F16>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 2: return launch_bits<2, F16>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 3: return launch_bits<3, F16>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 4: return launch_bits<4, F16>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 5: return launch_bits<5, F16>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 6: return launch_bits<6, F16>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 8: return launch_bits<8, F16>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        default: return hipErrorInvalidValue;
    }
}

template <bool F16>
hipError_t mfma_gather(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                       const uint16_t* biases, int64_t n, int64_t k, int group_size, int bits, uint16_t* y,
                       const Gather& g, hipStream_t stream) {
    const int64_t kb = k / 32;
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    switch (bits) {
        case 1: return launch_gather_bits<1, F16>(x, m, packed, scales, biases, n, kb, gshift, y, g, stream);
        case 2: return launch_gather_bits<2, F16>(x, m, packed, scales, biases, n, kb, gshift, y, g, stream);
        case 3: return launch_gather_bits<3, F16>(x, m, packed, scales, biases, n, kb, gshift, y, g, stream);
        case 4: return launch_gather_bits<4, F16>(x, m, packed, scales, biases, n, kb, gshift, y, g, stream);
        case 5: return launch_gather_bits<5, F16>(x, m, packed, scales, biases, n, kb, gshift, y, g, stream);
        case 6: return launch_gather_bits<6, F16>(x, m, packed, scales, biases, n, kb, gshift, y, g, stream);
        case 8: return launch_gather_bits<8, F16>(x, m, packed, scales, biases, n, kb, gshift, y, g, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace qaff
