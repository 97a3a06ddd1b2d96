// Quantized GEMM on bf16 MFMA: Y[m, n] = sum_k X[m, k] * w[n, k] for many rows of X (the prefill
// path of spark_runtime weights/mlx_int8.rs, `gemm`, which that page leaves as an untiled
// reference; the product itself is nuvec_core quantized.rs, `quantized_matmul` with transpose).
//
// Compute-bound (about 2.3 kflop per byte at the prefill shape). One kernel design serves every
// shape: 128 x 256 tiles of Y with each W element dequantized once, in registers, by the wave that
// multiplies it (below); a split of K over blocks when the tiles are too few to fill the chip; and
// the same tile body over the rows of each expert for gathered products sorted by expert.
#pragma once

#include "launch.h"
#include "mfma16.h"

#include <hip/hip_runtime.h>

namespace qaff {
namespace {

constexpr int BK = 64;        // codes of K per step (two 32-code blocks)
constexpr int LDK = BK + 8;   // LDS row pitch of X in bf16 elements (padding spreads rows over banks)

// ---- 128 x 256 tiles with W dequantized into registers ------------------------------------------
//
// At the prefill shape the products above are held back by what runs beside the matrix cores --
// the dequantization on the VALU and the traffic through LDS -- and by the power it all draws, not
// by HBM. This kernel keeps W out of LDS: each W element is dequantized once, by the one wave that
// multiplies it, straight into a register operand.
//  * A 512-thread block owns a 128 (M) x 256 (N) tile of Y. Wave w owns W rows 32 w .. 32 w + 31 of
//    the tile and all 128 rows of X: four 32 x 32 tiles of Y along M.
//  * K goes in steps of 64 codes (two 32-code blocks). In a step, lane l = 32 h + r holds block h of
//    W row r (BITS words, one load), and MFMA kk (0..3) of the step contracts codes 8 kk .. 8 kk + 7
//    of every lane's block. X follows the same order: lane (r, h) supplies
//    x[row][64 t + 32 h + 8 kk + e], e = 0..7, from LDS (the MFMA sums over all its k slots, so any
//    order that X and W share is the same product).
//  * X tiles go through LDS, double buffered, rows padded to 72 bf16 so that 16 rows read at one
//    offset fall on distinct banks. X is loaded two steps ahead, W three steps ahead.
//  * Scales and biases come in windows of 8 groups (16 bytes per row and array), one window ahead.
// Against dequantizing W tiles into LDS this halves the VALU work per flop and removes the W tile's
// LDS stores and reads; two waves per SIMD still hide the latencies. 4- and 8-bit codes enter the
// multiply-add as float16 mantissas (dequant8m): at the prefill shape 234 -> 225 us sustained.
// (A 256 x 128 tile with one wave per SIMD, which dequantizes each W element for 256 rows of X,
// measured 257-263 us: at the power limit its clock rose to 2.15-2.28 GHz, but the matrix cores
// idled more, and it moves half again as many bytes per flop from L2.)
// Shapes: K a multiple of 64 * kDirectBody (so of 8 groups) with 16-byte aligned scales and biases
// takes the kernel as above. Every other K (a multiple of 32) or alignment (2 bytes) takes the
// GENERAL variant: scale windows loaded element by element, and the K-steps past the last whole
// 1024-code chunk done one at a time after the main loop, X chunks and W blocks past K zeroed
// (K = 11008: 260 us with the earlier 256 x 128 kernel that dequantized W into LDS). Rows of X
// beyond m and rows of W beyond n are clamped, not zeroed: they only reach outputs that are not
// stored.
// Split K (PARTIAL): with few tiles, grid y splits K into `splits` ranges of whole 1024-code
// chunks; block (tile, s) sums its range and stores the float32 tile to part[s][m][n], and
// sum_partials_kernel adds the ranges in order.
//
// The 16-bit format (bf16 or float16, mfma16.h) is a template parameter: x, scales, biases and y in
// it, W dequantized and rounded to it, v_mfma_f32_32x32x16_bf16 or _f16.
//
// MFMA 32x32x16 layout: lane l supplies row l % 32 of A and of W (column of B), each as 8 values of
// k slot l / 32; result value v of lane l is row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.

constexpr int DBM = 128;
constexpr int DBN = 256;
constexpr int kDirectThreads = 512;
constexpr int kDirectBody = 16;  // K-steps per loop iteration (scale windows are 4, 8 or 16 steps)

// One (32 SUB) x 256 tile of Y (SUB = 4: 128 rows; 2: 64 rows): rows m0 .. m0 + 32 SUB - 1 of
// x [m, k] (rows past m clamped, not stored) against W rows n0 .. n0 + 255 of [n, k], over the K-steps of split `split` of `splits` (all of K
// when not PARTIAL), stored as bf16 into y [m, n] or as float32 into part[split][m][n]. `xl` is the
// block's LDS for the X tiles; the call opens with a barrier so that the block can run tiles back
// to back.
template <int BITS, int GSHIFT, bool PARTIAL, int SUB, bool GENERAL, bool F16>
__device__ __forceinline__ void direct_tile(
    const uint16_t* x, uint32_t m, const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
    uint32_t n, uint32_t kb, uint16_t* y, uint32_t m0, uint32_t n0, float* part, uint32_t split, uint32_t splits,
    uint16_t (&xl)[2][DBM * LDK]) {
    constexpr int TM = 32 * SUB;                  // tile rows
    constexpr int P = 4 << GSHIFT;                // K-steps per window of 8 groups
    constexpr int XPT = TM * 8 / kDirectThreads;   // 16-byte X chunks per thread and step

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    __syncthreads();  // the previous tile's reads of xl are done

    const uint32_t k = kb * 32;
    const uint32_t gpr = kb >> GSHIFT;  // groups per row
    // This block's K range: 1024-code chunks [c0, c1) of the kb / 32 (all of them unless split).
    const uint32_t chunks = kb >> 5;
    const uint32_t c0 = PARTIAL ? (uint32_t)((uint64_t)split * chunks / splits) : 0u;
    const uint32_t c1 = PARTIAL ? (uint32_t)((uint64_t)(split + 1) * chunks / splits) : chunks;
    const uint32_t kt_off = c0 * kDirectBody;               // first K-step
    const uint32_t ktiles = (c1 - c0) * kDirectBody;        // K-steps of the range
    const uint32_t nwin = ktiles / P;                       // scale windows of the range

    // X: chunk (xkc) of rows xrow + 64 i; 32-bit offsets within the tile's rows.
    const uint16_t* xb = x + (size_t)m0 * k + (size_t)kt_off * 64;
    const int xrow = tid >> 3;
    const int xkc = tid & 7;
    uint32_t xo[XPT];
    int xa[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        xo[i] = (min(m0 + xrow + 64 * i, m - 1) - m0) * k + xkc * 8;
        xa[i] = (xrow + 64 * i) * LDK + xkc * 8;
    }
    // W row of this lane, its block h of each step, and its scale and bias windows.
    const uint32_t wrow = min(n0 + 32 * wave + (lane & 31), n - 1);
    const uint32_t* wp = packed + (size_t)wrow * kb * BITS + h * BITS + (size_t)kt_off * 2 * BITS;
    const uint16_t* sp = scales + (size_t)wrow * gpr + (kt_off / P) * 8;
    const uint16_t* bp = biases + (size_t)wrow * gpr + (kt_off / P) * 8;

    auto load_x = [&](u32x4a (&xr)[XPT], uint32_t kt) {
        const uint16_t* p = xb + min(kt, ktiles - 1) * 64;
#pragma unroll
        for (int i = 0; i < XPT; ++i) xr[i] = *reinterpret_cast<const u32x4a*>(p + xo[i]);
    };
    auto store_x = [&](const u32x4a (&xr)[XPT], int buf) {
#pragma unroll
        for (int i = 0; i < XPT; ++i) *reinterpret_cast<u32x4a*>(&xl[buf][xa[i]]) = xr[i];
    };
    auto load_w = [&](uint32_t (&wr)[BITS], uint32_t kt) { load_block<BITS>(wp + (size_t)min(kt, ktiles - 1) * 2 * BITS, wr); };
    auto load_sb = [&](u32x4a (&r)[2], uint32_t win) {
        const uint32_t o = min(win, nwin - 1) * 8;
        if constexpr (GENERAL) {  // rows of scales need only 2-byte alignment: element loads
            uint32_t sv[4], bv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                sv[q] = (uint32_t)sp[o + 2 * q] | ((uint32_t)sp[o + 2 * q + 1] << 16);
                bv[q] = (uint32_t)bp[o + 2 * q] | ((uint32_t)bp[o + 2 * q + 1] << 16);
            }
            r[0] = u32x4a{sv[0], sv[1], sv[2], sv[3]};
            r[1] = u32x4a{bv[0], bv[1], bv[2], bv[3]};
        } else {
            r[0] = *reinterpret_cast<const u32x4a*>(sp + o);
            r[1] = *reinterpret_cast<const u32x4a*>(bp + o);
        }
    };

    f32x16 acc[SUB];
#pragma unroll
    for (int i = 0; i < SUB; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;

    // X operand of tile i, MFMA kk: row 32 i + lane % 32, k offset 32 h + 8 kk.
    const int aoff = (lane & 31) * LDK + h * 32;
    auto read_a = [&](const uint16_t* L, int kk, op8<F16> (&a)[SUB]) {
#pragma unroll
        for (int i = 0; i < SUB; ++i) a[i] = *reinterpret_cast<const op8<F16>*>(L + aoff + 32 * i * LDK + 8 * kk);
    };

    // Prologue: X of step 0 in LDS, X of steps 1 and 2 and W of steps 0..2 in flight, the first
    // scale window in flight. (GENERAL: K may hold no whole 1024-code chunk; the tail does it all.)
    if (!GENERAL || ktiles > 0) {
    u32x4a xr[2][XPT], sbc[2], sbn[2];
    uint32_t wr[4][BITS];
    load_sb(sbn, 0);
    load_w(wr[0], 0);
    load_w(wr[1], 1);
    load_w(wr[2], 2);
    load_x(xr[0], 0);
    load_x(xr[1], 1);
    store_x(xr[0], 0);
    load_x(xr[0], 2);
    __syncthreads();

    // Step kt: store X of step kt+1 into the free buffer and issue the loads of X and W of step
    // kt+3 (and of the next scale window at a window's first step), then multiply step kt. Register
    // sets are fixed by the position in the unrolled body: X by the step's parity, W by kt % 4.
    for (uint32_t kt0 = 0; kt0 < ktiles; kt0 += kDirectBody) {
#pragma unroll
        for (int u = 0; u < kDirectBody; ++u) {
            const uint32_t kt = kt0 + u;
            if (u % P == 0) {
                sbc[0] = sbn[0];
                sbc[1] = sbn[1];
            }
            store_x(xr[(u + 1) & 1], (u + 1) & 1);
            load_x(xr[(u + 1) & 1], kt + 3);
            load_w(wr[(u + 3) & 3], kt + 3);
            if (u % P == 0) load_sb(sbn, kt / P + 1);
            // Keep the loads here: the operands are read-only, so the compiler could otherwise sink
            // them towards their first use and lose the prefetch distance.
            asm volatile("" ::: "memory");
            // This lane's group in the window: block 2 u + h, i.e. group (2 u + h) >> GSHIFT.
            uint32_t sw, bw, sh;
            if constexpr (GSHIFT == 0) {
                sw = sbc[0][u % P];
                bw = sbc[1][u % P];
                sh = 16u * (uint32_t)h;
            } else {
                const int gi = (u % P) >> (GSHIFT - 1);
                sw = sbc[0][gi >> 1];
                bw = sbc[1][gi >> 1];
                sh = 16u * (uint32_t)(gi & 1);
            }
            const Dq dq = make_dq(half_to_f32<F16>(sw >> sh), half_to_f32<F16>(bw >> sh));
            const uint16_t* L = xl[u & 1];
            op8<F16> a[2][SUB];
            read_a(L, 0, a[0]);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk < 3) read_a(L, kk + 1, a[(kk + 1) & 1]);
                const op8<F16> bw8 = dequant_op<F16, BITS>(wr[u & 3], kk, dq);
#pragma unroll
                for (int i = 0; i < SUB; ++i) acc[i] = mfma32x32x16<F16>(a[kk & 1][i], bw8, acc[i]);
            }
            __syncthreads();
        }
    }
    }

    // GENERAL: the K-steps past the last whole 1024-code chunk (done by the last split), one at a
    // time with the loads of the next four steps in flight (register sets rotated by the step's
    // position in an unrolled group of four); X chunks and W blocks past K are zeros, and scales
    // and biases are single elements.
    if constexpr (GENERAL) {
        constexpr int D = 4;
        const uint32_t steps = (kb + 1) >> 1;
        uint32_t kt = chunks * kDirectBody;
        if ((!PARTIAL || split + 1 == splits) && kt < steps) {
            const uint16_t* xt = x + (size_t)m0 * k;
            const uint32_t* wt = packed + (size_t)wrow * kb * BITS;
            const uint16_t* st = scales + (size_t)wrow * gpr;
            const uint16_t* bt = biases + (size_t)wrow * gpr;
            u32x4a tx[D][XPT];
            uint32_t tw[D][BITS];
            float ts[D], tb[D];
            auto tload = [&](int d, uint32_t s) {
#pragma unroll
                for (int i = 0; i < XPT; ++i)
                    tx[d][i] = s * 64 + (uint32_t)xkc * 8 < k
                                   ? *reinterpret_cast<const u32x4a*>(xt + xo[i] + s * 64)
                                   : u32x4a{0u, 0u, 0u, 0u};
                const uint32_t jb = 2 * s + (uint32_t)h;
                if (jb < kb) {
                    load_block<BITS>(wt + (size_t)jb * BITS, tw[d]);
                    ts[d] = half_to_f32<F16>(st[jb >> GSHIFT]);
                    tb[d] = half_to_f32<F16>(bt[jb >> GSHIFT]);
                } else {
#pragma unroll
                    for (int q = 0; q < BITS; ++q) tw[d][q] = 0u;
                    ts[d] = 0.f;
                    tb[d] = 0.f;
                }
            };
#pragma unroll
            for (int d = 0; d < D; ++d)
                if (kt + d < steps) tload(d, kt + d);
            for (; kt < steps; kt += D) {
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    if (kt + d >= steps) break;
                    __syncthreads();  // the previous step's reads of xl are done
                    store_x(tx[d], 0);
                    uint32_t w[BITS];
#pragma unroll
                    for (int q = 0; q < BITS; ++q) w[q] = tw[d][q];
                    const Dq dq = make_dq(ts[d], tb[d]);
                    if (kt + d + D < steps) tload(d, kt + d + D);
                    __syncthreads();
                    op8<F16> a[SUB];
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        read_a(xl[0], kk, a);
                        const op8<F16> bw8 = dequant_op<F16, BITS>(w, kk, dq);
#pragma unroll
                        for (int i = 0; i < SUB; ++i) acc[i] = mfma32x32x16<F16>(a[i], bw8, acc[i]);
                    }
                }
            }
        }
    }

    const uint32_t gc = n0 + 32 * wave + (lane & 31);
    const int orow = 4 * h;
    if (gc < n) {
#pragma unroll
        for (int i = 0; i < SUB; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const uint32_t gm = m0 + 32 * i + 8 * (v >> 2) + orow + (v & 3);
                if (gm < m) {
                    if constexpr (PARTIAL)
                        part[((size_t)split * m + gm) * n + gc] = acc[i][v];
                    else
                        y[(size_t)gm * n + gc] = f32_to_half_bits<F16>(acc[i][v]);
                }
            }
    }
}

// SUB: 32-row sub-tiles per tile (4: 128-row tiles; 2: 64-row tiles, for split K at few rows).
template <int BITS, int GSHIFT, bool PARTIAL, bool GENERAL, bool F16, int SUB>
__global__ __launch_bounds__(kDirectThreads) void gemm_direct_kernel(
    const uint16_t* x, uint32_t m, const uint32_t* packed, const uint16_t* scales,
    const uint16_t* biases, uint32_t n, uint32_t kb, uint16_t* y, uint32_t tiles_m,
    uint32_t tiles_n, float* part, uint32_t splits) {
    __shared__ __attribute__((aligned(16))) uint16_t xl[2][DBM * LDK];
    // Tile order: block b runs on XCD b % 8, so each XCD gets a contiguous run of 32 tiles, laid
    // out as 4 tile rows x 8 tile columns where the grid allows, to share X and W in its L2. With
    // one or two tile rows the run goes down the columns instead, so that each XCD fetches whole W
    // tile columns (for both rows) and no W column is fetched by two XCDs (x [128, 14336] on
    // [4096, 14336] in 64-row tiles: about 60 MB against 77 MB across the L2s).
    const uint32_t tiles = tiles_m * tiles_n;
    uint32_t t = blockIdx.x;
    if ((tiles & 7u) == 0) t = (t & 7u) * (tiles >> 3) + (t >> 3);
    uint32_t tm, tn;
    if ((tiles_m & 3u) == 0 && (tiles_n & 7u) == 0) {
        const uint32_t st = t >> 5, w = t & 31u, stn = tiles_n >> 3;
        tm = (st / stn) * 4 + (w >> 3);
        tn = (st % stn) * 8 + (w & 7u);
    } else if (tiles_m <= 2) {
        tm = t % tiles_m;
        tn = t / tiles_m;
    } else {
        tm = t / tiles_n;
        tn = t % tiles_n;
    }
    direct_tile<BITS, GSHIFT, PARTIAL, SUB, GENERAL, F16>(x, m, packed, scales, biases, n, kb, y, tm * (32 * SUB),
                                                          tn * DBN, part, PARTIAL ? blockIdx.y : 0u, splits, xl);
}

// ---- gathered batches grouped by expert (nuvec_core quantized.rs, gather_qmm with sorted rhs) --
//
// Output batch r (one row of x each, no lhs) is x[r] . dequantize(W[rhs[r]])^T with rhs sorted,
// so the rows of expert e are [#(rhs < e), #(rhs < e + 1)): a plain GEMM of those rows against
// W[e]. Block (e, tile column, s) finds that range in the sorted indices and runs the expert's
// row tiles s, s + kGroupedSplit, ..., each with W[e] dequantized into registers as above. Experts
// of a few hundred rows take 64-row tiles (SUB = 2): less padding in each expert's last tile and
// more, smaller tiles to spread over the compute units, for twice the dequantization per flop.
// Expert w_count stands for the rows past every expert (an index out of range): they get NaN.
constexpr uint32_t kGroupedSplit = 3;  // blocks per expert and tile column

template <int BITS, int GSHIFT, int SUB, bool F16>
__global__ __launch_bounds__(kDirectThreads) void gemm_grouped_kernel(
    const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint16_t* biases, uint32_t n,
    uint32_t kb, uint16_t* y, const uint32_t* rhs, uint32_t batch, uint32_t w_count, uint32_t tiles_n,
    uint64_t w_stride, uint64_t sb_stride) {
    constexpr uint32_t TM = 32 * SUB;
    __shared__ __attribute__((aligned(16))) uint16_t xl[2][DBM * LDK];
    // Block b runs on XCD b % 8 (the grid is a multiple of 8): consecutive logical blocks -- those of
    // one expert -- go to one XCD, so that its L2 holds the expert's weights and rows for all of them.
    const uint32_t t = (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    if (t >= (w_count + 1) * tiles_n * kGroupedSplit) return;
    const uint32_t e = t / (tiles_n * kGroupedSplit);
    const uint32_t rem = t - e * tiles_n * kGroupedSplit;
    const uint32_t tn = rem / kGroupedSplit, s = rem % kGroupedSplit;
    const int lane = threadIdx.x & 63;
    uint32_t lo, hi;
    count_below2(rhs, batch, e, e + 1, lane, lo, hi);  // the same in every wave
    if (e == w_count) hi = batch;                       // rows past every expert
    if (lo >= hi) return;                               // block-uniform
    const uint32_t rows = hi - lo;
    if (e >= w_count) {
        // an index out of range: NaN over these rows' columns of this tile column
        const uint32_t cols = min(n - tn * DBN, (uint32_t)DBN);
        for (uint32_t o = s * kDirectThreads + threadIdx.x; o < rows * cols; o += kGroupedSplit * kDirectThreads)
            y[(size_t)(lo + o / cols) * n + tn * DBN + o % cols] = F16 ? 0x7e00u : 0x7fc0u;  // quiet NaN
        return;
    }
    const uint32_t k = kb * 32;
    for (uint32_t t = s; t * TM < rows; t += kGroupedSplit)
        direct_tile<BITS, GSHIFT, false, SUB, false, F16>(x + (size_t)lo * k, rows, packed + e * w_stride,
                                                          scales + e * sb_stride, biases + e * sb_stride, n, kb,
                                                          y + (size_t)lo * n, t * TM, tn * DBN, nullptr, 0u, 1u, xl);
}

// y[i] = half(part[0][i] + part[1][i] + ... + part[splits - 1][i]), in that order, for i < count.
template <bool F16>
__global__ __launch_bounds__(256) void sum_partials_kernel(const float* part, uint64_t count, uint32_t splits,
                                                           uint16_t* y) {
    const uint64_t i = ((uint64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= count) return;
    if (i + 4 <= count && (count & 3) == 0) {
        f32x4 acc = *reinterpret_cast<const f32x4*>(part + i);
        for (uint32_t s = 1; s < splits; ++s) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(part + (size_t)s * count + i);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        *reinterpret_cast<u32x2*>(y + i) = u32x2{pack_half2<F16>(acc.x, acc.y), pack_half2<F16>(acc.z, acc.w)};
        return;
    }
    for (uint64_t j = i; j < i + 4 && j < count; ++j) {
        float a = part[j];
        for (uint32_t s = 1; s < splits; ++s) a += part[(size_t)s * count + j];
        y[j] = f32_to_half_bits<F16>(a);
    }
}

// Tile rows of the split-K GEMM: 64-row tiles up to 128 rows of x (their partial sums are half
// those of a 14-way split of 128-row tiles: at x [128, 14336] on [4096, 14336], 27.9 against
// 29.9 us), 128-row tiles above.
inline int64_t split_tile_rows(int64_t m) { return m <= 128 ? 64 : DBM; }

template <int BITS, int GSHIFT, bool GENERAL, bool F16>
hipError_t launch_direct_g(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                           const uint16_t* biases, int64_t n, int64_t kb, uint16_t* y, int64_t tiles_m,
                           int64_t tiles_n, float* part, int64_t splits, hipStream_t stream) {
    if (splits > 1) {
        const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)splits);
        if (split_tile_rows(m) == 64)
            gemm_direct_kernel<BITS, GSHIFT, true, GENERAL, F16, 2><<<grid, dim3(kDirectThreads), 0, stream>>>(
                x, (uint32_t)m, packed, scales, biases, (uint32_t)n, (uint32_t)kb, y, (uint32_t)tiles_m,
                (uint32_t)tiles_n, part, (uint32_t)splits);
        else
            gemm_direct_kernel<BITS, GSHIFT, true, GENERAL, F16, 4><<<grid, dim3(kDirectThreads), 0, stream>>>(
                x, (uint32_t)m, packed, scales, biases, (uint32_t)n, (uint32_t)kb, y, (uint32_t)tiles_m,
                (uint32_t)tiles_n, part, (uint32_t)splits);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const uint64_t count = (uint64_t)m * (uint64_t)n;
        sum_partials_kernel<F16><<<dim3((unsigned)((count + 1023) / 1024)), dim3(256), 0, stream>>>(part, count,
                                                                                            (uint32_t)splits, y);
        return hipGetLastError();
    }
    gemm_direct_kernel<BITS, GSHIFT, false, GENERAL, F16, 4><<<dim3((unsigned)(tiles_m * tiles_n)),
                                                          dim3(kDirectThreads), 0, stream>>>(
        x, (uint32_t)m, packed, scales, biases, (uint32_t)n, (uint32_t)kb, y, (uint32_t)tiles_m, (uint32_t)tiles_n,
        nullptr, 1u);
    return hipGetLastError();
}

template <int BITS, bool GENERAL, bool F16>
hipError_t launch_direct_b(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                           const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, uint16_t* y,
                           int64_t tiles_m, int64_t tiles_n, float* part, int64_t splits, hipStream_t stream) {
    if (gshift == 0) return launch_direct_g<BITS, 0, GENERAL, F16>(x, m, packed, scales, biases, n, kb, y, tiles_m, tiles_n, part, splits, stream);
    if (gshift == 1) return launch_direct_g<BITS, 1, GENERAL, F16>(x, m, packed, scales, biases, n, kb, y, tiles_m, tiles_n, part, splits, stream);
    return launch_direct_g<BITS, 2, GENERAL, F16>(x, m, packed, scales, biases, n, kb, y, tiles_m, tiles_n, part, splits, stream);
}

template <bool GENERAL, bool F16>
hipError_t launch_direct_v(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                           const uint16_t* biases, int64_t n, int64_t kb, int bits, uint32_t gshift, uint16_t* y,
                           int64_t tiles_m, int64_t tiles_n, float* part, int64_t splits, hipStream_t stream) {
    switch (bits) {
        case 1: return launch_direct_b<1, GENERAL, F16>(x, m, packed, scales, biases, n, kb, gshift, y, tiles_m, tiles_n, part, splits, stream);
        case 2: return launch_direct_b<2, GENERAL, F16>(x, m, packed, scales, biases, n, kb, gshift, y, tiles_m, tiles_n, part, splits, stream);
        case 3: return launch_direct_b<3, GENERAL, F16>(x, m, packed, scales, biases, n, kb, gshift, y, tiles_m, tiles_n, part, splits, stream);
        case 4: return launch_direct_b<4, GENERAL, F16>(x, m, packed, scales, biases, n, kb, gshift, y, tiles_m, tiles_n, part, splits, stream);
        case 5: return launch_direct_b<5, GENERAL, F16>(x, m, packed, scales, biases, n, kb, gshift, y, tiles_m, tiles_n, part, splits, stream);
        case 6: return launch_direct_b<6, GENERAL, F16>(x, m, packed, scales, biases, n, kb, gshift, y, tiles_m, tiles_n, part, splits, stream);
        case 8: return launch_direct_b<8, GENERAL, F16>(x, m, packed, scales, biases, n, kb, gshift, y, tiles_m, tiles_n, part, splits, stream);
        default: return hipErrorInvalidValue;
    }
}

template <bool F16>
hipError_t launch_direct(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                         const uint16_t* biases, int64_t n, int64_t kb, int bits, uint32_t gshift, uint16_t* y,
                         int64_t tiles_m, int64_t tiles_n, float* part, int64_t splits, bool general,
                         hipStream_t stream) {
    if (general)
        return launch_direct_v<true, F16>(x, m, packed, scales, biases, n, kb, bits, gshift, y, tiles_m, tiles_n, part,
                                     splits, stream);
    return launch_direct_v<false, F16>(x, m, packed, scales, biases, n, kb, bits, gshift, y, tiles_m, tiles_n, part,
                                  splits, stream);
}

// K splits of whole 1024-code chunks (the last split also takes a K tail): at most one block
// per compute unit, then the fewest splits that keep the longest range as short (14 chunks over
// at most 8 splits: 7 ranges of two, so fewer partial sums for the same critical path).
int64_t direct_splits(int64_t m, int64_t n, int64_t k) {
    if (m <= 0 || n <= 0 || k < 64 * kDirectBody) return 1;
    const int64_t tiles_n = (n + DBN - 1) / DBN;
    const int64_t rows = split_tile_rows(m);
    const int64_t tiles = ((m + rows - 1) / rows) * tiles_n;
    if (tiles > 0x7fffffff / 2) return 1;
    const int64_t chunks = k / (64 * kDirectBody);
    int64_t s = (int64_t)device_cu_count() / tiles;
    if (s > chunks) s = chunks;
    if (s > 64) s = 64;
    if (s <= 1) return 1;
    const int64_t longest = (chunks + s - 1) / s;
    return (chunks + longest - 1) / longest;
}

template <int BITS, int GSHIFT, bool F16>
hipError_t launch_grouped_g(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                            int64_t n, int64_t kb, uint16_t* y, const uint32_t* rhs, int64_t batch, int64_t w_count,
                            uint64_t w_stride, uint64_t sb_stride, hipStream_t stream) {
    const int64_t tiles_n = (n + DBN - 1) / DBN;
    const unsigned blocks = (unsigned)(((w_count + 1) * tiles_n * kGroupedSplit + 7) / 8 * 8);
    // 64-row tiles while the experts average up to 256 rows
    if (batch <= 256 * w_count)
        gemm_grouped_kernel<BITS, GSHIFT, 2, F16><<<dim3(blocks), dim3(kDirectThreads), 0, stream>>>(
            x, packed, scales, biases, (uint32_t)n, (uint32_t)kb, y, rhs, (uint32_t)batch, (uint32_t)w_count,
            (uint32_t)tiles_n, w_stride, sb_stride);
    else
        gemm_grouped_kernel<BITS, GSHIFT, 4, F16><<<dim3(blocks), dim3(kDirectThreads), 0, stream>>>(
            x, packed, scales, biases, (uint32_t)n, (uint32_t)kb, y, rhs, (uint32_t)batch, (uint32_t)w_count,
            (uint32_t)tiles_n, w_stride, sb_stride);
    return hipGetLastError();
}

template <int BITS, bool F16>
hipError_t launch_grouped_b(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                            int64_t n, int64_t kb, uint32_t gshift, uint16_t* y, const uint32_t* rhs, int64_t batch,
                            int64_t w_count, uint64_t w_stride, uint64_t sb_stride, hipStream_t stream) {
    if (gshift == 0)
        return launch_grouped_g<BITS, 0, F16>(x, packed, scales, biases, n, kb, y, rhs, batch, w_count, w_stride, sb_stride, stream);
    if (gshift == 1)
        return launch_grouped_g<BITS, 1, F16>(x, packed, scales, biases, n, kb, y, rhs, batch, w_count, w_stride, sb_stride, stream);
    return launch_grouped_g<BITS, 2, F16>(x, packed, scales, biases, n, kb, y, rhs, batch, w_count, w_stride, sb_stride, stream);
}

template <bool F16>
hipError_t grouped_run(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                       int64_t n, int64_t k, int group_size, int bits, uint16_t* y, const uint32_t* rhs, int64_t batch,
                       int64_t w_count, uint64_t w_stride, uint64_t sb_stride, hipStream_t stream) {
    const int64_t kb = k / 32;
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    switch (bits) {
        case 1: return launch_grouped_b<1, F16>(x, packed, scales, biases, n, kb, gshift, y, rhs, batch, w_count, w_stride, sb_stride, stream);
        case 2: return launch_grouped_b<2, F16>(x, packed, scales, biases, n, kb, gshift, y, rhs, batch, w_count, w_stride, sb_stride, stream);
        case 3: return launch_grouped_b<3, F16>(x, packed, scales, biases, n, kb, gshift, y, rhs, batch, w_count, w_stride, sb_stride, stream);
        case 4: return launch_grouped_b<4, F16>(x, packed, scales, biases, n, kb, gshift, y, rhs, batch, w_count, w_stride, sb_stride, stream);
        case 5: return launch_grouped_b<5, F16>(x, packed, scales, biases, n, kb, gshift, y, rhs, batch, w_count, w_stride, sb_stride, stream);
        case 6: return launch_grouped_b<6, F16>(x, packed, scales, biases, n, kb, gshift, y, rhs, batch, w_count, w_stride, sb_stride, stream);
        case 8: return launch_grouped_b<8, F16>(x, packed, scales, biases, n, kb, gshift, y, rhs, batch, w_count, w_stride, sb_stride, stream);
        default: return hipErrorInvalidValue;
    }
}

template <bool F16>
hipError_t gemm_run(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                    const uint16_t* biases, int64_t n, int64_t k, int group_size, int bits, uint16_t* y,
                    hipStream_t stream, void* workspace, size_t workspace_bytes) {
    const int64_t kb = k / 32;
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    auto a16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
    // whole 1024-code chunks of K and 16-byte aligned scale rows: the kernel as designed; anything
    // else its GENERAL variant
    const bool general = !(k % (64 * kDirectBody) == 0 && a16(scales) && a16(biases));
    const int64_t tiles_n = (n + DBN - 1) / DBN;
    const int64_t max_rows = (int64_t)(0x7fffffff / tiles_n) * DBM;
    // split K where the workspace allows it (float32 partials of every split)
    const int64_t splits = direct_splits(m, n, k);
    if (splits > 1 && workspace && workspace_bytes >= (size_t)splits * (size_t)m * (size_t)n * sizeof(float))
        return launch_direct<F16>(x, m, packed, scales, biases, n, kb, bits, gshift, y,
                                  (m + split_tile_rows(m) - 1) / split_tile_rows(m), tiles_n,
                                  static_cast<float*>(workspace), splits, general, stream);
    for (int64_t m_off = 0; m_off < m; m_off += max_rows) {
        const int64_t mm = (m - m_off < max_rows) ? (m - m_off) : max_rows;
        const int64_t tiles_m = (mm + DBM - 1) / DBM;
        const hipError_t e = launch_direct<F16>(x + (size_t)m_off * k, mm, packed, scales, biases, n, kb, bits,
                                                gshift, y + (size_t)m_off * n, tiles_m, tiles_n, nullptr, 1, general,
                                                stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace
}  // namespace qaff
