// Quantized GEMM on bf16 MFMA: Y[m, n] = sum_k X[m, k] * w[n, k] for many rows of X (the prefill
// path of spark_runtime weights/mlx_int8.rs, `gemm`, which that page leaves as an untiled
// reference; the product itself is nuvec_core quantized.rs, `quantized_matmul` with transpose).
//
// Compute-bound (about 2.3 kflop per byte at the prefill shape). A 256-thread block owns a
// BM x BN tile of Y and walks K in steps of BK = 64 (two 32-code blocks, each with one scale and
// bias). Per step it stages the X tile (bf16, straight copy) and the W tile -- dequantized on the
// way in, w = s*c + b in float32 then rounded to bf16 -- into LDS, double buffered, and each of the
// four waves runs v_mfma_f32_16x16x32_bf16 over its 64 x 64 sub-tile with float32 accumulators.
//
// MFMA operand layout (16x16x32, bf16): lane l supplies row (l % 16) of A and column (l % 16) of B,
// each as the 8 consecutive k values starting at 8 * (l / 16); lane l receives D rows
// 4 * (l / 16) + 0..3 of column l % 16. Both A = X and B = W^T are read as 8 consecutive k of one
// row of X or W, i.e. one 16-byte LDS read each.
#include "launch.h"
#include "qaff_device.h"

#include <hip/hip_runtime.h>

namespace qaff {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int LDK = BK + 8;  // LDS row pitch in bf16 elements (padding spreads rows over banks)
constexpr int kThreads = 256;

template <int BITS>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint16_t* __restrict__ x, uint32_t m, const uint32_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases, uint32_t n,
    uint32_t kb, uint32_t gshift, uint16_t* __restrict__ y) {
#pragma clang fp contract(off)
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const uint32_t m0 = blockIdx.y * BM;
    const uint32_t n0 = blockIdx.x * BN;
    const uint32_t k = kb * 32;
    const uint32_t gpr = kb >> gshift;
    const uint32_t ktiles = (kb + 1) / 2;

    // Global -> register staging of the next tile.
    u32x4a xa[4];
    uint32_t wq[BITS];
    float ws = 0.f, wbias = 0.f;
    bool wvalid = false;
    const int brow = tid >> 1;  // W row of the tile this thread dequantizes
    const int bblk = tid & 1;   // which 32-code block of the step

    auto load_tile = [&](uint32_t kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + kThreads * i;
            const int row = c >> 3;
            const int col = (c & 7) * 8;
            const uint32_t gm = m0 + row;
            const uint32_t gk = kt * BK + col;
            if (gm < m && gk < k) xa[i] = *reinterpret_cast<const u32x4a*>(x + (size_t)gm * k + gk);
            else xa[i] = u32x4a{0u, 0u, 0u, 0u};
        }
        const uint32_t gn = n0 + brow;
        const uint32_t jb = kt * 2 + bblk;
        wvalid = gn < n && jb < kb;
        if (wvalid) {
            load_block<BITS>(packed + (size_t)gn * kb * BITS + (size_t)jb * BITS, wq);
            const size_t gi = (size_t)gn * gpr + (jb >> gshift);
            ws = bf16_to_f32(scales[gi]);
            wbias = bf16_to_f32(biases[gi]);
        }
    };

    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + kThreads * i;
            const int row = c >> 3;
            const int col = (c & 7) * 8;
            *reinterpret_cast<u32x4a*>(&As[buf][row * LDK + col]) = xa[i];
        }
        uint32_t d[16];
        if (wvalid) {
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const float lo = ws * (float)code_at<BITS>(wq, 2 * c) + wbias;
                const float hi = ws * (float)code_at<BITS>(wq, 2 * c + 1) + wbias;
                d[c] = pack_bf16x2(lo, hi);
            }
        } else {
#pragma unroll
            for (int c = 0; c < 16; ++c) d[c] = 0u;
        }
        u32x4a* dst = reinterpret_cast<u32x4a*>(&Bs[buf][brow * LDK + bblk * 32]);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = u32x4a{d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]};
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    load_tile(0);
    store_tile(0);
    __syncthreads();

    const int frow = lane & 15;
    const int fk = (lane >> 4) * 8;
    for (uint32_t kt = 0; kt < ktiles; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < ktiles) load_tile(kt + 1);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            bf16x8 a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *reinterpret_cast<const bf16x8*>(&As[buf][(wm * 64 + i * 16 + frow) * LDK + kk + fk]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(wn * 64 + j * 16 + frow) * LDK + kk + fk]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < ktiles) store_tile(buf ^ 1);
        __syncthreads();
    }

    const int orow = (lane >> 4) * 4;
    const int ocol = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint32_t gm = m0 + wm * 64 + i * 16 + orow + v;
                const uint32_t gn = n0 + wn * 64 + j * 16 + ocol;
                if (gm < m && gn < n) y[(size_t)gm * n + gn] = to_bf16_bits(acc[i][j][v]);
            }
}

// ---- 256 x 128 tiles for large m --------------------------------------------------------------
//
// One block of WM x WN waves owns a 256 x 128 tile of Y (each wave a (256/WM) x (128/WN) sub-tile)
// and walks K in steps of 64. With about one tile per compute unit at the prefill shape, latency is
// hidden by prefetching two K-steps ahead into registers: at step t a block stores step t+1 from
// registers into the free LDS buffer (dequantizing W on the way), issues the global loads of step
// t+3 into the register set that just emptied, then multiplies step t from the other LDS buffer.
// LDS rows are 64 bf16 = eight 16-byte chunks; chunk c of row r is stored at position c ^ (r % 8)
// so that the MFMA operand reads (16 rows at one chunk) and the tile writes spread over the banks.
// Blocks are ordered so that consecutive tiles along N share one 256-row band of X and each XCD
// (block index mod 8 on MI355X) gets one band: its 32 compute units then stream the same X rows
// through their shared L2.

constexpr int BM2 = 256;
constexpr int BN2 = 128;
constexpr int kLdsA = BM2 * BK;  // bf16 elements of one A buffer
constexpr int kLdsB = BN2 * BK;  // bf16 elements of one B buffer

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

// A thread's share of W per K-step is UC codes (BN2 * BK / threads: 16 or 32). A whole block (32)
// is BITS words. Half a block is BITS/2 whole words for even widths (16 * BITS bits); for odd
// widths it straddles a word, so the thread keeps the whole block and picks its half.
template <int BITS, int UC>
constexpr int kUnitWords = (UC == 32 || BITS % 2 == 1) ? BITS : BITS / 2;

template <int NW>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t (&w)[NW]) {
    if constexpr (NW == 1) {
        w[0] = p[0];
    } else if constexpr (NW == 2) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(p);
        w[0] = v.x; w[1] = v.y;
    } else if constexpr (NW == 3) {
        const u32x3 v = *reinterpret_cast<const u32x3*>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z;
    } else if constexpr (NW == 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (NW == 5) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w; w[4] = p[4];
    } else if constexpr (NW == 6) {
        const u32x3 v = *reinterpret_cast<const u32x3*>(p);
        const u32x3 u = *reinterpret_cast<const u32x3*>(p + 3);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = u.x; w[4] = u.y; w[5] = u.z;
    } else {
        static_assert(NW == 8, "unit words");
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
        const u32x4 u = *reinterpret_cast<const u32x4*>(p + 4);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        w[4] = u.x; w[5] = u.y; w[6] = u.z; w[7] = u.w;
    }
}

// Code j of a little-endian stream held in NW words (j compile-time after unrolling).
template <int BITS, int NW>
__device__ __forceinline__ uint32_t stream_code(const uint32_t (&w)[NW], int j) {
    const int bit = j * BITS, wi = bit >> 5, sh = bit & 31;
    const uint32_t mask = (1u << BITS) - 1u;
    if (sh + BITS <= 32) return (w[wi] >> sh) & mask;
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & mask;
}

// A thread's UC codes -> UC/2 dwords of bf16 pairs in column order, w = s*c + b rounded to nearest
// even (the float32 product is exact, so the fused multiply-add rounds once like mul-then-add).
template <int BITS, int UC>
__device__ __forceinline__ void dequant_unit(const uint32_t (&w)[kUnitWords<BITS, UC>], int half, float s, float b,
                                             uint32_t (&o)[UC / 2]) {
    constexpr int NW = kUnitWords<BITS, UC>;
    float v[UC];
    if constexpr (UC == 32 || BITS % 2 == 0) {
#pragma unroll
        for (int i = 0; i < UC; ++i) v[i] = (float)stream_code<BITS, NW>(w, i);
    } else {
#pragma unroll
        for (int i = 0; i < UC; ++i)
            v[i] = (float)(half ? stream_code<BITS, NW>(w, 16 + i) : stream_code<BITS, NW>(w, i));
    }
#pragma unroll
    for (int i = 0; i < UC / 2; ++i) o[i] = pack_bf16x2(__builtin_fmaf(s, v[2 * i], b), __builtin_fmaf(s, v[2 * i + 1], b));
}

template <int BITS, int UC, int NCH>
struct Stage {
    u32x4a xa[NCH];                      // chunks of 16 bytes of the X tile
    uint32_t wq[kUnitWords<BITS, UC>];  // this thread's words of W
    uint32_t sraw, braw;                 // the 4-byte words holding its scale and bias
};

template <int BITS, int WM, int WN>
// The operand pointers are deliberately not __restrict__: with them the compiler may move the
// prefetch loads across anything, including the empty asm that keeps them in place.
__global__ __launch_bounds__(64 * WM * WN) void gemm_big_kernel(
    const uint16_t* x, uint32_t m, const uint32_t* packed, const uint16_t* scales,
    const uint16_t* biases, uint32_t n, uint32_t kb, uint32_t gshift, uint16_t* y,
    uint32_t tiles_n, uint32_t tiles) {
    constexpr int kThreadsB = 64 * WM * WN;
    constexpr int TM = BM2 / WM;              // wave sub-tile rows
    constexpr int TN = BN2 / WN;              // wave sub-tile columns
    constexpr int FM = TM / 16, FN = TN / 16;  // 16 x 16 MFMA tiles per wave
    constexpr int NCH = BM2 * BK / 8 / kThreadsB;  // 16-byte X chunks per thread per step
    constexpr int UC = BN2 * BK / kThreadsB;       // W codes per thread per step
    constexpr int UPR = BK / UC;                   // W units per row of the tile
    constexpr int NW = kUnitWords<BITS, UC>;
    static_assert(UC == 16 || UC == 32, "W unit");
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][kLdsA + kLdsB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN;
    const int wn = wave % WN;

    // XCD-aware tile order: block b runs on XCD b % 8; give each XCD a contiguous run of tiles.
    uint32_t t = blockIdx.x;
    if ((tiles & 7u) == 0) t = (t & 7u) * (tiles >> 3) + (t >> 3);
    const uint32_t m0 = (t / tiles_n) * BM2;
    const uint32_t n0 = (t % tiles_n) * BN2;
    const uint32_t k = kb * 32;
    const uint32_t gpr = kb >> gshift;
    const uint32_t ktiles = (kb + 1) / 2;

    // this thread's W unit: row of the tile, block (0..1) of the step, half (0..1) when UC = 16
    const int wrow = tid / UPR;
    const int wsub = tid % UPR;
    const int wblk = wsub / (32 / UC);
    const int whalf = wsub % (32 / UC);
    const uint32_t gn = min(n0 + wrow, n - 1);
    const uint32_t* wrow_p = packed + (size_t)gn * kb * BITS;
    const bool wrow_ok = n0 + wrow < n;

    auto load = [&](Stage<BITS, UC, NCH>& st, uint32_t kt) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + kThreadsB * i;
            const int row = c >> 3;
            const int kc = c & 7;
            const uint32_t gm = min(m0 + row, m - 1);
            const uint32_t gk = min(kt * BK + kc * 8, k - 8);  // also clamps steps past the end
            st.xa[i] = *reinterpret_cast<const u32x4a*>(x + (size_t)gm * k + gk);
        }
        const uint32_t jb = min(kt * 2 + wblk, kb - 1);
        const uint32_t wofs = (NW == BITS) ? jb * BITS : jb * BITS + whalf * (BITS / 2);
        load_words<NW>(wrow_p + wofs, st.wq);
        // The 4-byte word holding the bf16 scale (bias): a 16-bit load would need a zero-extension
        // that the compiler places where it waits for the newest loads. The arrays are 4-byte
        // aligned on this path, so word e/2 holds element e. (Indexing keeps the loads in the
        // global address space; an integer round trip of the address would turn them into flat
        // loads, which the compiler can only wait for all at once.)
        const size_t e = (size_t)gn * gpr + (jb >> gshift);
        st.sraw = reinterpret_cast<const uint32_t*>(scales)[e >> 1];
        st.braw = reinterpret_cast<const uint32_t*>(biases)[e >> 1];
        // Keep the loads here: the operands are read-only, so the compiler would otherwise sink
        // them towards their first use a whole step later and lose the prefetch distance.
        asm volatile("" ::: "memory");
    };

    auto store = [&](const Stage<BITS, UC, NCH>& st, uint32_t kt, int buf) {
        uint16_t* A = lds[buf];
        uint16_t* B = lds[buf] + kLdsA;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + kThreadsB * i;
            const int row = c >> 3;
            const int kc = c & 7;
            const bool ok = m0 + row < m && kt * BK + kc * 8 < k;
            u32x4a v = st.xa[i];
            asm volatile("" : "+v"(v));  // as for W below: keep this step's work from moving up
            *reinterpret_cast<u32x4a*>(&A[swz(row, kc)]) = ok ? v : u32x4a{0u, 0u, 0u, 0u};
        }
        // The empty asm makes this step's W arithmetic start here: the values are otherwise free
        // to move, and the compiler hoists the next step's dequantization to the top of the loop,
        // where it has to wait for the newest loads.
        uint32_t wq[NW];
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            wq[i] = st.wq[i];
            asm volatile("" : "+v"(wq[i]));
        }
        uint32_t sr = st.sraw, br = st.braw;
        asm volatile("" : "+v"(sr), "+v"(br));
        const uint32_t odd = (uint32_t)((size_t)gn * gpr + (min(kt * 2 + wblk, kb - 1) >> gshift)) & 1u;
        sr = odd ? (sr >> 16) : (sr & 0xffffu);
        br = odd ? (br >> 16) : (br & 0xffffu);
        uint32_t o[UC / 2];
        dequant_unit<BITS, UC>(wq, whalf, bf16_to_f32(sr), bf16_to_f32(br), o);
        const bool ok = wrow_ok && kt * 2 + wblk < kb;
        const int chunk = wblk * 4 + whalf * 2;
#pragma unroll
        for (int q = 0; q < UC / 8; ++q)
            *reinterpret_cast<u32x4a*>(&B[swz(wrow, chunk + q)]) =
                ok ? u32x4a{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]} : u32x4a{0u, 0u, 0u, 0u};
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int frow = lane & 15;
    const int fchunk = lane >> 4;
    auto compute = [&](int buf) {
        const uint16_t* A = lds[buf];
        const uint16_t* B = lds[buf] + kLdsA;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 a[FM], b[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                a[i] = *reinterpret_cast<const bf16x8*>(&A[swz(wm * TM + i * 16 + frow, kk * 4 + fchunk)]);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                b[j] = *reinterpret_cast<const bf16x8*>(&B[swz(wn * TN + j * 16 + frow, kk * 4 + fchunk)]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };

    // Prologue: step 0 into LDS buffer 0, steps 1 and 2 in flight in the two register sets.
    // Loads and stores past the last step are not skipped: loads are clamped into the operands and
    // such stores write zeros into a buffer that no later step reads. A branch around them would
    // make the compiler wait for every outstanding load instead of only the two-step-old ones.
    Stage<BITS, UC, NCH> s0, s1;
    load(s0, 0);
    store(s0, 0, 0);
    load(s1, 1);
    load(s0, 2);
    __syncthreads();

    // Steady state, unrolled by two so each register set has fixed registers:
    //   even t: s1 holds t+1, s0 holds t+2;  odd t: s0 holds t+1, s1 holds t+2.
    // The loop always runs whole pairs: with an odd number of steps the last multiply reads a
    // buffer that was filled with zeros (a step past the end) and adds exact zeros. A branch out of
    // the middle would again cost the precise waits.
    for (uint32_t kt = 0; kt < ktiles; kt += 2) {
        store(s1, kt + 1, 1);
        load(s1, kt + 3);
        compute(0);
        __syncthreads();
        store(s0, kt + 2, 0);
        load(s0, kt + 4);
        compute(1);
        __syncthreads();
    }

    const int orow = (lane >> 4) * 4;
    const int ocol = lane & 15;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint32_t gm = m0 + wm * TM + i * 16 + orow + v;
                const uint32_t gc = n0 + wn * TN + j * 16 + ocol;
                if (gm < m && gc < n) y[(size_t)gm * n + gc] = to_bf16_bits(acc[i][j][v]);
            }
}

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
// Requirements (checked by the launcher): K a multiple of 64 * kDirectBody (so of 8 groups);
// scales and biases 16-byte aligned. Rows of X beyond m and rows of W beyond n are clamped, not
// zeroed: they only reach outputs that are not stored.
// Split K (PARTIAL): with few tiles, grid y splits K into `splits` ranges of whole 1024-code
// chunks; block (tile, s) sums its range and stores the float32 tile to part[s][m][n], and
// sum_partials_kernel adds the ranges in order.
//
// MFMA 32x32x16 (bf16) layout: lane l supplies row l % 32 of A and of W (column of B), each as 8
// values of k slot l / 32; result value v of lane l is row 8 (v / 4) + 4 (l / 32) + v % 4, column
// l % 32.

constexpr int DBM = 128;
constexpr int DBN = 256;
constexpr int kDirectThreads = 512;
constexpr int kDirectBody = 16;  // K-steps per loop iteration (scale windows are 4, 8 or 16 steps)

typedef float f32x16 __attribute__((ext_vector_type(16)));

// One (32 SUB) x 256 tile of Y (SUB = 4: 128 rows; 2: 64 rows): rows m0 .. m0 + 32 SUB - 1 of
// x [m, k] (rows past m clamped, not stored) against W rows n0 .. n0 + 255 of [n, k], over the K-steps of split `split` of `splits` (all of K
// when not PARTIAL), stored as bf16 into y [m, n] or as float32 into part[split][m][n]. `xl` is the
// block's LDS for the X tiles; the call opens with a barrier so that the block can run tiles back
// to back.
template <int BITS, int GSHIFT, bool PARTIAL, int SUB = 4>
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
        r[0] = *reinterpret_cast<const u32x4a*>(sp + o);
        r[1] = *reinterpret_cast<const u32x4a*>(bp + o);
    };

    f32x16 acc[SUB];
#pragma unroll
    for (int i = 0; i < SUB; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;

    // X operand of tile i, MFMA kk: row 32 i + lane % 32, k offset 32 h + 8 kk.
    const int aoff = (lane & 31) * LDK + h * 32;
    auto read_a = [&](const uint16_t* L, int kk, bf16x8 (&a)[SUB]) {
#pragma unroll
        for (int i = 0; i < SUB; ++i) a[i] = *reinterpret_cast<const bf16x8*>(L + aoff + 32 * i * LDK + 8 * kk);
    };

    // Prologue: X of step 0 in LDS, X of steps 1 and 2 and W of steps 0..2 in flight, the first
    // scale window in flight.
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
            const Dq dq = make_dq(__uint_as_float((sw >> sh) << 16), __uint_as_float((bw >> sh) << 16));
            const uint16_t* L = xl[u & 1];
            bf16x8 a[2][SUB];
            read_a(L, 0, a[0]);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk < 3) read_a(L, kk + 1, a[(kk + 1) & 1]);
                const bf16x8 bw8 = dequant8m<BITS>(wr[u & 3], kk, dq);
#pragma unroll
                for (int i = 0; i < SUB; ++i)
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk & 1][i], bw8, acc[i], 0, 0, 0);
            }
            __syncthreads();
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
                        y[(size_t)gm * n + gc] = to_bf16_bits(acc[i][v]);
                }
            }
    }
}

template <int BITS, int GSHIFT, bool PARTIAL>
__global__ __launch_bounds__(kDirectThreads) void gemm_direct_kernel(
    const uint16_t* x, uint32_t m, const uint32_t* packed, const uint16_t* scales,
    const uint16_t* biases, uint32_t n, uint32_t kb, uint16_t* y, uint32_t tiles_m,
    uint32_t tiles_n, float* part, uint32_t splits) {
    __shared__ __attribute__((aligned(16))) uint16_t xl[2][DBM * LDK];
    // Tile order: block b runs on XCD b % 8, so each XCD gets a contiguous run of 32 tiles, laid
    // out as 4 tile rows x 8 tile columns where the grid allows, to share X and W in its L2.
    const uint32_t tiles = tiles_m * tiles_n;
    uint32_t t = blockIdx.x;
    if ((tiles & 7u) == 0) t = (t & 7u) * (tiles >> 3) + (t >> 3);
    uint32_t tm, tn;
    if ((tiles_m & 3u) == 0 && (tiles_n & 7u) == 0) {
        const uint32_t st = t >> 5, w = t & 31u, stn = tiles_n >> 3;
        tm = (st / stn) * 4 + (w >> 3);
        tn = (st % stn) * 8 + (w & 7u);
    } else {
        tm = t / tiles_n;
        tn = t % tiles_n;
    }
    direct_tile<BITS, GSHIFT, PARTIAL>(x, m, packed, scales, biases, n, kb, y, tm * DBM, tn * DBN, part,
                                       PARTIAL ? blockIdx.y : 0u, splits, xl);
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

template <int BITS, int GSHIFT, int SUB>
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
            y[(size_t)(lo + o / cols) * n + tn * DBN + o % cols] = 0x7fc0u;
        return;
    }
    const uint32_t k = kb * 32;
    for (uint32_t t = s; t * TM < rows; t += kGroupedSplit)
        direct_tile<BITS, GSHIFT, false, SUB>(x + (size_t)lo * k, rows, packed + e * w_stride,
                                              scales + e * sb_stride, biases + e * sb_stride, n, kb,
                                              y + (size_t)lo * n, t * TM, tn * DBN, nullptr, 0u, 1u, xl);
}

// y[i] = bf16(part[0][i] + part[1][i] + ... + part[splits - 1][i]), in that order, for i < count.
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
        *reinterpret_cast<u32x2*>(y + i) = u32x2{pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w)};
        return;
    }
    for (uint64_t j = i; j < i + 4 && j < count; ++j) {
        float a = part[j];
        for (uint32_t s = 1; s < splits; ++s) a += part[(size_t)s * count + j];
        y[j] = to_bf16_bits(a);
    }
}

// Waves of the 256 x 128 tile along M (WN = 2 along N): 2 gives four 128 x 64 wave tiles, 4 gives
// eight 64 x 64 ones.
constexpr int kBigWM = 4;
constexpr int kBigWN = 2;

// m above this uses the 256 x 128 tiles; below, the 128 x 128 tiles waste less on padding.
constexpr int64_t kBigTileMinM = 256;

template <int BITS>
hipError_t launch_bits(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                       const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, uint16_t* y,
                       hipStream_t stream) {
    const bool sb_aligned = (reinterpret_cast<uintptr_t>(scales) % 4 == 0) && (reinterpret_cast<uintptr_t>(biases) % 4 == 0);
    if (m >= kBigTileMinM && sb_aligned) {
        const int64_t tiles_n = (n + BN2 - 1) / BN2;
        // one launch covers at most 2^31 tiles worth of rows; slice m beyond that
        const int64_t max_rows = (int64_t)(0x7fffffff / tiles_n) * BM2;
        for (int64_t m_off = 0; m_off < m; m_off += max_rows) {
            const int64_t mm = (m - m_off < max_rows) ? (m - m_off) : max_rows;
            const int64_t tiles = ((mm + BM2 - 1) / BM2) * tiles_n;
            gemm_big_kernel<BITS, kBigWM, kBigWN><<<dim3((unsigned)tiles), dim3(64 * kBigWM * kBigWN), 0, stream>>>(
                x + (size_t)m_off * kb * 32, (uint32_t)mm, packed, scales, biases, (uint32_t)n,
                (uint32_t)kb, gshift, y + (size_t)m_off * n, (uint32_t)tiles_n, (uint32_t)tiles);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const unsigned gx = (unsigned)((n + BN - 1) / BN);
    const int64_t max_rows = (int64_t)65535 * BM;
    for (int64_t m_off = 0; m_off < m; m_off += max_rows) {
        const int64_t mm = (m - m_off < max_rows) ? (m - m_off) : max_rows;
        const unsigned gy = (unsigned)((mm + BM - 1) / BM);
        gemm_kernel<BITS><<<dim3(gx, gy), dim3(kThreads), 0, stream>>>(
            x + (size_t)m_off * kb * 32, (uint32_t)mm, packed, scales, biases, (uint32_t)n,
            (uint32_t)kb, gshift, y + (size_t)m_off * n);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int BITS, int GSHIFT>
hipError_t launch_direct_g(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                           const uint16_t* biases, int64_t n, int64_t kb, uint16_t* y, int64_t tiles_m,
                           int64_t tiles_n, float* part, int64_t splits, hipStream_t stream) {
    if (splits > 1) {
        gemm_direct_kernel<BITS, GSHIFT, true><<<dim3((unsigned)(tiles_m * tiles_n), (unsigned)splits),
                                                 dim3(kDirectThreads), 0, stream>>>(
            x, (uint32_t)m, packed, scales, biases, (uint32_t)n, (uint32_t)kb, y, (uint32_t)tiles_m,
            (uint32_t)tiles_n, part, (uint32_t)splits);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const uint64_t count = (uint64_t)m * (uint64_t)n;
        sum_partials_kernel<<<dim3((unsigned)((count + 1023) / 1024)), dim3(256), 0, stream>>>(part, count,
                                                                                            (uint32_t)splits, y);
        return hipGetLastError();
    }
    gemm_direct_kernel<BITS, GSHIFT, false><<<dim3((unsigned)(tiles_m * tiles_n)), dim3(kDirectThreads), 0, stream>>>(
        x, (uint32_t)m, packed, scales, biases, (uint32_t)n, (uint32_t)kb, y, (uint32_t)tiles_m, (uint32_t)tiles_n,
        nullptr, 1u);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_direct_b(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                           const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, uint16_t* y,
                           int64_t tiles_m, int64_t tiles_n, float* part, int64_t splits, hipStream_t stream) {
    if (gshift == 0) return launch_direct_g<BITS, 0>(x, m, packed, scales, biases, n, kb, y, tiles_m, tiles_n, part, splits, stream);
    if (gshift == 1) return launch_direct_g<BITS, 1>(x, m, packed, scales, biases, n, kb, y, tiles_m, tiles_n, part, splits, stream);
    return launch_direct_g<BITS, 2>(x, m, packed, scales, biases, n, kb, y, tiles_m, tiles_n, part, splits, stream);
}

hipError_t launch_direct(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                         const uint16_t* biases, int64_t n, int64_t kb, int bits, uint32_t gshift, uint16_t* y,
                         int64_t tiles_m, int64_t tiles_n, float* part, int64_t splits, hipStream_t stream) {
    switch (bits) {
        case 1: return launch_direct_b<1>(x, m, packed, scales, biases, n, kb, gshift, y, tiles_m, tiles_n, part, splits, stream);
        case 2: return launch_direct_b<2>(x, m, packed, scales, biases, n, kb, gshift, y, tiles_m, tiles_n, part, splits, stream);
        case 3: return launch_direct_b<3>(x, m, packed, scales, biases, n, kb, gshift, y, tiles_m, tiles_n, part, splits, stream);
        case 4: return launch_direct_b<4>(x, m, packed, scales, biases, n, kb, gshift, y, tiles_m, tiles_n, part, splits, stream);
        case 5: return launch_direct_b<5>(x, m, packed, scales, biases, n, kb, gshift, y, tiles_m, tiles_n, part, splits, stream);
        case 6: return launch_direct_b<6>(x, m, packed, scales, biases, n, kb, gshift, y, tiles_m, tiles_n, part, splits, stream);
        case 8: return launch_direct_b<8>(x, m, packed, scales, biases, n, kb, gshift, y, tiles_m, tiles_n, part, splits, stream);
        default: return hipErrorInvalidValue;
    }
}

// Splits of K for the 128 x 256 kernel: enough K ranges (whole 1024-code chunks) for about one
// block per compute unit when the tiles alone are fewer, and only where the product fits one
// launch (one slice of m).
int64_t direct_splits(int64_t m, int64_t n, int64_t k) {
    if (m <= 0 || n <= 0 || k % (64 * kDirectBody) != 0) return 1;
    const int64_t tiles_n = (n + DBN - 1) / DBN;
    const int64_t tiles = ((m + DBM - 1) / DBM) * tiles_n;
    if (tiles > 0x7fffffff / 2) return 1;
    const int64_t chunks = k / (64 * kDirectBody);
    int64_t s = (int64_t)device_cu_count() / tiles;
    if (s > chunks) s = chunks;
    if (s > 64) s = 64;
    return s < 1 ? 1 : s;
}

template <int BITS, int GSHIFT>
hipError_t launch_grouped_g(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                            int64_t n, int64_t kb, uint16_t* y, const uint32_t* rhs, int64_t batch, int64_t w_count,
                            uint64_t w_stride, uint64_t sb_stride, hipStream_t stream) {
    const int64_t tiles_n = (n + DBN - 1) / DBN;
    const unsigned blocks = (unsigned)(((w_count + 1) * tiles_n * kGroupedSplit + 7) / 8 * 8);
    // 64-row tiles while the experts average up to 256 rows
    if (batch <= 256 * w_count)
        gemm_grouped_kernel<BITS, GSHIFT, 2><<<dim3(blocks), dim3(kDirectThreads), 0, stream>>>(
            x, packed, scales, biases, (uint32_t)n, (uint32_t)kb, y, rhs, (uint32_t)batch, (uint32_t)w_count,
            (uint32_t)tiles_n, w_stride, sb_stride);
    else
        gemm_grouped_kernel<BITS, GSHIFT, 4><<<dim3(blocks), dim3(kDirectThreads), 0, stream>>>(
            x, packed, scales, biases, (uint32_t)n, (uint32_t)kb, y, rhs, (uint32_t)batch, (uint32_t)w_count,
            (uint32_t)tiles_n, w_stride, sb_stride);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_grouped_b(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                            int64_t n, int64_t kb, uint32_t gshift, uint16_t* y, const uint32_t* rhs, int64_t batch,
                            int64_t w_count, uint64_t w_stride, uint64_t sb_stride, hipStream_t stream) {
    if (gshift == 0)
        return launch_grouped_g<BITS, 0>(x, packed, scales, biases, n, kb, y, rhs, batch, w_count, w_stride, sb_stride, stream);
    if (gshift == 1)
        return launch_grouped_g<BITS, 1>(x, packed, scales, biases, n, kb, y, rhs, batch, w_count, w_stride, sb_stride, stream);
    return launch_grouped_g<BITS, 2>(x, packed, scales, biases, n, kb, y, rhs, batch, w_count, w_stride, sb_stride, stream);
}

}  // namespace

bool gemm_grouped_supported(int64_t k, const uint16_t* scales, const uint16_t* biases, uint64_t sb_stride) {
    auto a16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
    return k > 0 && k % (64 * kDirectBody) == 0 && a16(scales) && a16(biases) && (sb_stride * 2) % 16 == 0;
}

hipError_t launch_gemm_grouped(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                               const uint16_t* biases, int64_t n, int64_t k, int group_size, int bits, uint16_t* y,
                               const uint32_t* rhs, int64_t batch, int64_t w_count, uint64_t w_stride,
                               uint64_t sb_stride, hipStream_t stream) {
    const int64_t kb = k / 32;
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    switch (bits) {
        case 1: return launch_grouped_b<1>(x, packed, scales, biases, n, kb, gshift, y, rhs, batch, w_count, w_stride, sb_stride, stream);
        case 2: return launch_grouped_b<2>(x, packed, scales, biases, n, kb, gshift, y, rhs, batch, w_count, w_stride, sb_stride, stream);
        case 3: return launch_grouped_b<3>(x, packed, scales, biases, n, kb, gshift, y, rhs, batch, w_count, w_stride, sb_stride, stream);
        case 4: return launch_grouped_b<4>(x, packed, scales, biases, n, kb, gshift, y, rhs, batch, w_count, w_stride, sb_stride, stream);
        case 5: return launch_grouped_b<5>(x, packed, scales, biases, n, kb, gshift, y, rhs, batch, w_count, w_stride, sb_stride, stream);
        case 6: return launch_grouped_b<6>(x, packed, scales, biases, n, kb, gshift, y, rhs, batch, w_count, w_stride, sb_stride, stream);
        case 8: return launch_grouped_b<8>(x, packed, scales, biases, n, kb, gshift, y, rhs, batch, w_count, w_stride, sb_stride, stream);
        default: return hipErrorInvalidValue;
    }
}

size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    const int64_t s = direct_splits(m, n, k);
    return s > 1 ? (size_t)s * (size_t)m * (size_t)n * sizeof(float) : 0;
}

hipError_t launch_gemm(const uint16_t* x, int64_t m, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                       int group_size, int bits, uint16_t* y, hipStream_t stream, void* workspace,
                       size_t workspace_bytes) {
    const int64_t kb = k / 32;
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    auto a16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
    // The 128 x 256 kernel that dequantizes W into registers takes every m when K allows it: below
    // 256 rows its one row of tiles still ran [4096, 14336] 4-bit g128 in 170 us at m = 17 ... 255,
    // where the 128 x 128 kernel took 297 - 320 us.
    if (k % (64 * kDirectBody) == 0 && a16(scales) && a16(biases)) {
        const int64_t tiles_n = (n + DBN - 1) / DBN;
        const int64_t max_rows = (int64_t)(0x7fffffff / tiles_n) * DBM;
        // split K where the workspace allows it (float32 partials of every split)
        const int64_t splits = direct_splits(m, n, k);
        if (splits > 1 && workspace && workspace_bytes >= gemm_workspace_bytes(m, n, k))
            return launch_direct(x, m, packed, scales, biases, n, kb, bits, gshift, y, (m + DBM - 1) / DBM, tiles_n,
                                 static_cast<float*>(workspace), splits, stream);
        for (int64_t m_off = 0; m_off < m; m_off += max_rows) {
            const int64_t mm = (m - m_off < max_rows) ? (m - m_off) : max_rows;
            const int64_t tiles_m = (mm + DBM - 1) / DBM;
            const hipError_t e = launch_direct(x + (size_t)m_off * k, mm, packed, scales, biases, n, kb, bits, gshift,
                                               y + (size_t)m_off * n, tiles_m, tiles_n, nullptr, 1, stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    switch (bits) {
        case 1: return launch_bits<1>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 2: return launch_bits<2>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 3: return launch_bits<3>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 4: return launch_bits<4>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 5: return launch_bits<5>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 6: return launch_bits<6>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        case 8: return launch_bits<8>(x, m, packed, scales, biases, n, kb, gshift, y, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qaff
