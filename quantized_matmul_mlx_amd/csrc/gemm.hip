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

// ---- 128 x 256 tiles for 4-bit codes ------------------------------------------------------------
//
// The prefill shape is limited by what the compute units pull through L2, not by HBM: X is re-read
// once per tile column and W once per tile row. A 128 (M) x 256 (N) tile halves the X traffic of
// the 256 x 128 tile at the price of twice the dequantization per multiply, and three changes keep
// the rest of the traffic in whole cache lines and the dequantization cheap:
//  * W is fetched one 128-byte line per row at a time, i.e. four K-steps (a "super-step") at once:
//    in load instruction i, the eight lanes of row group g read the eight 16-byte blocks of row
//    4 g + i, lane (q, b) block 2 ((q + i) & 3) + b. Every lane thereby holds exactly one block of
//    every K-step of the super-step, in register slot (u - q) & 3 for step u, and picks it with
//    three selects.
//  * Scales and biases arrive in windows of 8 groups (16 bytes per row), one window per thread,
//    and are kept in LDS as float32.
//  * The multiply uses v_mfma_f32_32x32x16_bf16, which leaves more issue slots for the
//    dequantization between matrix instructions than the 16x16x32 form, and each step's
//    dequantization is interleaved with its matrix instructions.
// Requirements (checked by the launcher): K a multiple of 8 groups and of 64 * kWideBody; W,
// scales and biases 16-byte aligned. Rows of X beyond m and rows of W beyond n are clamped, not
// zeroed: they only reach outputs that are not stored.
//
// MFMA 32x32x16 (bf16) layout: lane l supplies row l % 32 of A and of W (column of B), each as the
// 8 consecutive k starting at 8 * (l / 32); result value v of lane l is row 8 (v / 4) + 4 (l / 32)
// + v % 4, column l % 32. LDS rows are padded to 72 bf16 (144 bytes), which spreads 8 (16) rows
// read at one chunk over distinct banks and keeps the chunk offsets compile-time immediates.

constexpr int WBM = 128;
constexpr int WBN = 256;
constexpr int kWideThreads = 512;
constexpr int kWideA = WBM * LDK;  // bf16 elements of one A buffer
constexpr int kWideB = WBN * LDK;  // bf16 elements of one B buffer
constexpr int kSbPitch = 9;        // floats per row in the scale (bias) window: 8 groups + 1 padding
constexpr int kWideBody = 16;      // K-steps per loop iteration (windows are 4, 8 or 16 steps)

typedef float f32x16 __attribute__((ext_vector_type(16)));

// v_cndmask_b32 with a lane mask: `if_set` in the lanes of `mask`, `if_clear` elsewhere. Written
// out because the compiler turns chains of lane-dependent selects into divergent branches.
__device__ __forceinline__ uint32_t lane_select(uint64_t mask, uint32_t if_set, uint32_t if_clear) {
    uint32_t r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(if_clear), "v"(if_set), "s"(mask));
    return r;
}

template <int GSHIFT>
__global__ __launch_bounds__(kWideThreads) void gemm_wide_kernel(
    const uint16_t* x, uint32_t m, const uint32_t* packed, const uint16_t* scales,
    const uint16_t* biases, uint32_t n, uint32_t kb, uint16_t* y, uint32_t tiles_m,
    uint32_t tiles_n) {
    constexpr int P = (32 << GSHIFT) / 8;  // K-steps per window of 8 groups: 4, 8 or 16
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][kWideA + kWideB];
    __shared__ float sbl[2][2][WBN * kSbPitch];  // [buffer][scale, bias][row * 9 + group]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2;  // 64-row slice of the tile
    const int wn = wave & 3;   // 64-column slice

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
    const uint32_t m0 = tm * WBM;
    const uint32_t n0 = tn * WBN;
    const uint32_t k = kb * 32;
    const uint32_t gpr = kb >> GSHIFT;  // groups per row
    const uint32_t ktiles = kb >> 1;    // K-steps
    const uint32_t nsuper = kb >> 3;    // super-steps
    const uint32_t nwin = gpr >> 3;     // scale windows

    // Per-block bases (uniform) and 32-bit per-lane offsets: a tile spans far less than 4 GiB.
    const uint16_t* xb = x + (size_t)m0 * k;
    const uint32_t* wbase = packed + (size_t)n0 * (kb * 4);

    // X: two 16-byte chunks per thread and step, rows xrow and xrow + 64, chunk xkc.
    const int xrow = tid >> 3;
    const int xkc = tid & 7;
    const uint32_t xo0 = (min(m0 + xrow, m - 1) - m0) * k + xkc * 8;
    const uint32_t xo1 = (min(m0 + xrow + 64, m - 1) - m0) * k + xkc * 8;
    const int xa0 = xrow * LDK + xkc * 8;
    const int xa1 = (xrow + 64) * LDK + xkc * 8;

    // W: row group g, lane pair q, block b (see above).
    const int wg = tid >> 3;
    const int wq = (tid >> 1) & 3;
    const int wb = tid & 1;
    uint32_t wo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        wo[i] = (min(n0 + 4 * wg + i, n - 1) - n0) * (kb * 4) + (((wq + i) & 3) * 2 + wb) * 4;

    // Scale (threads 0..255) or bias (256..511) window of row sb_row.
    const int sb_arr = tid >> 8;
    const int sb_row = tid & 255;
    const uint16_t* sbp = (sb_arr ? biases : scales) + (size_t)min(n0 + sb_row, n - 1) * gpr;

    auto load_x = [&](u32x4a (&xr)[2], uint32_t kt) {
        const uint16_t* p = xb + min(kt, ktiles - 1) * BK;
        xr[0] = *reinterpret_cast<const u32x4a*>(p + xo0);
        xr[1] = *reinterpret_cast<const u32x4a*>(p + xo1);
    };
    auto load_w = [&](u32x4a (&wr)[4], uint32_t s) {
        const uint32_t* p = wbase + min(s, nsuper - 1) * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) wr[i] = *reinterpret_cast<const u32x4a*>(p + wo[i]);
    };
    auto load_sb = [&](u32x4a& r, uint32_t win) { r = *reinterpret_cast<const u32x4a*>(sbp + min(win, nwin - 1) * 8); };
    auto store_sb = [&](const u32x4a& r, int buf) {
        float* d = &sbl[buf][sb_arr][sb_row * kSbPitch];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            d[2 * e] = __uint_as_float(r[e] << 16);
            d[2 * e + 1] = __uint_as_float(r[e] & 0xffff0000u);
        }
    };
    auto store_x = [&](const u32x4a (&xr)[2], int buf) {
        *reinterpret_cast<u32x4a*>(&lds[buf][xa0]) = xr[0];
        *reinterpret_cast<u32x4a*>(&lds[buf][xa1]) = xr[1];
    };

    // Lanes whose register slot i (0..2) holds K-step u of a super-step: q == u - i.
    uint64_t sel[4][3];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 3; ++i) sel[u][i] = __builtin_amdgcn_ballot_w64(wq == ((u - i) & 3));

    // Dequantization of this lane's block of K-step dkt (u = dkt % 4) into B buffer dbuf, split in
    // four parts (one word, 8 codes, 16 bytes of the tile each) to interleave with the multiply.
    struct Deq {
        uint32_t w[4];
        float s, b;
        uint16_t* dst;
    };
    auto deq_begin = [&](const u32x4a (&wr)[4], uint32_t dkt, int u, int dbuf) {
        Deq d;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint32_t v = lane_select(sel[u][2], wr[2][c], wr[3][c]);
            v = lane_select(sel[u][1], wr[1][c], v);
            d.w[c] = lane_select(sel[u][0], wr[0][c], v);
        }
        const int row = 4 * wg + ((u - wq) & 3);
        const int grp = (int)(((dkt * 2 + wb) >> GSHIFT) & 7u);
        const int sbuf = (int)((dkt / P) & 1u);
        d.s = sbl[sbuf][0][row * kSbPitch + grp];
        d.b = sbl[sbuf][1][row * kSbPitch + grp];
        d.dst = lds[dbuf] + kWideA + row * LDK + wb * 32;
        return d;
    };
    auto deq_part = [&](const Deq& d, int c) {
        // even codes in the bytes of lo, odd codes in those of hi; the empty asm keeps the compiler
        // from turning the byte conversions back into one bit-field extract per code
        uint32_t lo = d.w[c] & 0x0f0f0f0fu;
        uint32_t hi = (d.w[c] >> 4) & 0x0f0f0f0fu;
        asm("" : "+v"(lo), "+v"(hi));
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = pack_bf16x2(__builtin_fmaf(d.s, (float)((lo >> (8 * j)) & 0xffu), d.b),
                               __builtin_fmaf(d.s, (float)((hi >> (8 * j)) & 0xffu), d.b));
        *reinterpret_cast<u32x4a*>(d.dst + 8 * c) = u32x4a{o[0], o[1], o[2], o[3]};
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // Operand rows: wm*64 + 32 i + lane % 32 of A, wn*64 + 32 j + lane % 32 of B; chunk 2 kk +
    // lane / 32 of the step is a constant offset from these.
    const int aoff = (wm * 64 + (lane & 31)) * LDK + (lane >> 5) * 8;
    const int boff = kWideA + (wn * 64 + (lane & 31)) * LDK + (lane >> 5) * 8;
    auto read_ops = [&](const uint16_t* L, int kk, bf16x8 (&a)[2], bf16x8 (&b)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const bf16x8*>(L + aoff + 32 * i * LDK + 16 * kk);
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const bf16x8*>(L + boff + 32 * j * LDK + 16 * kk);
    };
    // Multiplies step buffer cbuf while dequantizing the next step (d) into the other buffer.
    auto compute_deq = [&](int cbuf, const Deq& d) {
        const uint16_t* L = lds[cbuf];
        bf16x8 a[2][2], b[2][2];
        read_ops(L, 0, a[0], b[0]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if (kk < 3) read_ops(L, kk + 1, a[(kk + 1) & 1], b[(kk + 1) & 1]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk & 1][i], b[kk & 1][j], acc[i][j], 0, 0, 0);
            deq_part(d, kk);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Prologue: window 0 in LDS, step 0 in buffer 0, steps 1 and 2 of X in flight, super-steps 0
    // and 1 of W in registers.
    u32x4a xr[2][2], wr[2][4], sbr;
    load_sb(sbr, 0);
    load_w(wr[0], 0);
    load_w(wr[1], 1);
    load_x(xr[0], 0);
    load_x(xr[1], 1);
    store_sb(sbr, 0);
    store_x(xr[0], 0);
    load_x(xr[0], 2);
    __syncthreads();
    {
        const Deq d = deq_begin(wr[0], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < 4; ++c) deq_part(d, c);
    }
    __syncthreads();

    // Step kt: store X of step kt+1 into the free buffer and issue the loads of step kt+3 (of
    // super-step kt/4 + 2 at the end of a super-step; of the next scale window at the start of a
    // window, stored to LDS two steps before its first use), then multiply step kt while
    // dequantizing W of step kt+1 into the free buffer. Register sets are fixed by the position in
    // the unrolled body: X by the step's parity, W by the super-step's.
    for (uint32_t kt0 = 0; kt0 < ktiles; kt0 += kWideBody) {
#pragma unroll
        for (int u = 0; u < kWideBody; ++u) {
            const uint32_t kt = kt0 + u;
            const int nb = (u + 1) & 1;
            const int ws = ((u + 1) >> 2) & 1;  // W set of step kt+1
            store_x(xr[nb], nb);
            if (((u + 1) & 3) == 0) load_w(wr[ws ^ 1], (kt + 1) / 4 + 1);
            load_x(xr[nb], kt + 3);
            if (u % P == 0) load_sb(sbr, (kt + P) / P);
            // Keep the loads here: the operands are read-only, so the compiler could otherwise sink
            // them towards their first use and lose the prefetch distance.
            asm volatile("" ::: "memory");
            if (u % P == P - 2) store_sb(sbr, (int)(((kt + 2) / P) & 1u));
            const Deq d = deq_begin(wr[ws], kt + 1, (u + 1) & 3, nb);
            compute_deq(u & 1, d);
            __syncthreads();
        }
    }

    const int ocol = lane & 31;
    const int orow = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const uint32_t gm = m0 + wm * 64 + 32 * i + 8 * (v >> 2) + orow + (v & 3);
                const uint32_t gc = n0 + wn * 64 + 32 * j + ocol;
                if (gm < m && gc < n) y[(size_t)gm * n + gc] = to_bf16_bits(acc[i][j][v]);
            }
}

// Waves of the 256 x 128 tile along M (WN = 2 along N): 2 gives four 128 x 64 wave tiles, 4 gives
// eight 64 x 64 ones.
#ifndef QAFF_GEMM_WM
#define QAFF_GEMM_WM 4
#endif
constexpr int kBigWM = QAFF_GEMM_WM;
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

}  // namespace

hipError_t launch_gemm(const uint16_t* x, int64_t m, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                       int group_size, int bits, uint16_t* y, hipStream_t stream) {
    const int64_t kb = k / 32;
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    auto a16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
    if (bits == 4 && m >= kBigTileMinM && k % (64 * kWideBody) == 0 && k % (8 * (int64_t)group_size) == 0 &&
        a16(packed) && a16(scales) &&
        a16(biases)) {
        const int64_t tiles_n = (n + WBN - 1) / WBN;
        const int64_t max_rows = (int64_t)(0x7fffffff / tiles_n) * WBM;
        for (int64_t m_off = 0; m_off < m; m_off += max_rows) {
            const int64_t mm = (m - m_off < max_rows) ? (m - m_off) : max_rows;
            const int64_t tiles_m = (mm + WBM - 1) / WBM;
            const dim3 grid((unsigned)(tiles_m * tiles_n));
            const uint16_t* xs = x + (size_t)m_off * k;
            uint16_t* ys = y + (size_t)m_off * n;
            switch (gshift) {
                case 0: gemm_wide_kernel<0><<<grid, kWideThreads, 0, stream>>>(xs, (uint32_t)mm, packed, scales, biases, (uint32_t)n, (uint32_t)kb, ys, (uint32_t)tiles_m, (uint32_t)tiles_n); break;
                case 1: gemm_wide_kernel<1><<<grid, kWideThreads, 0, stream>>>(xs, (uint32_t)mm, packed, scales, biases, (uint32_t)n, (uint32_t)kb, ys, (uint32_t)tiles_m, (uint32_t)tiles_n); break;
                default: gemm_wide_kernel<2><<<grid, kWideThreads, 0, stream>>>(xs, (uint32_t)mm, packed, scales, biases, (uint32_t)n, (uint32_t)kb, ys, (uint32_t)tiles_m, (uint32_t)tiles_n); break;
            }
            const hipError_t e = hipGetLastError();
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
