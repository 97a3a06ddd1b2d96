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

template <int BITS>
hipError_t launch_bits(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                       const uint16_t* biases, int64_t n, int64_t kb, uint32_t gshift, uint16_t* y,
                       hipStream_t stream) {
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
    switch (bits) {
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
