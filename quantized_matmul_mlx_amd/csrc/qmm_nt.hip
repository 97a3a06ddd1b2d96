// The quantized product without the transpose (nuvec_core quantized.rs, `quantized_matmul` with
// transpose = false): y[m, n] = sum over k of x[m, k] * w[k, n], for a weight stored [k, n] whose
// rows (the k index) are bit streams of n codes in groups of G along n.
//
// The output runs along the weight's rows, so a lane owns one 32-column block (a whole group
// part: G >= 32) and walks down k. With w = s c + b of the row's group:
//     sum_k x[k] w[k, n] = sum_k (x[k] s[k]) c[k, n] + sum_k x[k] b[k]
// one multiply-add per code and x row, plus one per row for the bias term.
// There are only n/32 column blocks, so K is split over blocks too: each block writes float32
// partial sums of its K chunk to a caller-provided workspace, and a second kernel adds the chunks
// in order (deterministic) and rounds y.
//  * Block: 256 threads over 16 column blocks (512 columns) x 16 row phases, and a chunk of 128
//    rows of K: lane (cb, p) takes rows k0 + p + 16 i, i < 8, and issues all their loads (codes,
//    scale, bias, x for m <= 2 rows per launch) before any arithmetic: one wait per block.
//    (Measured at [4096, 4096] 4-bit, M = 1: 8 rows per lane 9.8 us, 16 rows 10.5, 4 rows 11.4.)
//  * The 16 phases' partial sums are added through LDS (rows padded to 33 floats against bank
//    conflicts).
// x and the scales and biases come in four forms (XK): bf16 x with bf16 scales, float32 x with
// bf16 scales, float16 x with float16 scales, or each of float32, bf16 or float16 as the launch
// says (the module's promotion of x, scales and biases to one float type); every value is widened
// to float32 exactly, so the sums are the same arithmetic in all four. The fixed-type forms issue
// a lane's loads back to back; the run-time form's per-load type switches take about twice as
// long at the decode shape.
#include "launch.h"
#include "qaff_device.h"

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

namespace qaff {
namespace {

// The float32 partial sums of qaff_qmm_nt_static (for callers that cannot allocate): one array per
// device, held until the process ends. Host code never names it after set-up; it uses the device
// address that hipGetSymbolAddress returns for the current device (qmm_nt_static_scratch).
static __device__ __align__(256) uint8_t scratch[kQmmNtStaticScratchBytes];

constexpr int kNtThreads = 256;
constexpr int kNtCols = 16;    // column blocks per thread block
constexpr int kNtPhases = 16;  // row phases per thread block
constexpr int kNtMaxM = 2;     // x rows per launch
constexpr int kNtPad = 33;     // floats per (phase, column block, row) in the LDS sums
// rows per lane and K chunk (all loaded at once: fewer for the wider codes, within the registers)
template <int BITS>
constexpr int kNtRows = 8;

// The 32 codes of a block as float32. 4-bit codes: the even and odd nibbles of each word go to the
// bytes of two words (one AND, one shift-AND), whose bytes convert directly (v_cvt_f32_ubyte0..3);
// the empty asm keeps the compiler from turning them back into one bit-field extract per code.
template <int BITS>
__device__ __forceinline__ void codes_f32(const uint32_t (&w)[BITS], float (&cf)[32]) {
    if constexpr (BITS == 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t lo = w[q] & 0x0f0f0f0fu;
            uint32_t hi = (w[q] >> 4) & 0x0f0f0f0fu;
            asm("" : "+v"(lo), "+v"(hi));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                cf[8 * q + 2 * e] = (float)((lo >> (8 * e)) & 0xffu);
                cf[8 * q + 2 * e + 1] = (float)((hi >> (8 * e)) & 0xffu);
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < 32; ++c) cf[c] = (float)code_at<BITS>(w, c);
    }
}

// XK: 0 bf16 x and bf16 scales, 1 float32 x and bf16 scales, 3 float16 x and float16 scales, 2 x
// of dtype code xd and scales and biases of sbd (0 float32, 1 bf16, 2 float16).
template <int BITS, int MB, int XK>
__global__ __launch_bounds__(kNtThreads) void qmm_nt_partial_kernel(
    const void* x, uint32_t m, const uint32_t* packed, const void* scales, const void* biases,
    uint32_t n, uint32_t k, uint32_t gshift, int xd, int sbd, float* ws) {
    __shared__ float red[kNtPhases * kNtCols * MB * kNtPad];  // [phase][column block][MB][kNtPad]
    const int tid = threadIdx.x;
    const int cbl = tid & (kNtCols - 1);
    const int phase = tid >> 4;
    const uint32_t ncb = n >> 5;
    const uint32_t cb = blockIdx.x * kNtCols + cbl;
    const uint32_t cbc = min(cb, ncb - 1);        // loads stay in bounds; stores are skipped
    constexpr int kRows = kNtRows<BITS>;
    const uint32_t k0 = blockIdx.y * (kNtPhases * kRows);
    const uint32_t gpr = n >> (5 + gshift);       // groups per weight row
    const uint32_t g = cbc >> gshift;             // this column block's group

    // 1. Every load first: the lane's kRows rows (k0 + phase + 16 i) of codes, scale, bias and x.
    //    Rows past k are clamped and get x = 0, so they add nothing.
    uint32_t w[kRows][BITS];
    uint32_t sraw[kRows], braw[kRows];  // XK 0, 1, 3: the 16-bit patterns
    float sv[kRows], bv[kRows];         // XK 2: widened at the load
    float xv[kRows][MB];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const uint32_t kk = k0 + phase + kNtPhases * i;
        const uint32_t kc = min(kk, k - 1);
        load_block<BITS>(packed + ((size_t)kc * ncb + cbc) * BITS, w[i]);
        const size_t si = (size_t)kc * gpr + g;
        if constexpr (XK == 2) {
            sv[i] = load_as_f32(scales, si, sbd);
            bv[i] = load_as_f32(biases, si, sbd);
        } else {
            sraw[i] = static_cast<const uint16_t*>(scales)[si];
            braw[i] = static_cast<const uint16_t*>(biases)[si];
        }
#pragma unroll
        for (int r = 0; r < MB; ++r) {
            const size_t o = (size_t)min((uint32_t)r, m - 1) * k + kc;
            const float v = XK == 2 ? load_as_f32(x, o, xd)
                          : XK == 1 ? static_cast<const float*>(x)[o]
                          : XK == 3 ? __half2float(__ushort_as_half(static_cast<const uint16_t*>(x)[o]))
                                    : bf16_to_f32(static_cast<const uint16_t*>(x)[o]);
            xv[i][r] = kk < k ? v : 0.f;
        }
    }

    // 2. The chunk's sums.
    float acc[MB][32];
    float bsum[MB];
#pragma unroll
    for (int r = 0; r < MB; ++r) {
        bsum[r] = 0.f;
#pragma unroll
        for (int c = 0; c < 32; ++c) acc[r][c] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const float s = XK == 2 ? sv[i]
                      : XK == 3 ? __half2float(__ushort_as_half((uint16_t)sraw[i])) : bf16_to_f32(sraw[i]);
        const float b = XK == 2 ? bv[i]
                      : XK == 3 ? __half2float(__ushort_as_half((uint16_t)braw[i])) : bf16_to_f32(braw[i]);
        float cf[32];
        codes_f32<BITS>(w[i], cf);
#pragma unroll
        for (int r = 0; r < MB; ++r) {
            const float xsv = xv[i][r] * s;
            bsum[r] = __builtin_fmaf(xv[i][r], b, bsum[r]);
#pragma unroll
            for (int c = 0; c < 32; ++c) acc[r][c] = __builtin_fmaf(xsv, cf[c], acc[r][c]);
        }
    }

    // 3. Add the 16 phases through LDS, then write the chunk's partial sums.
#pragma unroll
    for (int r = 0; r < MB; ++r)
#pragma unroll
        for (int c = 0; c < 32; ++c) red[((phase * kNtCols + cbl) * MB + r) * kNtPad + c] = acc[r][c] + bsum[r];
    __syncthreads();
    for (int o = tid; o < kNtCols * MB * 32; o += kNtThreads) {
        const int c = o & 31, r = (o >> 5) % MB, cl = o / (32 * MB);
        float sum = 0.f;
#pragma unroll
        for (int p = 0; p < kNtPhases; ++p) sum += red[((p * kNtCols + cl) * MB + r) * kNtPad + c];
        const uint32_t col = (blockIdx.x * kNtCols + cl) * 32 + c;
        if (col < n && (uint32_t)r < m) ws[((size_t)blockIdx.y * MB + r) * n + col] = sum;
    }
}

// y[r, col] = sum over the chunks of ws[chunk][r][col], in chunk order, stored as dtype code OUT
// (0 float32, 1 bf16, 2 float16; round to nearest even).
template <int OUT>
__global__ __launch_bounds__(256) void qmm_nt_reduce_kernel(const float* ws, uint32_t chunks, uint32_t mb,
                                                            uint32_t m, uint32_t n, void* y) {
    const uint32_t o = blockIdx.x * 256 + threadIdx.x;
    if (o >= m * n) return;
    const uint32_t r = o / n, col = o % n;
    // in chunk order, 32 loads in flight at a time (indices past the last chunk re-read it and
    // are not added)
    float sum = 0.f;
    for (uint32_t s = 0; s < chunks; s += 32) {
        float v[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) v[j] = ws[((size_t)min(s + j, chunks - 1) * mb + r) * n + col];
#pragma unroll
        for (int j = 0; j < 32; ++j)
            if (s + j < chunks) sum += v[j];
    }
    store_from_f32(y, o, OUT, sum);
}

}  // namespace

// The K chunking: chunks of kNtRows rows per row phase, one thread block per chunk and column
// tile.
int64_t qmm_nt_chunk_rows(int bits) {
    return (int64_t)kNtPhases * (bits >= 6 ? kNtRows<8> : kNtRows<4>);
}

void qmm_nt_plan(int64_t k, int64_t n, int bits, int64_t* kchunk, int64_t* chunks) {
    (void)n;
    *kchunk = qmm_nt_chunk_rows(bits);
    *chunks = (k + *kchunk - 1) / *kchunk;
}

size_t qmm_nt_workspace_bytes(int64_t m, int64_t k, int64_t n, int bits) {
    int64_t kc, chunks;
    qmm_nt_plan(k, n, bits, &kc, &chunks);
    const int64_t mb = m < kNtMaxM ? m : kNtMaxM;
    return (size_t)(chunks * mb * n) * sizeof(float);
}

namespace {

// The operand types of one launch: x and scales/biases dtype codes, y's, and the kernel form.
struct NtTypes {
    int xd, sbd, yd, xk;
};

template <int BITS, int MB, int XK>
hipError_t launch_slice(const void* x, int64_t m, const uint32_t* packed, const void* scales, const void* biases,
                        int64_t k, int64_t n, uint32_t gshift, int64_t chunks, const NtTypes& t, float* ws, void* y,
                        hipStream_t stream) {
    const unsigned gx = (unsigned)(((n / 32) + kNtCols - 1) / kNtCols);
    qmm_nt_partial_kernel<BITS, MB, XK><<<dim3(gx, (unsigned)chunks), kNtThreads, 0, stream>>>(
        x, (uint32_t)m, packed, scales, biases, (uint32_t)n, (uint32_t)k, gshift, t.xd, t.sbd, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned gr = (unsigned)((m * n + 255) / 256);
    if (t.yd == 1)
        qmm_nt_reduce_kernel<1><<<gr, 256, 0, stream>>>(ws, (uint32_t)chunks, MB, (uint32_t)m, (uint32_t)n, y);
    else if (t.yd == 2)
        qmm_nt_reduce_kernel<2><<<gr, 256, 0, stream>>>(ws, (uint32_t)chunks, MB, (uint32_t)m, (uint32_t)n, y);
    else
        qmm_nt_reduce_kernel<0><<<gr, 256, 0, stream>>>(ws, (uint32_t)chunks, MB, (uint32_t)m, (uint32_t)n, y);
    return hipGetLastError();
}

template <int BITS, int MB>
hipError_t launch_form(const void* x, int64_t m, const uint32_t* packed, const void* scales, const void* biases,
                       int64_t k, int64_t n, uint32_t gshift, int64_t chunks, const NtTypes& t, float* ws, void* y,
                       hipStream_t stream) {
    switch (t.xk) {
        case 0: return launch_slice<BITS, MB, 0>(x, m, packed, scales, biases, k, n, gshift, chunks, t, ws, y, stream);
        case 1: return launch_slice<BITS, MB, 1>(x, m, packed, scales, biases, k, n, gshift, chunks, t, ws, y, stream);
        case 3: return launch_slice<BITS, MB, 3>(x, m, packed, scales, biases, k, n, gshift, chunks, t, ws, y, stream);
        default: return launch_slice<BITS, MB, 2>(x, m, packed, scales, biases, k, n, gshift, chunks, t, ws, y, stream);
    }
}

template <int BITS>
hipError_t launch_bits(const void* x, int64_t m, const uint32_t* packed, const void* scales, const void* biases,
                       int64_t k, int64_t n, uint32_t gshift, const NtTypes& t, float* ws, void* y,
                       hipStream_t stream) {
    int64_t kchunk, chunks;
    qmm_nt_plan(k, n, BITS, &kchunk, &chunks);
    const size_t xsize = t.xd == 0 ? 4 : 2, ysize = t.yd == 0 ? 4 : 2;
    for (int64_t m0 = 0; m0 < m; m0 += kNtMaxM) {
        const int64_t mm = m - m0 < kNtMaxM ? m - m0 : kNtMaxM;
        const void* xs = static_cast<const uint8_t*>(x) + (size_t)m0 * k * xsize;
        void* ys = static_cast<uint8_t*>(y) + (size_t)m0 * n * ysize;
        const hipError_t e =
            mm == 1 ? launch_form<BITS, 1>(xs, mm, packed, scales, biases, k, n, gshift, chunks, t, ws, ys, stream)
                    : launch_form<BITS, 2>(xs, mm, packed, scales, biases, k, n, gshift, chunks, t, ws, ys, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t qmm_nt_static_scratch(void** ptr) {
    static std::mutex mu;
    static std::vector<void*> addr;  // per device; null until resolved
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current: its own copy
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_qmm_nt(const void* x, int x_dtype, int64_t m, const uint32_t* packed, const void* scales,
                         const void* biases, int sb_dtype, int64_t k, int64_t n, int group_size, int bits,
                         void* workspace, void* y, int y_dtype, hipStream_t stream) {
    const uint32_t gshift = group_size == 32 ? 0u : group_size == 64 ? 1u : 2u;
    float* ws = static_cast<float*>(workspace);
    // bf16 scales with a bf16 or float32 x (and y of x's type), and all-float16 operands, take the
    // fixed-type forms
    const int xk = sb_dtype == 1 && x_dtype == 1 && y_dtype == 1 ? 0
                 : sb_dtype == 1 && x_dtype == 0 && y_dtype == 0 ? 1
                 : sb_dtype == 2 && x_dtype == 2 && y_dtype == 2 ? 3 : 2;
    const NtTypes t{x_dtype, sb_dtype, y_dtype, xk};
    switch (bits) {
        case 1: return launch_bits<1>(x, m, packed, scales, biases, k, n, gshift, t, ws, y, stream);
        case 2: return launch_bits<2>(x, m, packed, scales, biases, k, n, gshift, t, ws, y, stream);
        case 3: return launch_bits<3>(x, m, packed, scales, biases, k, n, gshift, t, ws, y, stream);
        case 4: return launch_bits<4>(x, m, packed, scales, biases, k, n, gshift, t, ws, y, stream);
        case 5: return launch_bits<5>(x, m, packed, scales, biases, k, n, gshift, t, ws, y, stream);
        case 6: return launch_bits<6>(x, m, packed, scales, biases, k, n, gshift, t, ws, y, stream);
        case 8: return launch_bits<8>(x, m, packed, scales, biases, k, n, gshift, t, ws, y, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qaff
