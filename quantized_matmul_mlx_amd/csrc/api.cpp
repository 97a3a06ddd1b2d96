// The C ABI declared in include/qaff.h: argument checks (all on the host, before any HIP call),
// kernel dispatch and the per-thread error text.
//
// The checks follow the pages' own: nuvec_core quantized.rs `check_params` (group sizes 32/64/128;
// bit widths 1-6 and 8), rlx-moshi mlx_dequant.rs
// `dequantize_affine` (the group size divides the columns; the packed width is cols*bits/32) and
// spark_runtime weights/mlx_int8.rs `MlxInt8Weight::load` (scales and biases are [rows, cols/G]).
// Shapes are implied by the sizes passed in, so only sizes, pointers and alignment can be checked.
#include "qaff.h"

#include "launch.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

namespace {

thread_local std::string g_error;

qaff_status fail(qaff_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}

constexpr int kGemvMaxM = 16;
constexpr int kGemvMfmaMinM = 3;
// Past 4096 codes the VALU GEMV's long rows cost more: the matrix-core decode kernel wins from 2
// rows there ([4096, 14336] 4-bit at m = 2: 11.2 against 12.4 us with groups of 64).
int64_t gemv_mfma_min_m(int64_t k) { return k > 4096 ? 2 : kGemvMfmaMinM; }
// Gathered products grouped by expert take the GEMM over each expert's rows once the experts
// average this many rows (below, the matrix-core decode kernel's 16-row tiles).
constexpr int64_t kGroupedGemmRows = 32;

bool debug_sync() {
    static const bool on = [] {
        const char* v = std::getenv("QAFF_DEBUG_SYNC");
        return v && v[0] && std::strcmp(v, "0") != 0;
    }();
    return on;
}

qaff_status after_launch(const char* op, hipError_t e, hipStream_t stream) {
    if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(QAFF_ERR_DEVICE, "%s: %s", op, hipGetErrorString(e));
    return QAFF_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Bytes of one element of a dtype (x, y and outputs need this much alignment; 16-byte aligned ones
// take the vector kernels, the others the element-by-element ones).
uintptr_t esize_of(qaff_dtype d) { return d == QAFF_F32 ? 4 : 2; }

// Checks shared by every entry point: bits, group size, cols and the weight pointers.
qaff_status check_weight(const char* op, const uint32_t* packed, const uint16_t* scales,
                         const uint16_t* biases, int64_t rows, int64_t cols, int32_t group_size,
                         int32_t bits) {
    if (bits < 1 || bits > 8 || bits == 7)
        return fail(QAFF_ERR_UNSUPPORTED, "%s: %d bits are not supported (1, 2, 3, 4, 5, 6 or 8)", op, bits);
    if (group_size != 32 && group_size != 64 && group_size != 128)
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: group size %d is not supported (32, 64 or 128)", op, group_size);
    if (rows < 0 || cols < 0) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: negative size", op);
    if (cols % group_size != 0)
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: %lld columns are not a multiple of the group size %d", op,
                    (long long)cols, group_size);
    if (rows > 0 && cols > 0) {
        if (!packed || !scales || !biases) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null weight pointer", op);
        if (!aligned(packed, 4)) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: packed codes must be 4-byte aligned", op);
        if (!aligned(scales, 2) || !aligned(biases, 2))
            return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: scales and biases must be 2-byte aligned", op);
    }
    if (rows > 0xffffffffLL) return fail(QAFF_ERR_UNSUPPORTED, "%s: more than 2^32-1 weight rows", op);
    // the kernels address within a row's code stream (cols * bits bits) in 32 bits
    if (cols > 0xffffffffLL / bits)
        return fail(QAFF_ERR_UNSUPPORTED, "%s: a row of %lld %d-bit codes is 2^32 bits or longer", op, (long long)cols,
                    bits);
    return QAFF_OK;
}

bool valid_dtype(qaff_dtype d) { return d == QAFF_F32 || d == QAFF_BF16; }
bool any_dtype(qaff_dtype d) { return d == QAFF_F32 || d == QAFF_BF16 || d == QAFF_F16; }

qaff_status dequant_common(const char* op, const uint32_t* packed, const uint16_t* scales,
                           const uint16_t* biases, int64_t table_rows, int64_t cols,
                           int32_t group_size, int32_t bits, const uint32_t* indices,
                           int64_t out_rows, bool gather, void* out, qaff_dtype out_dtype,
                           hipStream_t stream) {
    g_error.clear();
    qaff_status st = check_weight(op, packed, scales, biases, table_rows, cols, group_size, bits);
    if (st != QAFF_OK) return st;
    if (!valid_dtype(out_dtype)) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: unknown output dtype %d", op, (int)out_dtype);
    if (out_rows < 0) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: negative number of indices", op);
    if (out_rows == 0 || cols == 0) return QAFF_OK;
    if (gather) {
        if (!indices) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null indices", op);
        if (!aligned(indices, 4)) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: indices must be 4-byte aligned", op);
        if (table_rows > 0 && (!packed || !scales || !biases))
            return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null weight pointer", op);
    }
    if (!out) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null output", op);
    if (!aligned(out, esize_of(out_dtype)))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: output must be aligned to its element size", op);
    if (out_rows * (cols / 32) >= (1LL << 31))
        return fail(QAFF_ERR_UNSUPPORTED, "%s: output of %lld x %lld is too large", op, (long long)out_rows, (long long)cols);
    // an output that is not 16-byte aligned is stored element by element (the same values)
    hipError_t e = aligned(out, 16)
        ? qaff::launch_dequant(packed, scales, biases, gather ? indices : nullptr, table_rows, out_rows, cols,
                               group_size, bits, out, out_dtype == QAFF_BF16, stream)
        : qaff::launch_dequant_typed(packed, scales, biases, (int)QAFF_BF16, out_rows, cols, group_size, bits, out,
                                     (int)out_dtype, stream, gather ? indices : nullptr, table_rows);
    return after_launch(op, e, stream);
}

}  // namespace

namespace qaff {

int device_cu_count() {
    static std::mutex mu;
    static std::vector<int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}

}  // namespace qaff

extern "C" {

qaff_status qaff_dequantize(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                            int64_t rows, int64_t cols, int32_t group_size, int32_t bits, void* out,
                            qaff_dtype out_dtype, hipStream_t stream) {
    return dequant_common("qaff_dequantize", packed, scales, biases, rows, cols, group_size, bits,
                          nullptr, rows, false, out, out_dtype, stream);
}

qaff_status qaff_dequant_rows(const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                              int64_t table_rows, int64_t cols, int32_t group_size, int32_t bits,
                              const uint32_t* indices, int64_t n_indices, void* out,
                              qaff_dtype out_dtype, hipStream_t stream) {
    return dequant_common("qaff_dequant_rows", packed, scales, biases, table_rows, cols, group_size,
                          bits, indices, n_indices, true, out, out_dtype, stream);
}

namespace {

// Decode-sized m that take the GEMM with K split when a workspace is given: K beyond the
// matrix-core decode kernel (more than 32768 codes) and a multiple of 1024, from kSplitMinM rows on,
// where the VALU GEMV's work per code and x row outweighs the GEMM's fixed cost.
constexpr int64_t kSplitMinM = 8;
bool split_gemv_range(int64_t m, int64_t k) {
    return m >= kSplitMinM && m <= kGemvMaxM && !qaff::gemv_mfma_supported(m, k) && k % 1024 == 0 && k > 4096;
}

// A few rows past the decode range, without K split through a workspace: 16-row slices through the
// decode kernels (each reads all of W) instead of one GEMM whose few tiles leave most compute units
// idle. Measured on [2048 | 4096 | 8192 | 11008 | 14336, 4096 | 8192 | 14336] weights, 3 to 8
// bits, against the unsplit GEMM: up to 3 slices win everywhere (17 rows of [4096, 14336] 4-bit:
// 24 against 171 us), up to 6 where n <= 8192 and up to 8 where n <= 4096 (128 rows of
// [4096, 14336] 4-bit: 134 against 171 us); past those they lose by up to a fifth.
bool decode_slices(int64_t m, int64_t n, int64_t k) {
    const int64_t slices = (m + kGemvMaxM - 1) / kGemvMaxM;
    if (m <= kGemvMaxM || slices > 8 || !qaff::gemv_mfma_supported(kGemvMaxM, k)) return false;
    return slices <= 3 || (slices <= 6 && n <= 8192) || n <= 4096;
}

// Where the slices also beat the GEMM with K split through a workspace, which then needs none:
// small weights at up to 2 slices ([4096, 4096] at 17 rows: 8.1 against 14.3 us for the split;
// wider or longer weights favour the split).
bool slices_over_split(int64_t m, int64_t n, int64_t k) {
    return decode_slices(m, n, k) && m <= 2 * kGemvMaxM && n <= 4096 && k <= 4096;
}

extern "C++" {
// The rows [m0, m0 + mm) of a decode-sized product (mm <= 16), as qaff_qmm's automatic path would
// run them alone: the matrix-core decode kernel from gemv_mfma_min_m(k) rows, else the VALU GEMV.
// F16: float16 x, scales, biases and y.
template <bool F16>
hipError_t decode_slice(const uint16_t* x, int64_t mm, const uint32_t* packed, const uint16_t* scales,
                        const uint16_t* biases, int64_t n, int64_t k, int32_t group_size, int32_t bits, uint16_t* y,
                        hipStream_t stream) {
    if (mm >= gemv_mfma_min_m(k)) {
        return F16 ? qaff::launch_gemv_mfma_f16(x, mm, packed, scales, biases, n, k, group_size, bits, y, stream)
                   : qaff::launch_gemv_mfma(x, mm, packed, scales, biases, n, k, group_size, bits, y, stream);
    }
    return F16 ? qaff::launch_gemv_f16(x, mm, packed, scales, biases, n, k, group_size, bits, y, stream)
               : qaff::launch_gemv(x, false, mm, packed, scales, biases, n, k, group_size, bits, y, stream);
}

template <bool F16>
hipError_t launch_decode_slices(const uint16_t* x, int64_t m, const uint32_t* packed, const uint16_t* scales,
                                const uint16_t* biases, int64_t n, int64_t k, int32_t group_size, int32_t bits,
                                uint16_t* y, hipStream_t stream) {
    for (int64_t m0 = 0; m0 < m; m0 += kGemvMaxM) {
        const int64_t mm = m - m0 < kGemvMaxM ? m - m0 : kGemvMaxM;
        // x and y offsets are multiples of 16 rows: still 16-byte aligned
        const hipError_t e = decode_slice<F16>(x + (size_t)m0 * k, mm, packed, scales, biases, n, k, group_size, bits,
                                               y + (size_t)m0 * n, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}
}  // extern "C++"

// qaff_qmm_ex, and qaff_qmm_ws with a workspace (ws non-null: the call needs ws_need bytes, checked
// by the caller; the GEMM path may split K into it).
qaff_status qmm_impl(const char* op, const void* x, qaff_dtype x_dtype, int64_t m, const uint32_t* packed,
                     const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                     int32_t group_size, int32_t bits, void* y, hipStream_t stream, qaff_path path,
                     void* ws, size_t ws_bytes) {
    g_error.clear();
    qaff_status st = check_weight(op, packed, scales, biases, n, k, group_size, bits);
    if (st != QAFF_OK) return st;
    if (m < 0) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: negative m", op);
    if (!valid_dtype(x_dtype)) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: unknown x dtype %d", op, (int)x_dtype);
    if (path != QAFF_PATH_AUTO && path != QAFF_PATH_GEMV && path != QAFF_PATH_GEMM && path != QAFF_PATH_GEMV_MFMA)
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: unknown path %d", op, (int)path);
    if (x_dtype == QAFF_F32 && (path == QAFF_PATH_GEMM || path == QAFF_PATH_GEMV_MFMA))
        return fail(QAFF_ERR_UNSUPPORTED, "%s: the MFMA paths take a bf16 x only", op);
    // the matrix-core decode kernel: m <= 16, its K range, scale words readable as 4-byte words
    const bool mfma_ok = x_dtype == QAFF_BF16 && m <= kGemvMaxM && qaff::gemv_mfma_supported(m, k) &&
                         aligned(scales, 4) && aligned(biases, 4);
    if (path == QAFF_PATH_GEMV_MFMA && m > 0 && n > 0 && k > 0 && !mfma_ok)
        return fail(QAFF_ERR_UNSUPPORTED, "%s: the matrix-core decode kernel takes 1 <= m <= 16, k a multiple "
                    "of 512 up to 32768 and 4-byte aligned scales and biases", op);
    if (m == 0 || n == 0) return QAFF_OK;
    const int64_t esize = (int64_t)esize_of(x_dtype);
    if (!y) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null y", op);
    if (!aligned(y, esize)) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: y must be aligned to its element size", op);
    if (k == 0) return after_launch(op, qaff::launch_fill_zero(y, m * n * esize, stream), stream);
    if (!x) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null x", op);
    if (!aligned(x, esize)) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: x must be aligned to its element size", op);
    if (n > 0x7fffffffLL || m > 0x7fffffffLL) return fail(QAFF_ERR_UNSUPPORTED, "%s: m or n above 2^31-1", op);
    if (!aligned(x, 16) || !aligned(y, 16)) {
        // x or y not 16-byte aligned: the element-by-element GEMV (any m)
        if (path == QAFF_PATH_GEMM || path == QAFF_PATH_GEMV_MFMA)
            return fail(QAFF_ERR_UNSUPPORTED, "%s: the MFMA paths need 16-byte aligned x and y", op);
        return after_launch(op, qaff::launch_gemv_scalar(x, (int)x_dtype, m, packed, scales, biases, (int)QAFF_BF16, n,
                                                         k, group_size, bits, y, (int)x_dtype, qaff::ScalarGemv{},
                                                         stream), stream);
    }

    bool use_gemm = false, use_mfma = false;
    if (x_dtype == QAFF_BF16) {
        use_gemm = path == QAFF_PATH_GEMM || (path == QAFF_PATH_AUTO && m > kGemvMaxM);
        use_mfma = path == QAFF_PATH_GEMV_MFMA || (path == QAFF_PATH_AUTO && m >= gemv_mfma_min_m(k) && mfma_ok);
        // with a workspace (qaff_qmm_ws sized it for these m, n, k), a few rows beyond the matrix-core
        // decode kernel's K range take the GEMM with K split, which beats the VALU GEMV there
        if (path == QAFF_PATH_AUTO && ws && m <= kGemvMaxM && !mfma_ok && split_gemv_range(m, k) &&
            aligned(scales, 16) && aligned(biases, 16))
            use_gemm = true;
    }
    // a GEMM with few tiles and no K split: 16-row slices through the decode kernels instead
    const bool gemm_splits = ws && !slices_over_split(m, n, k) && qaff::gemm_workspace_bytes(m, n, k) > 0 &&
                             ws_bytes >= qaff::gemm_workspace_bytes(m, n, k);
    if (x_dtype == QAFF_BF16 && path == QAFF_PATH_AUTO && use_gemm && m > kGemvMaxM && !gemm_splits &&
        decode_slices(m, n, k) && aligned(scales, 4) && aligned(biases, 4))
        return after_launch(op, launch_decode_slices<false>(static_cast<const uint16_t*>(x), m, packed, scales, biases,
                                                            n, k, group_size, bits, static_cast<uint16_t*>(y), stream),
                            stream);
    hipError_t e;
    if (use_mfma && !use_gemm) {
        e = qaff::launch_gemv_mfma(static_cast<const uint16_t*>(x), m, packed, scales, biases, n, k, group_size,
                                   bits, static_cast<uint16_t*>(y), stream);
    } else if (use_gemm) {
        e = qaff::launch_gemm(static_cast<const uint16_t*>(x), m, packed, scales, biases, n, k, group_size,
                              bits, static_cast<uint16_t*>(y), stream, ws, ws_bytes);
    } else {
        e = qaff::launch_gemv(x, x_dtype == QAFF_F32, m, packed, scales, biases, n, k, group_size, bits, y,
                              stream);
    }
    return after_launch(op, e, stream);
}

}  // namespace

qaff_status qaff_qmm_ex(const void* x, qaff_dtype x_dtype, int64_t m, const uint32_t* packed,
                        const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                        int32_t group_size, int32_t bits, void* y, hipStream_t stream, qaff_path path) {
    return qmm_impl("qaff_qmm", x, x_dtype, m, packed, scales, biases, n, k, group_size, bits, y, stream, path,
                    nullptr, 0);
}

size_t qaff_qmm_workspace_size(int64_t m, int64_t n, int64_t k, int32_t group_size, int32_t bits) {
    (void)group_size;
    (void)bits;
    if (n <= 0 || k <= 0) return 0;
    if (m <= kGemvMaxM && !split_gemv_range(m, k)) return 0;
    if (slices_over_split(m, n, k)) return 0;
    return qaff::gemm_workspace_bytes(m, n, k);
}

qaff_status qaff_qmm_ws(const void* x, qaff_dtype x_dtype, int64_t m, const uint32_t* packed,
                        const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                        int32_t group_size, int32_t bits, void* workspace, size_t workspace_bytes, void* y,
                        hipStream_t stream) {
    static const char* op = "qaff_qmm_ws";
    g_error.clear();
    const size_t need = qaff_qmm_workspace_size(m, n, k, group_size, bits);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: the workspace needs %zu bytes (qaff_qmm_workspace_size), got %zu",
                        op, need, workspace ? workspace_bytes : (size_t)0);
        if (!aligned(workspace, 16)) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: workspace must be 16-byte aligned", op);
    }
    return qmm_impl(op, x, x_dtype, m, packed, scales, biases, n, k, group_size, bits, y, stream, QAFF_PATH_AUTO,
                    need > 0 ? workspace : nullptr, need > 0 ? workspace_bytes : 0);
}

qaff_status qaff_gemv_gate_up(const void* x, int64_t m, const uint32_t* gate_packed,
                              const uint16_t* gate_scales, const uint16_t* gate_biases,
                              const uint32_t* up_packed, const uint16_t* up_scales,
                              const uint16_t* up_biases, int64_t n, int64_t k, int32_t group_size,
                              int32_t bits, void* gate_y, void* up_y, hipStream_t stream) {
    static const char* op = "qaff_gemv_gate_up";
    g_error.clear();
    qaff_status st = check_weight(op, gate_packed, gate_scales, gate_biases, n, k, group_size, bits);
    if (st != QAFF_OK) return st;
    st = check_weight(op, up_packed, up_scales, up_biases, n, k, group_size, bits);
    if (st != QAFF_OK) return st;
    if (m < 0) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: negative m", op);
    if (m > kGemvMaxM) return fail(QAFF_ERR_UNSUPPORTED, "%s: a decode product: m <= %d", op, kGemvMaxM);
    if (m == 0 || n == 0) return QAFF_OK;
    if (!gate_y || !up_y) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null output", op);
    if (!aligned(gate_y, 2) || !aligned(up_y, 2))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: outputs must be 2-byte aligned", op);
    if (k == 0) {
        hipError_t e = qaff::launch_fill_zero(gate_y, m * n * 2, stream);
        if (e == hipSuccess) e = qaff::launch_fill_zero(up_y, m * n * 2, stream);
        return after_launch(op, e, stream);
    }
    if (!x) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null x", op);
    if (!aligned(x, 2)) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: x must be 2-byte aligned", op);
    if (n > 0x7fffffffLL) return fail(QAFF_ERR_UNSUPPORTED, "%s: n above 2^31-1", op);
    if (!aligned(x, 16) || !aligned(gate_y, 16) || !aligned(up_y, 16)) {
        // element by element: the two products one after the other
        const qaff::ScalarGemv none{};
        hipError_t e = qaff::launch_gemv_scalar(x, (int)QAFF_BF16, m, gate_packed, gate_scales, gate_biases,
                                                (int)QAFF_BF16, n, k, group_size, bits, gate_y, (int)QAFF_BF16, none,
                                                stream);
        if (e == hipSuccess)
            e = qaff::launch_gemv_scalar(x, (int)QAFF_BF16, m, up_packed, up_scales, up_biases, (int)QAFF_BF16, n, k,
                                         group_size, bits, up_y, (int)QAFF_BF16, none, stream);
        return after_launch(op, e, stream);
    }
    qaff::GemvFused f{};
    f.packed2 = up_packed;
    f.scales2 = up_scales;
    f.biases2 = up_biases;
    f.y2 = static_cast<uint16_t*>(up_y);
    return after_launch(op, qaff::launch_gemv_fused(static_cast<const uint16_t*>(x), m, gate_packed, gate_scales,
                                                    gate_biases, n, k, group_size, bits,
                                                    static_cast<uint16_t*>(gate_y), f, stream), stream);
}

qaff_status qaff_gemv_silu_gate(const void* gate, const void* up, int64_t m, const uint32_t* packed,
                                const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                                int32_t group_size, int32_t bits, const void* resid, void* y,
                                hipStream_t stream) {
    static const char* op = "qaff_gemv_silu_gate";
    g_error.clear();
    qaff_status st = check_weight(op, packed, scales, biases, n, k, group_size, bits);
    if (st != QAFF_OK) return st;
    if (m < 0) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: negative m", op);
    if (m > kGemvMaxM) return fail(QAFF_ERR_UNSUPPORTED, "%s: a decode product: m <= %d", op, kGemvMaxM);
    if (m == 0 || n == 0) return QAFF_OK;
    if (!y) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null y", op);
    if (!aligned(y, 2)) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: y must be 2-byte aligned", op);
    if (resid && !aligned(resid, 2)) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: resid must be 2-byte aligned", op);
    if (k == 0) {  // y = bf16(0 + resid) = resid, or zeros
        if (resid) return after_launch(op, hipMemcpyAsync(y, resid, (size_t)(m * n * 2), hipMemcpyDeviceToDevice, stream), stream);
        return after_launch(op, qaff::launch_fill_zero(y, m * n * 2, stream), stream);
    }
    if (!gate || !up) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null gate or up", op);
    if (!aligned(gate, 2) || !aligned(up, 2))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: gate and up must be 2-byte aligned", op);
    if (n > 0x7fffffffLL) return fail(QAFF_ERR_UNSUPPORTED, "%s: n above 2^31-1", op);
    if (!aligned(gate, 16) || !aligned(up, 16) || !aligned(y, 16)) {
        qaff::ScalarGemv opt{};
        opt.up = static_cast<const uint16_t*>(up);
        opt.resid = static_cast<const uint16_t*>(resid);
        return after_launch(op, qaff::launch_gemv_scalar(gate, (int)QAFF_BF16, m, packed, scales, biases,
                                                         (int)QAFF_BF16, n, k, group_size, bits, y, (int)QAFF_BF16, opt,
                                                         stream), stream);
    }
    qaff::GemvFused f{};
    f.up = static_cast<const uint16_t*>(up);
    f.resid = static_cast<const uint16_t*>(resid);
    return after_launch(op, qaff::launch_gemv_fused(static_cast<const uint16_t*>(gate), m, packed, scales, biases,
                                                    n, k, group_size, bits, static_cast<uint16_t*>(y), f, stream),
                        stream);
}

qaff_status qaff_gather_qmm_ex(const void* x, qaff_dtype x_dtype, int64_t x_batches, int64_t m,
                               const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                               int64_t w_batches, int64_t n, int64_t k, int32_t group_size, int32_t bits,
                               const uint32_t* lhs_indices, const uint32_t* rhs_indices, int64_t batch,
                               int32_t sorted_indices, void* y, hipStream_t stream, qaff_path path) {
    static const char* op = "qaff_gather_qmm";
    g_error.clear();
    if (x_batches < 0 || w_batches < 0 || batch < 0 || m < 0)
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: negative size", op);
    // the weight as one matrix of w_batches * n rows
    qaff_status st = check_weight(op, packed, scales, biases, w_batches * n, k, group_size, bits);
    if (st != QAFF_OK) return st;
    if (!valid_dtype(x_dtype)) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: unknown x dtype %d", op, (int)x_dtype);
    if (path != QAFF_PATH_AUTO && path != QAFF_PATH_GEMV && path != QAFF_PATH_GEMV_MFMA && path != QAFF_PATH_GEMM)
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: unknown path %d", op, (int)path);
    if (!lhs_indices && batch > x_batches)
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: no lhs indices, but %lld batches of %lld x batches", op,
                    (long long)batch, (long long)x_batches);
    if (!rhs_indices && batch > w_batches)
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: no rhs indices, but %lld batches of %lld weight batches", op,
                    (long long)batch, (long long)w_batches);
    if ((lhs_indices && !aligned(lhs_indices, 4)) || (rhs_indices && !aligned(rhs_indices, 4)))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: indices must be 4-byte aligned", op);
    if (x_batches >= 0xffffffffLL || w_batches >= 0xffffffffLL || batch >= 0xffffffffLL)
        return fail(QAFF_ERR_UNSUPPORTED, "%s: 2^32-1 or more batches", op);
    const bool mfma_ok = x_dtype == QAFF_BF16 && qaff::gemv_mfma_gather_supported(k) && aligned(scales, 4) &&
                         aligned(biases, 4);
    if (path == QAFF_PATH_GEMV_MFMA && batch > 0 && m > 0 && n > 0 && k > 0 && !mfma_ok)
        return fail(QAFF_ERR_UNSUPPORTED, "%s: the matrix-core decode kernel takes a bf16 x, k a multiple of 512 "
                    "up to 4096 and 4-byte aligned scales and biases", op);
    if (batch == 0 || m == 0 || n == 0) return QAFF_OK;
    const int64_t esize = (int64_t)esize_of(x_dtype);
    if (!y) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null y", op);
    if (!aligned(y, esize)) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: y must be aligned to its element size", op);
    if (n > 0x7fffffffLL || m > 0x7fffffffLL) return fail(QAFF_ERR_UNSUPPORTED, "%s: m or n above 2^31-1", op);
    if (k == 0) return after_launch(op, qaff::launch_fill_zero(y, batch * m * n * esize, stream), stream);
    if (x_batches > 0 && !x) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null x", op);
    if (x && !aligned(x, esize)) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: x must be aligned to its element size", op);
    const bool vec = (!x || aligned(x, 16)) && aligned(y, 16);
    if (!vec && path == QAFF_PATH_GEMV_MFMA)
        return fail(QAFF_ERR_UNSUPPORTED, "%s: the matrix-core decode kernel needs 16-byte aligned x and y", op);

    qaff::Gather g{};
    g.lhs = lhs_indices;
    g.rhs = rhs_indices;
    g.x_count = (uint32_t)x_batches;
    g.w_count = (uint32_t)w_batches;
    g.batch = (uint32_t)batch;
    g.x_stride = (uint64_t)(m * k);
    g.w_stride = (uint64_t)(n * (k / 32) * bits);
    g.sb_stride = (uint64_t)(n * (k / group_size));
    g.y_stride = (uint64_t)(m * n);
    // sorted rows, one per output batch, gathered by expert
    const bool sorted_rows = sorted_indices != 0 && m == 1 && !lhs_indices && rhs_indices && x_dtype == QAFF_BF16;
    const bool groupable = sorted_rows && mfma_ok;
    // the GEMM over each expert's rows: forced, or once experts average kGroupedGemmRows rows
    const bool gemm_ok = sorted_rows && vec && qaff::gemm_grouped_supported(k, scales, biases, g.sb_stride) &&
                         (w_batches + 1) * ((n + 255) / 256) * 3 < (1LL << 31) - 8;  // its grid fits
    if (path == QAFF_PATH_GEMM && !gemm_ok)
        return fail(QAFF_ERR_UNSUPPORTED, "%s: the grouped GEMM takes sorted rhs with one bf16 x row per batch and no "
                    "lhs, k a multiple of 1024 and 16-byte aligned scales and biases of every weight batch", op);
    if (gemm_ok && (path == QAFF_PATH_GEMM || (path == QAFF_PATH_AUTO && batch >= kGroupedGemmRows * w_batches)))
        return after_launch(op, qaff::launch_gemm_grouped(static_cast<const uint16_t*>(x), packed, scales, biases, n, k,
                                                          group_size, bits, static_cast<uint16_t*>(y), rhs_indices,
                                                          batch, w_batches, g.w_stride, g.sb_stride, stream), stream);
    bool use_mfma = false;
    if (path == QAFF_PATH_GEMV_MFMA) {
        use_mfma = true;
        g.grouped = groupable;
    } else if (path == QAFF_PATH_AUTO && mfma_ok) {
        // grouped once experts average at least one row: each expert's weights are then read once
        g.grouped = groupable && batch >= w_batches;
        use_mfma = g.grouped || m >= kGemvMfmaMinM;
    }
    hipError_t e;
    if (!vec) {
        qaff::ScalarGemv opt{};
        opt.gather = true;
        opt.g = g;
        e = qaff::launch_gemv_scalar(x, (int)x_dtype, m, packed, scales, biases, (int)QAFF_BF16, n, k, group_size, bits,
                                     y, (int)x_dtype, opt, stream);
    } else if (use_mfma)
        e = qaff::launch_gemv_mfma_gather(static_cast<const uint16_t*>(x), m, packed, scales, biases, n, k, group_size,
                                          bits, static_cast<uint16_t*>(y), g, stream);
    else
        e = qaff::launch_gemv_gather(x, x_dtype == QAFF_F32, m, packed, scales, biases, n, k, group_size, bits, y, g,
                                     stream);
    return after_launch(op, e, stream);
}

qaff_status qaff_gather_qmm(const void* x, qaff_dtype x_dtype, int64_t x_batches, int64_t m,
                            const uint32_t* packed, const uint16_t* scales, const uint16_t* biases,
                            int64_t w_batches, int64_t n, int64_t k, int32_t group_size, int32_t bits,
                            const uint32_t* lhs_indices, const uint32_t* rhs_indices, int64_t batch,
                            int32_t sorted_indices, void* y, hipStream_t stream) {
    return qaff_gather_qmm_ex(x, x_dtype, x_batches, m, packed, scales, biases, w_batches, n, k, group_size, bits,
                              lhs_indices, rhs_indices, batch, sorted_indices, y, stream, QAFF_PATH_AUTO);
}

qaff_dtype qaff_promote_dtype(qaff_dtype a, qaff_dtype b) { return a == b ? a : QAFF_F32; }

qaff_status qaff_gather_qmm_typed(const void* x, qaff_dtype x_dtype, int64_t x_batches, int64_t m,
                                  const uint32_t* packed, const void* scales, const void* biases, qaff_dtype sb_dtype,
                                  int64_t w_batches, int64_t n, int64_t k, int32_t group_size, int32_t bits,
                                  const uint32_t* lhs_indices, const uint32_t* rhs_indices, int64_t batch,
                                  int32_t sorted_indices, void* y, hipStream_t stream) {
    static const char* op = "qaff_gather_qmm_typed";
    g_error.clear();
    if (!any_dtype(x_dtype) || !any_dtype(sb_dtype))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: unknown dtype (x %d, scales %d)", op, (int)x_dtype, (int)sb_dtype);
    // bf16 scales with a float32 or bf16 x: the plain gathered product (y in x's dtype, the promoted one)
    if (sb_dtype == QAFF_BF16 && x_dtype != QAFF_F16)
        return qaff_gather_qmm(x, x_dtype, x_batches, m, packed, static_cast<const uint16_t*>(scales),
                               static_cast<const uint16_t*>(biases), w_batches, n, k, group_size, bits, lhs_indices,
                               rhs_indices, batch, sorted_indices, y, stream);
    if (x_batches < 0 || w_batches < 0 || batch < 0 || m < 0)
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: negative size", op);
    qaff_status st = check_weight(op, packed, static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(biases),
                                  w_batches * n, k, group_size, bits);
    if (st != QAFF_OK) return st;
    if (!lhs_indices && batch > x_batches)
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: no lhs indices, but %lld batches of %lld x batches", op,
                    (long long)batch, (long long)x_batches);
    if (!rhs_indices && batch > w_batches)
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: no rhs indices, but %lld batches of %lld weight batches", op,
                    (long long)batch, (long long)w_batches);
    if ((lhs_indices && !aligned(lhs_indices, 4)) || (rhs_indices && !aligned(rhs_indices, 4)))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: indices must be 4-byte aligned", op);
    if (x_batches >= 0xffffffffLL || w_batches >= 0xffffffffLL || batch >= 0xffffffffLL)
        return fail(QAFF_ERR_UNSUPPORTED, "%s: 2^32-1 or more batches", op);
    const qaff_dtype y_dtype = qaff_promote_dtype(x_dtype, sb_dtype);
    if (batch == 0 || m == 0 || n == 0) return QAFF_OK;
    if (sb_dtype == QAFF_F32 && (!aligned(scales, 4) || !aligned(biases, 4)))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: float32 scales and biases must be 4-byte aligned", op);
    if (!y) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null y", op);
    if (!aligned(y, esize_of(y_dtype))) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: y must be aligned to its element size", op);
    if (n > 0x7fffffffLL || m > 0x7fffffffLL) return fail(QAFF_ERR_UNSUPPORTED, "%s: m or n above 2^31-1", op);
    if (k == 0) return after_launch(op, qaff::launch_fill_zero(y, batch * m * n * (int64_t)esize_of(y_dtype), stream), stream);
    if (x_batches > 0 && !x) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null x", op);
    if (x && !aligned(x, esize_of(x_dtype)))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: x must be aligned to its element size", op);
    qaff::Gather g{};
    g.lhs = lhs_indices;
    g.rhs = rhs_indices;
    g.x_count = (uint32_t)x_batches;
    g.w_count = (uint32_t)w_batches;
    g.batch = (uint32_t)batch;
    g.x_stride = (uint64_t)(m * k);
    g.w_stride = (uint64_t)(n * (k / 32) * bits);
    g.sb_stride = (uint64_t)(n * (k / group_size));
    g.y_stride = (uint64_t)(m * n);
    const bool vec = (!x || aligned(x, 16)) && aligned(y, 16);
    // float16 x, scales and biases: the matrix-core kernels of qaff_gather_qmm in float16, under
    // its rules (the grouped GEMM once experts average kGroupedGemmRows rows, the grouped decode
    // kernel once they average one, the batched one from kGemvMfmaMinM rows)
    if (x_dtype == QAFF_F16 && sb_dtype == QAFF_F16 && vec) {
        const uint16_t* s16 = static_cast<const uint16_t*>(scales);
        const uint16_t* b16 = static_cast<const uint16_t*>(biases);
        const bool sorted_rows = sorted_indices != 0 && m == 1 && !lhs_indices && rhs_indices;
        if (sorted_rows && batch >= kGroupedGemmRows * w_batches && qaff::gemm_grouped_supported(k, s16, b16, g.sb_stride) &&
            (w_batches + 1) * ((n + 255) / 256) * 3 < (1LL << 31) - 8)
            return after_launch(op, qaff::launch_gemm_grouped_f16(static_cast<const uint16_t*>(x), packed, s16, b16, n, k,
                                                                  group_size, bits, static_cast<uint16_t*>(y),
                                                                  rhs_indices, batch, w_batches, g.w_stride,
                                                                  g.sb_stride, stream), stream);
        if (qaff::gemv_mfma_gather_supported(k) && aligned(scales, 4) && aligned(biases, 4)) {
            g.grouped = sorted_rows && batch >= w_batches;
            if (g.grouped || m >= kGemvMfmaMinM)
                return after_launch(op, qaff::launch_gemv_mfma_gather_f16(static_cast<const uint16_t*>(x), m, packed, s16,
                                                                          b16, n, k, group_size, bits,
                                                                          static_cast<uint16_t*>(y), g, stream), stream);
        }
    }
    // sorted rows, one per output batch, gathered by expert: the grouped walk once experts average
    // 16 rows or more (each expert's weights are then read once; measured with float16 operands on
    // 128 experts of [768, 2048]: 4 rows per expert 279 against 204 us batched, 32 rows 1385
    // against 1506 us, 128 rows 5229 against 5957 us)
    g.grouped = sorted_indices != 0 && m == 1 && !lhs_indices && rhs_indices && batch >= 16 * w_batches;
    if (!vec) {  // the typed GEMV reads x in 16-byte loads
        g.grouped = 0;
        qaff::ScalarGemv opt{};
        opt.gather = true;
        opt.g = g;
        return after_launch(op, qaff::launch_gemv_scalar(x, (int)x_dtype, m, packed, scales, biases, (int)sb_dtype, n, k,
                                                         group_size, bits, y, (int)y_dtype, opt, stream), stream);
    }
    return after_launch(op, qaff::launch_gemv_typed(x, (int)x_dtype, m, packed, scales, biases, (int)sb_dtype, n, k,
                                                    group_size, bits, y, (int)y_dtype, stream, &g), stream);
}

qaff_status qaff_dequantize_typed(const uint32_t* packed, const void* scales, const void* biases, qaff_dtype sb_dtype,
                                  int64_t rows, int64_t cols, int32_t group_size, int32_t bits, void* out,
                                  qaff_dtype out_dtype, hipStream_t stream) {
    static const char* op = "qaff_dequantize_typed";
    g_error.clear();
    if (!any_dtype(sb_dtype) || !any_dtype(out_dtype))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: unknown dtype (%d, %d)", op, (int)sb_dtype, (int)out_dtype);
    if (sb_dtype == QAFF_BF16 && out_dtype != QAFF_F16)
        return qaff_dequantize(packed, static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(biases), rows,
                               cols, group_size, bits, out, out_dtype, stream);
    // the weight checks, with the scales' own alignment
    qaff_status st = check_weight(op, packed, static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(biases),
                                  rows, cols, group_size, bits);
    if (st != QAFF_OK) return st;
    if (rows == 0 || cols == 0) return QAFF_OK;
    if (sb_dtype == QAFF_F32 && (!aligned(scales, 4) || !aligned(biases, 4)))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: float32 scales and biases must be 4-byte aligned", op);
    if (!out) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null output", op);
    if (!aligned(out, esize_of(out_dtype)))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: output must be aligned to its element size", op);
    return after_launch(op, qaff::launch_dequant_typed(packed, scales, biases, (int)sb_dtype, rows, cols, group_size,
                                                       bits, out, (int)out_dtype, stream), stream);
}

qaff_status qaff_qmm_typed(const void* x, qaff_dtype x_dtype, int64_t m, const uint32_t* packed, const void* scales,
                           const void* biases, qaff_dtype sb_dtype, int64_t n, int64_t k, int32_t group_size,
                           int32_t bits, void* y, hipStream_t stream) {
    static const char* op = "qaff_qmm_typed";
    g_error.clear();
    if (!any_dtype(x_dtype) || !any_dtype(sb_dtype))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: unknown dtype (%d, %d)", op, (int)x_dtype, (int)sb_dtype);
    if (sb_dtype == QAFF_BF16 && x_dtype != QAFF_F16)
        return qaff_qmm_ex(x, x_dtype, m, packed, static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(biases),
                           n, k, group_size, bits, y, stream, QAFF_PATH_AUTO);
    qaff_status st = check_weight(op, packed, static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(biases),
                                  n, k, group_size, bits);
    if (st != QAFF_OK) return st;
    if (m < 0) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: negative m", op);
    if (m == 0 || n == 0) return QAFF_OK;
    if (sb_dtype == QAFF_F32 && k > 0 && (!aligned(scales, 4) || !aligned(biases, 4)))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: float32 scales and biases must be 4-byte aligned", op);
    const qaff_dtype yt = qaff_promote_dtype(x_dtype, sb_dtype);
    if (!y) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null y", op);
    if (!aligned(y, esize_of(yt))) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: y must be aligned to its element size", op);
    if (k == 0) return after_launch(op, qaff::launch_fill_zero(y, m * n * (int64_t)esize_of(yt), stream), stream);
    if (!x) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null x", op);
    if (!aligned(x, esize_of(x_dtype)))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: x must be aligned to its element size", op);
    if (n > 0x7fffffffLL || m > 0x7fffffffLL) return fail(QAFF_ERR_UNSUPPORTED, "%s: m or n above 2^31-1", op);
    if (!aligned(x, 16) || !aligned(y, 16))
        return after_launch(op, qaff::launch_gemv_scalar(x, (int)x_dtype, m, packed, scales, biases, (int)sb_dtype, n, k,
                                                         group_size, bits, y, (int)yt, qaff::ScalarGemv{}, stream),
                            stream);
    if (x_dtype == QAFF_F16 && sb_dtype == QAFF_F16) {
        // qaff_qmm's kernels in float16, under its rules: the GEMM past kGemvMaxM rows, the
        // matrix-core decode kernel from gemv_mfma_min_m(k) rows where it applies, else the GEMV
        const uint16_t* x16 = static_cast<const uint16_t*>(x);
        const uint16_t* s16 = static_cast<const uint16_t*>(scales);
        const uint16_t* b16 = static_cast<const uint16_t*>(biases);
        uint16_t* y16 = static_cast<uint16_t*>(y);
        hipError_t e;
        if (m > kGemvMaxM && decode_slices(m, n, k) && aligned(scales, 4) && aligned(biases, 4))
            e = launch_decode_slices<true>(x16, m, packed, s16, b16, n, k, group_size, bits, y16, stream);
        else if (m > kGemvMaxM)
            e = qaff::launch_gemm_f16(x16, m, packed, s16, b16, n, k, group_size, bits, y16, stream);
        else if (m >= gemv_mfma_min_m(k) && qaff::gemv_mfma_supported(m, k) && aligned(scales, 4) && aligned(biases, 4))
            e = qaff::launch_gemv_mfma_f16(x16, m, packed, s16, b16, n, k, group_size, bits, y16, stream);
        else
            e = qaff::launch_gemv_f16(x16, m, packed, s16, b16, n, k, group_size, bits, y16, stream);
        return after_launch(op, e, stream);
    }
    return after_launch(op, qaff::launch_gemv_typed(x, (int)x_dtype, m, packed, scales, biases, (int)sb_dtype, n, k,
                                                    group_size, bits, y, (int)yt, stream), stream);
}

size_t qaff_qmm_nt_workspace_size(int64_t m, int64_t k, int64_t n, int32_t bits) {
    if (m <= 0 || k <= 0 || n <= 0) return 0;
    return qaff::qmm_nt_workspace_bytes(m, k, n, bits);
}

namespace {

// qaff_qmm_nt (bf16 scales, typed = false) and qaff_qmm_nt_typed with the workspace given (ws) or,
// for qaff_qmm_nt_static (ws null), the library's static scratch array of the current device.
qaff_status qmm_nt_impl(const char* op, const void* x, qaff_dtype x_dtype, int64_t m, const uint32_t* packed,
                        const void* scales, const void* biases, qaff_dtype sb_dtype, bool typed, int64_t k,
                        int64_t n, int32_t group_size, int32_t bits, void* workspace, size_t workspace_bytes,
                        bool use_static, void* y, hipStream_t stream) {
    g_error.clear();
    if (typed ? !any_dtype(x_dtype) || !any_dtype(sb_dtype) : !valid_dtype(x_dtype))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: unknown dtype (x %d, scales %d)", op, (int)x_dtype, (int)sb_dtype);
    // the weight is [k, n]: k rows of n codes
    qaff_status st = check_weight(op, packed, static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(biases),
                                  k, n, group_size, bits);
    if (st != QAFF_OK) return st;
    if (m < 0) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: negative m", op);
    if (m == 0 || n == 0) return QAFF_OK;
    if (sb_dtype == QAFF_F32 && k > 0 && (!aligned(scales, 4) || !aligned(biases, 4)))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: float32 scales and biases must be 4-byte aligned", op);
    // the kernels load x and store y one element at a time: element alignment is enough
    const qaff_dtype y_dtype = qaff_promote_dtype(x_dtype, sb_dtype);
    const int64_t ysize = (int64_t)esize_of(y_dtype);
    if (!y) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null y", op);
    if (!aligned(y, ysize)) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: y must be aligned to its element size", op);
    if (k == 0) return after_launch(op, qaff::launch_fill_zero(y, m * n * ysize, stream), stream);
    if (!x) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null x", op);
    if (!aligned(x, esize_of(x_dtype)))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: x must be aligned to its element size", op);
    if (m * n >= (1LL << 31) || k > 0x7fffffffLL || n > 0x7fffffffLL)
        return fail(QAFF_ERR_UNSUPPORTED, "%s: %lld x %lld outputs or k = %lld is too large", op, (long long)m,
                    (long long)n, (long long)k);
    int64_t kchunk, chunks;
    qaff::qmm_nt_plan(k, n, bits, &kchunk, &chunks);
    if (chunks > 65535) return fail(QAFF_ERR_UNSUPPORTED, "%s: k = %lld is too large", op, (long long)k);
    const size_t need = qaff::qmm_nt_workspace_bytes(m, k, n, bits);
    if (use_static) {
        if (need > qaff::kQmmNtStaticScratchBytes)
            return fail(QAFF_ERR_UNSUPPORTED, "%s: these sizes need %zu bytes of partial sums, more than the static "
                        "scratch of %zu bytes (qaff_qmm_nt_static_max_bytes); use qaff_qmm_nt with a workspace",
                        op, need, qaff::kQmmNtStaticScratchBytes);
        const hipError_t e = qaff::qmm_nt_static_scratch(&workspace);
        if (e != hipSuccess) return fail(QAFF_ERR_DEVICE, "%s: static scratch: %s", op, hipGetErrorString(e));
    } else {
        if (!workspace || workspace_bytes < need)
            return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: the workspace needs %zu bytes (qaff_qmm_nt_workspace_size), got %zu",
                        op, need, workspace ? workspace_bytes : (size_t)0);
        if (!aligned(workspace, 16)) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: workspace must be 16-byte aligned", op);
    }
    return after_launch(op, qaff::launch_qmm_nt(x, (int)x_dtype, m, packed, scales, biases, (int)sb_dtype, k, n,
                                                group_size, bits, workspace, y, (int)y_dtype, stream), stream);
}

}  // namespace

qaff_status qaff_qmm_nt(const void* x, qaff_dtype x_dtype, int64_t m, const uint32_t* packed, const uint16_t* scales,
                        const uint16_t* biases, int64_t k, int64_t n, int32_t group_size, int32_t bits,
                        void* workspace, size_t workspace_bytes, void* y, hipStream_t stream) {
    return qmm_nt_impl("qaff_qmm_nt", x, x_dtype, m, packed, scales, biases, QAFF_BF16, false, k, n, group_size, bits,
                       workspace, workspace_bytes, false, y, stream);
}

qaff_status qaff_qmm_nt_typed(const void* x, qaff_dtype x_dtype, int64_t m, const uint32_t* packed, const void* scales,
                              const void* biases, qaff_dtype sb_dtype, int64_t k, int64_t n, int32_t group_size,
                              int32_t bits, void* workspace, size_t workspace_bytes, void* y, hipStream_t stream) {
    return qmm_nt_impl("qaff_qmm_nt_typed", x, x_dtype, m, packed, scales, biases, sb_dtype, true, k, n, group_size,
                       bits, workspace, workspace_bytes, false, y, stream);
}

qaff_status qaff_qmm_nt_static(const void* x, qaff_dtype x_dtype, int64_t m, const uint32_t* packed,
                               const uint16_t* scales, const uint16_t* biases, int64_t k, int64_t n,
                               int32_t group_size, int32_t bits, void* y, hipStream_t stream) {
    return qmm_nt_impl("qaff_qmm_nt_static", x, x_dtype, m, packed, scales, biases, QAFF_BF16, false, k, n, group_size,
                       bits, nullptr, 0, true, y, stream);
}

size_t qaff_qmm_nt_static_max_bytes(void) { return qaff::kQmmNtStaticScratchBytes; }

namespace {

qaff_status quantize_impl(const char* op, const void* w, qaff_dtype w_dtype, int64_t rows, int64_t cols,
                          int32_t group_size, int32_t bits, uint32_t* packed, void* scales, void* biases,
                          qaff_dtype sb_dtype, hipStream_t stream) {
    g_error.clear();
    if (!any_dtype(w_dtype) || !any_dtype(sb_dtype))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: unknown dtype (w %d, scales %d)", op, (int)w_dtype, (int)sb_dtype);
    // the outputs are checked as a weight would be, with the scales' own alignment
    qaff_status st = check_weight(op, packed, static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(biases),
                                  rows, cols, group_size, bits);
    if (st != QAFF_OK) return st;
    if (rows == 0 || cols == 0) return QAFF_OK;
    if (sb_dtype == QAFF_F32 && (!aligned(scales, 4) || !aligned(biases, 4)))
        return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: float32 scales and biases must be 4-byte aligned", op);
    if (!w) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: null w", op);
    if (!aligned(w, esize_of(w_dtype))) return fail(QAFF_ERR_INVALID_ARGUMENT, "%s: w must be aligned to its element size", op);
    if (rows * (cols / 32) >= (1LL << 37))
        return fail(QAFF_ERR_UNSUPPORTED, "%s: %lld x %lld is too large", op, (long long)rows, (long long)cols);
    return after_launch(op, qaff::launch_quantize(w, (int)w_dtype, rows, cols, group_size, bits, packed, scales, biases,
                                                  (int)sb_dtype, stream), stream);
}

}  // namespace

qaff_status qaff_quantize(const void* w, qaff_dtype w_dtype, int64_t rows, int64_t cols, int32_t group_size,
                          int32_t bits, uint32_t* packed, uint16_t* scales, uint16_t* biases, hipStream_t stream) {
    return quantize_impl("qaff_quantize", w, w_dtype, rows, cols, group_size, bits, packed, scales, biases, QAFF_BF16,
                         stream);
}

qaff_status qaff_quantize_typed(const void* w, qaff_dtype w_dtype, int64_t rows, int64_t cols, int32_t group_size,
                                int32_t bits, uint32_t* packed, void* scales, void* biases, qaff_dtype sb_dtype,
                                hipStream_t stream) {
    return quantize_impl("qaff_quantize_typed", w, w_dtype, rows, cols, group_size, bits, packed, scales, biases,
                         sb_dtype, stream);
}

qaff_status qaff_qmm(const void* x, qaff_dtype x_dtype, int64_t m, const uint32_t* packed,
                     const uint16_t* scales, const uint16_t* biases, int64_t n, int64_t k,
                     int32_t group_size, int32_t bits, void* y, hipStream_t stream) {
    return qaff_qmm_ex(x, x_dtype, m, packed, scales, biases, n, k, group_size, bits, y, stream,
                       QAFF_PATH_AUTO);
}

const char* qaff_last_error(void) { return g_error.c_str(); }

const char* qaff_status_string(qaff_status status) {
    switch (status) {
        case QAFF_OK: return "QAFF_OK";
        case QAFF_ERR_INVALID_ARGUMENT: return "QAFF_ERR_INVALID_ARGUMENT";
        case QAFF_ERR_UNSUPPORTED: return "QAFF_ERR_UNSUPPORTED";
        case QAFF_ERR_DEVICE: return "QAFF_ERR_DEVICE";
        default: return "QAFF_ERR_UNKNOWN";
    }
}

int qaff_abi_version(void) { return QAFF_ABI_VERSION; }

int qaff_gemv_max_m(void) { return kGemvMaxM; }

int qaff_gemv_mfma_min_m(void) { return kGemvMfmaMinM; }

}  // extern "C"
