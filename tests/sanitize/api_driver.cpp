// Drives the C ABI's host code (quantized_matmul_mlx_amd/csrc/api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer without a GPU: the launchers of launch.h and the few HIP runtime calls
// that api.cpp makes are replaced by stubs that record what would have been launched. Every entry
// point is called with arguments that validation must refuse (nothing may be launched) and with
// arguments it must accept (the expected launcher must be reached). Exit status 0 when every check
// holds. Test infrastructure.
#include "qaff.h"
#include "launch.h"

#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

static std::vector<std::string> g_calls;
static int failures = 0;
#define CHECK(c)                                                             \
    do {                                                                     \
        if (!(c)) {                                                          \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

static hipError_t rec(const char* name) {
    g_calls.push_back(name);
    return hipSuccess;
}

// ---- stubs for the device side ----
extern "C" {
hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) { *v = 256; return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stub error"; }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) { return rec("memcpy"); }
}

namespace qaff {
hipError_t launch_dequant(const uint32_t*, const uint16_t*, const uint16_t*, const uint32_t* idx, int64_t, int64_t,
                          int64_t, int, int, void*, bool, hipStream_t) { return rec(idx ? "dequant_rows" : "dequant"); }
hipError_t launch_gemv(const void*, bool, int64_t, const uint32_t*, const uint16_t*, const uint16_t*, int64_t, int64_t,
                       int, int, void*, hipStream_t) { return rec("gemv"); }
hipError_t launch_gemv_fused(const uint16_t*, int64_t, const uint32_t*, const uint16_t*, const uint16_t*, int64_t,
                             int64_t, int, int, uint16_t*, const GemvFused&, hipStream_t) { return rec("gemv_fused"); }
hipError_t launch_gemv_f16(const uint16_t*, int64_t, const uint32_t*, const uint16_t*, const uint16_t*, int64_t,
                           int64_t, int, int, uint16_t*, hipStream_t) { return rec("gemv_f16"); }
hipError_t launch_gemv_gather(const void*, bool, int64_t, const uint32_t*, const uint16_t*, const uint16_t*, int64_t,
                              int64_t, int, int, void*, const Gather&, hipStream_t) { return rec("gemv_gather"); }
bool gemv_mfma_supported(int64_t m, int64_t k) { return m >= 1 && m <= 16 && k % 512 == 0 && k > 0 && k <= 32768; }
bool gemv_mfma_gather_supported(int64_t k) { return k % 512 == 0 && k > 0 && k <= 4096; }
hipError_t launch_gemv_mfma(const uint16_t*, int64_t, const uint32_t*, const uint16_t*, const uint16_t*, int64_t,
                            int64_t, int, int, uint16_t*, hipStream_t) { return rec("gemv_mfma"); }
hipError_t launch_gemv_mfma_f16(const uint16_t*, int64_t, const uint32_t*, const uint16_t*, const uint16_t*, int64_t,
                                int64_t, int, int, uint16_t*, hipStream_t) { return rec("gemv_mfma_f16"); }
hipError_t launch_gemv_mfma_gather_f16(const uint16_t*, int64_t, const uint32_t*, const uint16_t*, const uint16_t*,
                                       int64_t, int64_t, int, int, uint16_t*, const Gather& g, hipStream_t) {
    return rec(g.grouped ? "gemv_mfma_gather_f16_grouped" : "gemv_mfma_gather_f16");
}
hipError_t launch_gemm_f16(const uint16_t*, int64_t, const uint32_t*, const uint16_t*, const uint16_t*, int64_t, int64_t,
                           int, int, uint16_t*, hipStream_t) { return rec("gemm_f16"); }
hipError_t launch_gemm_grouped_f16(const uint16_t*, const uint32_t*, const uint16_t*, const uint16_t*, int64_t, int64_t,
                                   int, int, uint16_t*, const uint32_t*, int64_t, int64_t, uint64_t, uint64_t,
                                   hipStream_t) { return rec("gemm_grouped_f16"); }
hipError_t launch_gemv_mfma_gather(const uint16_t*, int64_t, const uint32_t*, const uint16_t*, const uint16_t*, int64_t,
                                   int64_t, int, int, uint16_t*, const Gather& g, hipStream_t) {
    return rec(g.grouped ? "gemv_mfma_gather_grouped" : "gemv_mfma_gather");
}
hipError_t launch_gemm(const uint16_t*, int64_t, const uint32_t*, const uint16_t*, const uint16_t*, int64_t, int64_t,
                       int, int, uint16_t*, hipStream_t, void* ws, size_t) { return rec(ws ? "gemm_split" : "gemm"); }
bool gemm_grouped_supported(int64_t k, const uint16_t*, const uint16_t*, uint64_t) { return k % 1024 == 0; }
hipError_t launch_gemm_grouped(const uint16_t*, const uint32_t*, const uint16_t*, const uint16_t*, int64_t, int64_t,
                               int, int, uint16_t*, const uint32_t*, int64_t, int64_t, uint64_t, uint64_t,
                               hipStream_t) { return rec("gemm_grouped"); }
size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    return (m <= 256 && k % 1024 == 0) ? (size_t)(m * n * 4 * 2) : 0;
}
hipError_t launch_quantize(const void*, int, int64_t, int64_t, int, int, uint32_t*, void*, void*, int,
                           hipStream_t) { return rec("quantize"); }
void qmm_nt_plan(int64_t k, int64_t, int, int64_t* kchunk, int64_t* chunks) { *kchunk = 128; *chunks = (k + 127) / 128; }
size_t qmm_nt_workspace_bytes(int64_t m, int64_t k, int64_t n, int) {
    return (size_t)(((k + 127) / 128) * (m < 2 ? m : 2) * n) * 4;
}
hipError_t launch_qmm_nt(const void*, int, int64_t, const uint32_t*, const void*, const void*, int, int64_t,
                         int64_t, int, int, void* ws, void*, int, hipStream_t) { return rec(ws ? "qmm_nt" : "qmm_nt_null_ws"); }
static uint8_t fake_scratch[64];
hipError_t qmm_nt_static_scratch(void** ptr) { *ptr = fake_scratch; return rec("static_scratch"); }
hipError_t launch_dequant_typed(const uint32_t*, const void*, const void*, int, int64_t, int64_t, int, int, void*, int,
                                hipStream_t, const uint32_t*, int64_t) { return rec("dequant_typed"); }
hipError_t launch_gemv_typed(const void*, int, int64_t, const uint32_t*, const void*, const void*, int, int64_t,
                             int64_t, int, int, void*, int, hipStream_t, const Gather*) { return rec("gemv_typed"); }
hipError_t launch_fill_zero(void*, int64_t, hipStream_t) { return rec("fill_zero"); }
hipError_t launch_gemv_scalar(const void*, int, int64_t, const uint32_t*, const void*, const void*, int, int64_t,
                              int64_t, int, int, void*, int, const ScalarGemv&, hipStream_t) { return rec("gemv_scalar"); }
}  // namespace qaff

// fake device addresses: never dereferenced
static void* const A16 = reinterpret_cast<void*>(0x10000);
static void* const A2 = reinterpret_cast<void*>(0x10002);
static void* const A1 = reinterpret_cast<void*>(0x10001);
static const uint32_t* const P16 = reinterpret_cast<const uint32_t*>(0x20000);
static const uint16_t* const S16 = reinterpret_cast<const uint16_t*>(0x30000);
static const uint16_t* const B16 = reinterpret_cast<const uint16_t*>(0x40000);
static const uint16_t* const B2 = reinterpret_cast<const uint16_t*>(0x40002);  // 2-byte aligned biases
static const uint32_t* const I16 = reinterpret_cast<const uint32_t*>(0x50000);

// Runs a call and checks its status and what it launched ("" = nothing).
template <typename F>
static void expect(int line, qaff_status want, const char* launched, F&& call) {
    g_calls.clear();
    const qaff_status got = call();
    const std::string last = g_calls.empty() ? "" : g_calls.back();
    if (got != want || last != launched) {
        std::fprintf(stderr, "line %d: status %d (want %d), launched '%s' (want '%s'), error '%s'\n", line, (int)got,
                     (int)want, last.c_str(), launched, qaff_last_error());
        ++failures;
    }
    if (got != QAFF_OK) CHECK(std::strlen(qaff_last_error()) > 0);
}
#define EXPECT(want, launched, expr) expect(__LINE__, want, launched, [&] { return (expr); })

int main() {
    const qaff_status OK = QAFF_OK, INV = QAFF_ERR_INVALID_ARGUMENT, UNS = QAFF_ERR_UNSUPPORTED;
    // dequantize / dequant_rows
    EXPECT(OK, "dequant", qaff_dequantize(P16, S16, B16, 4, 64, 32, 4, A16, QAFF_F32, nullptr));
    EXPECT(UNS, "", qaff_dequantize(P16, S16, B16, 4, 64, 32, 7, A16, QAFF_F32, nullptr));
    EXPECT(INV, "", qaff_dequantize(P16, S16, B16, 4, 64, 48, 4, A16, QAFF_F32, nullptr));
    EXPECT(INV, "", qaff_dequantize(P16, S16, B16, 4, 96, 64, 4, A16, QAFF_F32, nullptr));
    EXPECT(INV, "", qaff_dequantize(P16, S16, B16, -1, 64, 32, 4, A16, QAFF_F32, nullptr));
    EXPECT(INV, "", qaff_dequantize(nullptr, S16, B16, 4, 64, 32, 4, A16, QAFF_F32, nullptr));
    EXPECT(INV, "", qaff_dequantize(P16, S16, B16, 4, 64, 32, 4, A16, (qaff_dtype)9, nullptr));
    EXPECT(OK, "", qaff_dequantize(P16, S16, B16, 0, 64, 32, 4, A16, QAFF_BF16, nullptr));
    EXPECT(OK, "dequant_rows", qaff_dequant_rows(P16, S16, B16, 10, 64, 32, 4, I16, 5, A16, QAFF_BF16, nullptr));
    EXPECT(INV, "", qaff_dequant_rows(P16, S16, B16, 10, 64, 32, 4, nullptr, 5, A16, QAFF_BF16, nullptr));
    EXPECT(INV, "", qaff_dequant_rows(P16, S16, B16, 10, 64, 32, 4, I16, -2, A16, QAFF_BF16, nullptr));
    // qmm: dispatch by m and dtype, forced paths, k = 0
    EXPECT(OK, "gemv", qaff_qmm(A16, QAFF_BF16, 1, P16, S16, B16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemv_mfma", qaff_qmm(A16, QAFF_BF16, 4, P16, S16, B16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemv_mfma", qaff_qmm(A16, QAFF_BF16, 2, P16, S16, B16, 64, 4096 + 512 * 2, 64, 4, A16, nullptr));
    EXPECT(OK, "gemv", qaff_qmm(A16, QAFF_BF16, 1, P16, S16, B16, 64, 4096 + 512 * 2, 64, 4, A16, nullptr));
    EXPECT(OK, "gemv", qaff_qmm(A16, QAFF_BF16, 4, P16, S16, B16, 64, 32768 + 1024, 64, 4, A16, nullptr));
    // 17 to 128 rows without a K split: 16-row slices (the last slice's rows decide the last launch)
    EXPECT(OK, "gemv", qaff_qmm(A16, QAFF_BF16, 17, P16, S16, B16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemv_mfma", qaff_qmm(A16, QAFF_BF16, 48, P16, S16, B16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemv_mfma", qaff_qmm(A16, QAFF_BF16, 64, P16, S16, B16, 8192, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemm", qaff_qmm(A16, QAFF_BF16, 64, P16, S16, B16, 8256, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemv", qaff_qmm(A16, QAFF_BF16, 65, P16, S16, B16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemv_mfma", qaff_qmm(A16, QAFF_BF16, 96, P16, S16, B16, 8192, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemm", qaff_qmm(A16, QAFF_BF16, 97, P16, S16, B16, 8192, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemv_mfma", qaff_qmm(A16, QAFF_BF16, 128, P16, S16, B16, 4096, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemm", qaff_qmm(A16, QAFF_BF16, 129, P16, S16, B16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemm", qaff_qmm(A16, QAFF_BF16, 17, P16, S16, B16, 64, 4096 + 64, 64, 4, A16, nullptr));  // K % 512
    EXPECT(OK, "gemm", qaff_qmm_ex(A16, QAFF_BF16, 17, P16, S16, B16, 64, 4096, 64, 4, A16, nullptr, QAFF_PATH_GEMM));
    EXPECT(OK, "gemv", qaff_qmm(A16, QAFF_F32, 300, P16, S16, B16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(UNS, "", qaff_qmm_ex(A16, QAFF_F32, 300, P16, S16, B16, 64, 4096, 64, 4, A16, nullptr, QAFF_PATH_GEMM));
    EXPECT(INV, "", qaff_qmm_ex(A16, QAFF_BF16, 3, P16, S16, B16, 64, 4096, 64, 4, A16, nullptr, (qaff_path)7));
    EXPECT(OK, "fill_zero", qaff_qmm(A16, QAFF_BF16, 3, P16, S16, B16, 64, 0, 64, 4, A16, nullptr));
    EXPECT(OK, "", qaff_qmm(A16, QAFF_BF16, 0, P16, S16, B16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(INV, "", qaff_qmm(A16, QAFF_BF16, -1, P16, S16, B16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(INV, "", qaff_qmm(nullptr, QAFF_BF16, 2, P16, S16, B16, 64, 4096, 64, 4, A16, nullptr));
    // operands that are not 16-byte aligned: the element-by-element kernel, or UNSUPPORTED when forced
    EXPECT(OK, "gemv_scalar", qaff_qmm(A2, QAFF_BF16, 4, P16, S16, B16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemv_scalar", qaff_qmm(A16, QAFF_BF16, 300, P16, S16, B16, 64, 4096, 64, 4, A2, nullptr));
    EXPECT(UNS, "", qaff_qmm_ex(A2, QAFF_BF16, 300, P16, S16, B16, 64, 4096, 64, 4, A16, nullptr, QAFF_PATH_GEMM));
    EXPECT(INV, "", qaff_qmm(A1, QAFF_BF16, 4, P16, S16, B16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "dequant_typed", qaff_dequantize(P16, S16, B16, 4, 64, 32, 4, A2, QAFF_BF16, nullptr));
    EXPECT(OK, "dequant_typed", qaff_dequant_rows(P16, S16, B16, 10, 64, 32, 4, I16, 5, A2, QAFF_BF16, nullptr));
    EXPECT(INV, "", qaff_dequantize(P16, S16, B16, 4, 64, 32, 4, A2, QAFF_F32, nullptr));
    EXPECT(OK, "gemv_scalar", qaff_gemv_gate_up(A2, 1, P16, S16, B16, P16, S16, B16, 64, 4096, 64, 4, A16, A16, nullptr));
    EXPECT(OK, "gemv_scalar", qaff_gemv_silu_gate(A16, A16, 1, P16, S16, B16, 64, 4096, 64, 4, A2, A2, nullptr));
    EXPECT(OK, "gemv_scalar", qaff_gather_qmm(A2, QAFF_BF16, 2, 1, P16, S16, B16, 4, 64, 4096, 64, 4, I16, I16, 3, 0,
                                              A16, nullptr));
    EXPECT(OK, "gemv_scalar", qaff_qmm_typed(A2, QAFF_F16, 1, P16, S16, B16, QAFF_F16, 64, 4096, 64, 4, A16, nullptr));
    // float16 x, scales and biases: qaff_qmm's kernels in float16
    EXPECT(OK, "gemv_f16", qaff_qmm_typed(A16, QAFF_F16, 2, P16, S16, B16, QAFF_F16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemv_mfma_f16", qaff_qmm_typed(A16, QAFF_F16, 3, P16, S16, B16, QAFF_F16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemv_mfma_f16", qaff_qmm_typed(A16, QAFF_F16, 2, P16, S16, B16, QAFF_F16, 64, 5120, 64, 4, A16, nullptr));
    EXPECT(OK, "gemv_f16", qaff_qmm_typed(A16, QAFF_F16, 3, P16, S16, B2, QAFF_F16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemv_f16", qaff_qmm_typed(A16, QAFF_F16, 17, P16, S16, B16, QAFF_F16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemm_f16", qaff_qmm_typed(A16, QAFF_F16, 129, P16, S16, B16, QAFF_F16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemv_typed", qaff_qmm_typed(A16, QAFF_F16, 17, P16, S16, B16, QAFF_F32, 64, 4096, 64, 4, A16, nullptr));
    // ... and qaff_gather_qmm's: grouped GEMM, grouped and batched decode kernels, else the typed GEMV
    EXPECT(OK, "gemm_grouped_f16", qaff_gather_qmm_typed(A16, QAFF_F16, 256, 1, P16, S16, B16, QAFF_F16, 4, 64, 4096, 64,
                                                         4, nullptr, I16, 256, 1, A16, nullptr));
    EXPECT(OK, "gemv_mfma_gather_f16_grouped", qaff_gather_qmm_typed(A16, QAFF_F16, 8, 1, P16, S16, B16, QAFF_F16, 4, 64,
                                                                     4096, 64, 4, nullptr, I16, 8, 1, A16, nullptr));
    EXPECT(OK, "gemv_mfma_gather_f16", qaff_gather_qmm_typed(A16, QAFF_F16, 2, 3, P16, S16, B16, QAFF_F16, 4, 64, 4096,
                                                             64, 4, I16, I16, 3, 0, A16, nullptr));
    EXPECT(OK, "gemv_typed", qaff_gather_qmm_typed(A16, QAFF_F16, 2, 1, P16, S16, B16, QAFF_F16, 4, 64, 4096, 64, 4,
                                                   I16, I16, 3, 0, A16, nullptr));
    EXPECT(OK, "qmm_nt", qaff_qmm_nt(A2, QAFF_BF16, 2, P16, S16, B16, 4096, 4096, 64, 4, A16, 1 << 20, A2, nullptr));
    // qmm with a workspace: the split GEMM where the size calls for one, a short workspace refused
    const size_t need = qaff_qmm_workspace_size(128, 64, 4096, 64, 4);
    CHECK(need > 0);
    EXPECT(OK, "gemm_split", qaff_qmm_ws(A16, QAFF_BF16, 128, P16, S16, B16, 64, 4096, 64, 4, A16, need, A16, nullptr));
    EXPECT(INV, "", qaff_qmm_ws(A16, QAFF_BF16, 128, P16, S16, B16, 64, 4096, 64, 4, A16, need - 1, A16, nullptr));
    EXPECT(INV, "", qaff_qmm_ws(A16, QAFF_BF16, 128, P16, S16, B16, 64, 4096, 64, 4, nullptr, need, A16, nullptr));
    // fused decode products
    EXPECT(OK, "gemv_fused", qaff_gemv_gate_up(A16, 2, P16, S16, B16, P16, S16, B16, 64, 4096, 64, 4, A16, A16, nullptr));
    EXPECT(UNS, "", qaff_gemv_gate_up(A16, 17, P16, S16, B16, P16, S16, B16, 64, 4096, 64, 4, A16, A16, nullptr));
    EXPECT(OK, "gemv_fused", qaff_gemv_silu_gate(A16, A16, 1, P16, S16, B16, 64, 4096, 64, 4, A16, A16, nullptr));
    EXPECT(OK, "memcpy", qaff_gemv_silu_gate(A16, A16, 1, P16, S16, B16, 64, 0, 64, 4, A16, A16, nullptr));
    EXPECT(OK, "gemv_fused", qaff_gemv_silu_gate(A16, A16, 1, P16, S16, B16, 64, 4096, 64, 4, A2, A16, nullptr));
    EXPECT(INV, "", qaff_gemv_silu_gate(A16, A16, 1, P16, S16, B16, 64, 4096, 64, 4, A1, A16, nullptr));
    // gathered products
    EXPECT(OK, "gemv_gather", qaff_gather_qmm(A16, QAFF_BF16, 2, 1, P16, S16, B16, 4, 64, 4096, 64, 4, I16, I16, 3, 0,
                                              A16, nullptr));
    EXPECT(OK, "gemv_mfma_gather_grouped", qaff_gather_qmm(A16, QAFF_BF16, 8, 1, P16, S16, B16, 4, 64, 4096, 64, 4,
                                                           nullptr, I16, 8, 1, A16, nullptr));
    EXPECT(INV, "", qaff_gather_qmm(A16, QAFF_BF16, 2, 1, P16, S16, B16, 4, 64, 4096, 64, 4, nullptr, I16, 3, 0, A16,
                                    nullptr));
    // sorted rows averaging 32 or more per expert: the grouped GEMM (forced or automatic)
    EXPECT(OK, "gemm_grouped", qaff_gather_qmm(A16, QAFF_BF16, 512, 1, P16, S16, B16, 16, 64, 4096, 64, 4, nullptr, I16,
                                               512, 1, A16, nullptr));
    EXPECT(OK, "gemv_mfma_gather_grouped", qaff_gather_qmm(A16, QAFF_BF16, 500, 1, P16, S16, B16, 16, 64, 4096, 64, 4,
                                                           nullptr, I16, 500, 1, A16, nullptr));
    EXPECT(OK, "gemm_grouped", qaff_gather_qmm_ex(A16, QAFF_BF16, 20, 1, P16, S16, B16, 16, 64, 4096, 64, 4, nullptr,
                                                  I16, 20, 1, A16, nullptr, QAFF_PATH_GEMM));
    EXPECT(UNS, "", qaff_gather_qmm_ex(A16, QAFF_BF16, 2, 1, P16, S16, B16, 4, 64, 4096, 64, 4, I16, I16, 2, 0, A16,
                                       nullptr, QAFF_PATH_GEMM));
    // quantize
    EXPECT(OK, "quantize", qaff_quantize(A16, QAFF_BF16, 4, 128, 64, 4, const_cast<uint32_t*>(P16),
                                         const_cast<uint16_t*>(S16), const_cast<uint16_t*>(B16), nullptr));
    EXPECT(OK, "quantize", qaff_quantize(A2, QAFF_BF16, 4, 128, 64, 4, const_cast<uint32_t*>(P16),
                                         const_cast<uint16_t*>(S16), const_cast<uint16_t*>(B16), nullptr));
    EXPECT(INV, "", qaff_quantize(A1, QAFF_BF16, 4, 128, 64, 4, const_cast<uint32_t*>(P16), const_cast<uint16_t*>(S16),
                                  const_cast<uint16_t*>(B16), nullptr));
    EXPECT(OK, "quantize", qaff_quantize_typed(A2, QAFF_F16, 4, 128, 64, 4, const_cast<uint32_t*>(P16), A16, A16,
                                               QAFF_F32, nullptr));
    EXPECT(INV, "", qaff_quantize_typed(A16, QAFF_F16, 4, 128, 64, 4, const_cast<uint32_t*>(P16), A2, A16, QAFF_F32,
                                        nullptr));  // float32 scales need 4-byte alignment
    EXPECT(INV, "", qaff_quantize_typed(A16, QAFF_F16, 4, 128, 64, 4, const_cast<uint32_t*>(P16), A16, A16,
                                        (qaff_dtype)3, nullptr));
    // the product without the transpose, with a workspace and with the static scratch
    const size_t nt = qaff_qmm_nt_workspace_size(2, 4096, 4096, 4);
    CHECK(nt > 0);
    EXPECT(OK, "qmm_nt", qaff_qmm_nt(A16, QAFF_BF16, 2, P16, S16, B16, 4096, 4096, 64, 4, A16, nt, A16, nullptr));
    EXPECT(INV, "", qaff_qmm_nt(A16, QAFF_BF16, 2, P16, S16, B16, 4096, 4096, 64, 4, A16, nt - 4, A16, nullptr));
    EXPECT(OK, "qmm_nt", qaff_qmm_nt_static(A16, QAFF_BF16, 2, P16, S16, B16, 4096, 4096, 64, 4, A16, nullptr));
    EXPECT(UNS, "", qaff_qmm_nt_static(A16, QAFF_BF16, 2, P16, S16, B16, 128 * 300, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "qmm_nt", qaff_qmm_nt_typed(A2, QAFF_F16, 2, P16, S16, B16, QAFF_F16, 4096, 4096, 64, 4, A16, nt,
                                                 A2, nullptr));
    EXPECT(OK, "qmm_nt", qaff_qmm_nt_typed(A16, QAFF_F16, 2, P16, S16, B16, QAFF_BF16, 4096, 4096, 64, 4, A16, nt, A16,
                                           nullptr));  // float32 y
    EXPECT(INV, "", qaff_qmm_nt_typed(A16, QAFF_F16, 2, P16, S16, B16, QAFF_BF16, 4096, 4096, 64, 4, A16, nt, A2,
                                      nullptr));  // the float32 y needs 4-byte alignment
    EXPECT(INV, "", qaff_qmm_nt_typed(A16, QAFF_F16, 2, P16, reinterpret_cast<const uint16_t*>(A2), B16, QAFF_F32, 4096,
                                      4096, 64, 4, A16, nt, A16, nullptr));  // float32 scales need 4-byte alignment
    EXPECT(INV, "", qaff_qmm_nt_typed(A16, (qaff_dtype)3, 2, P16, S16, B16, QAFF_F16, 4096, 4096, 64, 4, A16, nt, A16,
                                      nullptr));
    EXPECT(INV, "", qaff_qmm_nt(A16, QAFF_F16, 2, P16, S16, B16, 4096, 4096, 64, 4, A16, nt, A16, nullptr));
    EXPECT(INV, "", qaff_qmm_nt_typed(A16, QAFF_F16, 2, P16, S16, B16, QAFF_F16, 4096, 4096, 64, 4, A16, nt - 4, A16,
                                      nullptr));
    // other float types
    EXPECT(OK, "dequant_typed", qaff_dequantize_typed(P16, S16, B16, QAFF_F16, 4, 64, 32, 4, A16, QAFF_F32, nullptr));
    EXPECT(OK, "dequant", qaff_dequantize_typed(P16, S16, B16, QAFF_BF16, 4, 64, 32, 4, A16, QAFF_F32, nullptr));
    EXPECT(OK, "gemv_f16", qaff_qmm_typed(A16, QAFF_F16, 1, P16, S16, B16, QAFF_F16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(OK, "gemv_typed", qaff_qmm_typed(A16, QAFF_F32, 1, P16, S16, B16, QAFF_F16, 64, 4096, 64, 4, A16, nullptr));
    EXPECT(INV, "", qaff_qmm_typed(A16, (qaff_dtype)5, 1, P16, S16, B16, QAFF_F16, 64, 4096, 64, 4, A16, nullptr));
    CHECK(qaff_promote_dtype(QAFF_BF16, QAFF_F16) == QAFF_F32);
    EXPECT(OK, "gemv_typed", qaff_gather_qmm_typed(A16, QAFF_F16, 2, 1, P16, A16, A16, QAFF_F32, 4, 64, 4096, 64, 4,
                                                   I16, I16, 3, 0, A16, nullptr));
    EXPECT(OK, "gemv_scalar", qaff_gather_qmm_typed(A2, QAFF_F16, 2, 1, P16, A16, A16, QAFF_F16, 4, 64, 4096, 64, 4,
                                                    I16, I16, 3, 0, A16, nullptr));
    EXPECT(OK, "gemv_gather", qaff_gather_qmm_typed(A16, QAFF_BF16, 2, 1, P16, A16, A16, QAFF_BF16, 4, 64, 4096, 64,
                                                    4, I16, I16, 3, 0, A16, nullptr));  // the plain gathered product
    EXPECT(INV, "", qaff_gather_qmm_typed(A16, QAFF_F16, 2, 1, P16, A2, A16, QAFF_F32, 4, 64, 4096, 64, 4, I16, I16, 3,
                                          0, A16, nullptr));
    EXPECT(INV, "", qaff_gather_qmm_typed(A16, QAFF_F16, 2, 1, P16, A16, A16, QAFF_F32, 4, 64, 4096, 64, 4, nullptr,
                                          I16, 3, 0, A16, nullptr));  // 3 batches of 2 x batches without lhs
    // the error text of a failure, then cleared by the next call
    qaff_dequantize(P16, S16, B16, 4, 64, 32, 7, A16, QAFF_F32, nullptr);
    CHECK(std::strstr(qaff_last_error(), "bits") != nullptr);
    qaff_dequantize(P16, S16, B16, 4, 64, 32, 4, A16, QAFF_F32, nullptr);
    CHECK(qaff_last_error()[0] == 0);
    CHECK(std::strcmp(qaff_status_string(QAFF_ERR_DEVICE), "QAFF_ERR_DEVICE") == 0);
    CHECK(qaff_abi_version() == QAFF_ABI_VERSION);
    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("api driver: all checks passed\n");
    return 0;
}
