// Measurement aids declared in include/qaff_bench.h: a plain streaming read (the ceiling of a
// memory-bound kernel over the same bytes) and a device timestamp for timing inside a graph.
#include "qaff_bench.h"

#include <hip/hip_runtime.h>

namespace {

typedef uint32_t u32x4a __attribute__((ext_vector_type(4)));

// Block b reads chunks [b * 256 * U, (b + 1) * 256 * U), thread t those t + 256 u: every wave
// instruction covers 1 KiB of consecutive bytes. All U loads are issued before any is used.
// With `out`, every wave also folds its lanes' words together and its first lane stores the low
// 16 bits to out[wave % out_count]: one dependent 2-byte result per wave, as a product writes.
template <int U, bool NT>
__global__ __launch_bounds__(256) void read_kernel(const u32x4a* __restrict__ src, uint64_t chunks, uint32_t magic,
                                                   uint32_t* sink, uint16_t* out, uint32_t out_count) {
    const uint64_t base = (uint64_t)blockIdx.x * (256 * U) + threadIdx.x;
    u32x4a v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t c = base + 256 * u;
        if (c < chunks) v[u] = NT ? __builtin_nontemporal_load(src + c) : src[c];
        else v[u] = u32x4a{0u, 0u, 0u, 0u};
    }
    uint32_t acc = 0u;
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    if (out) {
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, d, 64);
        const uint64_t wave = ((uint64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
        if ((threadIdx.x & 63) == 0) out[wave % out_count] = (uint16_t)acc;
    } else if (acc == magic) {
        sink[0] = acc;
    }
}

__global__ void stamp_kernel(uint64_t* slot) { *slot = (uint64_t)wall_clock64(); }

template <int U>
hipError_t launch_read(const void* src, uint64_t chunks, bool nt, uint32_t magic, uint32_t* sink, uint16_t* out,
                       uint32_t out_count, hipStream_t stream) {
    const uint64_t blocks = (chunks + 256 * U - 1) / (256 * U);
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffULL) return hipErrorInvalidValue;
    if (nt)
        read_kernel<U, true><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(static_cast<const u32x4a*>(src), chunks,
                                                                               magic, sink, out, out_count);
    else
        read_kernel<U, false><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(static_cast<const u32x4a*>(src), chunks,
                                                                                magic, sink, out, out_count);
    return hipGetLastError();
}

hipError_t read_any(const void* src, size_t bytes, int chunks_per_thread, int nontemporal, uint32_t magic,
                    uint32_t* sink, uint16_t* out, uint32_t out_count, hipStream_t stream) {
    const uint64_t chunks = bytes / 16;
    switch (chunks_per_thread) {
        case 1: return launch_read<1>(src, chunks, nontemporal != 0, magic, sink, out, out_count, stream);
        case 2: return launch_read<2>(src, chunks, nontemporal != 0, magic, sink, out, out_count, stream);
        case 4: return launch_read<4>(src, chunks, nontemporal != 0, magic, sink, out, out_count, stream);
        case 8: return launch_read<8>(src, chunks, nontemporal != 0, magic, sink, out, out_count, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

extern "C" {

hipError_t qaff_bench_read(const void* src, size_t bytes, int chunks_per_thread, int nontemporal, uint32_t magic,
                           uint32_t* sink, hipStream_t stream) {
    if (!src || !sink || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(sink) % 4 != 0)
        return hipErrorInvalidValue;
    return read_any(src, bytes, chunks_per_thread, nontemporal, magic, sink, nullptr, 1, stream);
}

hipError_t qaff_bench_read_store(const void* src, size_t bytes, int chunks_per_thread, int nontemporal,
                                 uint16_t* out, uint32_t out_count, hipStream_t stream) {
    if (!src || !out || out_count == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(out) % 2 != 0)
        return hipErrorInvalidValue;
    return read_any(src, bytes, chunks_per_thread, nontemporal, 0u, nullptr, out, out_count, stream);
}

hipError_t qaff_bench_stamp(uint64_t* slot, hipStream_t stream) {
    if (!slot || reinterpret_cast<uintptr_t>(slot) % 8 != 0) return hipErrorInvalidValue;
    stamp_kernel<<<dim3(1), dim3(1), 0, stream>>>(slot);
    return hipGetLastError();
}

int qaff_bench_wall_clock_khz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return khz;
}

}  // extern "C"
