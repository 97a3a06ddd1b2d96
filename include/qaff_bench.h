/*
 * qaff_bench -- measurement aids for the benchmark of libqaff (libqaff_bench.so). Nothing here is
 * part of the quantized-matmul path; the product library neither links nor calls it.
 *
 *   - A plain streaming read: the time any kernel needs just to read the same bytes once under the
 *     same launch and timing conditions, the ceiling against which a memory-bound product of those
 *     bytes is judged.
 *   - A device timestamp: a one-thread kernel that writes the GPU's constant-rate wall clock, so that
 *     a captured graph can be timed from its first to its last node without the graph's own launch.
 *
 * All pointers are device pointers owned by the caller; calls are asynchronous on `stream` and
 * return hipSuccess or the launch error.
 */
#ifndef QAFF_BENCH_H
#define QAFF_BENCH_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes at `src` (16-byte aligned, bytes a multiple of 16) once, with 16-byte
 * loads, `chunks_per_thread` (1, 2, 4 or 8) of them per thread of 256-thread blocks, non-temporal
 * when `nontemporal` is non-zero. The loaded words are folded by XOR and compared with `magic`; a
 * thread whose fold equals it writes it to sink[0] (this keeps the loads; the caller passes a
 * writable uint32). hipErrorInvalidValue for other arguments. */
hipError_t qaff_bench_read(const void* src, size_t bytes, int chunks_per_thread, int nontemporal,
                           uint32_t magic, uint32_t* sink, hipStream_t stream);

/* qaff_bench_read that also writes what a product writes: every wave folds its 64 lanes' loaded
 * words together and its first lane stores the low 16 bits to out[wave % out_count] (`out`: uint16,
 * out_count > 0 elements, 2-byte aligned; which wave's value an element keeps is unspecified).
 * The ceiling of a kernel that reads the bytes once and then writes one dependent result per
 * wave. hipErrorInvalidValue for other arguments. */
hipError_t qaff_bench_read_store(const void* src, size_t bytes, int chunks_per_thread, int nontemporal,
                                 uint16_t* out, uint32_t out_count, hipStream_t stream);

/* Writes the device wall clock (ticks at qaff_bench_wall_clock_khz() kHz) to *slot. */
hipError_t qaff_bench_stamp(uint64_t* slot, hipStream_t stream);

/* Rate of that clock in kHz on the current device, or 0 if it cannot be read. */
int qaff_bench_wall_clock_khz(void);

#ifdef __cplusplus
}
#endif

#endif /* QAFF_BENCH_H */
