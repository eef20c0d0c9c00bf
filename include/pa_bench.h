/*
 * pa_bench.h -- measurement helpers that sit beside libpa.so (not part of the
 * decode path).  They give the HBM bandwidth a plain streaming kernel reaches
 * on the device, and a copy of known size whose hardware counter readings
 * calibrate the FETCH_SIZE / WRITE_SIZE figures of other kernels.
 *
 * All pointers are caller-owned device memory; calls enqueue on `stream`
 * (a hipStream_t, NULL = default) and return without waiting.  Return value:
 * 0 on success, otherwise the hipError_t of the failed launch (or -1 for a
 * NULL pointer / a size that is not a multiple of 16 bytes).
 */
#ifndef PA_BENCH_H
#define PA_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16) from src with 16-byte loads spread over the
 * whole chip; each workgroup stores one 32-bit checksum to sink[workgroup]
 * (sink must hold pa_bench_read_grid() uint32 values). */
int pa_bench_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Number of workgroups pa_bench_read launches (the size of its sink). */
int pa_bench_read_grid(void);

/* dst[0:bytes] = src[0:bytes] with 16-byte loads and stores (bytes % 16 == 0). */
int pa_bench_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_BENCH_H */
