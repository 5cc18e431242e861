/*
 * pa_bench.h -- measurement helpers of libpa (not part of the attention
 * path): what the benchmark needs to relate the path's bandwidth to what the
 * GPU can do.
 */
#ifndef PA_BENCH_H
#define PA_BENCH_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of device memory at buf (16-byte aligned, a multiple
 * of 16) once, with 16-byte non-temporal loads spread over `workgroups`
 * workgroups of 256 threads, on `stream`; no other memory traffic (sink,
 * workgroups * 256 uint32 of device memory, is practically never written).
 * Bytes / duration is the plain streaming-read bandwidth of the device. */
pa_status pa_bench_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                               int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_BENCH_H */
