/*
 * vwl_bench.h -- measurement helper shipped beside libvwl.so in
 * libvwl_bench.so.  Not part of the verification path: it gives the HBM
 * read rate a plain streaming kernel reaches on the same device, the
 * practical ceiling the row kernels' bandwidth is reported against.
 */
#ifndef VWL_BENCH_H
#define VWL_BENCH_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (rounded down to 16-byte vectors) of device memory at `src`
 * (16-byte aligned) once, asynchronously on `stream`: `grid` workgroups of
 * `block` threads (64..512, a multiple of 64), each thread with `unroll`
 * (4, 8 or 16) 16-byte loads in flight per loop turn.  `sink` (device, 4-byte
 * aligned, one uint32) is written only if the xor of every loaded word
 * equals one fixed improbable value.  Returns 0, 1 for a null or misaligned
 * pointer, 2 for a bad launch shape, 3 for a launch failure. */
int vwl_bench_stream_read(const void *src, size_t bytes, void *sink, int grid, int block, int unroll,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* VWL_BENCH_H */
