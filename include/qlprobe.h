/*
 * qlprobe.h -- C ABI of libqlprobe.so, the measurement helpers that the
 * benchmark uses to put the layer's kernels in context. Nothing here is a step
 * of the method; the layer library (libqlora.so, include/qlora.h) neither
 * contains nor calls these kernels.
 *
 * Conventions as in qlora.h: device pointers owned by the caller, work enqueued
 * on `stream` (a hipStream_t passed as void*, NULL = the null stream), return
 * value 0 or a negative status (-1 NULL pointer, -2 bad size, -4 misaligned
 * pointer, -6 launch refused), arguments checked on the host before anything
 * is enqueued.
 */
#ifndef QLPROBE_H
#define QLPROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Plain streaming read of `bytes` bytes at the device pointer `data`: the
 * achievable read rate for a byte count, against which the decode forward's
 * packed-weight stream is compared. Each wave load instruction covers 1 KB
 * contiguous (16 bytes per lane); `loads` in {1, 2, 4, 8, 16} is the number of
 * such loads each thread keeps in flight (a work group of 256 threads reads
 * 4 KB * loads). bytes > 0 and a multiple of 16; data 16-byte aligned; sink a
 * device pointer to one uint32 (4-byte aligned) that may receive an
 * unspecified value.                                                           */
int ql_read_probe(const void* data, int64_t bytes, int loads, uint32_t* sink, void* stream);

/* An empty kernel of `groups` work groups of `threads` threads (1..1024): the
 * launch-and-drain floor of a grid of that size.                               */
int ql_empty_probe(int64_t groups, int threads, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLPROBE_H */
