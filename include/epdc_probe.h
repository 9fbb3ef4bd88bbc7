/*
 * epdc_probe.h -- C ABI of libepdc_probe.so: three streaming kernels that
 * measure what the card's HBM delivers reading only, writing only, and
 * copying one to one.  They are measurement tools beside the dispatch and
 * combine library (libepdc.so), not part of the method: the benchmark times
 * them on buffers much larger than the last-level cache and prices each
 * dispatch or combine kernel's reads and writes at those rates.
 *
 * Conventions:
 *  - `src` and `dst` are device pointers on the current device, 16-byte
 *    aligned; `bytes` is a positive multiple of 16.  The caller allocates and
 *    owns them; the library allocates nothing.
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream.  The
 *    kernel is enqueued and the call returns without waiting.
 *  - Status codes are those of include/epdc.h (EPDC_SUCCESS,
 *    EPDC_ERR_INVALID_ARGS, EPDC_ERR_GPU_OP); epdc_probe_last_error() gives a
 *    thread-local message for the last failed call.
 */
#ifndef EPDC_PROBE_H
#define EPDC_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "epdc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` of `src` once with 16-byte nontemporal loads, 32 KiB per
 * 256-thread block.  A block whose loaded words XOR to `magic` writes `magic`
 * to flag[0] (a 4-byte device word); that keeps the loads, and the caller
 * chooses a `magic` its data cannot produce (e.g. 1 for an all-zero buffer). */
epdc_status epdc_probe_read(const void *src, size_t bytes, uint32_t magic, uint32_t *flag,
                            void *stream);

/* Write `bytes` of `dst` once, one 16-byte store per thread, 4 KiB per
 * 256-thread block; word i of each vector holds value ^ i. */
epdc_status epdc_probe_write(void *dst, size_t bytes, uint32_t value, void *stream);

/* Copy `bytes` from `src` to `dst` (buffers must not overlap), four 16-byte
 * vectors per thread: nontemporal loads, ordinary stores. */
epdc_status epdc_probe_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Message of the calling thread's last failed call ("" if none). */
const char *epdc_probe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EPDC_PROBE_H */
