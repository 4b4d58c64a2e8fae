/*
 * kvattn_measure.h -- measurement utilities of libkvattn (not part of the
 * attention path; the operations are declared in kvattn.h).
 *
 * They exist so that a benchmark can time the kernel that streams the KV
 * cache on its own, and compare it with a plain streaming read of the same
 * device memory.  Both return the status codes of kvattn.h.
 */
#ifndef KVATTN_MEASURE_H
#define KVATTN_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "kvattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Measurement utility: the next decode call (any kvattn_*_decode* entry point)
 * made on the calling thread records `start_event` when its split-K kernel
 * (the kernel that reads the cache) starts executing and `stop_event` when it
 * ends, so the caller can time that kernel alone with hipEventElapsedTime.
 * Both are hipEvent_t handles the caller created with timing enabled (both
 * non-NULL, or both NULL to disarm).  The setting is consumed by that next
 * call whether or not it succeeds; the log-sum-exp merge kernel the call may
 * add afterwards, and the MLA plan kernel before it, are outside the two
 * events.
 */
kvattn_status kvattn_time_next_kernel(void* start_event, void* stop_event);

/*
 * Measurement utility, not part of the attention path: stream `bytes` bytes
 * of device memory at `buf` through 16-byte loads with `workgroups`
 * workgroups of 256 threads, to measure the device's practical HBM read
 * bandwidth (time it with events on `stream`).  `bytes` must be a positive
 * multiple of 16 and `buf` 16-byte aligned; `sink` is a device uint32 the
 * kernel may write (it keeps the loads from being optimised away).
 */
kvattn_status kvattn_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups,
                                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVATTN_MEASURE_H */
