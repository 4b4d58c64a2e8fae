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
 * Measurement utility: the next kvattn_mla_decode call made on the calling
 * thread has the first wave of its split kernel's workgroup 0 store four
 * uint64 values at `stamps` (device memory, 8-byte aligned, owned by the
 * caller): the shader clock counter (s_memtime) and the 100 MHz real-time
 * counter (s_memrealtime) when its tile loop starts, then both again when
 * it ends.  The ratio of the two differences is the shader clock the kernel
 * ran at, from which a matrix-core peak at the measured clock follows.
 * NULL disarms.  Consumed by that next call whether or not it succeeds;
 * nothing is stored if the call fails before its launch or its workgroup 0
 * has no tokens.
 */
kvattn_status kvattn_clock_next_mla(uint64_t* stamps);

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
