/*
 * q4mv_probe.h -- C ABI of libq4mv_probe.so: reference kernels for measurement only. They
 * are not part of the GEMV path; the benchmark times them next to it to give the ceilings
 * its figures are read against. Same conventions as q4mv.h: caller-owned HIP device
 * pointers, work enqueued asynchronously on `stream`, host-side validation before any launch,
 * negative status (the Q4MV_ERR_* values of q4mv.h) on failure.
 */
#ifndef Q4MV_PROBE_H
#define Q4MV_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * q4mv_probe_read -- the streaming-read ceiling: reads `bytes` of `src` once, with 16-byte
 * non-temporal loads (the GEMV's weight loads), grid-stride over blocks_per_cu workgroups of
 * 256 threads per compute unit with four loads in flight per thread, and stores one XOR of
 * the words each thread read into sink[thread] (so no load can be dropped).
 *   src  : bytes of device memory, 16-byte aligned; bytes > 0 and a multiple of 16
 *   sink : u32 [q4mv_probe_sink_words(blocks_per_cu)]
 *   blocks_per_cu : 1..16
 * Errors: NULL pointer (NULL), bad bytes or blocks_per_cu (SHAPE), src not 16-byte or sink
 * not 4-byte aligned (ALIGN), launch failure (LAUNCH).
 */
int q4mv_probe_read(const void *src, int64_t bytes, uint32_t *sink, int blocks_per_cu,
                    void *stream);

/* Words the sink of q4mv_probe_read needs (blocks_per_cu x compute units x 256); negative
   status for blocks_per_cu outside 1..16. */
int64_t q4mv_probe_sink_words(int blocks_per_cu);

/*
 * q4mv_probe_empty -- the launch floor: `blocks` workgroups of 256 threads whose kernel does
 * nothing. Timed back to back it gives the cost of a launch with no memory traffic.
 * Errors: blocks outside 1..2^20 (SHAPE), launch failure (LAUNCH).
 */
int q4mv_probe_empty(int blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4MV_PROBE_H */
