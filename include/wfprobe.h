/* wfprobe.h -- measurement probes beside the attention library (libwfprobe.so).
 *
 * Not part of the attention path.  The benchmark reads the attention's exponentials per second
 * (the online softmax takes one 2^x per visible (query row, key, head) triple) against the rate
 * at which the chip retires v_exp_f32 when nothing else runs, which wfprobe_exp_rate measures;
 * and a profiling run scales its memory counters by what they read for wfprobe_copy, a plain
 * copy of known size.
 */
#ifndef WFPROBE_H
#define WFPROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueues `blocks` workgroups of 256 lanes on `stream` (a hipStream_t passed as void*; NULL is
 * the null stream).  Each lane iterates x <- 2^(-x) on 8 independent values, `iters` times, and
 * stores their sum to out[block * 256 + lane]; out (device memory, caller-owned) must hold
 * blocks * 256 floats.  Asynchronous: time it with events on the same stream.
 * Returns the number of exponentials one launch retires (blocks * 256 * 8 * iters), or -1 when
 * out is NULL, blocks < 1, iters < 1 (checked before any HIP call) or the launch fails. */
int64_t wfprobe_exp_rate(float* out, int32_t blocks, int32_t iters, void* stream);

/* Enqueues on `stream` a plain copy of `bytes` bytes from src to dst (device memory, caller-owned,
 * not overlapping): one kernel, every 16-byte granule read once and written once.  Returns 0, or
 * -1 when a pointer is NULL or not 16-byte aligned, bytes is not a positive multiple of 16
 * (checked before any HIP call) or the launch fails. */
int32_t wfprobe_copy(void* dst, const void* src, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WFPROBE_H */
