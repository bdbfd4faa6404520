/* ds4probes.h - measurement probes of the device's achievable peaks.
 *
 * Not part of the attention step: the benchmark runs these beside the published
 * MI355X figures (HBM3E 8 TB/s, dense float16 matrix throughput 2.5 PFLOP/s) so
 * that every roofline fraction can also be read against what the device reaches.
 *
 * All pointers are device memory; `stream` is a hipStream_t (NULL = default).
 * Return value: 0 on success, 1 for an invalid argument (nothing launched), 2 when
 * the launch failed.  Calls are asynchronous on `stream`; the caller times them. */
#ifndef DS4PROBES_H
#define DS4PROBES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16, buffer 16-byte aligned) once with `grid`
 * workgroups of 256 threads.  `sink` receives grid*256 uint32 words (XORs of the
 * data, so that no load is elided). */
int ds4probe_stream_read(const void *buf, int64_t bytes, uint32_t *sink, int32_t grid, void *stream);

/* `grid` workgroups of 4 waves; each wave runs `iters` x 8 independent
 * v_mfma_f32_16x16x32_f16 with register operands (no memory traffic).  `out`
 * receives grid*256 floats; `clocks` receives per wave (shader-clock cycles,
 * 100 MHz reference ticks) over the loop: 2*grid*4 uint64. */
int ds4probe_mfma_loop(int32_t iters, float *out, unsigned long long *clocks, int32_t grid, void *stream);

/* Floating-point operations of one ds4probe_mfma_loop launch. */
int64_t ds4probe_mfma_loop_flops(int32_t iters, int32_t grid);

#ifdef __cplusplus
}
#endif

#endif
