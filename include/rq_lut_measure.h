/*
 * rq_lut_measure.h -- measurement aids exported by librq_lut.so. None of them is
 * part of the method or of the serving calls in rq_lut.h: they exist so that a
 * benchmark can time one kernel by its own dispatch, measure the HBM
 * stream-read ceiling of this GPU, and report which tiling a call will use.
 *
 * rq_set_stage_events keeps a one-shot, thread-local hook (the only state the
 * library holds between calls); the other functions are stateless.
 */
#ifndef RQ_LUT_MEASURE_H
#define RQ_LUT_MEASURE_H

#include "rq_lut.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Measurement aid, not part of the method: reads bytes [src, src + bytes)
 * once with 16-byte loads and nothing else, so that its rate is the HBM
 * stream-read ceiling this GPU reaches; the lookup+sum pass's bandwidth is
 * reported against it as well as against the specification.
 *   config  0 .. rq_stream_read_configs()-1: a grid size (256 to 2048
 *           workgroups of 1024 threads) and a count of loads each thread
 *           keeps in flight (1, 2, 4 or 8); the caller keeps the fastest
 *   src     device buffer, 16-byte aligned; bytes a multiple of 16
 *   sink    device uint32 [rq_stream_read_sink_words(config)]: word w is
 *           the XOR of every 32-bit word workgroup w read, so the XOR of
 *           all sink words is the XOR of every word of the buffer
 * bytes == 0 is a no-op. NULL buffers return RQ_ERR_NULL, misalignment
 * RQ_ERR_ALIGN, an unknown config RQ_ERR_SHAPE.
 */
int32_t rq_stream_read_configs(void);
size_t rq_stream_read_sink_words(int32_t config);
rq_status rq_stream_read(const void* src, size_t bytes, int32_t config, uint32_t* sink, hipStream_t stream);

/*
 * Measurement hook. The next lookup+sum kernel that rq_lut_logits or
 * rq_lut_matvec launches from the calling thread (or the next
 * rq_stream_read kernel) is launched with
 * hipExtLaunchKernelGGL(..., before, after, ...): the events take the start
 * and end of that kernel's own dispatch on its stream, so that
 * hipEventElapsedTime(before, after) is that one kernel's duration (the
 * selection/epilogue kernels of the same call fall outside; like a profiler's
 * kernel trace, it excludes the cache release at the kernel's end). The
 * hook is one-shot and thread-local: it is cleared when used, and by a call
 * with both events NULL. The events stay owned by the caller and must have
 * been created (hipEventCreate) without hipEventDisableTiming.
 */
rq_status rq_set_stage_events(hipEvent_t before, hipEvent_t after);

/*
 * The tiling rq_lut_logits uses for this matrix, batch and table dtype (a pure
 * function of the shapes). plan[0..9] = { batch values per staged table entry,
 * pairs per staged chunk, chunks, chunks per group, groups (partial sums per
 * output), row steps per lane, rows per step, row slabs, row sets per slab,
 * batch tiles }. Returns RQ_OK, or the status of the same argument checks as
 * rq_lut_logits (RQ_ERR_SHAPE when no tiling fits on chip).
 */
rq_status rq_lut_logits_plan(const rq_matrix* W, int32_t B, int32_t lut_dtype, int32_t plan[10]);

#ifdef __cplusplus
}
#endif

#endif /* RQ_LUT_MEASURE_H */
