/*
 * rq_lut_measure.h -- measurement aids exported by librq_lut.so. None of them is
 * part of the method or of the serving calls in rq_lut.h: they exist so that a
 * benchmark can time one kernel by its own dispatch, measure the HBM
 * stream-read ceiling and the LDS random-gather roof of this GPU, and report
 * which tiling a call will use.
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
 * rq_stream_read or rq_lds_gather kernel) is launched with
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
 * Measurement aid: the LDS random-gather roof. One workgroup of 1024 threads
 * per CU (256) fills 128 KB of LDS with 32-bit word i = i * 2654435761 (mod
 * 2^32), then each thread runs 8 independent sequences x <- x * 1664525 +
 * 1013904223 (mod 2^32), seeded x = 8 * (1024 * workgroup + thread) + chain,
 * and for each of `reps` steps of every sequence reads the `width`-byte entry
 * (2, 4, 8 or 16) whose index is the top log2(128 KB / width) bits of the new
 * x, XOR-folding its 32-bit words (a 2-byte entry: its 16 bits) into one
 * accumulator. sink[w] (rq_lds_gather_sink_words() words) is the XOR of the
 * accumulators of workgroup w's threads. 256 * 1024 * 8 * reps lookups in all.
 * Bad width or reps < 0: RQ_ERR_SHAPE; NULL sink: RQ_ERR_NULL.
 */
size_t rq_lds_gather_sink_words(void);
rq_status rq_lds_gather(int32_t width, int32_t reps, uint32_t* sink, hipStream_t stream);

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
