/*
 * moe_ceiling.h -- measurement helpers of libmoe (not part of the layer).
 *
 * The benchmark compares the layer's kernels with the MI355X vendor peaks
 * (dense bf16 matrix cores 2.5 PFLOP/s, HBM3E 8 TB/s) and, beside them, with
 * what the chip reaches on this machine in the simplest kernels of each kind.
 * Every call only enqueues one kernel on `stream` (a hipStream_t) and
 * returns; the caller times it with HIP events on the same stream.
 */
#ifndef MOE_CEILING_H
#define MOE_CEILING_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Matrix-core loop: `blocks` workgroups of 4 wavefronts, each wavefront
 * issuing iters x 8 v_mfma_f32_32x32x16_bf16 on register operands (four
 * independent accumulators, no memory traffic). sink: device fp32 [blocks]
 * (written). Returns the flops enqueued, or -1 on a bad argument or launch.
 */
long long moe_ceiling_mfma(int blocks, int iters, float* sink, void* stream);

/*
 * Streaming copy dst[0..bytes) = src[0..bytes) with 16-byte non-temporal
 * loads and stores over a grid of `blocks` x 256 threads. bytes % 16 == 0,
 * 16-byte aligned device pointers. Returns 0, or -1 on a bad argument.
 */
int moe_ceiling_copy(const void* src, void* dst, long long bytes, int blocks, void* stream);

/*
 * Streaming read of src[0..bytes) (16-byte loads folded into a checksum that
 * is practically never stored). sink: device uint32 [blocks]. Returns 0, or
 * -1 on a bad argument.
 */
int moe_ceiling_read(const void* src, long long bytes, unsigned* sink, int blocks, void* stream);

#ifdef __cplusplus
}
#endif
#endif
