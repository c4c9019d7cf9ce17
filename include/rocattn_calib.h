/*
 * rocattn_calib.h -- C ABI of librocattn_calib.so: microbenchmarks that
 * measure what the MI355X sustains on the two units the attention kernels
 * are bound by, so that the benchmark can quote an achieved rate against a
 * measured ceiling beside the published peak (2.5166 PFLOP/s dense bf16
 * MFMA, 8.0 TB/s HBM3E).  The roofline those peaks define is the one
 * "Transformer" (ai-notes) -- Discussion (Compute) implies: the two matrix
 * products of attention are compute, the K/V stream of a cached step is
 * memory.
 *
 * Conventions: device pointers, caller-owned; `stream` is a hipStream_t;
 * work is only enqueued (time it with events on that stream).  Returns 0,
 * -1 for a bad size or NULL pointer, -2 for overlapping buffers, -7 for a
 * pointer that is not 16-byte aligned, -9 for a launch error.
 */
#ifndef ROCATTN_CALIB_H
#define ROCATTN_CALIB_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * calib_mfma_loop -- n_workgroups workgroups of 4 waves; every wave issues
 * iters rounds of 4 independent v_mfma_f32_32x32x16_bf16 on register
 * operands and nothing else.  sink: float32 [n_workgroups], written only to
 * keep the loop alive (contents unspecified).  The FLOPs of one launch are
 * calib_mfma_loop_flops(n_workgroups, iters).
 */
int calib_mfma_loop(int n_workgroups, int iters, float* sink, void* stream);
double calib_mfma_loop_flops(int n_workgroups, int iters);

/*
 * calib_stream_read -- read `bytes` (a multiple of 16) from src once with
 * 16-byte loads, grid-stride over n_workgroups workgroups of 256 lanes;
 * sink: float32 [n_workgroups], one value per workgroup.
 */
int calib_stream_read(const void* src, size_t bytes, int n_workgroups, float* sink, void* stream);

/*
 * calib_stream_copy -- dst[0 .. bytes) = src[0 .. bytes) with 16-byte loads
 * and stores (bytes a multiple of 16; the buffers must not overlap).
 */
int calib_stream_copy(const void* src, void* dst, size_t bytes, int n_workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ROCATTN_CALIB_H */
