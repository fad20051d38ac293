/*
 * gdn_probe.h -- measurement helper of the benchmark, not part of the gated
 * delta rule's API: the dense bf16 and fp32 matrix-core rates of the GPU it runs on, so
 * that the benchmark can state fractions of a measured peak next to the
 * datasheet one.  Built as libgdn_probe.so, beside libgdn.so.
 */
#ifndef GDN_PROBE_H
#define GDN_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Enqueue n_blocks workgroups of 256 threads, each wave issuing `iters` x 4
 * independent v_mfma_f32_16x16x32_bf16 (16*16*32*2 FLOP each) on register
 * operands, with no memory traffic but one store per thread of the sums to
 * `out` (device, 256 * n_blocks floats, so that nothing is optimised away).
 * Total work: n_blocks * 4 waves * 4 * iters * 16384 FLOP.  Returns 0, or 1 for
 * bad arguments, 2 if the launch failed.
 */
int32_t gdn_probe_mfma_bf16(float *out, int32_t n_blocks, int32_t iters, void *stream);

/* The same with v_mfma_f32_16x16x4_f32 (16*16*4*2 FLOP each): the fp32
 * matrix-core rate the backward pass's products run at. */
int32_t gdn_probe_mfma_f32(float *out, int32_t n_blocks, int32_t iters, void *stream);

#ifdef __cplusplus
}
#endif

#endif
