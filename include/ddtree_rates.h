/*
 * ddtree_rates.h -- C ABI of libddtree_rates.so: achievable-rate probes for
 * MI355X (gfx950), used to read the verify path's roofline fractions against
 * what the chip sustains on the same box.  Not part of the verify path.
 *
 * Both calls only enqueue one kernel on `stream` (a hipStream_t as void*) and
 * return 0, or -1 for an invalid argument (nothing enqueued), -4 when the
 * launch fails.  The caller times the launch (HIP events on the same stream).
 */
#ifndef DDTREE_RATES_H
#define DDTREE_RATES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Back-to-back bf16 MFMA loop: `workgroups` workgroups of 4 waves (256 per CU
 * fill the chip's 256 CUs once; 512 put two waves on every SIMD), each wave
 * issuing 4 independent v_mfma_f32_32x32x16_bf16 per iteration for `iters`
 * iterations.  sink: device float32 [workgroups * 4] (one value per wave). */
int ddtree_rates_mfma_loop(int32_t workgroups, int32_t iters, float* sink, void* stream);

/* Dense bf16 flops one ddtree_rates_mfma_loop launch performs. */
int64_t ddtree_rates_mfma_loop_flops(int32_t workgroups, int32_t iters);

/* Read-only HBM stream: reads `bytes` (a multiple of 16, 16-byte aligned src)
 * once with 16-byte nontemporal loads, each of the `workgroups` workgroups
 * (256 threads) one contiguous span of about bytes / workgroups.
 * sink: device uint32 [workgroups * 256]. */
int ddtree_rates_stream_read(const void* src, int64_t bytes, int32_t workgroups, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DDTREE_RATES_H */
