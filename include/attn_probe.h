/*
 * attn_probe.h -- measurement probe of libattn_probe.so.  Not part of the
 * attention path: it measures how fast the bf16 matrix cores run on this
 * chip under the data the benchmark uses, the ceiling the attention kernel's
 * rate is read against ("Verify tiled attention", section "Separate storage
 * savings from runtime": measure the selected runtime backend rather than
 * assume a speedup).
 *
 * attn_probe_mfma -- enqueue one launch of `grid` workgroups of 256 threads
 *   (four 64-wide waves) on `stream`, each wave issuing 16 * iters
 *   v_mfma_f32_32x32x16_bf16 instructions:
 *     kind 0: operands in registers, all zero (no bit toggling);
 *     kind 1: operands in registers, random bf16 of magnitude 0.25-1;
 *     kind 2: A operands read from LDS, 1 KiB per MFMA per wave, all zero;
 *     kind 3: as 2 with random bf16 data in LDS and in the B operands.
 *   `out` is a device buffer of at least `grid` floats that the probe never
 *   writes in practice (a store guarded by a result test that fails);
 *   owned by the caller.  Returns 0, 1 for invalid arguments (nothing
 *   enqueued) or 4 when the launch failed.
 *
 * attn_probe_mfma_flops -- FLOPs of one such launch (2 * 32 * 32 * 16 per
 *   MFMA); host only.
 */
#ifndef ATTN_PROBE_H
#define ATTN_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

int attn_probe_mfma(int kind, int iters, int grid, float* out, void* stream);
double attn_probe_mfma_flops(int kind, int iters, int grid);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H */
