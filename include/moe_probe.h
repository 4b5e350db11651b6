/* moe_probe.h - measurement probes beside the MoE layer library (libmoe_probe.so).
 *
 * Not part of the layer: bench.py reports what these reach as context for the
 * datasheet fractions of the layer's kernels.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Register-only bf16 matrix-core loop: `blocks` workgroups of 256 threads
 * (two per CU fit), each wave running `iters` rounds of 8 independent
 * 32x32x16 bf16 MFMAs with fp32 accumulation, no memory traffic. Enqueued on
 * `stream` (a hipStream_t as void*, NULL = the null stream); returns 0, -1 for
 * bad arguments (blocks outside [1, 65536], iters < 1, sink NULL; nothing is
 * enqueued) or -2 for a failed launch.
 * sink [blocks * 256] fp32  device, written (one sum per thread; keeps the work live)
 */
int moe_probe_mfma_bf16(int blocks, int iters, float* sink, void* stream);

/* Floating-point operations one moe_probe_mfma_bf16 call performs. */
double moe_probe_mfma_bf16_flops(int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
