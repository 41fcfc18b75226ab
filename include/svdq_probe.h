/* Peak-rate probes for the benchmark harness.  They are not part of the
 * layer: they measure, on the device at hand, the dense matrix-core rates
 * that the layer's kernels are priced against, so that achieved rates can be
 * stated against both the published peak and the measured one. */
#ifndef SVDQ_PROBE_H
#define SVDQ_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

#define SVDQ_PROBE_MFMA_I8 0  /* v_mfma_i32_32x32x32_i8 (int8, the INT4 layer's product type) */
#define SVDQ_PROBE_MFMA_FP4 1 /* v_mfma_scale_f32_32x32x64_f8f6f4, both operands FP4 E2M1 */
#define SVDQ_PROBE_MFMA_FP6 2 /* v_mfma_scale_f32_32x32x64_f8f6f4, both operands FP6 E3M2 (the 6-bit
                                 route's MFMA), eight independent 32 x 32 tiles per iteration */
#define SVDQ_PROBE_DEQUANT 3  /* fp32 VALU only: the 6-bit route's dequantization of eight 32 x 32
                                 tiles per iteration, acc = fma(p * s_x, s_w, acc) on 16 values per lane */
#define SVDQ_PROBE_FP6_DEQUANT 4 /* the 6-bit route's mix: per tile one FP6 MFMA while the previous
                                    tile's result is dequantized, eight tiles per iteration */

/* Device, asynchronous.  Launches `blocks` blocks of 256 threads on `stream`
 * (NULL: the default stream); each wave runs `iters` iterations of
 * independent accumulation chains of the MFMA form `kind` on register
 * operands (no memory traffic in the loop) and writes its accumulators to
 * `sink`: a caller-owned device buffer, 16-byte aligned, of at least
 * blocks * 256 * 64 bytes, whose contents are unspecified afterwards.  The
 * dense operations performed are svdq_probe_mfma_ops(kind, blocks, iters).
 * Kinds 2-4 process eight 32 x 32 tiles per wave and iteration; they run at
 * most two waves per SIMD (launch 2 x CUs blocks for two), as the 6-bit
 * kernel 2 does.
 * Errors: SVDQ_ERR_INVALID_ARG (unknown kind, blocks or iters below 1, null
 * or misaligned sink), SVDQ_ERR_UNSUPPORTED_DEVICE, SVDQ_ERR_HIP. */
int svdq_probe_mfma(int kind, int blocks, int iters, void* sink, void* stream);

/* Host.  Dense operations (two per multiply-add) of the MFMAs of one
 * svdq_probe_mfma launch (for SVDQ_PROBE_DEQUANT: its fp32 flops, three per
 * dequantized value); 0 for an unknown kind or a count below 1. */
double svdq_probe_mfma_ops(int kind, int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_PROBE_H */
