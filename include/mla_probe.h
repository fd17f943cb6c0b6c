/*
 * Measurement probe shipped beside libmla.so as libmla_probe.so.  It is not part of
 * the MLA path: it measures the bf16 matrix-core rate the device sustains, which
 * the benchmark reports next to the rated peak.
 */
#ifndef MLA_PROBE_H
#define MLA_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Launch `blocks` workgroups of 512 threads (two waves per SIMD at one workgroup
 * per compute unit), each wave issuing `iters` rounds of four independent
 * v_mfma_f32_32x32x16_bf16.  out: device buffer of blocks * 512 floats (written,
 * so the work is kept).  Asynchronous on `stream`; 0, -1 for bad arguments, -5 if
 * the launch fails. */
int mla_probe_mfma_bf16(int blocks, int iters, float *out, void *stream);

/* FLOP one such launch performs (2 * 32 * 32 * 16 per MFMA). */
double mla_probe_mfma_bf16_flop(int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif
