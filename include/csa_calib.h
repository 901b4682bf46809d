/* Calibration probes of libcsa_calib.so: measurement tools built beside the
 * CSA library, not part of it and not a step of the method.  Same status
 * codes and stream type as include/csa.h; no csa_last_error (a probe either
 * launches or returns CSA_ERR_INVALID_ARG / CSA_ERR_LAUNCH). */
#ifndef CSA_CALIB_H
#define CSA_CALIB_H

#include "csa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* csa_read_probe: read every byte of buf (device, 16-byte aligned, the first
 *   bytes / 16 * 16 of them) once with plain streaming loads, as one launch:
 *   timed over large buffers it gives the practical HBM read ceiling of one
 *   launch that memory-bound kernels can be compared with.  sink: one
 *   unsigned of device memory (rarely written).  Bad arguments:
 *   CSA_ERR_INVALID_ARG. */
int csa_read_probe(const void *buf, long long bytes, unsigned *sink, csa_stream stream);

/* csa_mfma_probe: the matrix cores' issue ceiling.  waves_per_simd (1..8)
 *   workgroups of 256 threads per compute unit; every wave runs iters
 *   (1..2^24) rounds of four independent v_mfma_f32_16x16x32_bf16 chains,
 *   with valu_per_mfma (0..3) float FMAs on other registers after each MFMA.
 *   One launch performs (CUs x waves_per_simd x 4 waves) x iters x 4 x 16,384
 *   FLOP; timed, it gives the bf16 matrix rate a kernel with that much vector
 *   work per MFMA can reach.  sink: one float of device memory (rarely
 *   written).  Bad arguments: CSA_ERR_INVALID_ARG. */
int csa_mfma_probe(float *sink, int waves_per_simd, int iters, int valu_per_mfma, csa_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_CALIB_H */
