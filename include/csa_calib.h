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

/* csa_probe_workgroups: the grid of csa_queue_probe (two 256-thread
 *   workgroups per compute unit, as the index scan launches). */
int csa_probe_workgroups(void);

/* csa_queue_probe: when does a row that every workgroup reads arrive while
 *   the workgroups' own loads fill the memory system?  Each workgroup loads
 *   the 16 KB at row (the same for all, 16-byte aligned), then tiles (0, 2,
 *   4 or 8) rounds of 4 KB of its own slice of buf (workgroup w reads bytes
 *   w * tiles * 16 KB .. of it; buf_bytes >= csa_probe_workgroups() * tiles *
 *   16 KB), waits for the row, then for the rest.  stamps [wgs][4] int64
 *   (n_stamps >= 4 * wgs): (start, row arrived, everything arrived, unused)
 *   in wall-clock ticks (100 MHz).  This is the pattern of the index scan's
 *   first loads (query, then the key ring).  sink: one unsigned of device
 *   memory (rarely written).  Bad arguments: CSA_ERR_INVALID_ARG. */
int csa_queue_probe(const void *row, const void *buf, long long buf_bytes, int tiles, long long *stamps,
                    long long n_stamps, unsigned *sink, csa_stream stream);

/* csa_handoff_probe: the cost of handing data to one workgroup inside a
 *   launch.  wgs (1..65535) workgroups of 256 threads each write 256 floats
 *   to data (n_floats >= 256 wgs); with handoff != 0 each then (after a
 *   workgroup barrier, one thread) releases them device-wide with a fence
 *   and takes a ticket from *counter, and the last one
 *   reads all of them after an acquire fence, writes 256 sums to out (256
 *   floats) and resets *counter to 0.  *counter must be 0 before the first
 *   launch.  Timed with and without the hand-off, the difference is what
 *   a kernel pays to pass its workgroups' results to a final workgroup
 *   without a second launch.  Bad arguments: CSA_ERR_INVALID_ARG. */
int csa_handoff_probe(float *data, long long n_floats, unsigned *counter, float *out, int wgs, int handoff,
                      csa_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_CALIB_H */
