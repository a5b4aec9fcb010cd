/*
 * mo_probe.h -- measured roofline denominators of the GPU the library runs
 * on (a separate library, libmoprobe.so, used by the benchmark).
 *
 * The Muon step's products are bf16 matrix-core contractions and its
 * elementwise kernels stream HBM, so their roofline fractions are quoted
 * against the datasheet peaks (2.5 PFLOP/s dense bf16, 8 TB/s).  These
 * probes measure what the chip actually sustains for each unit on its own:
 * the clock a matrix-core-only load runs at, and the bandwidth of plain
 * streaming kernels, so that the fractions can also be read against
 * achieved ceilings.  Not part of the optimizer's ABI.
 *
 * Both calls allocate and free their own device memory, synchronise the
 * device and time with HIP events on an internal stream.  They return
 * 0 on success and a negative value on a HIP error (the message is then
 * available from mo_probe_last_error()).
 */
#ifndef MO_PROBE_H
#define MO_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* bf16 matrix-core rate: every wave of a grid of 8 workgroups per CU (two
 * waves per SIMD) issues `iters` x 8 v_mfma_f32_32x32x16_bf16 on register
 * operands (four independent accumulators), no memory traffic.
 * *tflops = 32768 flop x MFMAs / seconds; best of `reps` launches. */
int mo_probe_mfma_bf16(int iters, int reps, double* tflops);

/* The same grid and issue pattern on operands that switch like a product of
 * random matrices: each lane cycles through eight A and eight B register
 * operands of random bf16 values (random sign and mantissa, magnitudes
 * 2^-8 .. 1), so consecutive MFMAs never see the same inputs.  The
 * constant-like operands of mo_probe_mfma_bf16 toggle few bits; this rate
 * is what the matrix cores sustain within the chip's power budget on real
 * data, still with no memory traffic.  Same units and outputs. */
int mo_probe_mfma_bf16_random(int iters, int reps, double* tflops);

/* HBM rates over a buffer of `bytes` (rounded down to 64 KiB):
 * *read_gbs: a read-only reduction of the whole buffer (16-byte loads);
 * *copy_gbs: a copy into a second buffer, counted as read + write bytes.
 * Each stream runs in four launch shapes (1, 2 or 4 loads in flight per
 * thread; 4 to 64 workgroups of 256 threads per CU), since the fastest
 * shape differs from box to box by 10-20%; the best of `reps` launches of
 * every shape is reported. */
int mo_probe_hbm(size_t bytes, int reps, double* read_gbs, double* copy_gbs);

/* Message of the last failure on this thread. */
const char* mo_probe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MO_PROBE_H */
