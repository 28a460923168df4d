/* Measurement and test helpers of libcpattn (not part of the attention
 * method).
 *
 * The benchmark reports the attention kernel's throughput against the
 * published dense bf16 peak and, beside it, against what this part's
 * matrix cores sustain on a pure MFMA stream; two calls provide that
 * second denominator and the device's compute-unit count and clock.  A
 * third fills the LDS for the memory-safety tests. */
#ifndef CPATTN_PROBE_H
#define CPATTN_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Pure-MFMA rate probe, device.  Launches 'blocks' workgroups of 512 lanes
 * (two waves per SIMD, one workgroup per CU at a time); each wave runs
 * iters * 16 v_mfma_f32_32x32x16_bf16 over eight independent accumulators
 * on operands read once from 'operands' (device, 4096 bf16 values, 16-byte
 * aligned; random values give the operand toggling of real data), then
 * writes one float per lane to 'out' (device, blocks * 512 floats).  FLOPs
 * per launch: blocks * 8 * iters * 16 * 32768.  Enqueued on 'stream';
 * returns 0, or 1 for invalid arguments or a failed launch. */
int cpattn_probe_mfma(const void *operands, float *out, int blocks, int iters, void *stream);

/* LDS fill, device, for tests: launches 'blocks' workgroups of 256 lanes,
 * each holding the whole 160 KiB of LDS a workgroup can take (so one runs
 * per CU at a time) and setting every 32-bit word of it to 'pattern'.  The
 * LDS keeps its contents after a kernel ends; a test runs this before an
 * attention launch (with a NaN pattern) to show that the launch reads no
 * LDS it did not write.  Enqueued on 'stream'; returns 0, or 1 for
 * blocks < 1 or a failed launch. */
int cpattn_probe_fill_lds(unsigned pattern, int blocks, void *stream);

/* Compute units and maximum engine clock (kHz) of the current device, host.
 * Returns 0, or 1 for NULL pointers or a failed query. */
int cpattn_device_info(int *compute_units, int *max_clock_khz);

#ifdef __cplusplus
}
#endif

#endif
