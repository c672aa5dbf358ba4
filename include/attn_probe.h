/* Sustained-rate probes for the measurement harness (libattn_probe.so).
 *
 * Not part of the attention library: these kernels exist so that the ceilings the
 * attention kernels are measured against can be re-measured on the board at hand.
 * The published peak of the chip assumes its 2.4 GHz peak shader clock.  Under a
 * dense matrix-core load the board holds a lower, power-limited clock.  These probes
 * report what one compute unit sustains at that clock:
 *   - bf16 v_mfma_f32_32x32x16 back to back on every SIMD, with register operands
 *     loaded from a caller-chosen buffer (random data switch more bits, and so draw
 *     more power, than constant data);
 *   - LDS reads of the three forms the attention kernels use (16-byte ds_read_b128,
 *     8-byte ds_read_b64, and the transposing ds_read_b64_tr_b16), all addresses
 *     free of bank conflicts.
 *
 * Every call enqueues one kernel on `stream` and returns 0, or a negative code for
 * bad arguments (nothing is enqueued then).  Pointers are device pointers.  Calls that
 * overlap on one device share nothing.
 */
#ifndef ATTN_PROBE_H
#define ATTN_PROBE_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_PROBE_API __attribute__((visibility("default")))

/* Matrix-core probe.  `blocks` workgroups of 4 waves (two waves per SIMD, like the
 * attention forward); each wave issues 8 * iters v_mfma_f32_32x32x16_bf16 in four
 * independent accumulator chains, with operands taken from `ops`: 256 * 8 pieces of
 * 16 bytes (bf16x8), piece 8 t + f for thread t of every workgroup, f = 0..3 the A
 * operands and 4..7 the B operands.  Writes one float per thread (a sum of its
 * accumulators, so that nothing is optimised away) to out[blocks * 256].
 * Flops per call: blocks * 4 * iters * 8 * 32768.
 * Errors: -1 if a pointer is null, -2 if blocks < 1 or iters < 1, -4 if the launch fails. */
ATTN_PROBE_API int attn_probe_mfma_bf16(const void *ops, float *out, int blocks, int iters,
                                        hipStream_t stream);

/* LDS read probe.  `blocks` workgroups of 8 waves with 64 KiB of LDS each; every lane
 * first writes its share of the workgroup's LDS, then issues 8 * iters reads of the
 * form `mode` selects: 0 = ds_read_b128 (16 bytes a lane), 1 = ds_read_b64 (8 bytes),
 * 2 = ds_read_b64_tr_b16 (8 bytes; each 16-lane group returns the transpose of a
 * 4 x 16 block of 16-bit elements).  A wave's lanes read consecutive pieces (1 KiB or
 * 512 bytes per instruction), a different window of the LDS for every read.  Writes
 * one word per thread (a word of its last read) to out[blocks * 512].
 * Bytes read per call: blocks * 512 * iters * 8 * (16, 8 or 8).
 * Errors: -1 if out is null, -2 if blocks < 1 or iters < 1, -3 for another mode, -4 if
 * the launch fails. */
ATTN_PROBE_API int attn_probe_lds_read(unsigned *out, int blocks, int iters, int mode, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H */
