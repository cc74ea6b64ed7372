/* Measurement probes of the GPU's sustained rates (not part of the attention
 * path).  The benchmark reports each kernel's rate both against MI355X's
 * published peaks and against what these probes measure on the same GPU in
 * the same run: a dense bf16 MFMA loop and a streaming HBM read.
 *
 * Conventions as in swa.h: device pointers, the call returns SWA_OK or a
 * negative swa_status_t, argument checks run on the host before any launch,
 * and the work is queued on `stream` (the call does not synchronize).
 */
#ifndef SWA_PROBE_H
#define SWA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Dense bf16 matrix rate: `workgroups` workgroups of 512 threads (8 waves);
 * each wave runs `iters` rounds of 32 v_mfma_f32_32x32x16_bf16 (32 x 32 x 16,
 * 32768 FLOP each) on four independent accumulators, the A and B operands
 * changing from one product to the next; one workgroup per CU.  `operands`: 512 x 8 bf16 values
 * (8 KiB, 16-byte aligned; random values give the power draw of real data),
 * read once.  `out`: workgroups * 512 floats (the accumulators' sums, so the
 * products cannot be dropped).  FLOP per call: workgroups * 8 * iters * 32 *
 * 32768.  SWA_ERR_INVALID_ARG for null or misaligned pointers, workgroups
 * outside [1, 65535] or iters outside [1, 2^24]. */
int swa_probe_mfma_bf16(const void *operands, float *out, int workgroups, int iters, hipStream_t stream);

/* Streaming read: `bytes` bytes at `buf` (16-byte aligned, bytes a positive
 * multiple of 16) read once with 16-byte loads by `workgroups` workgroups of
 * 256 threads, each over a contiguous share.  `out`: workgroups * 256 words (an XOR of the
 * data read, so the loads cannot be dropped).  SWA_ERR_INVALID_ARG for null
 * or misaligned pointers, a bad size or workgroups outside [1, 65535]. */
int swa_probe_stream_read(const void *buf, size_t bytes, uint32_t *out, int workgroups, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SWA_PROBE_H */
