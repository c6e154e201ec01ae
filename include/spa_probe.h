/*
 * spa_probe.h -- rate probes of the device, beside the attention library's
 * C ABI (same library, same conventions as spa.h: device pointers owned by
 * the caller, asynchronous on the caller's stream, host-side validation
 * before anything is enqueued, spa_status results).
 *
 * They measure what a kernel with nothing else to do reaches on this GPU, so
 * that the attention kernels can be reported against the achievable rates as
 * well as against the vendor peaks.  Neither computes anything of the method:
 * time a call with events on the stream it runs on and divide.
 */
#ifndef SPA_PROBE_H_
#define SPA_PROBE_H_

#include <stddef.h>

#include "spa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * HBM read rate.  Reads `bytes` bytes of `buf` once with 16-byte non-temporal
 * loads (the policy of the decode gather), four in flight per lane, spread
 * over `workgroups` workgroups of 256 threads striding by the whole grid.
 * Rate = bytes / time.  Use a buffer well beyond the 256 MB Infinity Cache
 * (1 GiB or more) so that the reads come from HBM.
 *   buf:        device, 16-byte aligned, contents arbitrary (only read)
 *   bytes:      > 0, a multiple of 16
 *   workgroups: 1 .. 2^20 (a few per compute unit fills the chip)
 *   sink:       device, one uint32; written only if the XOR of everything read
 *               equals a fixed 32-bit pattern (practically never), which keeps
 *               the loads from being optimised away
 * Errors: SPA_ERR_INVALID_ARG for a null or misaligned pointer or a size out
 * of range; SPA_ERR_HIP if the launch fails.
 */
spa_status spa_probe_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink, void* stream);

/*
 * Dense bf16 MFMA rate.  `workgroups` workgroups of four waves each run
 * `iters` rounds of four independent v_mfma_f32_32x32x16_bf16 accumulator
 * chains, 131,072 flops per wave and round:
 *     flops = workgroups * 4 * iters * 131072, rate = flops / time.
 *   workgroups: 1 .. 2^20 (two per compute unit put two waves on every SIMD)
 *   iters:      1 .. 2^24
 *   sink:       device, one float; written only if the accumulated sum is
 *               negative, which it never is (all operands are positive)
 * Errors: SPA_ERR_INVALID_ARG for a null pointer or a count out of range;
 * SPA_ERR_HIP if the launch fails.
 */
spa_status spa_probe_mfma_bf16(int workgroups, int iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPA_PROBE_H_ */
