/*
 * kvc_peaks.h -- measurement kernels of libkvc.so: the machine ceilings the correction
 * kernels are compared against (HBM streaming, bf16 MFMA, LDS reads, fp32 VALU), measured
 * on the device rather than taken from a data sheet.  A kernel's algorithmic bytes or flops
 * divided by its time, over the ceiling measured here, says how close it runs to what this
 * GPU can actually sustain; the copy kernel also calibrates HBM byte counters (its traffic
 * is exactly `bytes` read plus `bytes` written).
 *
 * Conventions: as in kvc.h (caller-owned device buffers, 16-byte aligned; work enqueued on
 * `stream`; host-side validation, kvc_status result, kvc_last_error() for the reason).
 * Every kernel here touches only the buffers passed in, within the sizes stated.
 */
#ifndef KVC_PEAKS_H_
#define KVC_PEAKS_H_

#include <stddef.h>
#include <stdint.h>

#include "kvc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0..bytes) = src[0..bytes): a grid-stride 16-byte copy that streams HBM at its
 * sustained rate.  bytes must be a positive multiple of 16; dst and src must not overlap
 * (KVC_E_ALIAS).  Traffic: bytes read + bytes written. */
kvc_status kvc_peak_copy(void* dst, const void* src, size_t bytes, void* stream);

/* n_blocks work-groups of 256 threads, each wave running `iters` rounds of 4 independent
 * v_mfma_f32_32x32x16_bf16 chains on register operands: 4 * 32768 * iters flops per wave,
 * n_blocks * 4 waves.  sink: device float [n_blocks * 256], written once per thread so the
 * work cannot be elided.  1 <= n_blocks <= 65536, 1 <= iters <= 1 << 20. */
kvc_status kvc_peak_mfma_bf16(float* sink, int32_t n_blocks, int32_t iters, void* stream);

/* n_blocks work-groups of 256 threads, each thread reading `iters` x 8 conflict-free
 * 16-byte LDS words (ds_read_b128): 128 * 256 * iters bytes per work-group.
 * sink: device uint32 [n_blocks * 256].  Same limits as above. */
kvc_status kvc_peak_lds_read(uint32_t* sink, int32_t n_blocks, int32_t iters, void* stream);

/* n_blocks work-groups of 256 threads, each thread running `iters` rounds of 8 independent
 * unpacked fp32 adds: 8 * iters lane-ops per thread.  sink: device float [n_blocks * 256].
 * Same limits as above. */
kvc_status kvc_peak_valu(float* sink, int32_t n_blocks, int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_PEAKS_H_ */
