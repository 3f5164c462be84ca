/*
 * Practical-peak probes for the roofline of the group-wise fake-quant linear
 * (measurement utilities; not part of the method). Status codes as in qat.h:
 * 0 ok, 1 bad argument (nothing launched), 7 launch failed.
 */
#ifndef QAT_PEAKS_H
#define QAT_PEAKS_H
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/*
 * A register-resident loop of v_mfma_f32_16x16x32_bf16: `blocks` workgroups
 * of 8 waves (two per SIMD), each wave `iters` x 8 independent MFMAs, no
 * memory traffic. Time it with events; qat_peak_mfma_flops(blocks, iters) is
 * the work it does. scratch: device, >= qat_peak_scratch_bytes(blocks) bytes
 * (one float per thread is written so the loop is not removed).
 */
int64_t qat_peak_mfma_flops(int32_t blocks, int32_t iters);
size_t qat_peak_scratch_bytes(int32_t blocks);
int32_t qat_peak_mfma(int32_t blocks, int32_t iters, float* scratch, hipStream_t stream);

/*
 * A grid-stride read of `bytes` (16-byte aligned, device) by `blocks`
 * 256-thread workgroups; one partial sum per thread goes to scratch
 * (>= blocks * 256 floats). Time it with events over a buffer larger than
 * the 256 MiB MALL for the HBM read ceiling.
 */
int32_t qat_peak_read(const void* buf, size_t bytes, int32_t blocks, float* scratch, hipStream_t stream);

/*
 * A grid-stride store over the first bytes / 16 * 16 bytes of buf (16-byte
 * aligned, device; its contents are overwritten) by `blocks` 256-thread
 * workgroups. Time it with events over a buffer larger than the 256 MiB MALL
 * for the HBM write ceiling.
 */
int32_t qat_peak_write(void* buf, size_t bytes, int32_t blocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* QAT_PEAKS_H */
