/*
 * qat.h -- C ABI of the MI355X (gfx950) group-wise fake-quantised linear.
 *
 * The operations are those of EfficientQAT (arXiv 2407.11062):
 *   Block-AP: per-group min-max init, the quantiser
 *     W_int = clamp(round(W/s) + z, 0, 2^N - 1)          (Eq. 1)
 *   and dequantiser W_hat = (W_int - z) * s               (Eq. 2),
 *   a bf16 GEMM forward and the straight-through backward;
 *   E2E-QP: packed integer weights and frozen zero points, only the step
 *   sizes train, with the exact gradient dW_hat/ds = W_int - z.
 * Sources: "EfficientQAT" Paper-Notes (zhaoyang97, ACL2025), method details
 * (Eq. 1, Eq. 2, E2E-QP gradient); "EfficientQAT, low-bit training on a single
 * GPU" (modelfoundations.com), Phase 1 (min-max init, ~4096 steps per block)
 * and Phase 2 (exact scale gradient), and its "Paper vs. code" section (float
 * zero point rounded straight-through, hard-rounded at pack; FP32 blocks);
 * paperlayer.ai summary of arXiv 2407.11062v3, Appendix A (straight-through
 * estimator; gradients for s, z and W) and Appendix D (one step size and one
 * N-bit zero point per group of g weights).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Shapes: W is [out, in] row-major (nn.Linear). Groups are `group`
 *   consecutive elements of a row along `in`: 32, 64 or 128 (the sizes the
 *   paperlayer.ai summary's Appendix F ablates; 64 is the default of every
 *   workload here), or group == in for channel-wise quantisation (one group
 *   per row). group must divide in; G = in / group groups per row.
 *   s, z, ds, dz are [out, G] fp32 row-major. X is [M, in], Y and dY are
 *   [M, out], dX is [M, in]; all bf16 passed as uint16_t bit patterns.
 * - bits N in {2, 3, 4}; K = 2^N - 1. in is a multiple of 64. The GEMM calls
 *   (fake-quant fwd/bwd, dequant-GEMM fwd/bwd) take any out with out % 4 == 0
 *   (so that bf16 rows of out elements, Y and dY, are 8-byte aligned); out
 *   need not fill a tile: when it is not a multiple of 64, dY is read by 4-byte
 *   DMA and the dX contraction over out is zero-filled past its end. M is any
 *   positive count of tokens. Every operand must be smaller than 2 GiB.
 * - All tensor pointers are DEVICE pointers owned by the caller. The library
 *   never allocates, frees or keeps them beyond the enqueued work.
 * - Inputs are const and never written. Outputs are fully overwritten (never
 *   accumulated) and must not overlap inputs or each other.
 * - Every call is asynchronous on `stream` (0 = the null stream) and performs
 *   no device synchronisation.
 * - Every tensor pointer must be 16-byte aligned.
 * - Arguments are validated on the host BEFORE anything is enqueued; on error
 *   nothing is launched and no output is touched. No exception crosses the ABI.
 * - Numerics: s, z and u = W/s are IEEE fp32 results of single correctly
 *   rounded operations; round() is round-half-to-even; W_hat is rounded
 *   fp32 -> bf16 (nearest-even) as the GEMM operand; GEMMs accumulate in fp32.
 *
 * Return value: QAT_OK or one of the QAT_ERR_* codes below.
 */
#ifndef QAT_H
#define QAT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  QAT_OK = 0,
  QAT_ERR_NULL = 1,      /* a required pointer is NULL                                   */
  QAT_ERR_SHAPE = 2,     /* a dimension <= 0, in not a multiple of 64, out not a multiple
                            of 4 (GEMM calls), or an operand of 2 GiB or more               */
  QAT_ERR_BITS = 3,      /* bits not in {2, 3, 4}                                          */
  QAT_ERR_GROUP = 4,     /* group not 32, 64, 128 or in, or not dividing in                */
  QAT_ERR_ALIGN = 5,     /* a pointer is not 16-byte aligned                               */
  QAT_ERR_WORKSPACE = 6, /* workspace NULL or smaller than the size query returns          */
  QAT_ERR_HIP = 7,       /* a HIP launch failed; qat_last_error() has the HIP message      */
  QAT_ERR_ALIAS = 8,     /* an output overlaps an input or another output                  */
  QAT_ERR_SCRATCH = 9    /* the problem exceeds the static scratch of the no-allocation
                            entry point (qat_noalloc_max_weights)                          */
};

/* Text of a status code (static storage). */
const char* qat_status_string(int32_t status);

/* HIP error text of the last QAT_ERR_HIP on the calling thread ("" if none). */
const char* qat_last_error(void);

/*
 * a1. Per-group min-max init (modelfoundations.com note, Phase 1):
 *   for each row o and group j of W:
 *     d = fl32(max - min);  s = max(fl32(d / K), fl32(1e-5));  z = rint(fl32(-min / s)).
 * W [out, in] fp32 in; s, z [out, G] fp32 out (z is integer valued).
 */
int32_t qat_init_minmax(const float* W, int64_t out, int64_t in, int32_t group, int32_t bits,
                        float* s, float* z, hipStream_t stream);

/*
 * a2+a3 as a standalone export (Paper-Notes, Eq. 1 and Eq. 2):
 *   zr = clamp(rint(z), 0, K); u = fl32(W / s); q = clamp(rint(u) + zr, 0, K);
 *   codes = q (uint8, [out, in]); W_hat = bf16(fl32((q - zr) * s)) ([out, in]).
 * Either output may be NULL (not both).
 */
int32_t qat_quant_codes(const float* W, const float* s, const float* z, int64_t out, int64_t in,
                        int32_t group, int32_t bits, uint8_t* codes, uint16_t* W_hat,
                        hipStream_t stream);

/* Workspace bytes that qat_fakequant_linear_fwd / _bwd need for these sizes: one bf16 W_hat
 * [out, in] (rounded up to 256 bytes); the same at every bit width. 0 for invalid sizes. */
size_t qat_fakequant_ws_bytes(int64_t out, int64_t in, int32_t bits);

/*
 * a2-a4. Fake-quantised linear forward: Y = X * W_hat^T, with W_hat from
 * W, s, z exactly as in qat_quant_codes (the zero point is rounded and clamped
 * straight-through, as the "Paper vs. code" section of the modelfoundations.com
 * note describes). X [M, in] bf16, Y [M, out] bf16; fp32 accumulation.
 * ws: NULL selects the fused kernel that quantises fp32 W tiles directly into
 * LDS (no workspace; the quantiser runs once per 256-token tile, VALU-bound);
 * otherwise >= qat_fakequant_ws_bytes(out, in, bits) bytes of device memory that
 * receive a bf16 W_hat staged once per call and read by the GEMM. After the
 * call the workspace holds that W_hat, [out, in] row-major from its first
 * byte: the tensor a training step saves for its backward
 * (qat_fakequant_linear_bwd_saved).
 */
int32_t qat_fakequant_linear_fwd(const uint16_t* X, const float* W, const float* s, const float* z,
                                 int64_t M, int64_t out, int64_t in, int32_t group, int32_t bits,
                                 uint16_t* Y, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid allocation): the forward of
 * qat_fakequant_linear_fwd with a workspace, bit-identical to it, whose W_hat
 * is staged in a static device array of qat_noalloc_max_weights() bf16 values
 * (48 Mi, 96 MiB) that the library holds on each GPU it runs on until the
 * process ends. Allocates nothing. Returns QAT_ERR_SCRATCH when out * in
 * exceeds that maximum (nothing enqueued), and QAT_ERR_HIP if the array's
 * device address cannot be looked up. Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be ordered by the caller. The array keeps the last
 * call's W_hat; nothing in it has to start at zero.
 */
int64_t qat_noalloc_max_weights(void);
int32_t qat_fakequant_linear_fwd_noalloc(const uint16_t* X, const float* W, const float* s, const float* z,
                                         int64_t M, int64_t out, int64_t in, int32_t group, int32_t bits,
                                         uint16_t* Y, hipStream_t stream);

/*
 * a5-a7. Straight-through backward (paperlayer.ai summary, Appendix A; the
 * gradient formulas follow from Eq. 1-2 with identity derivative for round):
 *   dX = dY * W_hat                                  [M, in]  bf16
 *   Gw = dY^T * X;  m = [0 <= rint(u) + zr <= K]
 *   dW = Gw * m                                      [out, in] fp32
 *   ds[o,j] = sum_{i in j} Gw[o,i] * (m_i ? rint(u_i) - u_i : q_i - zr)
 *   dz[o,j] = -s[o,j] * sum_{i in j, m_i = 0} Gw[o,i]  [out, G] fp32
 * Any of dX, dW, ds, dz may be NULL to skip it (ds and dz come together: both
 * NULL or both set). ws, when dX is wanted: NULL recomputes W_hat from W, s,
 * z inside the dX GEMM (W's rows quantised straight into LDS, no workspace);
 * otherwise >= qat_fakequant_ws_bytes(out, in, bits) bytes of scratch that
 * receive the bf16 W_hat transposed, [in][out], so that the dX GEMM reads
 * both operands K-contiguous. Both give the same dX bit for bit. ws is unused
 * when dX is NULL. dY and X are read in place (the dW GEMM contracts over
 * tokens reading both with LDS transpose loads), so no transposed copies are
 * made.
 */
int32_t qat_fakequant_linear_bwd(const uint16_t* dY, const uint16_t* X, const float* W,
                                 const float* s, const float* z, int64_t M, int64_t out, int64_t in,
                                 int32_t group, int32_t bits, uint16_t* dX, float* dW, float* ds,
                                 float* dz, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The same backward on the W_hat its forward staged (what autograd saves for
 * dX = dY * W_hat): w_hat, bf16 [out, in], is the workspace of a
 * qat_fakequant_linear_fwd call on the same W, s, z (or qat_quant_codes'
 * W_hat), read in place by the dX GEMM; nothing is staged and no workspace is
 * needed. w_hat is required when dX is wanted (else it may be NULL) and must
 * not overlap an output. Results are those of qat_fakequant_linear_bwd.
 */
int32_t qat_fakequant_linear_bwd_saved(const uint16_t* dY, const uint16_t* X, const float* W,
                                       const float* s, const float* z, const uint16_t* w_hat, int64_t M,
                                       int64_t out, int64_t in, int32_t group, int32_t bits, uint16_t* dX,
                                       float* dW, float* ds, float* dz, hipStream_t stream);

/*
 * a8. Pack (modelfoundations.com note: a trained block is quantised in place;
 * zero points are hard-rounded at pack time): zp = clamp(rint(z), 0, K),
 * codes as in qat_quant_codes with zp, written as a per-row LSB-first
 * bitstream: code i occupies bits [N*i, N*i+N) of the row; row stride in*N/8
 * bytes. Wq [out, in*N/8] uint8 out; z_round [out, G] fp32 out (may be NULL).
 */
int32_t qat_pack(const float* W, const float* s, const float* z, int64_t out, int64_t in,
                 int32_t group, int32_t bits, uint8_t* Wq, float* z_round, hipStream_t stream);

/* Workspace bytes that qat_dequant_gemm_fwd / _bwd_s need: one bf16 W_hat [out, in]
 * (rounded up to 256 bytes); 0 for invalid sizes. */
size_t qat_dequant_ws_bytes(int64_t out, int64_t in, int32_t bits);

/*
 * a9. E2E-QP forward (modelfoundations.com note, Phase 2; Paper-Notes, E2E-QP):
 * W_hat = bf16(fl32((q - z) * s)) with q unpacked from Wq and z used as stored
 * (frozen, integer valued); Y = X * W_hat^T.
 * ws: NULL selects the fused kernel that dequantises packed codes straight
 * into LDS inside the GEMM (no workspace; the dequantisation runs once per
 * 128- or 256-token tile); otherwise >= qat_dequant_ws_bytes(out, in, bits)
 * bytes that receive the bf16 W_hat, staged once per call; after the call the
 * workspace holds it, [out, in] row-major from its first byte
 * (qat_dequant_gemm_bwd_s_saved reads it).
 */
int32_t qat_dequant_gemm_fwd(const uint16_t* X, const uint8_t* Wq, const float* s, const float* z,
                             int64_t M, int64_t out, int64_t in, int32_t group, int32_t bits,
                             uint16_t* Y, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * a10. E2E-QP backward with the exact scale gradient dW_hat/ds = q - z:
 *   dX = dY * W_hat (may be NULL);
 *   ds[o,j] = sum_{i in j} Gw[o,i] * (q_i - z[o,j]),  Gw = dY^T X (never stored);
 *   dz[o,j] = -s[o,j] * sum_{i in j} Gw[o,i]  (the train-s-and-z variant of the
 *   Paper-Notes ablation table; may be NULL).
 * ws, when dX is wanted: NULL dequantises the packed codes inside the dX
 * GEMM (straight into LDS, no workspace); otherwise >= qat_dequant_ws_bytes(
 * out, in, bits) bytes of scratch that receive the dequantised bf16 W_hat
 * transposed, [in][out]. Both give the same dX bit for bit. ws is unused when
 * dX is NULL.
 */
int32_t qat_dequant_gemm_bwd_s(const uint16_t* dY, const uint16_t* X, const uint8_t* Wq,
                               const float* s, const float* z, int64_t M, int64_t out, int64_t in,
                               int32_t group, int32_t bits, uint16_t* dX, float* ds, float* dz,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The same backward on the W_hat its forward staged: w_hat, bf16 [out, in],
 * is the workspace of a qat_dequant_gemm_fwd call on the same Wq, s, z, read
 * in place by the dX GEMM (required when dX is wanted, else it may be NULL;
 * must not overlap an output). Results are those of qat_dequant_gemm_bwd_s.
 */
int32_t qat_dequant_gemm_bwd_s_saved(const uint16_t* dY, const uint16_t* X, const uint8_t* Wq,
                                     const float* s, const float* z, const uint16_t* w_hat, int64_t M,
                                     int64_t out, int64_t in, int32_t group, int32_t bits, uint16_t* dX,
                                     float* ds, float* dz, hipStream_t stream);

/*
 * Deployment format (paperlayer.ai summary of EfficientQAT, Appendix D: each
 * group of g weights shares an FP16 step size and an N-bit zero point).
 * From fp32 s, z [out, G] (G = in / group):
 *   s16[o][j] = fp16(s[o][j]), round to nearest even (beyond the fp16 range:
 *               infinity), [out, G] uint16 bit patterns;
 *   zq         = clamp(rint(z), 0, K) as N-bit fields of an LSB-first bitstream
 *               per row, field j in bits [N j, N j + N), row stride
 *               qat_deploy_zq_stride(in, group, bits) = ceil(G N / 8) bytes,
 *               padding bits zero.
 * The codes stay qat_pack's Wq. Outputs are caller-owned device memory; same
 * checks and status codes as the other calls (out may be any row count).
 */
int64_t qat_deploy_zq_stride(int64_t in, int32_t group, int32_t bits);
int32_t qat_deploy_qparams(const float* s, const float* z, int64_t out, int64_t in, int32_t group,
                           int32_t bits, uint16_t* s16, uint8_t* zq, hipStream_t stream);

/*
 * The deployed model's linear layer (summary, Appendix A and section 4: the
 * INT2 model's linear-layer matrix-vector product, against the FP16 linear):
 *   Y[m][o] = fp16( sum_k X[m][k] * W_hat[o][k] ),  W_hat[o][k] = fp16((q - z) s16)
 * with q from Wq [out, in N / 8], s16 and zq as above, X fp16 [M, in], Y fp16
 * [M, out] (16-bit patterns), fp32 accumulation, one rounding to fp16 at the
 * end. 1 <= M <= 16 (QAT_ERR_SHAPE otherwise; larger batches are GEMMs); out
 * may be any row count. No workspace; the call allocates nothing. Needs
 * |s16| * 2^N below the fp16 range (any trained step size is far below).
 */
int32_t qat_deploy_gemv(const uint16_t* X, const uint8_t* Wq, const uint16_t* s16, const uint8_t* zq,
                        int64_t M, int64_t out, int64_t in, int32_t group, int32_t bits, uint16_t* Y,
                        hipStream_t stream);

/*
 * Kernel timing, for benchmarks. qat_timing_enable(1) clears earlier records
 * and starts bracketing every kernel the library launches with two HIP events
 * on its stream; qat_timing_enable(0) stops. qat_timing_count() waits for the
 * recorded events and returns the number of distinct kernel labels (or
 * -QAT_ERR_HIP); qat_timing_get(i, ...) returns label i (copied into `label`,
 * truncated to label_len), its summed elapsed milliseconds and its launch
 * count. Timing adds one event pair per launch; off, it costs nothing.
 * qat_timing_select(label) restricts the events to launches of that kernel
 * label (NULL: every launch), so one kernel can be timed inside a run of
 * the whole path at the cost of its own event pairs only.
 */
int32_t qat_timing_enable(int32_t on);
int32_t qat_timing_select(const char* label);
int32_t qat_timing_count(void);
int32_t qat_timing_get(int32_t i, char* label, size_t label_len, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* QAT_H */
