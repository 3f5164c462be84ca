/*
 * qat_block.h -- C ABI of one Block-AP training step on a Llama-2 decoder
 * block whose seven linears are group-wise fake-quantised (gfx950).
 *
 * Sources (page title -- section):
 *   "EfficientQAT, low-bit training on a single GPU" (modelfoundations.com),
 *   Phase 1 (Block-AP): each transformer block is trained on its own, all of
 *   its linear weights together with their step sizes and zero points, to a
 *   mean-squared error against the full-precision block's outputs; weights
 *   and quantisation parameters have their own learning rates (2e-5 and
 *   1e-4 at 2 bits), each on a cosine schedule, with AdamW; "The recipe in
 *   numbers" (2048-token samples, batch 2).
 *   paperlayer.ai summary of arXiv 2407.11062v3, Appendix A: gradients reach
 *   W, s and z through the rounding by the straight-through estimator (the
 *   linears are those of qat.h: qat_fakequant_linear_fwd / _bwd).
 *
 * The block (readings where the pages name no architecture): Llama-2's
 *   h1 = RMSNorm(x) g1;  q, k, v = fq(h1);  q, k = RoPE(q, k) (base 10000,
 *   each head's halves rotated as pairs);  A = causal softmax(q k^T /
 *   sqrt(128)) per (sequence, head);  x2 = x + fq_o(A v);
 *   h2 = RMSNorm(x2) g2;  y = x2 + fq_down(SiLU(fq_gate(h2)) * fq_up(h2));
 *   loss = mean over all elements of (y - target)^2.  RMSNorm epsilon 1e-5.
 *   fq(X) = X W_hat^T with W_hat from Eq. 1 and Eq. 2 of qat.h. Trained:
 *   W, s, z of the seven linears; g1 and g2 are frozen.
 *
 * Layouts (row-major, device pointers owned by the caller, 16-byte aligned):
 *   x, target   [batch * seq][hidden] bf16 (uint16_t bit patterns); token
 *               t of sequence b is row b * seq + t.
 *   g1, g2      [hidden] fp32.
 *   linear i (QAT_BLOCK_Q .. QAT_BLOCK_DOWN): W [out][in], s, z [out][in /
 *   group] fp32 with (out, in) = (H, H) for q, k, v, o; (I, H) for gate, up;
 *   (H, I) for down. Gradients dW, ds, dz and the AdamW moments m_*, v_*
 *   have the shapes of their parameters.
 *
 * Precision: activations that feed an MFMA are bf16 (h1, q, k, v, P, the
 *   attention output, h2, gate, up, the SiLU product and every gradient that
 *   enters a GEMM); scores, probabilities before rounding, the residual
 *   stream x2, y, the outputs of o and down, the norms' statistics and the
 *   loss are fp32; GEMMs accumulate in fp32; W_hat is rounded to bf16 as in
 *   qat.h. The optimiser works in fp32 on fp32 parameters and moments.
 *
 * Shapes: hidden H a multiple of 128, at most 8192, with H / heads == 128
 *   (Llama-2's head size); inter I a multiple of 64; seq T a multiple of 64,
 *   at most 4096; batch >= 1; bits 2..4; group 32, 64 or 128 dividing H and
 *   I. Every linear weight below 2 GiB of fp32 and batch * seq * I * 2 bytes
 *   below 2 GiB.
 *
 * Calls are asynchronous on `stream`, validate everything before the first
 * launch (nothing is enqueued on error), allocate nothing, and use only the
 * caller's workspace (qat_block_ws_bytes bytes, 256-byte aligned offsets
 * inside). Two calls that share a workspace must not overlap in time.
 * Return value: QAT_OK or a QAT_ERR_* code of qat.h.
 */
#ifndef QAT_BLOCK_H
#define QAT_BLOCK_H

#include "qat.h"

#ifdef __cplusplus
extern "C" {
#endif

enum {
  QAT_BLOCK_Q = 0,
  QAT_BLOCK_K = 1,
  QAT_BLOCK_V = 2,
  QAT_BLOCK_O = 3,
  QAT_BLOCK_GATE = 4,
  QAT_BLOCK_UP = 5,
  QAT_BLOCK_DOWN = 6,
  QAT_BLOCK_LINEARS = 7
};

typedef struct qat_block_shape {
  int64_t hidden;  /* H */
  int64_t heads;   /* attention heads, H / heads == 128 */
  int64_t inter;   /* I, the MLP width */
  int64_t seq;     /* T, tokens per sequence */
  int64_t batch;   /* B, sequences per step */
  int32_t bits;    /* N in {2, 3, 4} */
  int32_t group;   /* 32, 64 or 128 */
} qat_block_shape;

typedef struct qat_block_linear {
  float* W;        /* parameters: read by the step, then updated in place */
  float* s;
  float* z;
  float* dW;       /* this step's gradients (outputs). dW may be NULL in a step (W's update
                      then never materialises it); all three may be NULL in
                      qat_block_forward */
  float* ds;
  float* dz;
  float* m_W;      /* AdamW first and second moments (updated in place) */
  float* v_W;
  float* m_s;
  float* v_s;
  float* m_z;
  float* v_z;
} qat_block_linear;

/*
 * AdamW as in torch.optim.AdamW (decoupled weight decay p <- p (1 - lr wd);
 * m <- b1 m + (1 - b1) g; v <- b2 v + (1 - b2) g^2; p <- p - lr / (1 - b1^t)
 * * m / (sqrt(v / (1 - b2^t)) + eps), t = step + 1) with two parameter
 * groups: W at lr_weight, s and z at lr_quant, each scaled by the cosine
 * schedule of optimizer step `step` (0-based) over total_steps:
 * lr = lr0 (1 + cos(pi step / total_steps)) / 2 (computed on the host in
 * double precision).
 */
typedef struct qat_block_adamw {
  double lr_weight;
  double lr_quant;
  double beta1;
  double beta2;
  double eps;
  double weight_decay;
  int64_t step;
  int64_t total_steps;
} qat_block_adamw;

/* Workspace bytes of one step or forward at this shape (0 if the shape is invalid). */
size_t qat_block_ws_bytes(const qat_block_shape* shape);

/*
 * The block's forward and loss: y (fp32 [B*T][H], may be NULL) and *loss
 * (one fp32 in device memory). Reads the seven linears' W, s, z only.
 */
int32_t qat_block_forward(const qat_block_shape* shape, const qat_block_linear* lin, const float* g1,
                          const float* g2, const uint16_t* x, const uint16_t* target, float* y, float* loss,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * One Block-AP step: forward and loss (as qat_block_forward, before the
 * update), the straight-through backward into every linear's dW, ds, dz,
 * then AdamW on W, s, z and their moments. ds and dz are required; dW is
 * optional: W's update is made in the epilogue of its gradient product, from
 * the masked gradient in registers. lin points to QAT_BLOCK_LINEARS entries in
 * the order of the enum above.
 */
int32_t qat_block_ap_step(const qat_block_shape* shape, const qat_block_linear* lin, const float* g1,
                          const float* g2, const uint16_t* x, const uint16_t* target, const qat_block_adamw* opt,
                          float* y, float* loss, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QAT_BLOCK_H */
