// Internal launchers of the gfx950 kernels (not part of the C ABI).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qat {

// Names the kernel launched in its scope (by QAT_LAUNCH) for the library's
// timing (qat_timing_enable): while timing is on for this label it holds two
// HIP events that the launch binds to its own dispatch, so they time the
// kernel from its start to its end without adding packets to the stream; a
// single branch otherwise.
class LaunchTimer {
 public:
  LaunchTimer(const char* label, hipStream_t st);
  ~LaunchTimer();

 private:
  const char* label_;
  void* start_ = nullptr;
  void* stop_ = nullptr;
};

// The events of the innermost LaunchTimer of the calling thread that no launch
// has taken yet (both null if none), for the next launch.
void timing_events(hipEvent_t* start, hipEvent_t* stop);

}  // namespace qat

// hipLaunchKernelGGL's arguments; the launch carries the scope's timing events.
#define QAT_LAUNCH(kernel, grid, block, shmem, stream, ...)                                      \
  do {                                                                                           \
    hipEvent_t qat_e0_ = nullptr, qat_e1_ = nullptr;                                             \
    qat::timing_events(&qat_e0_, &qat_e1_);                                                      \
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, qat_e0_, qat_e1_, 0, __VA_ARGS__); \
  } while (0)

namespace qat {

// Status of the launches a C-ABI call has just enqueued: QAT_OK, or QAT_ERR_HIP
// with the HIP error text kept for qat_last_error (qat_api.hip).
int32_t finish_call();

// ---- HBM-bound kernels (qat_elementwise.hip) ----
// `group` is 32, 64, 128 or in (channel-wise); in % group == 0.
void launch_init_minmax(const float* W, int64_t out, int64_t in, int group, int bits, float* s, float* z,
                        hipStream_t st);
void launch_quant_codes(const float* W, const float* s, const float* z, int64_t out, int64_t in, int group,
                        int bits, uint8_t* codes, uint16_t* w_hat, hipStream_t st);
void launch_pack(const float* W, const float* s, const float* z, int64_t out, int64_t in, int group, int bits,
                 uint8_t* Wq, float* zround, hipStream_t st);
void launch_dequant(const uint8_t* Wq, const float* s, const float* z, int64_t out, int64_t in, int group,
                    int bits, uint16_t* w_hat, hipStream_t st);
// W_hat^T [in][out] bf16 for the dX GEMM (needs out % 64 == 0): from the fp32
// master weight (fake-quant) or from packed codes (E2E-QP).
void launch_w_hat_t(const float* W, const float* s, const float* z, int64_t out, int64_t in, int group,
                    int bits, uint16_t* w_hat_t, hipStream_t st);
void launch_dequant_t(const uint8_t* Wq, const float* s, const float* z, int64_t out, int64_t in, int group,
                      int bits, uint16_t* w_hat_t, hipStream_t st);
// p[0 .. n) = 0 with a plain store kernel (usable under stream capture).
void launch_fill_zero(float* p, int64_t n, hipStream_t st);

// ---- Deployment format and the inference linear (qat_deploy.hip) ----
// s16 = fp16(s) [out][G]; zq = N-bit clamp(rint(z), 0, K), LSB-first per row,
// row stride ceil(G*N/8) bytes.
void launch_deploy_qparams(const float* s, const float* z, int64_t out, int64_t in, int group, int bits,
                           uint16_t* s16, uint8_t* zq, hipStream_t st);
// Y[M][out] fp16 = X[M][in] fp16 times fp16((q - z) s16)^T, M <= 16.
void launch_deploy_gemv(const uint16_t* X, const uint8_t* Wq, const uint16_t* s16, const uint8_t* zq, int64_t M,
                        int64_t out, int64_t in, int group, int bits, uint16_t* Y, hipStream_t st);

// ---- MFMA GEMMs (qat_gemm.hip) ----
// C[M, N] = sum_k A[m, k] * B[n, k] in bf16 with fp32 accumulation. Each operand
// is either K-contiguous ([rows][ld], ld >= K) or MN-contiguous ([K][ld] with
// the operand's rows contiguous). K-contiguous operands need K % 64 == 0;
// with MN-contiguous operands K may be ragged (k beyond K reads as zero).
struct GemmArgs {
  const uint16_t* A;
  int64_t lda;
  const void* B;       // bf16 rows, fp32 master weight [N][ldb], or packed codes [N][ldb bytes]
  int64_t ldb;
  int M, N, K;
  const float* s;      // [weight rows][G] step sizes (fused loaders / epilogues)
  const float* z;
  int64_t G;           // groups per weight row
  int group;           // elements per group: 32, 64, 128, or the row length (channel-wise)
  float Kq;            // 2^bits - 1
  uint16_t* C;         // bf16 output [M][ldc]
  int64_t ldc;
  const float* W;      // fp32 master weight [M][ldw] for the straight-through epilogue
  int64_t ldw;
  const uint8_t* Wq;   // packed codes [M][ldq bytes] for the E2E epilogue
  int64_t ldq;
  float* dW;           // [M][ldw] fp32, may be null
  float* ds;           // [M][G], may be null
  float* dz;           // [M][G], may be null
  float* Cf;           // fp32 output [M][ldc] (kStoreF32)
  // Batched products (plain bf16 loads and the store epilogues only): with
  // batch_h > 0 the grid's y index z = b * batch_h + h selects the problem
  // whose A, B and C start at b * s?_b + h * s?_h elements from the given
  // pointers (the per-(sequence, head) products of attention).
  int batch_h;
  int batches;
  int64_t sa_b, sa_h, sb_b, sb_h, sc_b, sc_h;
  // Causal structure of attention products (rows m and the contraction index
  // k are token positions of one sequence): 0 none; kCausalLower: k runs over
  // [0, end of the row tile).
  int causal;
  // kSteAdam: AdamW on the weight in the straight-through epilogue. W (the
  // same array as the const W above) and its moments mW, vW are updated in
  // place from the masked gradient; dW is still stored when non-null.
  float* Wupd;
  float* mW;
  float* vW;
  float adam_b1, adam_b2, adam_isbc2, adam_eps, adam_step, adam_decay;
  // kResidMse: the scale of the loss gradient (2 / n).
  float escale;
  // kResidMse: y = resid + product (fp32, [M][ldc]; stored to Cf when
  // non-null), d = y - target (bf16 target), C = bf16(escale d), and one fp32
  // partial of sum d^2 per workgroup at partial[blockIdx.x].
  const float* resid;
  const uint16_t* target;
  float* partial;
};

enum Causal { kCausalNone = 0, kCausalLower = 1 };

enum BLoad { kBf16 = 0, kFp32Quant = 1, kPacked = 2 };
enum Epi { kStoreBf16 = 0, kSteGrads = 1, kE2eScaleGrad = 2, kStoreF32 = 3, kSteAdam = 4, kResidMse = 5 };
// Operand layouts of the GEMM: K-contiguous ([rows][ld]) or MN-contiguous
// ([K][ld], the operand's rows contiguous); the D variants load by 4-byte DMA
// for rows that are only 4-byte aligned (kKContigD also zero-fills the
// contraction's tail per lane).
enum Layout { kKContig = 0, kMNContig = 1, kKContigD = 2, kMNContigD = 3 };

// Forward-type GEMM with bf16 output: Y = X W_hat^T. bload selects the B source.
void launch_gemm_fwd(const GemmArgs& a, int bload, int bits, hipStream_t st);
// dX = dY W_hat: A = dY [M][out], B = W_hat^T [in][out], both K-contiguous.
void launch_gemm_dx(const GemmArgs& a, hipStream_t st);
// The same product on W_hat [out][in] read in place (B MN-contiguous, ldb = in).
void launch_gemm_dx_mn(const GemmArgs& a, hipStream_t st);
// The same product with W_hat made in LDS from the weight itself (no
// workspace): bload kFp32Quant (a.B the fp32 master weight [out][ldb]) or
// kPacked (a.B the packed codes, ldb bytes per row); a.s, a.z, a.G, a.group,
// a.Kq as for the fused forward; K = out must be a multiple of 32.
void launch_gemm_dx_fused(const GemmArgs& a, int bload, int bits, hipStream_t st);
// The forward product (K-contiguous operands) with the kResidMse epilogue;
// returns the number of workgroups launched (one loss partial each), at most
// gemm_fwd_max_workgroups(M, N).
int64_t launch_gemm_fwd_mse(const GemmArgs& a, hipStream_t st);
int64_t gemm_fwd_max_workgroups(int64_t M, int64_t N);
// Gradient GEMM over tokens, Gw = dY^T X with both operands MN-contiguous;
// epi = kSteGrads (dW, ds, dz), kSteAdam (the same, and AdamW on W, m, v in
// place; groups of 32 to 256 that divide 256) or kE2eScaleGrad (ds, dz).
void launch_gemm_grads(const GemmArgs& a, int epi, int bits, hipStream_t st);
// Forward-type GEMM on a staged bf16 W_hat with fp32 output (a.Cf).
void launch_gemm_fwd_f32(const GemmArgs& a, hipStream_t st);
// The linear's backward GEMMs (argument set-up shared by the C-ABI calls and
// the block step): dX = dY W_hat from W_hat^T [in][out] bf16, and the
// gradient GEMM's arguments Gw = dY^T X over M tokens (epilogue fields W, Wq,
// dW, ds, dz left to the caller).
void launch_linear_dx(const uint16_t* dY, const uint16_t* w_hat_t, int64_t M, int64_t out, int64_t in,
                      uint16_t* dX, hipStream_t st);
void launch_linear_dx_saved(const uint16_t* dY, const uint16_t* w_hat, int64_t M, int64_t out, int64_t in,
                            uint16_t* dX, hipStream_t st);
void launch_linear_dx_fused(const uint16_t* dY, const void* B, int64_t ldb, const float* s, const float* z, int64_t M,
                            int64_t out, int64_t in, int group, int bits, uint16_t* dX, int bload, hipStream_t st);
GemmArgs linear_grads_args(const uint16_t* dY, const uint16_t* X, const float* s, const float* z, int64_t M,
                           int64_t out, int64_t in, int group, int bits);
// Fused causal attention forward (qat_attn.hip): O [B*T][H] bf16 and the
// rows' base-2 log-sum-exp lse [B*nh][T] of S / sqrt(128) from q, k, v
// [B*T][H] bf16 (head size 128, T a multiple of 64).
void launch_flash_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse, int B, int T,
                      int H, hipStream_t st);
// Fused causal attention backward for dK and dV (qat_attn.hip) from q, k, v,
// the output's gradient dO [B*T][H] bf16, the forward's lse and the row terms
// D = rowsum(dO O) [B*nh][T]; also writes dS^T [B*nh][T][T] bf16 ([key][query],
// zero above the diagonal within every 128-query tile) for the dQ product.
void launch_flash_bwd_kv(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dO,
                         const float* lse, const float* D, uint16_t* dk, uint16_t* dv, uint16_t* dsT, int B, int T,
                         int H, hipStream_t st);
// The dQ product of attention, batched (a.batches problems, a.batch_h per
// sequence): C bf16 = A B with A and B MN-contiguous (dS^T [key][query], k
// [key][d]); a.causal kCausalLower.
void launch_gemm_attn(const GemmArgs& a, hipStream_t st);

}  // namespace qat
