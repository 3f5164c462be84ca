// Internal launchers of the gfx950 kernels (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qat {

// ---- HBM-bound kernels (qat_elementwise.hip) ----
void launch_init_minmax(const float* W, int64_t out, int64_t in, int bits, float* s, float* z,
                        hipStream_t st);
void launch_quant_codes(const float* W, const float* s, const float* z, int64_t out, int64_t in,
                        int bits, uint8_t* codes, uint16_t* w_hat, hipStream_t st);
void launch_pack(const float* W, const float* s, const float* z, int64_t out, int64_t in, int bits,
                 uint8_t* Wq, float* zround, hipStream_t st);
void launch_quant_t(const float* W, const float* s, const float* z, int64_t out, int64_t in, int bits,
                    uint16_t* Wt, hipStream_t st);
void launch_dequant_t(const uint8_t* Wq, const float* s, const float* z, int64_t out, int64_t in,
                      int bits, uint16_t* Wt, hipStream_t st);
void launch_transpose_bf16(const uint16_t* src, int64_t R, int64_t C, uint16_t* dst, int64_t Rp,
                           hipStream_t st);

// ---- MFMA GEMMs (qat_gemm.hip) ----
// All compute C[M, N] = sum_k A[m, k] * B[n, k] with A bf16 [M][lda] K-contiguous and
// K % 64 == 0; they differ in where B comes from and what the epilogue does.
struct GemmArgs {
  const uint16_t* A;
  int64_t lda;
  const void* B;       // bf16 [N][ldb], fp32 W [N][ldb] or packed codes [N][ldb bytes]
  int64_t ldb;
  int M, N, K;
  const float* s;      // [N-or-M rows][G] step sizes (fused loaders / epilogues)
  const float* z;
  int64_t G;           // groups per weight row
  float Kq;            // 2^bits - 1
  uint16_t* C;         // bf16 output [M][ldc]
  int64_t ldc;
  const float* W;      // fp32 master weight [M][ldw] for the straight-through epilogue
  int64_t ldw;
  const uint8_t* Wq;   // packed codes [M][ldq bytes] for the E2E epilogue
  int64_t ldq;
  float* dW;           // [M][ldw] fp32, may be null
  float* ds;           // [M][G]
  float* dz;           // [M][G], may be null for E2E
};

enum BLoad { kBf16 = 0, kFp32Quant = 1, kPacked = 2 };
enum Epi { kStoreBf16 = 0, kSteGrads = 1, kE2eScaleGrad = 2 };

// Y = X W_hat^T style (bf16 output). bload selects the B source; bits used by fused loaders.
void launch_gemm_bf16_out(const GemmArgs& a, int bload, int bits, hipStream_t st);
// Straight-through gradient GEMM: rows = out, cols = in, epilogue writes dW, ds, dz.
void launch_gemm_ste_grads(const GemmArgs& a, hipStream_t st);
// E2E scale-gradient GEMM: rows = out, cols = in, epilogue writes ds (and dz).
void launch_gemm_e2e_grads(const GemmArgs& a, int bits, hipStream_t st);

}  // namespace qat
