// Tile choice and launches of the MFMA GEMM (kernel template in qat_gemm_kernel.h).
//
// Configurations (measured on the Llama-2 shapes of this path):
//   A  256x256, BK 32, 4 stages   large outputs (>= 256 tiles): gradient GEMMs,
//                                 MLP-sized and 70B-sized forwards
//   B  128x256, BK 64, 3 stages   about one tile per CU at 128x256
//   C  128x128, BK 64, 4 stages   small problems
// Fused B operands go through an LDS ring beside the bf16 stages: packed codes
// (E2E-QP forward) with 256-row B tiles, BK = 32, 4 stages; the fp32 master
// weight (forward without workspace) with 128-row B tiles, BK = 32, 3 stages.
#include "qat_gemm_kernel.h"

namespace qat {

namespace {

int64_t tiles(const GemmArgs& a, int bm, int bn) {
  return (int64_t)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
}

template <int BL, int EP>
constexpr const char* gemm_label(bool mn_b) {
  if (EP == kSteGrads) return "gemm_ste_grads";
  if (EP == kE2eScaleGrad) return "gemm_e2e_grads";
  if (BL == kFp32Quant) return "gemm_fwd_fused_fp32";
  if (BL == kPacked) return "gemm_fwd_packed";
  return mn_b ? "gemm_dx" : "gemm_fwd";
}

template <int BM, int BN, int BK, int S, int AMN, int BMN, int BL, int EP, int NB>
void launch_cfg(const GemmArgs& a, hipStream_t st) {
  LaunchTimer t(gemm_label<BL, EP>(BMN == kMNContig), st);
  hipLaunchKernelGGL((k_gemm<BM, BN, BK, S, 0, AMN, BMN, BL, EP, NB>), dim3((unsigned)tiles(a, BM, BN)),
                     dim3(256), 0, st, a);
}

template <int AMN, int BMN, int BL, int EP, int NB>
void launch_pick(const GemmArgs& a, hipStream_t st) {
  if constexpr (BL == kBf16) {
    if (tiles(a, 256, 256) >= 256) launch_cfg<256, 256, 32, 4, AMN, BMN, BL, EP, NB>(a, st);
    else if (tiles(a, 128, 256) >= 192) launch_cfg<128, 256, 64, 3, AMN, BMN, BL, EP, NB>(a, st);
    else launch_cfg<128, 128, 64, 4, AMN, BMN, BL, EP, NB>(a, st);
  } else if constexpr (BL == kPacked) {
    if (tiles(a, 256, 256) >= 256) launch_cfg<256, 256, 32, 4, AMN, BMN, BL, EP, NB>(a, st);
    else launch_cfg<128, 256, 32, 4, AMN, BMN, BL, EP, NB>(a, st);
  } else {
    if (tiles(a, 256, 128) >= 256) launch_cfg<256, 128, 32, 3, AMN, BMN, BL, EP, NB>(a, st);
    else launch_cfg<128, 128, 32, 3, AMN, BMN, BL, EP, NB>(a, st);
  }
}

}  // namespace

void launch_gemm_fwd(const GemmArgs& a, int bload, int bits, hipStream_t st) {
  if (bload == kBf16) launch_pick<kKContig, kKContig, kBf16, kStoreBf16, 0>(a, st);
  else if (bload == kFp32Quant) launch_pick<kKContig, kKContig, kFp32Quant, kStoreBf16, 0>(a, st);
  else if (bits == 2) launch_pick<kKContig, kKContig, kPacked, kStoreBf16, 2>(a, st);
  else if (bits == 3) launch_pick<kKContig, kKContig, kPacked, kStoreBf16, 3>(a, st);
  else launch_pick<kKContig, kKContig, kPacked, kStoreBf16, 4>(a, st);
}

void launch_gemm_dx(const GemmArgs& a, hipStream_t st) {
  launch_pick<kKContig, kMNContig, kBf16, kStoreBf16, 0>(a, st);
}

void launch_gemm_grads(const GemmArgs& a, int epi, int bits, hipStream_t st) {
  if (epi == kSteGrads) launch_pick<kMNContig, kMNContig, kBf16, kSteGrads, 0>(a, st);
  else if (bits == 2) launch_pick<kMNContig, kMNContig, kBf16, kE2eScaleGrad, 2>(a, st);
  else if (bits == 3) launch_pick<kMNContig, kMNContig, kBf16, kE2eScaleGrad, 3>(a, st);
  else launch_pick<kMNContig, kMNContig, kBf16, kE2eScaleGrad, 4>(a, st);
}

}  // namespace qat
