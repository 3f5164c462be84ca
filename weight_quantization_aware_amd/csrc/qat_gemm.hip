// Tile choice and launches of the MFMA GEMMs (kernels in qat_gemm_kernel.h).
//
// bf16 operands (k_gemm, BK = 64), measured on the Llama-2 shapes of this path:
//   256x256, 2 stages   outputs of >= 256 such tiles (one per CU or more):
//                       gradient GEMMs, MLP- and 70B-sized forwards; 8 waves
//                       (two per SIMD) up to K = 4096, 4 waves beyond
//   128x256, 3 stages   about one 128x256 tile per CU (2048-token q_proj);
//                       8 waves
//   128x128, 4 stages   small problems; 4 waves
// Fused B operands (k_gemm_fused) go through an LDS ring beside the bf16
// stages: packed codes (E2E-QP forward without workspace) with 256-row B tiles,
// BK = 32, 4 stages; the fp32 master weight (fake-quant forward without
// workspace) with 128-row B tiles, BK = 32, 3 stages.
#include "qat_gemm_kernel.h"

namespace qat {

namespace {

int64_t tiles(const GemmArgs& a, int bm, int bn) {
  return (int64_t)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
}

// With the store epilogues the NB template argument only tags the launch: 0
// the forward, 1 the dX GEMM, 5 the products of attention (same code,
// distinct kernel symbols so that profiles can tell them apart).
constexpr int kTagAttn = 5;
template <int BL, int EP, int NB>
constexpr const char* gemm_label() {
  if (EP == kSteGrads) return "gemm_ste_grads";
  if (EP == kSteAdam) return "gemm_ste_grads_adamw";
  if (EP == kE2eScaleGrad) return "gemm_e2e_grads";
  if (BL == kFp32Quant) return "gemm_fwd_fused_fp32";
  if (BL == kPacked) return "gemm_fwd_packed";
  if (EP == kResidMse) return "gemm_fwd_mse";
  if (NB == kTagAttn) return "attn_gemm_bf16";
  if (EP == kStoreF32) return "gemm_fwd_f32";
  return NB == 1 ? "gemm_dx" : "gemm_fwd";
}

int batches(const GemmArgs& a) { return a.batch_h > 0 ? a.batches : 1; }

template <int BM, int BN, int S, int WGM, int WGN, int AMN, int BMN, int EP, int NB, int GM = 0>
void launch_bf16(const GemmArgs& a, hipStream_t st) {
  LaunchTimer t(gemm_label<kBf16, EP, NB>(), st);
  hipLaunchKernelGGL((k_gemm<BM, BN, 64, S, WGM, WGN, GM, AMN, BMN, EP, NB>),
                     dim3((unsigned)tiles(a, BM, BN), (unsigned)batches(a)), dim3(64 * WGM * WGN), 0, st, a);
}

template <int BM, int BN, int BK, int S, int BL, int NB>
void launch_fused(const GemmArgs& a, hipStream_t st) {
  LaunchTimer t(gemm_label<BL, kStoreBf16, NB>(), st);
  hipLaunchKernelGGL((k_gemm_fused<BM, BN, BK, S, 0, BL, NB>), dim3((unsigned)tiles(a, BM, BN)), dim3(256), 0,
                     st, a);
}

// Returns the number of workgroups launched.
template <int AMN, int BMN, int EP, int NB>
int64_t launch_pick(const GemmArgs& a, hipStream_t st) {
  if (tiles(a, 256, 256) >= 256) {
    if (a.K <= 4096) launch_bf16<256, 256, 2, 2, 4, AMN, BMN, EP, NB>(a, st);
    else launch_bf16<256, 256, 2, 2, 2, AMN, BMN, EP, NB>(a, st);
    return tiles(a, 256, 256);
  } else if (tiles(a, 128, 256) >= 192) {
    launch_bf16<128, 256, 3, 2, 4, AMN, BMN, EP, NB>(a, st);
    return tiles(a, 128, 256);
  } else {
    launch_bf16<128, 128, 4, 2, 2, AMN, BMN, EP, NB>(a, st);
    return tiles(a, 128, 128);
  }
}

// Gradient GEMMs for groups other than 64: two tile configurations. Groups
// of 32 (GM 1) and groups that tile BN (GM 2: 128, or a short whole row) are
// stored directly; whole rows wider than BN (GM 3) are accumulated per tile
// into ds and dz, zero-filled here first.
template <int EP, int NB, int GM>
void launch_pick_grads_gm(const GemmArgs& a, hipStream_t st) {
  if (tiles(a, 256, 256) >= 256) launch_bf16<256, 256, 2, 2, 4, kMNContig, kMNContig, EP, NB, GM>(a, st);
  else launch_bf16<128, 128, 4, 2, 2, kMNContig, kMNContig, EP, NB, GM>(a, st);
}

// The weight-updating epilogue streams whole 256-column tile rows (groups of
// 32 to 256 columns that divide 256): always 256x256 tiles on 8 waves, also
// for problems of fewer tiles than CUs.
void launch_grads_adam(const GemmArgs& a, hipStream_t st) {
  launch_bf16<256, 256, 2, 2, 4, kMNContig, kMNContig, kSteAdam, 0, 0>(a, st);
}

template <int EP, int NB>
void launch_grads(const GemmArgs& a, hipStream_t st) {
  if (a.group == 64) {
    launch_pick<kMNContig, kMNContig, EP, NB>(a, st);
  } else if (a.group == 32) {
    launch_pick_grads_gm<EP, NB, 1>(a, st);
  } else {
    const int bn = tiles(a, 256, 256) >= 256 ? 256 : 128;
    if (bn % a.group == 0) {
      launch_pick_grads_gm<EP, NB, 2>(a, st);
    } else {
      const int64_t n = (int64_t)a.M * a.G;
      if (a.ds) launch_fill_zero(a.ds, n, st);
      if (a.dz) launch_fill_zero(a.dz, n, st);
      launch_pick_grads_gm<EP, NB, 3>(a, st);
    }
  }
}

template <int BL, int NB>
void launch_pick_fused(const GemmArgs& a, hipStream_t st) {
  if constexpr (BL == kPacked) {
    if (tiles(a, 256, 256) >= 256) launch_fused<256, 256, 32, 4, BL, NB>(a, st);
    else launch_fused<128, 256, 32, 4, BL, NB>(a, st);
  } else {
    if (tiles(a, 256, 128) >= 256) launch_fused<256, 128, 32, 3, BL, NB>(a, st);
    else launch_fused<128, 128, 32, 3, BL, NB>(a, st);
  }
}

}  // namespace

void launch_gemm_fwd(const GemmArgs& a, int bload, int bits, hipStream_t st) {
  if (bload == kBf16) launch_pick<kKContig, kKContig, kStoreBf16, 0>(a, st);
  else if (bload == kFp32Quant) launch_pick_fused<kFp32Quant, 0>(a, st);
  else if (bits == 2) launch_pick_fused<kPacked, 2>(a, st);
  else if (bits == 3) launch_pick_fused<kPacked, 3>(a, st);
  else launch_pick_fused<kPacked, 4>(a, st);
}

void launch_gemm_fwd_f32(const GemmArgs& a, hipStream_t st) {
  launch_pick<kKContig, kKContig, kStoreF32, 0>(a, st);
}

// The dQ product of attention (N = head size 128): 128x128 tiles.
void launch_gemm_attn(const GemmArgs& a, hipStream_t st) {
  launch_bf16<128, 128, 4, 2, 2, kMNContig, kMNContig, kStoreBf16, kTagAttn>(a, st);
}

void launch_gemm_dx(const GemmArgs& a, hipStream_t st) {
  launch_pick<kKContig, kKContig, kStoreBf16, 1>(a, st);
}

// W_hat read in place costs the same as a staged W_hat^T on the Llama-2-7B
// block's shapes (4096 tokens) and 4% more at 2048 tokens (128x256 tiles);
// 8 waves also beyond K = 4096 (measured faster with this loader at
// K = 11008).
void launch_gemm_dx_mn(const GemmArgs& a, hipStream_t st) {
  if (tiles(a, 256, 256) >= 256) launch_bf16<256, 256, 2, 2, 4, kKContig, kMNContig, kStoreBf16, 1>(a, st);
  else if (tiles(a, 128, 256) >= 192) launch_bf16<128, 256, 3, 2, 4, kKContig, kMNContig, kStoreBf16, 1>(a, st);
  else launch_bf16<128, 128, 4, 2, 2, kKContig, kMNContig, kStoreBf16, 1>(a, st);
}

int64_t launch_gemm_fwd_mse(const GemmArgs& a, hipStream_t st) {
  return launch_pick<kKContig, kKContig, kResidMse, 0>(a, st);
}

int64_t gemm_fwd_max_workgroups(int64_t M, int64_t N) { return ((M + 127) / 128) * ((N + 127) / 128); }

void launch_gemm_grads(const GemmArgs& a, int epi, int bits, hipStream_t st) {
  if (epi == kSteGrads) launch_grads<kSteGrads, 0>(a, st);
  else if (epi == kSteAdam) launch_grads_adam(a, st);
  else if (bits == 2) launch_grads<kE2eScaleGrad, 2>(a, st);
  else if (bits == 3) launch_grads<kE2eScaleGrad, 3>(a, st);
  else launch_grads<kE2eScaleGrad, 4>(a, st);
}

}  // namespace qat
