// Tile choice and launches of the MFMA GEMMs (kernels in qat_gemm_kernel.h).
//
// bf16 operands (k_gemm, BK = 64), measured on the Llama-2 shapes of this path:
//   256x256, 2 stages   outputs of >= 256 such tiles (one per CU or more):
//                       gradient GEMMs, MLP- and 70B-sized forwards; 8 waves
//                       (two per SIMD) up to K = 4096, 4 waves beyond
//   128x256, 3 stages   about one 128x256 tile per CU (2048-token q_proj);
//                       8 waves
//   128x128, 4 stages   small problems; 4 waves
// Fused B operands (the fp32 master weight or packed codes turned into bf16
// W_hat in LDS by converter waves beside the MFMA waves; the calls without a
// workspace): the forward in k_gemm_fused_fwd and dX in k_gemm_fused_dx (raw
// weights through converter registers, the activations' DMA on the MFMA
// waves); 256x128 or 128x128 tiles, BK = 32.
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
template <int BL, int EP, int NB, int BT = 0>
constexpr const char* gemm_label() {
  if (BT == 1) return BL == kFp32Quant ? "gemm_dx_fused_fp32" : "gemm_dx_packed";
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
  QAT_LAUNCH((k_gemm<BM, BN, 64, S, WGM, WGN, GM, AMN, BMN, EP, NB>),
                     dim3((unsigned)tiles(a, BM, BN), (unsigned)batches(a)), dim3(64 * WGM * WGN), 0, st, a);
}

template <int BM, int BN, int BL, int NB, int ADW>
void launch_fused_dx(const GemmArgs& a, hipStream_t st) {
  LaunchTimer t(gemm_label<BL, kStoreBf16, NB, 1>(), st);
  QAT_LAUNCH((k_gemm_fused_dx<BM, BN, BL, NB, ADW>), dim3((unsigned)tiles(a, BM, BN)), dim3(512), 0, st, a);
}

// 256x256 tiles (8 waves) or 128x256 (8 waves) for a product with at least
// one round of 256x256 tiles on the 256 CUs: whichever needs less time,
// counting whole rounds of tiles. A 256x256 tile takes ~1.7x as long as a
// 128x256 one (measured at K = 4096), so the bigger tiles lose where their
// last round is mostly empty: 2048 x 11008 has 344 tiles of 256x256 (two
// rounds, the second 34% full) but 688 of 128x256 (three rounds), and ran
// 168-183 us on 256x256 tiles against 147-170 us on 128x256.
bool prefer_256x256(const GemmArgs& a) {
  const int64_t t256 = tiles(a, 256, 256), t128 = tiles(a, 128, 256);
  return t256 >= 256 && ((t256 + 255) / 256) * 17 <= ((t128 + 255) / 256) * 10;
}

// Returns the number of workgroups launched.
template <int AMN, int BMN, int EP, int NB>
int64_t launch_pick(const GemmArgs& a, hipStream_t st) {
  if (prefer_256x256(a)) {
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
template <int EP, int NB, int GM, int AL = kMNContig>
void launch_pick_grads_gm(const GemmArgs& a, hipStream_t st) {
  if (tiles(a, 256, 256) >= 256) launch_bf16<256, 256, 2, 2, 4, AL, kMNContig, EP, NB, GM>(a, st);
  else launch_bf16<128, 128, 4, 2, 2, AL, kMNContig, EP, NB, GM>(a, st);
}

// The weight-updating epilogue streams whole 256-column tile rows (groups of
// 32 to 256 columns that divide 256): always 256x256 tiles on 8 waves, also
// for problems of fewer tiles than CUs.
void launch_grads_adam(const GemmArgs& a, hipStream_t st) {
  launch_bf16<256, 256, 2, 2, 4, kMNContig, kMNContig, kSteAdam, 0, 0>(a, st);
}

// AL: the layout of A = dY^T (kMNContigD when dY's rows of `out` elements
// are not 16-byte aligned).
template <int EP, int NB, int AL>
void launch_grads_al(const GemmArgs& a, hipStream_t st) {
  if (a.group == 64) {
    launch_pick<AL, kMNContig, EP, NB>(a, st);
  } else if (a.group == 32) {
    launch_pick_grads_gm<EP, NB, 1, AL>(a, st);
  } else {
    const int bn = tiles(a, 256, 256) >= 256 ? 256 : 128;
    if (bn % a.group == 0) {
      launch_pick_grads_gm<EP, NB, 2, AL>(a, st);
    } else {
      const int64_t n = (int64_t)a.M * a.G;
      if (a.ds) launch_fill_zero(a.ds, n, st);
      if (a.dz) launch_fill_zero(a.dz, n, st);
      launch_pick_grads_gm<EP, NB, 3, AL>(a, st);
    }
  }
}

template <int EP, int NB>
void launch_grads(const GemmArgs& a, hipStream_t st) {
  if (a.lda % 8 == 0) launch_grads_al<EP, NB, kMNContig>(a, st);
  else launch_grads_al<EP, NB, kMNContigD>(a, st);
}

template <int BM, int BN, int BL, int NB>
void launch_fused_fwd(const GemmArgs& a, hipStream_t st) {
  LaunchTimer t(gemm_label<BL, kStoreBf16, NB, 0>(), st);
  QAT_LAUNCH((k_gemm_fused_fwd<BM, BN, BL, NB>), dim3((unsigned)tiles(a, BM, BN)), dim3(512), 0, st, a);
}

// The forward with a fused B operand (k_gemm_fused_fwd, 4 MFMA + 4 converter
// waves, BK = 32): 256 x 128 tiles where the output has at least one per CU,
// else 128 x 128. (512 x 64 tiles, which halve the conversions per MFMA,
// measured no faster for fp32 weights and 18% slower for packed codes at
// 2048 x 4096 x 4096: the larger A tile costs more LDS traffic.)
template <int BL, int NB>
void launch_pick_fused(const GemmArgs& a, hipStream_t st) {
  if (tiles(a, 256, 128) >= 256) launch_fused_fwd<256, 128, BL, NB>(a, st);
  else launch_fused_fwd<128, 128, BL, NB>(a, st);
}

// dX = dY W_hat with W_hat^T made in LDS from the weight's rows
// (k_gemm_fused_dx).
// ADW: dY by 4-byte DMA with the contraction's tail masked (out not a
// multiple of 64). Its 256x128 instance needs more than the 256 VGPRs of two
// waves per SIMD (328 bytes of scratch per lane, spills inside the main
// loop): 2.5-5x slower than 128x128 tiles at out = 4100 and 11000, so ragged
// contractions always take 128x128.
template <int BL, int NB, int ADW>
void launch_pick_dx_fused_a(const GemmArgs& a, hipStream_t st) {
  if (ADW == 0 && tiles(a, 256, 128) >= 256) launch_fused_dx<256, 128, BL, NB, ADW>(a, st);
  else launch_fused_dx<128, 128, BL, NB, ADW>(a, st);
}

template <int BL, int NB>
void launch_pick_dx_fused(const GemmArgs& a, hipStream_t st) {
  if (a.K % 64 == 0 && a.lda % 8 == 0) launch_pick_dx_fused_a<BL, NB, 0>(a, st);
  else launch_pick_dx_fused_a<BL, NB, 1>(a, st);
}

}  // namespace

void launch_gemm_dx_fused(const GemmArgs& a, int bload, int bits, hipStream_t st) {
  if (bload == kFp32Quant) launch_pick_dx_fused<kFp32Quant, 0>(a, st);
  else if (bits == 2) launch_pick_dx_fused<kPacked, 2>(a, st);
  else if (bits == 3) launch_pick_dx_fused<kPacked, 3>(a, st);
  else launch_pick_dx_fused<kPacked, 4>(a, st);
}

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
template <int AL>
void launch_gemm_dx_mn_al(const GemmArgs& a, hipStream_t st) {
  // with dY by 4-byte DMA (kKContigD) the 256x256 eight-wave instance spills
  // inside its main loop; 128x256 tiles measured 1.3-1.6x faster there
  // (M = 4096, out = 4100 and 11000)
  if (AL == kKContig && prefer_256x256(a)) launch_bf16<256, 256, 2, 2, 4, AL, kMNContig, kStoreBf16, 1>(a, st);
  else if (tiles(a, 128, 256) >= 192) launch_bf16<128, 256, 3, 2, 4, AL, kMNContig, kStoreBf16, 1>(a, st);
  else launch_bf16<128, 128, 4, 2, 2, AL, kMNContig, kStoreBf16, 1>(a, st);
}

// dY by 4-byte DMA with the contraction's tail masked when out (K) is not a
// multiple of 64; W_hat's k-rows at or beyond K read as zero either way.
void launch_gemm_dx_mn(const GemmArgs& a, hipStream_t st) {
  if (a.K % 64 == 0 && a.lda % 8 == 0) launch_gemm_dx_mn_al<kKContig>(a, st);
  else launch_gemm_dx_mn_al<kKContigD>(a, st);
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
