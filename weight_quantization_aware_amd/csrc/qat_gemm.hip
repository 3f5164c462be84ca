// MFMA GEMMs of the group-wise fake-quant linear on gfx950.
//
// One kernel template computes C[M, N] = sum_k A[m, k] * B[n, k] with bf16
// operands that are both K-contiguous, fp32 accumulation in
// v_mfma_f32_16x16x32_bf16, and a 256-thread workgroup (4 wave64s in a 2x2
// grid) owning a BM x BN output tile. K advances in slabs of 64, which is
// exactly one quantisation group when B is the weight, so a fused loader needs
// one (s, z) pair per weight row and slab.
//
//   B sources (BLoad):  bf16 rows; fp32 master weight quantised and
//                       dequantised on the way into LDS (Eq. 1 + Eq. 2);
//                       packed N-bit codes dequantised on the way into LDS.
//   Epilogues (Epi):    bf16 store; straight-through gradients (dW, ds, dz);
//                       E2E-QP exact scale gradient (ds, dz).
//
// LDS: per operand a [rows][64] bf16 slab, 128 B per row as 8 chunks of 16 B
// with chunk c of row r stored at position c ^ (r & 7), so that the 16-byte
// fragment reads of 8 consecutive rows hit distinct banks. Two slabs per
// operand (double buffering); global loads for slab k+1 are issued before the
// MFMAs of slab k and written to LDS after them.
#include "qat_device.h"
#include "qat_internal.h"

namespace qat {

constexpr int kBK = 64;

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

// Workgroup id -> output tile. Consecutive workgroup ids are dealt round-robin
// to the 8 XCDs, so tile p is given to the XCD that owns a contiguous range of
// p; inside it tiles run in groups of 8 tile-rows so neighbours share B tiles
// in that XCD's L2.
__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int per = T / 8, rem = T % 8;
  const int xcd = b & 7, idx = b >> 3;
  const int p = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  constexpr int GM = 8;
  const int gsize = GM * tiles_n;
  const int gid = p / gsize;
  const int first = gid * GM;
  const int gm = min(tiles_m - first, GM);
  const int in_g = p - gid * gsize;
  tm = first + in_g % gm;
  tn = in_g / gm;
}

// ---------------------------------------------------------------------------
// B-operand loaders: load(k-slab) into registers, then store() into LDS.
// Thread t covers chunk (t & 7) of rows (t >> 3) + 32 p, p < PASSES.
// ---------------------------------------------------------------------------
template <int ROWS>
struct LoadBf16 {
  static constexpr int P = ROWS / 32;
  uint4 r[P];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int64_t ld, int row0, int nrows,
                                       int k0) {
    const int c = threadIdx.x & 7, rr = threadIdx.x >> 3;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int row = row0 + rr + 32 * p;
      r[p] = make_uint4(0, 0, 0, 0);
      if (row < nrows) r[p] = *(const uint4*)(src + (int64_t)row * ld + k0 + c * 8);
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds) const {
    const int c = threadIdx.x & 7, rr = threadIdx.x >> 3;
#pragma unroll
    for (int p = 0; p < P; ++p) *(uint4*)(lds + lds_off(rr + 32 * p, c)) = r[p];
  }
};

// fp32 master weight -> fused quantise / dequantise -> bf16 in LDS.
// u = w * fl32(1/s) is within 3 ulp of fl32(w/s); only where that interval can
// hold a rounding tie (a half-integer) is the element redone with the correctly
// rounded division, so the codes equal those of the exact fp32 quantiser.
template <int ROWS>
struct LoadFp32Quant {
  static constexpr int P = ROWS / 32;
  float4 r[P][2];
  float sv[P], zr[P];
  bool ok[P];
  float K;
  __device__ __forceinline__ void load(const float* __restrict__ W, int64_t ld, int row0, int nrows, int k0,
                                       const float* __restrict__ s, const float* __restrict__ z, int64_t G,
                                       float Kq) {
    const int c = threadIdx.x & 7, rr = threadIdx.x >> 3;
    K = Kq;
    const int kt = k0 / kBK;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int row = row0 + rr + 32 * p;
      ok[p] = row < nrows;
      if (ok[p]) {
        const float4* src = (const float4*)(W + (int64_t)row * ld + k0 + c * 8);
        r[p][0] = src[0];
        r[p][1] = src[1];
        sv[p] = s[(int64_t)row * G + kt];
        zr[p] = z[(int64_t)row * G + kt];
      }
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds) const {
    const int c = threadIdx.x & 7, rr = threadIdx.x >> 3;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      uint4 o = make_uint4(0, 0, 0, 0);
      if (ok[p]) {
        const float s_ = sv[p];
        const float z_ = round_clamp_zero(zr[p], K);
        const float rs = 1.0f / s_;
        float w[8] = {r[p][0].x, r[p][0].y, r[p][0].z, r[p][0].w,
                      r[p][1].x, r[p][1].y, r[p][1].z, r[p][1].w};
        float h[8];
        bool near_tie = false;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float u = w[k] * rs;
          const float fr = u - floorf(u);
          near_tie |= fabsf(fr - 0.5f) <= fabsf(u) * 0x1p-20f + 0x1p-60f;
          const float q = fminf(fmaxf(__builtin_rintf(u) + z_, 0.0f), K);
          h[k] = (q - z_) * s_;
        }
        if (near_tie) {
#pragma unroll
          for (int k = 0; k < 8; ++k) h[k] = quant_elem(w[k], s_, z_, K).w_hat;
        }
        o = make_uint4(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]),
                       pack_bf16x2(h[6], h[7]));
      }
      *(uint4*)(lds + lds_off(rr + 32 * p, c)) = o;
    }
  }
};

// Packed N-bit codes -> (q - z) * s -> bf16 in LDS (E2E-QP; z as stored).
template <int ROWS, int NB>
struct LoadPacked {
  static constexpr int P = ROWS / 32;
  uint32_t word[P];
  float sv[P], zv[P];
  bool ok[P];
  __device__ __forceinline__ void load(const uint8_t* __restrict__ Wq, int64_t ldq, int row0, int nrows,
                                       int k0, const float* __restrict__ s, const float* __restrict__ z,
                                       int64_t G) {
    const int c = threadIdx.x & 7, rr = threadIdx.x >> 3;
    const int kt = k0 / kBK;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int row = row0 + rr + 32 * p;
      ok[p] = row < nrows;
      if (ok[p]) {
        const uint8_t* src = Wq + (int64_t)row * ldq + (int64_t)kt * 8 * NB + c * NB;
        if constexpr (NB == 2) word[p] = *(const uint16_t*)src;
        else if constexpr (NB == 4) word[p] = *(const uint32_t*)src;
        else word[p] = (uint32_t)src[0] | ((uint32_t)src[1] << 8) | ((uint32_t)src[2] << 16);
        sv[p] = s[(int64_t)row * G + kt];
        zv[p] = z[(int64_t)row * G + kt];
      }
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds) const {
    const int c = threadIdx.x & 7, rr = threadIdx.x >> 3;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      uint4 o = make_uint4(0, 0, 0, 0);
      if (ok[p]) {
        float h[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float q = (float)((word[p] >> (NB * k)) & ((1u << NB) - 1));
          h[k] = (q - zv[p]) * sv[p];
        }
        o = make_uint4(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]),
                       pack_bf16x2(h[6], h[7]));
      }
      *(uint4*)(lds + lds_off(rr + 32 * p, c)) = o;
    }
  }
};

template <int ROWS, int BL, int NB>
struct BLoaderOf;
template <int ROWS, int NB>
struct BLoaderOf<ROWS, kBf16, NB> { using T = LoadBf16<ROWS>; };
template <int ROWS, int NB>
struct BLoaderOf<ROWS, kFp32Quant, NB> { using T = LoadFp32Quant<ROWS>; };
template <int ROWS, int NB>
struct BLoaderOf<ROWS, kPacked, NB> { using T = LoadPacked<ROWS, NB>; };

template <int BL, class L>
__device__ __forceinline__ void load_b(L& l, const GemmArgs& a, int n0, int k0) {
  if constexpr (BL == kBf16) l.load((const uint16_t*)a.B, a.ldb, n0, a.N, k0);
  else if constexpr (BL == kFp32Quant) l.load((const float*)a.B, a.ldb, n0, a.N, k0, a.s, a.z, a.G, a.Kq);
  else l.load((const uint8_t*)a.B, a.ldb, n0, a.N, k0, a.s, a.z, a.G);
}

// Code i of a packed row (LSB-first bitstream).
template <int NB>
__device__ __forceinline__ float code_at(const uint8_t* __restrict__ row, int64_t i) {
  const int64_t bit = i * NB;
  const int64_t byte = bit >> 3;
  const int sh = (int)(bit & 7);
  uint32_t v = row[byte];
  if (NB == 3 && sh > 5) v |= (uint32_t)row[byte + 1] << 8;
  return (float)((v >> sh) & ((1u << NB) - 1));
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
template <int BM, int BN, int BL, int EP, int NB>
__global__ __launch_bounds__(256) void k_gemm(const GemmArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TI = WM / 16, TJ = WN / 16;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (A_BYTES + B_BYTES)];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
  const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  LoadBf16<BM> la;
  typename BLoaderOf<BN, BL, NB>::T lb;
  // Buffer b holds the A slab at smem + b * STAGE and the B slab right after it.
  constexpr int STAGE = A_BYTES + B_BYTES;

  la.load(a.A, a.lda, m0, a.M, 0);
  load_b<BL>(lb, a, n0, 0);
  la.store(smem);
  lb.store(smem + A_BYTES);
  __syncthreads();

  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = a.K / kBK;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(a.A, a.lda, m0, a.M, (kt + 1) * kBK);
      load_b<BL>(lb, a, n0, (kt + 1) * kBK);
    }
    const uint8_t* pa = smem + cur * STAGE;
    const uint8_t* pb = pa + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int chunk = ks * 4 + (lane >> 4);
      bf16x8 af[TI], bfr[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) af[i] = *(const bf16x8*)(pa + lds_off(wm0 + i * 16 + (lane & 15), chunk));
#pragma unroll
      for (int j = 0; j < TJ; ++j) bfr[j] = *(const bf16x8*)(pb + lds_off(wn0 + j * 16 + (lane & 15), chunk));
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      uint8_t* nxt = smem + (cur ^ 1) * STAGE;
      la.store(nxt);
      lb.store(nxt + A_BYTES);
    }
    __syncthreads();
  }

  // acc[i][j][r] is C[m0 + wm0 + 16 i + 4 (lane >> 4) + r][n0 + wn0 + 16 j + (lane & 15)].
  const int rq = 4 * (lane >> 4), cl = lane & 15;
  if constexpr (EP == kStoreBf16) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm0 + i * 16 + rq + r;
        if (row >= a.M) continue;
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int col = n0 + wn0 + j * 16 + cl;
          if (col < a.N) a.C[(int64_t)row * a.ldc + col] = bf16_bits(acc[i][j][r]);
        }
      }
  } else {
    // Rows are weight rows o, columns are inputs i; a group is 64 columns = 4 j-tiles
    // of one wave, so every group sum is a 16-lane row reduction after a local sum.
    constexpr int NG = WN / 64;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = m0 + wm0 + i * 16 + rq + r;
        const bool row_ok = o < a.M;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const int c0 = n0 + wn0 + g * 64;
          const bool ok = row_ok && c0 < a.N;
          const int64_t gi = (int64_t)o * a.G + c0 / 64;
          float ps = 0.f, pz = 0.f, sv = 0.f;
          if (ok) {
            sv = a.s[gi];
            if constexpr (EP == kSteGrads) {
              const float zr = round_clamp_zero(a.z[gi], a.Kq);
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                const int col = c0 + jj * 16 + cl;
                const float gw = acc[i][g * 4 + jj][r];
                const QElem e = quant_elem(a.W[(int64_t)o * a.ldw + col], sv, zr, a.Kq);
                if (a.dW) a.dW[(int64_t)o * a.ldw + col] = e.m ? gw : 0.0f;
                ps += gw * (e.m ? (__builtin_rintf(e.u) - e.u) : (e.q - zr));
                pz += e.m ? 0.0f : gw;
              }
            } else {
              const float zv = a.z[gi];
              const uint8_t* qrow = a.Wq + (int64_t)o * a.ldq;
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                const int col = c0 + jj * 16 + cl;
                const float gw = acc[i][g * 4 + jj][r];
                ps += gw * (code_at<NB>(qrow, col) - zv);
                pz += gw;
              }
            }
          }
          ps = row16_sum(ps);
          pz = row16_sum(pz);
          if (ok && cl == 0 && a.ds) {
            a.ds[gi] = ps;
            if (a.dz) a.dz[gi] = -sv * pz;
          }
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Tile choice and launch
// ---------------------------------------------------------------------------
// Prefer the largest tile that still gives at least one tile per CU (256 CUs).
static int pick_tile(int M, int N) {
  auto tiles = [&](int bm, int bn) { return (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (tiles(256, 256) >= 256) return 0;
  if (tiles(256, 128) >= 256) return 1;
  return 2;
}

template <int BM, int BN, int BL, int EP, int NB>
static void launch_cfg(const GemmArgs& a, hipStream_t st) {
  const int T = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((k_gemm<BM, BN, BL, EP, NB>), dim3(T), dim3(256), 0, st, a);
}

template <int BL, int EP, int NB>
static void launch_pick(const GemmArgs& a, hipStream_t st) {
  switch (pick_tile(a.M, a.N)) {
    case 0: launch_cfg<256, 256, BL, EP, NB>(a, st); break;
    case 1: launch_cfg<256, 128, BL, EP, NB>(a, st); break;
    default: launch_cfg<128, 128, BL, EP, NB>(a, st); break;
  }
}

void launch_gemm_bf16_out(const GemmArgs& a, int bload, int bits, hipStream_t st) {
  if (bload == kBf16) launch_pick<kBf16, kStoreBf16, 0>(a, st);
  else if (bload == kFp32Quant) launch_pick<kFp32Quant, kStoreBf16, 0>(a, st);
  else if (bits == 2) launch_pick<kPacked, kStoreBf16, 2>(a, st);
  else if (bits == 3) launch_pick<kPacked, kStoreBf16, 3>(a, st);
  else launch_pick<kPacked, kStoreBf16, 4>(a, st);
}

void launch_gemm_ste_grads(const GemmArgs& a, hipStream_t st) {
  launch_pick<kBf16, kSteGrads, 0>(a, st);
}

void launch_gemm_e2e_grads(const GemmArgs& a, int bits, hipStream_t st) {
  if (bits == 2) launch_pick<kBf16, kE2eScaleGrad, 2>(a, st);
  else if (bits == 3) launch_pick<kBf16, kE2eScaleGrad, 3>(a, st);
  else launch_pick<kBf16, kE2eScaleGrad, 4>(a, st);
}

}  // namespace qat
