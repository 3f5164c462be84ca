// HBM-bound kernels of the group-wise fake-quant linear (gfx950, wave64):
// min-max init, code export (also the bf16 W_hat staging of the forward and
// backward GEMMs), pack, and the E2E-QP dequantisation of packed codes.
#include "qat_device.h"
#include "qat_internal.h"

namespace qat {

// ---------------------------------------------------------------------------
// a1: per-group min-max init (modelfoundations.com EfficientQAT note, Phase 1).
// A wave reads 4 KiB fully coalesced (lane l loads float4 j*64 + l of the
// wave's window, j = 0..3). In chunk j a group of GS elements covers GS/4
// consecutive lanes (8, 16 or 32), which reduce min / max with DPP (and one
// cross-row shuffle for 32 lanes); the first four lanes of each group's lane
// set write the groups of chunks 0..3.
// ---------------------------------------------------------------------------
template <int GS>
__global__ __launch_bounds__(256) void k_init_minmax(const float4* __restrict__ W, int64_t ngroups,
                                                     float K, float* __restrict__ s,
                                                     float* __restrict__ z) {
  constexpr int LPG = GS / 4;                           // lanes per group within a chunk
  constexpr int GPC = 64 / LPG;                         // groups per chunk
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nvec = ngroups * LPG;
  // Groups never straddle the end (in % GS == 0): a window past the end holds
  // whole groups that are not stored, so its zero fill is never used.
  float4 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t idx = wave * 256 + j * 64 + lane;
    v[j] = idx < nvec ? W[idx] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float mn[4], mx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = fminf(fminf(v[j].x, v[j].y), fminf(v[j].z, v[j].w));
    const float b = fmaxf(fmaxf(v[j].x, v[j].y), fmaxf(v[j].z, v[j].w));
    if constexpr (LPG == 8) {
      mn[j] = row8_min(a);
      mx[j] = row8_max(b);
    } else {
      mn[j] = row16_min(a);
      mx[j] = row16_max(b);
      if constexpr (LPG == 32) {
        mn[j] = fminf(mn[j], __shfl_xor(mn[j], 16));
        mx[j] = fmaxf(mx[j], __shfl_xor(mx[j], 16));
      }
    }
  }
  const int sel = lane % LPG;
  if (sel < 4) {
    const float a = sel == 0 ? mn[0] : sel == 1 ? mn[1] : sel == 2 ? mn[2] : mn[3];
    const float b = sel == 0 ? mx[0] : sel == 1 ? mx[1] : sel == 2 ? mx[2] : mx[3];
    const int64_t g = wave * 4 * GPC + sel * GPC + lane / LPG;
    if (g < ngroups) {
      const float sv = fmaxf((b - a) / K, kSMin);
      s[g] = sv;
      z[g] = __builtin_rintf(-a / sv);
    }
  }
}

// Channel-wise init (one group per weight row): a wave per row.
__global__ __launch_bounds__(256) void k_init_rows(const float4* __restrict__ W, int64_t out, int64_t vpr,
                                                   float K, float* __restrict__ s, float* __restrict__ z) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= out) return;                               // uniform per wave
  const float4* p = W + row * vpr;
  float a = __builtin_inff(), b = -__builtin_inff();
#pragma unroll 4
  for (int64_t i = lane; i < vpr; i += 64) {
    const float4 v = p[i];
    a = fminf(a, fminf(fminf(v.x, v.y), fminf(v.z, v.w)));
    b = fmaxf(b, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
  }
  a = row16_min(a);
  b = row16_max(b);
  a = fminf(a, __shfl_xor(a, 16));
  b = fmaxf(b, __shfl_xor(b, 16));
  a = fminf(a, __shfl_xor(a, 32));
  b = fmaxf(b, __shfl_xor(b, 32));
  if (lane == 0) {
    const float sv = fmaxf((b - a) / K, kSMin);
    s[row] = sv;
    z[row] = __builtin_rintf(-a / sv);
  }
}

// ---------------------------------------------------------------------------
// a2+a3 export: codes (u8) and W_hat (bf16 bits), 4 elements per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_codes(const float4* __restrict__ W,
                                                     const float* __restrict__ s,
                                                     const float* __restrict__ z, int64_t nvec,
                                                     FastDiv vpg, float K, uint32_t* __restrict__ codes,
                                                     uint2* __restrict__ w_hat) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nvec) return;
  int64_t g = vpg.div((uint32_t)i);      // float4 -> group (group / 4 float4 per group)
  float sv = s[g];
  float zr = round_clamp_zero(z[g], K);
  float4 w = W[i];
  QElem e0 = quant_elem(w.x, sv, zr, K), e1 = quant_elem(w.y, sv, zr, K);
  QElem e2 = quant_elem(w.z, sv, zr, K), e3 = quant_elem(w.w, sv, zr, K);
  if (codes)
    codes[i] = (uint32_t)e0.q | ((uint32_t)e1.q << 8) | ((uint32_t)e2.q << 16) | ((uint32_t)e3.q << 24);
  if (w_hat)
    w_hat[i] = make_uint2(pack_bf16x2(e0.w_hat, e1.w_hat), pack_bf16x2(e2.w_hat, e3.w_hat));
}

// ---------------------------------------------------------------------------
// a8: pack. 8 lanes per group, 8 codes per lane -> N bytes per lane, so the
// packed stream of a wave is contiguous. zp = clamp(rint(z), 0, K).
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(256) void k_pack(const float4* __restrict__ W, const float* __restrict__ s,
                                              const float* __restrict__ z, int64_t nchunks, FastDiv cpg,
                                              uint32_t cpg_n, uint8_t* __restrict__ Wq,
                                              float* __restrict__ zround) {
  constexpr float K = (float)((1 << N) - 1);
  int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;   // chunk of 8 elements
  if (c >= nchunks) return;
  int64_t g = cpg.div((uint32_t)c);                        // group / 8 chunks per group
  float sv = s[g];
  float zr = round_clamp_zero(z[g], K);
  float4 a = W[2 * c], b = W[2 * c + 1];
  float w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t word = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) word |= ((uint32_t)quant_elem(w[k], sv, zr, K).q) << (N * k);
  uint8_t* dst = Wq + c * N;
  if constexpr (N == 2) {
    *(uint16_t*)dst = (uint16_t)word;
  } else if constexpr (N == 4) {
    *(uint32_t*)dst = word;
  } else {
    dst[0] = (uint8_t)word;
    dst[1] = (uint8_t)(word >> 8);
    dst[2] = (uint8_t)(word >> 16);
  }
  if (zround && c == g * cpg_n) zround[g] = zr;           // first chunk of the group
}

// ---------------------------------------------------------------------------
// E2E-QP operand staging: packed codes -> W_hat = bf16(fl32((q - z) * s)),
// z as stored, [out, in] bf16. One chunk of 8 codes (N bytes in, 16 B out) per
// thread, so both streams are contiguous across a wave.
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ Wq, const float* __restrict__ s,
                                                 const float* __restrict__ z, int64_t nchunks, FastDiv cpg,
                                                 uint4* __restrict__ w_hat) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nchunks) return;
  const int64_t g = cpg.div((uint32_t)c);
  const float sv = s[g], zv = z[g];
  const uint8_t* src = Wq + c * N;
  uint32_t word;
  if constexpr (N == 2) word = *(const uint16_t*)src;
  else if constexpr (N == 4) word = *(const uint32_t*)src;
  else word = (uint32_t)src[0] | ((uint32_t)src[1] << 8) | ((uint32_t)src[2] << 16);
  float h[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) h[k] = ((float)((word >> (N * k)) & ((1u << N) - 1)) - zv) * sv;
  w_hat[c] = make_uint4(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]),
                        pack_bf16x2(h[6], h[7]));
}

// ---------------------------------------------------------------------------
// W_hat^T staging for the backward dX GEMM: the bf16 W_hat of a7 (fp32 master
// weight, SRC = 0: Eq. 1-2 with zr = clamp(rint(z), 0, K)) or of a9 (packed
// N-bit codes, SRC = 1: (q - z) * s) written transposed, [in][out], so that
// dX = dY W_hat contracts two K-contiguous operands. A workgroup transposes a
// 128 (out) x 64 (in) tile through LDS: every thread quantises two rows x 8
// columns per item (rows read 256 or N*8 bytes contiguous per 8 lanes), stores
// the row pairs as 4-byte words of the transposed tile, and the tile leaves as
// 256-byte rows of W_hat^T. out % 64 == 0 and in % 64 == 0.
// ---------------------------------------------------------------------------
template <int SRC, int N>
__global__ __launch_bounds__(256) void k_w_hat_t(const void* __restrict__ Wsrc, const float* __restrict__ s,
                                                 const float* __restrict__ z, int64_t out, int64_t in, int64_t G,
                                                 FastDiv gdiv, float K, uint16_t* __restrict__ w_hat_t) {
  constexpr int TO = 128, TIN = 64;                      // tile rows (out), cols (in)
  // LDS tile T[c][o] (c: input column, o: output row; 256 bytes per c). The
  // 16-byte chunk h of row c sits at h ^ (c / 8) ^ 8 (h & 1): the 64 four-byte
  // writes of one instruction (8 columns x 8 row pairs) fall on 64 distinct
  // banks, and so do the 32 of each half-wave on 32 banks (the former h ^ 2
  // (c / 8) put two of them on one bank there); a row is still read as whole
  // 16-byte chunks, every bank used equally.
  __shared__ __attribute__((aligned(16))) uint16_t T[TIN * TO];
  const int bo = SRC == 1 ? blockIdx.x : blockIdx.y, bi = SRC == 1 ? blockIdx.y : blockIdx.x;
  const int64_t o0 = (int64_t)bo * TO, i0 = (int64_t)bi * TIN;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int item = threadIdx.x + 256 * q;
    const int rp = item >> 3, co = item & 7;            // row pair, column octet
    const int64_t o = o0 + 2 * rp;
    const int64_t g = gdiv.div((uint32_t)(i0 + co * 8));  // the octet's group
    float h[2][8];
    if (o < out) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const float sv = s[(o + r) * G + g];
        if constexpr (SRC == 0) {
          const float zr = round_clamp_zero(z[(o + r) * G + g], K);
          const float4* src = (const float4*)((const float*)Wsrc + (o + r) * in + i0 + co * 8);
          const float4 w0 = src[0], w1 = src[1];
          const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
          for (int k = 0; k < 8; ++k) h[r][k] = quant_elem(w[k], sv, zr, K).w_hat;
        } else {
          const float zv = z[(o + r) * G + g];
          const uint8_t* src = (const uint8_t*)Wsrc + (o + r) * (in * N / 8) + (i0 + co * 8) * N / 8;
          uint32_t word;
          if constexpr (N == 2) word = *(const uint16_t*)src;
          else if constexpr (N == 4) word = *(const uint32_t*)src;
          else word = (uint32_t)src[0] | ((uint32_t)src[1] << 8) | ((uint32_t)src[2] << 16);
#pragma unroll
          for (int k = 0; k < 8; ++k) h[r][k] = ((float)((word >> (N * k)) & ((1u << N) - 1)) - zv) * sv;
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int k = 0; k < 8; ++k) h[r][k] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = co * 8 + k;
      const int hc = rp >> 2;                                                 // chunk of rows 2rp, 2rp+1
      const int dw = ((hc ^ (c >> 3) ^ ((hc & 1) << 3)) << 2) | (rp & 3);   // their swizzled 4-byte slot
      *(uint32_t*)&T[c * TO + 2 * dw] = pack_bf16x2(h[0][k], h[1][k]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = threadIdx.x + 256 * q;
    const int row = idx >> 4, ch = idx & 15;            // row of W_hat^T in the tile, 8-element chunk
    const int64_t oc = o0 + ch * 8;
    if (oc < out)
      *(uint4*)(w_hat_t + (i0 + row) * out + oc) = *(const uint4*)&T[row * TO + ((ch ^ (row >> 3) ^ ((ch & 1) << 3)) * 8)];
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline unsigned blocks_for(int64_t n, int64_t per) { return (unsigned)((n + per - 1) / per); }

// Zero fill (the accumulation target of the gradient epilogues for whole-row
// groups wider than one GEMM tile).
__global__ __launch_bounds__(256) void k_fill_zero(float4* __restrict__ p, int64_t n4, float* __restrict__ tail,
                                                   int ntail) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (i < ntail) tail[i] = 0.f;
}

void launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  const int64_t n4 = n / 4;
  LaunchTimer t("fill_zero", st);
  QAT_LAUNCH(k_fill_zero, dim3(blocks_for(n4 > 0 ? n4 : 1, 256)), dim3(256), 0, st, (float4*)p, n4,
                     p + n4 * 4, (int)(n - n4 * 4));
}

void launch_init_minmax(const float* W, int64_t out, int64_t in, int group, int bits, float* s, float* z,
                        hipStream_t st) {
  const int64_t ngroups = out * (in / group);
  const float K = (float)((1 << bits) - 1);
  LaunchTimer t("init_minmax", st);
  if (group == in && group != 32 && group != 64 && group != 128) {
    QAT_LAUNCH(k_init_rows, dim3(blocks_for(out, 4)), dim3(256), 0, st, (const float4*)W, out, in / 4, K,
                       s, z);
  } else if (group == 32) {
    QAT_LAUNCH(k_init_minmax<32>, dim3(blocks_for(ngroups, 128)), dim3(256), 0, st, (const float4*)W,
                       ngroups, K, s, z);
  } else if (group == 64) {
    QAT_LAUNCH(k_init_minmax<64>, dim3(blocks_for(ngroups, 64)), dim3(256), 0, st, (const float4*)W,
                       ngroups, K, s, z);
  } else {
    QAT_LAUNCH(k_init_minmax<128>, dim3(blocks_for(ngroups, 32)), dim3(256), 0, st, (const float4*)W,
                       ngroups, K, s, z);
  }
}

void launch_quant_codes(const float* W, const float* s, const float* z, int64_t out, int64_t in, int group,
                        int bits, uint8_t* codes, uint16_t* w_hat, hipStream_t st) {
  int64_t nvec = out * in / 4;
  LaunchTimer t(codes ? "quant_codes" : "quant_w_hat", st);
  QAT_LAUNCH(k_quant_codes, dim3(blocks_for(nvec, 256)), dim3(256), 0, st,
                     (const float4*)W, s, z, nvec, FastDiv::make((uint32_t)group / 4), (float)((1 << bits) - 1),
                     (uint32_t*)codes, (uint2*)w_hat);
}

void launch_pack(const float* W, const float* s, const float* z, int64_t out, int64_t in, int group, int bits,
                 uint8_t* Wq, float* zround, hipStream_t st) {
  int64_t nchunks = out * in / 8;
  dim3 grid(blocks_for(nchunks, 256));
  const uint32_t cpg = (uint32_t)group / 8;
  const FastDiv fd = FastDiv::make(cpg);
  LaunchTimer t("pack", st);
  if (bits == 2)
    QAT_LAUNCH(k_pack<2>, grid, dim3(256), 0, st, (const float4*)W, s, z, nchunks, fd, cpg, Wq, zround);
  else if (bits == 3)
    QAT_LAUNCH(k_pack<3>, grid, dim3(256), 0, st, (const float4*)W, s, z, nchunks, fd, cpg, Wq, zround);
  else
    QAT_LAUNCH(k_pack<4>, grid, dim3(256), 0, st, (const float4*)W, s, z, nchunks, fd, cpg, Wq, zround);
}

void launch_dequant(const uint8_t* Wq, const float* s, const float* z, int64_t out, int64_t in, int group,
                    int bits, uint16_t* w_hat, hipStream_t st) {
  const int64_t nchunks = out * in / 8;
  dim3 grid(blocks_for(nchunks, 256));
  const FastDiv fd = FastDiv::make((uint32_t)group / 8);
  LaunchTimer t("dequant", st);
  if (bits == 2) QAT_LAUNCH(k_dequant<2>, grid, dim3(256), 0, st, Wq, s, z, nchunks, fd, (uint4*)w_hat);
  else if (bits == 3) QAT_LAUNCH(k_dequant<3>, grid, dim3(256), 0, st, Wq, s, z, nchunks, fd, (uint4*)w_hat);
  else QAT_LAUNCH(k_dequant<4>, grid, dim3(256), 0, st, Wq, s, z, nchunks, fd, (uint4*)w_hat);
}

void launch_w_hat_t(const float* W, const float* s, const float* z, int64_t out, int64_t in, int group,
                    int bits, uint16_t* w_hat_t, hipStream_t st) {
  const dim3 grid((unsigned)(in / 64), (unsigned)((out + 127) / 128));
  LaunchTimer t("quant_w_hat_t", st);
  QAT_LAUNCH((k_w_hat_t<0, 0>), grid, dim3(256), 0, st, W, s, z, out, in, in / group,
                     FastDiv::make((uint32_t)group), (float)((1 << bits) - 1), w_hat_t);
}

void launch_dequant_t(const uint8_t* Wq, const float* s, const float* z, int64_t out, int64_t in, int group,
                      int bits, uint16_t* w_hat_t, hipStream_t st) {
  const dim3 grid((unsigned)((out + 127) / 128), (unsigned)(in / 64));
  const float K = (float)((1 << bits) - 1);
  const int64_t G = in / group;
  const FastDiv fd = FastDiv::make((uint32_t)group);
  LaunchTimer t("dequant_t", st);
  if (bits == 2) QAT_LAUNCH((k_w_hat_t<1, 2>), grid, dim3(256), 0, st, Wq, s, z, out, in, G, fd, K, w_hat_t);
  else if (bits == 3) QAT_LAUNCH((k_w_hat_t<1, 3>), grid, dim3(256), 0, st, Wq, s, z, out, in, G, fd, K, w_hat_t);
  else QAT_LAUNCH((k_w_hat_t<1, 4>), grid, dim3(256), 0, st, Wq, s, z, out, in, G, fd, K, w_hat_t);
}

}  // namespace qat
