// HBM-bound kernels of the group-wise fake-quant linear (gfx950, wave64):
// min-max init, code export (also the bf16 W_hat staging of the forward and
// backward GEMMs), pack, and the E2E-QP dequantisation of packed codes.
#include "qat_device.h"
#include "qat_internal.h"

namespace qat {

// ---------------------------------------------------------------------------
// a1: per-group min-max init (modelfoundations.com EfficientQAT note, Phase 1).
// A wave reads 4 KiB fully coalesced (lane l loads float4 j*64 + l of the
// wave's window, j = 0..3), i.e. 16 groups; the 16 lanes that share a group
// reduce min / max with DPP inside their row. Lane (l & 15) == j of row
// (l >> 4) writes group j*4 + (l >> 4).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_init_minmax(const float4* __restrict__ W, int64_t ngroups,
                                                     float K, float* __restrict__ s,
                                                     float* __restrict__ z) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t base_vec = wave * 256;            // 256 float4 = 16 groups per wave
  const int64_t nvec = ngroups * 16;
  float4 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int64_t idx = base_vec + j * 64 + lane;
    if (idx < nvec) v[j] = W[idx];
    else v[j] = make_float4(__builtin_inff(), __builtin_inff(), __builtin_inff(), __builtin_inff());
  }
  float mn[4], mx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int64_t idx = base_vec + j * 64 + lane;
    bool ok = idx < nvec;
    float a = fminf(fminf(v[j].x, v[j].y), fminf(v[j].z, v[j].w));
    float b = fmaxf(fmaxf(v[j].x, v[j].y), fmaxf(v[j].z, v[j].w));
    mn[j] = row16_min(a);
    mx[j] = row16_max(ok ? b : -__builtin_inff());
  }
  const int sel = lane & 15;
  if (sel < 4) {
    float a = mn[0], b = mx[0];
    if (sel == 1) { a = mn[1]; b = mx[1]; }
    if (sel == 2) { a = mn[2]; b = mx[2]; }
    if (sel == 3) { a = mn[3]; b = mx[3]; }
    int64_t g = wave * 16 + sel * 4 + (lane >> 4);
    if (g < ngroups) {
      float d = b - a;
      float sv = fmaxf(d / K, kSMin);
      s[g] = sv;
      z[g] = __builtin_rintf(-a / sv);
    }
  }
}

// ---------------------------------------------------------------------------
// a2+a3 export: codes (u8) and W_hat (bf16 bits), 4 elements per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_codes(const float4* __restrict__ W,
                                                     const float* __restrict__ s,
                                                     const float* __restrict__ z, int64_t nvec,
                                                     float K, uint32_t* __restrict__ codes,
                                                     uint2* __restrict__ w_hat) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nvec) return;
  int64_t g = i >> 4;                    // 16 float4 per group of 64
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
                                              const float* __restrict__ z, int64_t nchunks,
                                              uint8_t* __restrict__ Wq, float* __restrict__ zround) {
  constexpr float K = (float)((1 << N) - 1);
  int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;   // chunk of 8 elements
  if (c >= nchunks) return;
  int64_t g = c >> 3;
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
  if (zround && (c & 7) == 0) zround[g] = zr;
}

// ---------------------------------------------------------------------------
// E2E-QP operand staging: packed codes -> W_hat = bf16(fl32((q - z) * s)),
// z as stored, [out, in] bf16. One chunk of 8 codes (N bytes in, 16 B out) per
// thread, so both streams are contiguous across a wave.
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ Wq, const float* __restrict__ s,
                                                 const float* __restrict__ z, int64_t nchunks,
                                                 uint4* __restrict__ w_hat) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nchunks) return;
  const int64_t g = c >> 3;
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
// Launchers
// ---------------------------------------------------------------------------
static inline unsigned blocks_for(int64_t n, int64_t per) { return (unsigned)((n + per - 1) / per); }

void launch_init_minmax(const float* W, int64_t out, int64_t in, int bits, float* s, float* z,
                        hipStream_t st) {
  int64_t ngroups = out * (in / kGroup);
  LaunchTimer t("init_minmax", st);
  hipLaunchKernelGGL(k_init_minmax, dim3(blocks_for(ngroups, 64)), dim3(256), 0, st,
                     (const float4*)W, ngroups, (float)((1 << bits) - 1), s, z);
}

void launch_quant_codes(const float* W, const float* s, const float* z, int64_t out, int64_t in,
                        int bits, uint8_t* codes, uint16_t* w_hat, hipStream_t st) {
  int64_t nvec = out * in / 4;
  LaunchTimer t(codes ? "quant_codes" : "quant_w_hat", st);
  hipLaunchKernelGGL(k_quant_codes, dim3(blocks_for(nvec, 256)), dim3(256), 0, st,
                     (const float4*)W, s, z, nvec, (float)((1 << bits) - 1), (uint32_t*)codes,
                     (uint2*)w_hat);
}

void launch_pack(const float* W, const float* s, const float* z, int64_t out, int64_t in, int bits,
                 uint8_t* Wq, float* zround, hipStream_t st) {
  int64_t nchunks = out * in / 8;
  dim3 grid(blocks_for(nchunks, 256));
  LaunchTimer t("pack", st);
  if (bits == 2)
    hipLaunchKernelGGL(k_pack<2>, grid, dim3(256), 0, st, (const float4*)W, s, z, nchunks, Wq, zround);
  else if (bits == 3)
    hipLaunchKernelGGL(k_pack<3>, grid, dim3(256), 0, st, (const float4*)W, s, z, nchunks, Wq, zround);
  else
    hipLaunchKernelGGL(k_pack<4>, grid, dim3(256), 0, st, (const float4*)W, s, z, nchunks, Wq, zround);
}

void launch_dequant(const uint8_t* Wq, const float* s, const float* z, int64_t out, int64_t in, int bits,
                    uint16_t* w_hat, hipStream_t st) {
  const int64_t nchunks = out * in / 8;
  dim3 grid(blocks_for(nchunks, 256));
  LaunchTimer t("dequant", st);
  if (bits == 2) hipLaunchKernelGGL(k_dequant<2>, grid, dim3(256), 0, st, Wq, s, z, nchunks, (uint4*)w_hat);
  else if (bits == 3) hipLaunchKernelGGL(k_dequant<3>, grid, dim3(256), 0, st, Wq, s, z, nchunks, (uint4*)w_hat);
  else hipLaunchKernelGGL(k_dequant<4>, grid, dim3(256), 0, st, Wq, s, z, nchunks, (uint4*)w_hat);
}

}  // namespace qat
