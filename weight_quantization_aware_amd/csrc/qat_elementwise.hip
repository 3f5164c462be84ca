// HBM-bound kernels of the group-wise fake-quant linear (gfx950, wave64):
// min-max init, code export, pack, and the transposed W_hat / operand staging
// that lets every GEMM of the path read K-contiguous operands.
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
// Transposed operand staging through LDS, 64x64 tiles, 256 threads.
// Source tile rows r (64) x columns c (64); the destination holds the tile
// transposed. Values go through LDS as fp32 in a [64][65] array (the +1 pad
// keeps column reads free of bank conflicts).
// ---------------------------------------------------------------------------

// Store a 64x64 fp32 tile held in `t` transposed as bf16: dst[(c0 + c) * ldd + r0 + r].
// Thread layout on the way out: column c = tid % 64, rows seg*16 .. +15 with seg = tid / 64.
__device__ __forceinline__ void store_tile_t(float (*t)[65], uint16_t* __restrict__ dst, int64_t ldd,
                                             int64_t c0, int64_t r0) {
  const int c = threadIdx.x & 63, seg = threadIdx.x >> 6;
  uint32_t p[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) p[k] = pack_bf16x2(t[seg * 16 + 2 * k][c], t[seg * 16 + 2 * k + 1][c]);
  uint4* o = (uint4*)(dst + (c0 + c) * ldd + r0 + seg * 16);
  o[0] = make_uint4(p[0], p[1], p[2], p[3]);
  o[1] = make_uint4(p[4], p[5], p[6], p[7]);
}

// W [out, in] fp32 -> W_hat^T [in, out] bf16 (Eq. 1 + Eq. 2, straight-through zero point).
__global__ __launch_bounds__(256) void k_quant_t(const float* __restrict__ W, const float* __restrict__ s,
                                                 const float* __restrict__ z, int64_t out, int64_t in,
                                                 float K, uint16_t* __restrict__ Wt) {
  __shared__ float t[64][65];
  const int64_t o0 = (int64_t)blockIdx.y * 64, i0 = (int64_t)blockIdx.x * 64;
  const int64_t G = in / kGroup;
  const int cv = threadIdx.x & 15, r = threadIdx.x >> 4;   // float4 column, row 0..15
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    int rr = r + 16 * p;
    int64_t o = o0 + rr;
    float sv = s[o * G + blockIdx.x];
    float zr = round_clamp_zero(z[o * G + blockIdx.x], K);
    float4 w = *(const float4*)(W + o * in + i0 + cv * 4);
    t[rr][cv * 4 + 0] = quant_elem(w.x, sv, zr, K).w_hat;
    t[rr][cv * 4 + 1] = quant_elem(w.y, sv, zr, K).w_hat;
    t[rr][cv * 4 + 2] = quant_elem(w.z, sv, zr, K).w_hat;
    t[rr][cv * 4 + 3] = quant_elem(w.w, sv, zr, K).w_hat;
  }
  __syncthreads();
  store_tile_t(t, Wt, out, i0, o0);
}

// Packed Wq [out, in*N/8] -> W_hat^T [in, out] bf16 with W_hat = fl32((q - z) * s), z as stored.
template <int N>
__global__ __launch_bounds__(256) void k_dequant_t(const uint8_t* __restrict__ Wq,
                                                   const float* __restrict__ s,
                                                   const float* __restrict__ z, int64_t out,
                                                   int64_t in, uint16_t* __restrict__ Wt) {
  __shared__ float t[64][65];
  const int64_t o0 = (int64_t)blockIdx.y * 64, i0 = (int64_t)blockIdx.x * 64;
  const int64_t G = in / kGroup;
  const int64_t rowbytes = in * N / 8;
  const int c8 = threadIdx.x & 7, r = threadIdx.x >> 3;     // 8-code chunk, row 0..31
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    int rr = r + 32 * p;
    int64_t o = o0 + rr;
    float sv = s[o * G + blockIdx.x];
    float zv = z[o * G + blockIdx.x];
    const uint8_t* src = Wq + o * rowbytes + (i0 / 8) * N + c8 * N;
    uint32_t word;
    if constexpr (N == 2) word = *(const uint16_t*)src;
    else if constexpr (N == 4) word = *(const uint32_t*)src;
    else word = (uint32_t)src[0] | ((uint32_t)src[1] << 8) | ((uint32_t)src[2] << 16);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float q = (float)((word >> (N * k)) & ((1u << N) - 1));
      t[rr][c8 * 8 + k] = (q - zv) * sv;
    }
  }
  __syncthreads();
  store_tile_t(t, Wt, out, i0, o0);
}

// bf16 [R, C] (row stride ldsrc) -> [C, Rp] (row stride Rp), rows R..Rp-1 zero.
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ src, int64_t R,
                                                        int64_t C, int64_t ldsrc,
                                                        uint16_t* __restrict__ dst, int64_t Rp) {
  __shared__ float t[64][65];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int c8 = threadIdx.x & 7, r = threadIdx.x >> 3;      // 8-element chunk, row 0..31
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    int rr = r + 32 * p;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + rr < R) v = *(const uint4*)(src + (r0 + rr) * ldsrc + c0 + c8 * 8);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      t[rr][c8 * 8 + 2 * k] = __builtin_bit_cast(float, w[k] << 16);
      t[rr][c8 * 8 + 2 * k + 1] = __builtin_bit_cast(float, w[k] & 0xFFFF0000u);
    }
  }
  __syncthreads();
  store_tile_t(t, dst, Rp, c0, r0);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline unsigned blocks_for(int64_t n, int64_t per) { return (unsigned)((n + per - 1) / per); }

void launch_init_minmax(const float* W, int64_t out, int64_t in, int bits, float* s, float* z,
                        hipStream_t st) {
  int64_t ngroups = out * (in / kGroup);
  hipLaunchKernelGGL(k_init_minmax, dim3(blocks_for(ngroups, 64)), dim3(256), 0, st,
                     (const float4*)W, ngroups, (float)((1 << bits) - 1), s, z);
}

void launch_quant_codes(const float* W, const float* s, const float* z, int64_t out, int64_t in,
                        int bits, uint8_t* codes, uint16_t* w_hat, hipStream_t st) {
  int64_t nvec = out * in / 4;
  hipLaunchKernelGGL(k_quant_codes, dim3(blocks_for(nvec, 256)), dim3(256), 0, st,
                     (const float4*)W, s, z, nvec, (float)((1 << bits) - 1), (uint32_t*)codes,
                     (uint2*)w_hat);
}

void launch_pack(const float* W, const float* s, const float* z, int64_t out, int64_t in, int bits,
                 uint8_t* Wq, float* zround, hipStream_t st) {
  int64_t nchunks = out * in / 8;
  dim3 grid(blocks_for(nchunks, 256));
  if (bits == 2)
    hipLaunchKernelGGL(k_pack<2>, grid, dim3(256), 0, st, (const float4*)W, s, z, nchunks, Wq, zround);
  else if (bits == 3)
    hipLaunchKernelGGL(k_pack<3>, grid, dim3(256), 0, st, (const float4*)W, s, z, nchunks, Wq, zround);
  else
    hipLaunchKernelGGL(k_pack<4>, grid, dim3(256), 0, st, (const float4*)W, s, z, nchunks, Wq, zround);
}

void launch_quant_t(const float* W, const float* s, const float* z, int64_t out, int64_t in, int bits,
                    uint16_t* Wt, hipStream_t st) {
  hipLaunchKernelGGL(k_quant_t, dim3((unsigned)(in / 64), (unsigned)(out / 64)), dim3(256), 0, st, W,
                     s, z, out, in, (float)((1 << bits) - 1), Wt);
}

void launch_dequant_t(const uint8_t* Wq, const float* s, const float* z, int64_t out, int64_t in,
                      int bits, uint16_t* Wt, hipStream_t st) {
  dim3 grid((unsigned)(in / 64), (unsigned)(out / 64));
  if (bits == 2)
    hipLaunchKernelGGL(k_dequant_t<2>, grid, dim3(256), 0, st, Wq, s, z, out, in, Wt);
  else if (bits == 3)
    hipLaunchKernelGGL(k_dequant_t<3>, grid, dim3(256), 0, st, Wq, s, z, out, in, Wt);
  else
    hipLaunchKernelGGL(k_dequant_t<4>, grid, dim3(256), 0, st, Wq, s, z, out, in, Wt);
}

void launch_transpose_bf16(const uint16_t* src, int64_t R, int64_t C, uint16_t* dst, int64_t Rp,
                           hipStream_t st) {
  hipLaunchKernelGGL(k_transpose_bf16, dim3((unsigned)(C / 64), (unsigned)(Rp / 64)), dim3(256), 0, st,
                     src, R, C, C, dst, Rp);
}

}  // namespace qat
