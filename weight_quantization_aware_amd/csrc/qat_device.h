// Device helpers shared by the gfx950 kernels of the group-wise fake-quant linear.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qat {

constexpr int kGroup = 64;           // the default quantisation group (elements along `in`)
constexpr float kSMin = 1e-5f;       // floor for the step size of a constant group

// Unsigned division of n < 2^31 by a runtime divisor d >= 1 with one multiply
// (the round-up reciprocal of Granlund and Montgomery): l = ceil(log2 d),
// m = floor(2^32 (2^l - d) / d) + 1, q = (umulhi(n, m) + n) >> l. The sum
// stays below 2^32 because umulhi(n, m) <= n < 2^31.
struct FastDiv {
  uint32_t m, l;
  __host__ __device__ static FastDiv make(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return FastDiv{(uint32_t)m, l};
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const { return (__umulhi(n, m) + n) >> l; }
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)bf16_bits(lo) | ((uint32_t)bf16_bits(hi) << 16);
}

// DPP lane exchanges inside a row of 16 lanes.
enum : int {
  kDppXor1 = 0xB1,          // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,          // quad_perm [2,3,0,1]
  kDppRowMirror = 0x140,    // lane i <-> 15 - i
  kDppRowHalfMirror = 0x141 // lane i <-> 7 - i (within each half row)
};

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// Sum / min / max over the 16 lanes of a DPP row; every lane gets the result.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppRowHalfMirror>(v);
  v += dpp<kDppRowMirror>(v);
  return v;
}
__device__ __forceinline__ float row16_min(float v) {
  v = fminf(v, dpp<kDppXor1>(v));
  v = fminf(v, dpp<kDppXor2>(v));
  v = fminf(v, dpp<kDppRowHalfMirror>(v));
  v = fminf(v, dpp<kDppRowMirror>(v));
  return v;
}
// Min / max over the 8 lanes of each half row.
__device__ __forceinline__ float row8_min(float v) {
  v = fminf(v, dpp<kDppXor1>(v));
  v = fminf(v, dpp<kDppXor2>(v));
  v = fminf(v, dpp<kDppRowHalfMirror>(v));
  return v;
}
__device__ __forceinline__ float row8_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp<kDppRowMirror>(v));
  return v;
}

// Quantiser of one element (Eq. 1 and Eq. 2 of the EfficientQAT paper notes):
//   u = fl32(w / s); v = rint(u) + zr; q = clamp(v, 0, K); m = 0 <= v <= K;
//   w_hat = fl32((q - zr) * s).
// zr is the already rounded and clamped zero point. Plain '/' is the IEEE
// correctly rounded fp32 division (no fast-math anywhere in this library).
struct QElem {
  float u, q, w_hat;
  bool m;
};

__device__ __forceinline__ QElem quant_elem(float w, float s, float zr, float K) {
  QElem e;
  e.u = w / s;
  float v = __builtin_rintf(e.u) + zr;
  e.m = (v >= 0.0f) && (v <= K);
  e.q = fminf(fmaxf(v, 0.0f), K);
  e.w_hat = (e.q - zr) * s;
  return e;
}

// Marks the rare branch it sits in: an empty volatile asm statement cannot be
// hoisted out of its branch, so the code after it (the exact division of a
// near-tie) stays behind the branch, skipped when no lane of the wave takes
// it, instead of being computed for every element and selected.
__device__ __forceinline__ void rare_branch(float& x) { asm volatile("" : "+v"(x)); }

// quant_elem with the quotient from a reciprocal: u0 = w * r (r = fl32(1/s)),
// refined by one residual step u = u0 + (w - u0 s) r (the residual is exact
// with an FMA), which lands within an ulp of fl32(w / s). The code decision
// rint(u) can only differ from the one of the correctly rounded quotient when
// u is within a few ulps of a half-integer; there the element is redone with
// the division, so q, m and w_hat are exactly quant_elem's and u is within an
// ulp of it.
__device__ __forceinline__ QElem quant_elem_rcp(float w, float s, float r, float zr, float K) {
  const float u0 = w * r;
  const float u = __builtin_fmaf(__builtin_fmaf(-u0, s, w), r, u0);
  const float fr = u - __builtin_floorf(u);
  if (__builtin_fabsf(fr - 0.5f) <= __builtin_fabsf(u) * 0x1p-20f + 0x1p-60f) {
    rare_branch(w);
    return quant_elem(w, s, zr, K);
  }
  QElem e;
  e.u = u;
  const float v = __builtin_rintf(u) + zr;
  e.m = (v >= 0.0f) && (v <= K);
  e.q = fminf(fmaxf(v, 0.0f), K);
  e.w_hat = (e.q - zr) * s;
  return e;
}

__device__ __forceinline__ float round_clamp_zero(float z, float K) {
  return fminf(fmaxf(__builtin_rintf(z), 0.0f), K);
}

}  // namespace qat
