// The MFMA GEMM kernels of the group-wise fake-quant linear (gfx950).
//
// C[M, N] = sum_k A[m, k] * B[n, k] in bf16 with fp32 accumulation in
// v_mfma_f32_16x16x32_bf16. A 256-thread workgroup (4 wave64s, 2x2, one per
// SIMD) owns a BM x BN tile; K advances in slabs of BK.
//
// The MFMA's first operand is the B fragment and its second the A fragment, so
// the 16x16 result a lane holds is 4 consecutive output COLUMNS of one row:
// acc[j][i][r] = C[m0 + wm0 + 16 i + (lane & 15)][n0 + wn0 + 16 j + 4 (lane >> 4) + r].
// Stores are then 8-byte (bf16) or 16-byte (fp32) vectors, and a 64-column
// quantisation group is 4 j-tiles x 4 registers of one lane plus a reduction
// over the 4 lanes that share (lane & 15).
//
// LDS: per operand and stage a slab of the tile, filled by direct-to-LDS DMA.
// K-contiguous tiles are [rows][BK] bf16 with 16-byte chunk c of row r at
// position c ^ ((r / RPL) & (CH - 1)); MN-contiguous tiles are [BK][rows] read
// with LDS transpose loads. Both spread a fragment read over distinct bank
// slots.
#pragma once
#include <type_traits>

#include "qat_device.h"
#include "qat_dma.h"
#include "qat_internal.h"

namespace qat {

// Workgroup id -> output tile. Consecutive workgroup ids go round-robin to the
// 8 XCDs; each XCD gets a contiguous range of tiles, walked in groups of 8
// tile-rows so that neighbouring workgroups share operand tiles in its L2.
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

// Row tiles of a causal product whose contraction ends at its row tile's end
// (kCausalLower: tile m contracts over [0, (m + 1) BM)): boustrophedon order,
// every other group of 8 row tiles reversed, so the XCD that takes a short
// tile in one group takes a long one in the next. With the problem's tiles on
// one XCD (grouped), the longest tiles go first instead (the XCD's CUs take
// workgroups in order as they free up).
__device__ __forceinline__ void causal_tile_of(int b, bool grouped, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int p = b / tiles_n;
  tn = b % tiles_n;
  if (grouped) {
    tm = tiles_m - 1 - p;
    return;
  }
  const int g = p / 8;
  const int end = min(8 * g + 8, tiles_m);
  tm = (g & 1) ? 8 * g + (end - 1 - p) : p;
}

// Workgroup -> (tile id, problem) of a launch. Batched launches whose problem
// count is a multiple of 8 keep all tiles of one problem on one XCD
// (workgroups go round-robin to the 8 XCDs in dispatch order, x fastest), so
// its shared operands are fetched into one L2: in each run of 8 x tiles
// consecutive workgroups, XCD j takes every tile of problem j of the run.
__device__ __forceinline__ void work_of(const GemmArgs& a0, int& tile, int& prob, bool& grouped) {
  tile = blockIdx.x;
  prob = blockIdx.y;
  grouped = a0.batch_h > 0 && (a0.batches & 7) == 0;
  if (grouped) {
    const int nt = gridDim.x;
    const int w = blockIdx.x + blockIdx.y * nt;
    const int r = w % (8 * nt);
    prob = 8 * (w / (8 * nt)) + (r & 7);
    tile = r >> 3;
  }
}

// The problem of a batched launch (see GemmArgs::batch_h).
__device__ __forceinline__ GemmArgs batch_view(const GemmArgs& a0, int z) {
  GemmArgs a = a0;
  if (a.batch_h > 0) {
    const int b = z / a.batch_h, h = z - b * a.batch_h;
    a.A += b * a.sa_b + h * a.sa_h;
    a.B = (const uint16_t*)a.B + b * a.sb_b + h * a.sb_h;
    const int64_t oc = b * a.sc_b + h * a.sc_h;
    if (a.C) a.C += oc;
    if (a.Cf) a.Cf += oc;
  }
  return a;
}

// LDS bank slots (16-byte chunks) served per cycle; the swizzle period. Eight
// measures free of bank conflicts for these fragment reads on gfx950.
constexpr int kLdsSlots = 8;

template <int BK, int SLOTS>
struct LdsLayout {
  static constexpr int CH = BK / 8;                      // 16-byte chunks per row
  static constexpr int PITCH = BK * 2;                   // bytes per row
  static constexpr int RPL = SLOTS / CH > 0 ? SLOTS / CH : 1;
  __device__ static __forceinline__ int off(int row, int chunk) {
    return row * PITCH + ((chunk ^ ((row / RPL) & (CH - 1))) << 4);
  }
};

// ---------------------------------------------------------------------------
// Direct-to-LDS operand tiles (bf16, K-contiguous rows).
// buffer_load_dwordx4 ... lds writes 64 lanes x 16 B = 1 KiB of LDS starting at
// M0; lane l lands at byte 16 l, i.e. row l / CH, chunk position l % CH of the
// instruction's rows, so lane l fetches the logical chunk that the swizzle maps
// to that position. The loads are issued from inline asm because the
// compiler's own LDS-DMA tracking waits for every outstanding DMA before any
// LDS read, which would collapse the multi-stage pipeline; the kernel waits on
// vmcnt itself. Rows at or beyond nrows read as zero (buffer range check).
// ---------------------------------------------------------------------------
// DWD = 1: the same tile by 4-byte DMA (64 lanes x 4 B = 256 B per
// instruction, 4 lanes per 16-byte chunk) for rows that are only 4-byte
// aligned (ld % 8 != 0), and the contraction's tail masked per lane: a dword
// at k >= kdim is fetched from an offset beyond the buffer's range and reads
// as zero, so rows whose kdim is not a multiple of the slab contract over
// exactly kdim elements (kdim even).
template <int ROWS, int BK, int SLOTS, int NW = 4, int DWD = 0>
struct DmaTileK {
  using L = LdsLayout<BK, SLOTS>;
  static constexpr int IB = DWD ? 256 : 1024;            // bytes per DMA instruction
  static constexpr int RPI = IB / L::PITCH;              // rows per DMA instruction
  static constexpr int NI = ROWS / RPI / NW;             // instructions per wave per slab
  static_assert(RPI >= 1 && NI * RPI * NW == ROWS, "tile rows must split over the waves");
  i32x4 rs;
  uint32_t voff[NI];
  uint32_t lrow[NI];                                     // wave-uniform LDS byte offsets
  int kc[DWD ? NI : 1];                                  // DWD: the lane's k within the slab
  int kdim;
  // src is [rows][ld] with K contiguous; rows >= nrows read as zero. The
  // range ends with the last row's kdim-th element, so a view into a wider
  // tensor (one head's columns) reads nothing past that tensor.
  // wave_: the wave's index among the NW loading waves (default: its index
  // in the workgroup).
  __device__ __forceinline__ void init(const uint16_t* src, int64_t ld, int row0, int nrows, int kdim_,
                                       int wave_ = -1) {
    kdim = kdim_;
    rs = buffer_rsrc(src + (int64_t)row0 * ld, ((int64_t)(nrows - 1 - row0) * ld + kdim) * 2);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(wave_ < 0 ? (int)(threadIdx.x >> 6) : wave_);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int r0 = (wave * NI + q) * RPI;
      const int lpc = DWD ? 4 : 1;                       // lanes per 16-byte chunk
      const int row = r0 + lane / (L::CH * lpc);
      const int pos = (lane / lpc) % L::CH;
      const int d = lane % lpc;                          // DWD: dword of the chunk
      const int chunk = pos ^ ((row / L::RPL) & (L::CH - 1));
      voff[q] = (uint32_t)(row * ld * 2 + chunk * 16 + d * 4);
      lrow[q] = (uint32_t)(r0 * L::PITCH);
      if constexpr (DWD) kc[q] = chunk * 8 + d * 2;
    }
  }
  __device__ __forceinline__ void issue_q(uint32_t lds_tile, int k0, int q) const {
    if constexpr (DWD) {
      const uint32_t off = k0 + kc[q] < kdim ? voff[q] + (uint32_t)k0 * 2 : 0x80000000u;
      dma4(rs, lds_tile + lrow[q], off);
    } else {
      dma16(rs, lds_tile + lrow[q], voff[q] + (uint32_t)k0 * 2);
    }
  }
  __device__ __forceinline__ void issue(uint32_t lds_tile, int k0) const {
#pragma unroll
    for (int q = 0; q < NI; ++q) issue_q(lds_tile, k0, q);
  }
  // The same with the slab's column offset in the scalar offset field: rows
  // at or beyond nrows are out of range by their row offset alone.
  __device__ __forceinline__ void issue_so_q(uint32_t lds_tile, int k0, int q) const {
    const uint32_t so = (uint32_t)k0 * 2;
    if constexpr (DWD) dma4s(rs, lds_tile + lrow[q], k0 + kc[q] < kdim ? voff[q] : 0x80000000u, so);
    else dma16s(rs, lds_tile + lrow[q], voff[q], so);
  }
  __device__ __forceinline__ void issue_so(uint32_t lds_tile, int k0) const {
#pragma unroll
    for (int q = 0; q < NI; ++q) issue_so_q(lds_tile, k0, q);
  }
  // Per-lane byte offset of fragment 0 (tile rows r0 .. r0 + 15) for k-step ks.
  // The swizzle term (row / RPL) & (CH - 1) repeats every 16 rows (RPL * CH
  // divides 16), so fragment f of the same k-step sits f * 16 * PITCH further.
  __device__ __forceinline__ static int frag_base(int r0, int ks, int lane) {
    return L::off(r0 + (lane & 15), ks * 4 + (lane >> 4));
  }
  static constexpr int FRAG_STRIDE = 16 * L::PITCH;
  // Fragment of tile row r (= 16 t + (lane & 15)) for k-step ks: 8 consecutive k.
  __device__ __forceinline__ static bf16x8 frag(const uint8_t* tile, int r, int ks, int lane) {
    return *(const bf16x8*)(tile + L::off(r, ks * 4 + (lane >> 4)));
  }
};


// MN-contiguous operand: global [K][ld] with the operand's rows contiguous
// (e.g. dY or X as operands of dY^T X, or W_hat [out][in] as the operand of
// dY W_hat). LDS keeps the natural [BK][ROWS] layout; 16-byte chunk c of k-row
// k sits at position c ^ (2 (k & 3)) ^ (8 ((k >> 3) & 1)): a 64-lane transpose
// read touches k-rows k0 + 8 g + (0..3), g = 0..3, and this spreads them over
// all 64 banks, two dwords each (the minimum for 512 bytes). Fragments are read with
// ds_read_b64_tr_b16: in each 16-lane group, lane j addresses the 4 elements
// (k0 + j / 4, r0 + 4 (j % 4) .. +3) and lane i receives element i % 4 of
// lane 4 e + i / 4's row for e = 0..3, i.e. rows r0 + i at k0 .. k0 + 3. Two
// reads (k0 and k0 + 4) give the same 8 consecutive k as the K-contiguous
// fragment. k-rows at or beyond kdim read as zero; rows beyond the operand's
// extent hold other data and only feed outputs that are never stored.
// DWD = 1: the same tile by 4-byte DMA (256 B of the [BK][ROWS] tile per
// instruction, 4 lanes per 16-byte chunk), for k-rows that are only 4-byte
// aligned (ld % 8 != 0).
template <int ROWS, int BK, int NW = 4, int DWD = 0>
struct DmaTileMN {
  static constexpr int CHR = ROWS / 8;                   // 16-byte chunks per k-row
  static constexpr int PITCH = ROWS * 2;
  static constexpr int IB = DWD ? 256 : 1024;            // bytes per DMA instruction
  static constexpr int NI = BK * PITCH / IB / NW;        // instructions per wave per slab
  static_assert(CHR >= 16 && NI * IB * NW == BK * PITCH && IB % 256 == 0, "tile shape");
  i32x4 rs;
  uint32_t voff[NI];
  uint32_t lrow[NI];
  uint32_t kstride;                                      // bytes per k-row in global memory
  __device__ static __forceinline__ int swz(int k) { return ((k & 3) << 1) ^ (((k >> 3) & 1) << 3); }
  __device__ static __forceinline__ int off(int k, int chunk) { return k * PITCH + ((chunk ^ swz(k)) << 4); }
  // The range ends with the last k-row's row nrows (rounded up to a whole
  // 16-byte chunk), so a view into a wider tensor reads nothing past it.
  __device__ __forceinline__ void init(const uint16_t* src, int64_t ld, int row0, int nrows, int kdim) {
    const int64_t end = min((int64_t)kdim * ld, (int64_t)(kdim - 1) * ld + ((nrows + 7) & ~7));
    rs = buffer_rsrc(src + row0, (end - row0) * 2);
    kstride = (uint32_t)(ld * 2);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int b0 = (wave * NI + q) * IB;               // the instruction's first byte of the tile
      const int b = b0 + lane * (IB / 64);               // this lane's
      const int kr = b / PITCH;
      const int pos = (b % PITCH) / 16;
      const int chunk = pos ^ swz(kr);
      voff[q] = (uint32_t)(kr * ld * 2 + chunk * 16 + (b % 16));
      lrow[q] = (uint32_t)b0;
    }
  }
  __device__ __forceinline__ void issue_q(uint32_t lds_tile, int k0, int q) const {
    if constexpr (DWD) dma4(rs, lds_tile + lrow[q], voff[q] + (uint32_t)k0 * kstride);
    else dma16(rs, lds_tile + lrow[q], voff[q] + (uint32_t)k0 * kstride);
  }
  __device__ __forceinline__ void issue(uint32_t lds_tile, int k0) const {
#pragma unroll
    for (int q = 0; q < NI; ++q) issue_q(lds_tile, k0, q);
  }
  // The lane's byte offset, within the tile, of its first read of the
  // fragment of rows r0 .. r0 + 15 (r0 a multiple of 16) at k-step 0. The
  // second read (k + 4) lies 4 k-rows further and k-step ks 32 ks k-rows
  // further, both at a constant distance: the lane's k-row differs from kb
  // only in bits 2 and 5, which the swizzle does not use.
  __device__ __forceinline__ static int frag_off(int r0, int lane) {
    const int j = lane & 15;
    const int kb = 8 * (lane >> 4) + (j >> 2);
    const int e = r0 + 4 * (j & 3);
    return off(kb, e >> 3) + ((e >> 2) & 1) * 8;
  }
  // The fragment whose first read is at p (tile + frag_off + 32 ks PITCH).
  __device__ __forceinline__ static bf16x8 frag_at(const uint8_t* p) {
    const __attribute__((address_space(3))) uint8_t* t = (const __attribute__((address_space(3))) uint8_t*)p;
    typedef short i16x4_ __attribute__((ext_vector_type(4)));
    const i16x4_ lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_*)t);
    const i16x4_ hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_*)(t + 4 * PITCH));
    typedef short i16x8_ __attribute__((ext_vector_type(8)));
    const i16x8_ v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  }
  __device__ __forceinline__ static bf16x8 frag(const uint8_t* tile, int r, int ks, int lane) {
    const int j = lane & 15;
    const int kb = ks * 32 + 8 * (lane >> 4) + (j >> 2);
    const int e = (r & ~15) + 4 * (j & 3);                  // first of the 4 elements this lane addresses
    const int c = e >> 3, half = (e >> 2) & 1;
    const __attribute__((address_space(3))) uint8_t* t = (const __attribute__((address_space(3))) uint8_t*)tile;
    typedef short i16x4_ __attribute__((ext_vector_type(4)));
    const i16x4_ lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_*)(t + off(kb, c) + half * 8));
    const i16x4_ hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_*)(t + off(kb + 4, c) + half * 8));
    typedef short i16x8_ __attribute__((ext_vector_type(8)));
    const i16x8_ v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  }
};

template <int ROWS, int BK, int MN, int NW = 4>
struct DmaTileOf { using T = DmaTileK<ROWS, BK, kLdsSlots, NW>; };
template <int ROWS, int BK, int NW>
struct DmaTileOf<ROWS, BK, kMNContig, NW> { using T = DmaTileMN<ROWS, BK, NW>; };
template <int ROWS, int BK, int NW>
struct DmaTileOf<ROWS, BK, kKContigD, NW> { using T = DmaTileK<ROWS, BK, kLdsSlots, NW, 1>; };
template <int ROWS, int BK, int NW>
struct DmaTileOf<ROWS, BK, kMNContigD, NW> { using T = DmaTileMN<ROWS, BK, NW, 1>; };

// K-contiguous operand layouts (read as [rows][BK] fragments), as opposed to
// the MN-contiguous ones (read with transpose loads).
constexpr bool k_contig(int layout) { return layout == kKContig || layout == kKContigD; }

// The quantiser of the fused loaders, on its fast path: u = w * rcp with rcp
// = v_rcp_f32(s) (within an ulp of 1/s), so |u - w/s| < 2^-22.4 |w/s| and
// |u - fl32(w/s)| < 2^-21.7 |w/s|; q - zr = med3(rint(u), -zr, K - zr)
// (exactly clamp(rint(u) + zr, 0, K) - zr, small integers); W_hat =
// fma(q - zr, s, +0), one rounding of the exact product like (q - zr) * s,
// with +0 where that product is a zero (as the subtraction q - zr gives).
// With K <= 15 and 0 <= zr <= K the code depends on rint only where |w/s| <
// 16.5 (beyond, both neighbouring integers clamp to the same end), and there
// u is within 2^-17.7 of fl32(w/s): rint(u) can differ from the correctly
// rounded quotient's only if |u - rint(u)| >= 0.5 - 2^-17 (a near-tie, also
// set for non-finite u). The caller redoes near-ties with quant_elem (the
// exact division), so the codes are exactly the fp32 quantiser's. Callers
// keep the running maximum of |u - rint(u)| (v_maximum3, which propagates a
// NaN, two weights per instruction) and take the rare path when any lane's
// maximum fails the margin: five and a half VALU operations per weight and
// one ballot per slab.
constexpr float kNearTie = 0.5f - 0x1p-17f;

struct QRow {
  float s, rcp, zr, lo, hi;
};

__device__ __forceinline__ QRow qrow(float s, float z, float K) {
  QRow r;
  r.s = s;
  r.rcp = __builtin_amdgcn_rcpf(s);
  r.zr = round_clamp_zero(z, K);
  r.lo = -r.zr;
  r.hi = K - r.zr;
  return r;
}

// W_hat on the fast path; res = |u - rint(u)| (the near-tie measure).
__device__ __forceinline__ float qfast(float w, const QRow& r, float& res) {
  const float u = w * r.rcp;
  const float ru = __builtin_rintf(u);
  res = __builtin_fabsf(u - ru);
  return __builtin_fmaf(__builtin_amdgcn_fmed3f(ru, r.lo, r.hi), r.s, 0.0f);
}

// Whether any lane of the wave saw a near-tie (or a non-finite u): m is the
// lane's running maximum of the residuals (NaN if one was NaN).
__device__ __forceinline__ bool wave_near_tie(float m) {
  return __builtin_amdgcn_ballot_w64(!(m < kNearTie)) != 0;
}

// The near-tie test of qfast alone (the rare path's per-element decision).
__device__ __forceinline__ bool qnear_tie(float w, const QRow& r) {
  const float u = w * r.rcp;
  return !(__builtin_fabsf(u - __builtin_rintf(u)) < kNearTie);
}

// Two floats to bf16 (round to nearest even) in one v_cvt_pk_bf16_f32, lo in bits 0-15.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  typedef float f2_ __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_ __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_{lo, hi}, b2_));
}

// bf16 W_hat = bf16(fl32((q - z) s)) of 2-bit codes by table: the group's
// four values are made once per call, with the per-element arithmetic, and
// v_perm_b32 (byte k of {S0, S1} is byte k of S1 for k < 4, of S0 - 4 for
// k >= 4) picks each pair's two bf16 from them. lo holds the low bytes of the
// four values, hi their high bytes; for codes (a, b) (4 bits t = a + 4 b) the
// selector bytes are (a, 4 + a, b, 4 + b): t times 1 + 2^8 + 2^14 + 2^22 puts
// copies of t at bits 0, 8, 14 and 22 (disjoint, no carries), the mask keeps
// a at bits 0-1 and 8-9 and b at bits 16-17 and 24-25. Four VALU operations
// per pair instead of an extraction, a conversion, a subtraction and a
// multiplication per code. x: codes LSB-first from bit 0; dword m of o is
// codes 2m, 2m + 1 (the first in the low half); dead (live false) gives +0.
template <int NP>
__device__ __forceinline__ void lut2_pairs(uint32_t x, float sv, float zv, bool live, uint32_t (&o)[NP]) {
  const uint32_t p01 = pack2_bf16((0.f - zv) * sv, (1.f - zv) * sv);
  const uint32_t p23 = pack2_bf16((2.f - zv) * sv, (3.f - zv) * sv);
  const uint32_t lo = live ? __builtin_amdgcn_perm(p23, p01, 0x06040200u) : 0u;
  const uint32_t hi = live ? __builtin_amdgcn_perm(p23, p01, 0x07050301u) : 0u;
  // the mask in an SGPR and the high-half bits in a VGPR (opaque to the
  // compiler, so that the two fold into one v_and_or_b32, whose VOP3 form
  // takes no literals)
  uint32_t kmask, kor;
  asm("s_mov_b32 %0, 0x03030303" : "=s"(kmask));
  asm("v_mov_b32 %0, 0x04000400" : "=v"(kor));
#pragma unroll
  for (int m = 0; m < NP; ++m) {
    const uint32_t t = (x >> (4 * m)) & 15u;
    const uint32_t sel = ((t * 0x00404101u) & kmask) | kor;
    o[m] = __builtin_amdgcn_perm(hi, lo, sel);
  }
}

// A DMA instruction index of a slab loaded by 4 waves: instruction q of wave
// cw; where the slab has fewer instructions than 4 x NI the last one repeats
// (the same bytes to the same place), so every wave issues NI.
template <int NTOT, int NI>
__device__ __forceinline__ int dma_index(int cw, int q) {
  return min(cw * NI + q, NTOT - 1);
}

// The forward's weight operand without an LDS ring: each of the 256 converter
// threads owns WPT weights of one row (a BN-row tile: TPR = 256 / BN threads
// per row, WPT = 32 / TPR: row tid / TPR, weights WPT (tid % TPR) .. of every
// 32-wide slab) and loads them straight into registers -- fp32: WPT / 4
// 16-byte loads; packed codes: the row's whole 4 N-byte slab (the TPR threads
// of a row load it, one instruction) -- several slabs ahead of their
// conversion. The loads are the compiler's own (it waits for them before the
// conversion reads the registers); rows at or beyond nrows read as zero
// through the buffer range, the slab's offset rides in the scalar offset.
template <int KIND, int NB, int WPT>
struct WSlab {
  static constexpr int ND = KIND == kPacked ? NB : WPT;  // dwords per thread and slab
  uint32_t d[ND];
};

template <int KIND, int NB, int WPT>
struct WRowLoader {
  static constexpr int TPR = 32 / WPT;                    // threads per weight row
  static constexpr int NL = KIND == kPacked ? 1 : WPT / 4; // load instructions per slab
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff;
  __device__ __forceinline__ void init(const void* W, int64_t row_bytes, int row0, int nrows, int tid) {
    int64_t n = (int64_t)(nrows - row0) * row_bytes;
    n = n < 0 ? 0 : (n > 0x7FFFFFF0 ? 0x7FFFFFF0 : n);
    rs = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)W + (int64_t)row0 * row_bytes), (short)0,
                                           (int)n, 0x00020000);
    const int row = tid / TPR, q = tid % TPR;
    voff = (uint32_t)(row * row_bytes) + (KIND == kPacked ? 0u : (uint32_t)(q * WPT * 4));
  }
  __device__ __forceinline__ void load(WSlab<KIND, NB, WPT>& w, int k0) const {
    typedef int v4i_ __attribute__((ext_vector_type(4)));
    typedef int v3i_ __attribute__((ext_vector_type(3)));
    typedef int v2i_ __attribute__((ext_vector_type(2)));
    if constexpr (KIND == kPacked) {
      const int so = k0 * NB / 8;
      if constexpr (NB == 2) {
        const v2i_ v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)voff, so, 0);
        w.d[0] = v.x, w.d[1] = v.y;
      } else if constexpr (NB == 3) {
        const v3i_ v = __builtin_amdgcn_raw_buffer_load_b96(rs, (int)voff, so, 0);
        w.d[0] = v.x, w.d[1] = v.y, w.d[2] = v.z;
      } else {
        const v4i_ v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, so, 0);
        w.d[0] = v.x, w.d[1] = v.y, w.d[2] = v.z, w.d[3] = v.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < WPT / 4; ++j) {
        const v4i_ v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff + 16 * j, k0 * 4, 0);
        w.d[4 * j] = v.x, w.d[4 * j + 1] = v.y, w.d[4 * j + 2] = v.z, w.d[4 * j + 3] = v.w;
      }
    }
  }
};

// The rows' s and z in chunks of CG = 4 consecutive groups: s[ROWS][CG] then
// z[ROWS][CG], 16 rows x 4 groups per dword DMA instruction (16 cache lines,
// where one group's ROWS values would touch ROWS / 4 per instruction), into
// one of three chunk entries, issued with the weights of the chunk's first
// slab. A slab lies inside one group (groups of 32, 64, 128 or a whole row).
template <int ROWS>
struct SzChunks {
  static constexpr int CG = 4;
  static constexpr int SZ_BYTES = 2 * ROWS * CG * 4, ENTRIES = 3;
  static constexpr int NC = SZ_BYTES / 256, NI = NC / 4;   // instructions per chunk, per converter wave
  static_assert(NI * 4 == NC, "chunk shape");
  i32x4 rsz[2];
  uint32_t vc[NI], dc[NI];
  int which[NI];
  int group;
  float K;
  FastDiv gdiv;
  __device__ __forceinline__ void init(const float* s, const float* z, int row0, int nrows, int64_t G, int group_,
                                       float K_, int cw) {
    group = group_;
    K = K_;
    gdiv = FastDiv::make((uint32_t)group_);
    rsz[0] = buffer_rsrc(s + (int64_t)row0 * G, (int64_t)(nrows - row0) * G * 4);
    rsz[1] = buffer_rsrc(z + (int64_t)row0 * G, (int64_t)(nrows - row0) * G * 4);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int idx = cw * NI + q;                                       // 0 .. NC - 1
      const int r = (idx % (NC / 2)) * 16 + lane / CG;                   // row of the chunk
      which[q] = idx / (NC / 2);                                         // 0: s, 1: z (uniform)
      // groups past a row's end read the next row's (never used) or, at the
      // last row, zeros (buffer range); the group offset stays per lane
      vc[q] = (uint32_t)((r * G + lane % CG) * 4);
      dc[q] = (uint32_t)(idx * 256);
    }
  }
  // The chunk DMA if the slab at k0 starts a chunk.
  __device__ __forceinline__ void issue(uint32_t lds_sz, int k0) const {
    const int g = (int)gdiv.div((uint32_t)k0);
    if (g % CG == 0 && k0 == g * group) {
      const uint32_t e = lds_sz + (uint32_t)(((g / CG) % ENTRIES) * SZ_BYTES);
#pragma unroll
      for (int q = 0; q < NI; ++q) {
        i32x4 r = which[q] ? rsz[1] : rsz[0];
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = __builtin_amdgcn_readfirstlane(r[j]);
        dma4(r, e + dc[q], vc[q] + (uint32_t)g * 4);
      }
    }
  }
  // Byte offset in LDS of row's s for the slab at k0 (z sits ROWS CG 4 further).
  __device__ __forceinline__ int at(int sz, int row, int k0) const {
    const int g = (int)gdiv.div((uint32_t)k0);
    return sz + ((g / CG) % ENTRIES) * SZ_BYTES + row * (CG * 4) + (g % CG) * 4;
  }
};

// One converter thread's WPT weights of the slab (registers w) into the
// K-contiguous bf16 B stage at byte b (row tid / TPR, 8-weight chunks
// (WPT / 8) (tid % TPR) ..): packed, W_hat = (q - z) s with z as stored;
// fp32, Eq. 1 then Eq. 2 by qfast, near-ties redone by quant_elem.
template <int KIND, int NB, int WPT>
__device__ __forceinline__ void convert_slab(const WSlab<KIND, NB, WPT>& w, float sv, float zv, float K,
                                             uint8_t* smem, int b, int tid) {
  using L = LdsLayout<32, kLdsSlots>;
  constexpr int TPR = 32 / WPT;
  const int row = tid / TPR, q = tid % TPR;
  float h[WPT];
  if constexpr (KIND == kPacked) {
    // this thread's WPT codes start at bit WPT N q of the row's slab; selects
    // (not an index) pick the two dwords around them, so the slab stays in
    // registers (the empty asm keeps the dwords values, so that the selects
    // are not turned back into an indexed load, which would move the slabs
    // to LDS)
    uint32_t d[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      d[i] = w.d[i];
      asm volatile("" : "+v"(d[i]));
    }
    const int bit = q * WPT * NB, k = bit >> 5;
    uint32_t lo = d[0], hi = NB > 1 ? d[1] : 0u;
#pragma unroll
    for (int i = 1; i < NB; ++i) {
      lo = k == i ? d[i] : lo;
      hi = k + 1 == i ? d[i] : hi;
    }
    const uint64_t x = ((uint64_t)hi << 32 | lo) >> (bit & 31);
    if constexpr (NB == 2) {
      uint32_t o[WPT / 2];
      lut2_pairs<WPT / 2>((uint32_t)x, sv, zv, true, o);
#pragma unroll
      for (int m = 0; m < WPT / 8; ++m)
        *(uint4*)&smem[b + L::off(row, (WPT / 8) * q + m)] = make_uint4(o[4 * m], o[4 * m + 1], o[4 * m + 2],
                                                                        o[4 * m + 3]);
      return;
    }
#pragma unroll
    for (int e = 0; e < WPT; ++e) h[e] = ((float)(uint32_t)((x >> (NB * e)) & ((1u << NB) - 1)) - zv) * sv;
  } else {
    const QRow r = qrow(sv, zv, K);
    float res[WPT];
#pragma unroll
    for (int e = 0; e < WPT; ++e) h[e] = qfast(__builtin_bit_cast(float, w.d[e]), r, res[e]);
    float m = res[0];                                          // the lane's largest residual
#pragma unroll
    for (int e = 1; e < WPT; ++e) m = __builtin_elementwise_maximum(m, res[e]);
    if (wave_near_tie(m)) {                                    // near a rounding tie: exact division
#pragma unroll
      for (int e = 0; e < WPT; ++e) {
        float wt = __builtin_bit_cast(float, w.d[e]);
        rare_branch(wt);
        if (qnear_tie(wt, r)) h[e] = quant_elem(wt, sv, r.zr, K).w_hat;
      }
    }
  }
#pragma unroll
  for (int m = 0; m < WPT / 8; ++m)
    *(uint4*)&smem[b + L::off(row, (WPT / 8) * q + m)] =
        make_uint4(pack2_bf16(h[8 * m], h[8 * m + 1]), pack2_bf16(h[8 * m + 2], h[8 * m + 3]),
                   pack2_bf16(h[8 * m + 4], h[8 * m + 5]), pack2_bf16(h[8 * m + 6], h[8 * m + 7]));
}

// The weight as the B operand of dX = dY W_hat without an LDS ring: B[n][k] =
// W_hat[k][n], so a slab is BK = 32 weight rows k0 .. k0 + 31 (the
// contraction) by ROWS = 128 weight columns n0 .. (dX's columns). Converter
// thread tid (0..255) owns row k0 + tid / 8 and its 16 columns n0 + 16
// (tid % 8) .., loaded straight into registers -- fp32: four 16-byte loads;
// packed codes: the 2 N bytes that hold them (one or two dwords) -- with the
// row's s and z of their group (a group of 32 or more columns holds all 16).
// Every offset, the slab's row included, is in the per-lane offset, so rows
// at or beyond kdim are out of the buffer's range and read as zero; the
// conversion zeroes them. Columns at or beyond the weight's width only feed
// dX columns that are never stored.
template <int KIND, int NB>
struct WColSlab {
  static constexpr int ND = KIND == kPacked ? (NB == 2 ? 1 : 2) : 16;
  uint32_t d[ND];
  float s, z;
};

template <int KIND, int NB>
struct WColLoader {
  static constexpr int NL = (KIND == kPacked ? 1 : 4) + 2;  // load instructions per slab
  __amdgpu_buffer_rsrc_t rw, rs, rz;
  uint32_t vw, vsz;
  uint32_t wrow, grow;                                     // bytes per weight row, per (s, z) row
  int sh;                                                  // 3-bit codes: bit of the first code in d
  __device__ __forceinline__ void init(const void* W, int64_t row_bytes, int n0, int kdim, const float* s,
                                       const float* z, int64_t G, int group, int tid) {
    const int r = tid / 8, c16 = tid % 8;
    wrow = (uint32_t)row_bytes;
    grow = (uint32_t)(G * 4);
    const int64_t cb = KIND == kPacked ? (int64_t)n0 * NB / 8 : (int64_t)n0 * 4;
    int64_t n = (int64_t)kdim * row_bytes - cb;
    n = n < 0 ? 0 : (n > 0x7FFFFFF0 ? 0x7FFFFFF0 : n);
    rw = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)W + cb), (short)0, (int)n, 0x00020000);
    int64_t ns = (int64_t)kdim * G * 4;
    ns = ns > 0x7FFFFFF0 ? 0x7FFFFFF0 : ns;
    rs = __builtin_amdgcn_make_buffer_rsrc((void*)s, (short)0, (int)ns, 0x00020000);
    rz = __builtin_amdgcn_make_buffer_rsrc((void*)z, (short)0, (int)ns, 0x00020000);
    if constexpr (KIND == kPacked) {
      const int bit = c16 * 16 * NB;
      vw = (uint32_t)(r * row_bytes + (bit >> 5) * 4);
      sh = bit & 31;
    } else {
      vw = (uint32_t)(r * row_bytes + c16 * 64);
      sh = 0;
    }
    vsz = (uint32_t)(r * G * 4 + (int64_t)((n0 + 16 * c16) / group) * 4);
  }
  __device__ __forceinline__ void load(WColSlab<KIND, NB>& w, int k0) const {
    typedef int v4i_ __attribute__((ext_vector_type(4)));
    typedef int v2i_ __attribute__((ext_vector_type(2)));
    const uint32_t ow = vw + (uint32_t)k0 * wrow;
    if constexpr (KIND == kPacked) {
      if constexpr (NB == 2) {
        w.d[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rw, (int)ow, 0, 0);
      } else {
        const v2i_ v = __builtin_amdgcn_raw_buffer_load_b64(rw, (int)ow, 0, 0);
        w.d[0] = v.x, w.d[1] = v.y;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4i_ v = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(ow + 16 * j), 0, 0);
        w.d[4 * j] = v.x, w.d[4 * j + 1] = v.y, w.d[4 * j + 2] = v.z, w.d[4 * j + 3] = v.w;
      }
    }
    const uint32_t os = vsz + (uint32_t)k0 * grow;
    w.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (int)os, 0, 0));
    w.z = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rz, (int)os, 0, 0));
  }
};

// One converter thread's 16 weights of a slab row as bf16 W_hat (pk, two
// 16-byte pieces of 8 columns): packed, W_hat = (q - z) s with z as stored;
// fp32, Eq. 1 then Eq. 2 by qfast, near-ties redone by quant_elem; zero for a
// row at or beyond the contraction's end (live false).
template <int KIND, int NB>
__device__ __forceinline__ void convert_cols(const WColSlab<KIND, NB>& w, float K, bool live, int sh,
                                             uint4 (&pk)[2]) {
  float h[16];
  if constexpr (KIND == kPacked && NB == 2) {
    uint32_t o[8];
    lut2_pairs<8>(w.d[0], w.s, w.z, live, o);
    pk[0] = make_uint4(o[0], o[1], o[2], o[3]);
    pk[1] = make_uint4(o[4], o[5], o[6], o[7]);
    return;
  }
  if constexpr (KIND == kPacked) {
    uint64_t x;
    if constexpr (NB == 2) x = w.d[0];
    else if constexpr (NB == 3) x = ((uint64_t)w.d[1] << 32 | w.d[0]) >> sh;
    else x = (uint64_t)w.d[1] << 32 | w.d[0];
#pragma unroll
    for (int e = 0; e < 16; ++e) h[e] = ((float)(uint32_t)((x >> (NB * e)) & ((1u << NB) - 1)) - w.z) * w.s;
  } else {
    const QRow r = qrow(w.s, w.z, K);
    float res[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) h[e] = qfast(__builtin_bit_cast(float, w.d[e]), r, res[e]);
    float m = res[0];                                          // the lane's largest residual
#pragma unroll
    for (int e = 1; e < 16; ++e) m = __builtin_elementwise_maximum(m, res[e]);
    if (wave_near_tie(m)) {                                    // near a rounding tie: exact division
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float wt = __builtin_bit_cast(float, w.d[e]);
        rare_branch(wt);
        if (qnear_tie(wt, r)) h[e] = quant_elem(wt, w.s, r.zr, K).w_hat;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) h[e] = live ? h[e] : 0.0f;
#pragma unroll
  for (int m = 0; m < 2; ++m)
    pk[m] = make_uint4(pack2_bf16(h[8 * m], h[8 * m + 1]), pack2_bf16(h[8 * m + 2], h[8 * m + 3]),
                       pack2_bf16(h[8 * m + 4], h[8 * m + 5]), pack2_bf16(h[8 * m + 6], h[8 * m + 7]));
}


// Four consecutive codes c0..c0+3 (c0 % 4 == 0) of a packed row.
template <int NB>
__device__ __forceinline__ uint32_t codes4(const uint8_t* __restrict__ row, int64_t c0) {
  const int64_t bit = c0 * NB;
  if constexpr (NB == 2) return row[bit >> 3];
  else if constexpr (NB == 4) return *(const uint16_t*)(row + (bit >> 3));
  else {
    const uint32_t lo = row[bit >> 3], hi = row[(bit >> 3) + 1];
    return ((lo | (hi << 8)) >> (bit & 7)) & 0xFFFu;
  }
}

template <int TI, int TJ>
struct Frags {
  bf16x8 a[TI], b[TJ];
};

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// v_mfma_f32_16x16x32_bf16 with the accumulator pinned to AGPRs: keeps the
// register allocator from mixing accumulators and fragments in one class
// (which spills at 128x128 accumulators per wave). The hazard recogniser does
// not look inside the asm, so code that reads the accumulators afterwards
// first waits out the MFMA latency (mfma_drain).
__device__ __forceinline__ void mfma_acc(f32x4& c, const bf16x8& b, const bf16x8& a) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
}
// Waits out the MFMA write-back latency before the epilogue reads the
// accumulators; the scheduling fence keeps every later instruction (the
// accumulator reads included) after the wait.
__device__ __forceinline__ void mfma_drain() {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// Epilogues. acc[j][i] holds C[m0 + wm0 + 16 i + (lane & 15)][n0 + wn0 + 16 j
// + 4 (lane >> 4) + r], r = 0..3.
//   kStoreBf16:    C (bf16) = acc.
//   kResidMse:     y = resid + acc, dy = bf16(escale (y - target)), and the
//                  workgroup's sum of (y - target)^2.
//   kStoreF32:     Cf (fp32) = acc.
//   kSteGrads:     rows are weight rows o (A = dY^T), columns inputs c (B =
//                  X^T); Gw = acc. dW = Gw * m and the group sums of ds, dz of
//                  the straight-through estimator, from W, s, z re-quantised
//                  here (quant_elem).
//   kE2eScaleGrad: as above with packed codes: ds = sum Gw (q - z), dz = -s
//                  sum Gw.
// A 64-column quantisation group is 4 j-tiles x 4 registers of one lane plus a
// reduction over the 4 lanes that share (lane & 15).
// ---------------------------------------------------------------------------
// Inputs of one (row, 64-column chunk) step of the gradient epilogues: the
// chunk's group(s) s and z (two groups when groups are 32 wide).
template <int EP>
struct EpiIn {
  float s[2], z[2];
  float4 w[4];          // kSteGrads: W[o][cg + 16 jj + cq .. + 3]
  uint32_t c[4];        // kE2eScaleGrad: the same four codes per jj
};

// Group modes of the gradient epilogues (GM): 0 groups of 64 columns, one per
// chunk; 1 groups of 32, two per chunk (j-tiles 0-1 and 2-3); 2 groups of
// 64 c columns that tile BN (128, or a whole row no wider than the tile): the
// chunk sums meet in LDS (`red`, free once the main loop has drained) and
// one thread per (row, group) adds the group's c chunks and stores; 3 whole
// rows wider than the tile: the same LDS sum over all of the tile's chunks,
// then one atomic add per row and tile into ds and dz, which the launcher
// zero-fills first.
template <int EP, int NB, int GM, int BM, int BN, int TI, int TJ, int WN>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& a, const f32x4 (&acc)[TJ][TI], int m0, int n0,
                                              int wm0, int wn0, int lane, float* red) {
  const int rl = lane & 15, cq = 4 * (lane >> 4);
  if constexpr (EP == kResidMse) {
    // y = resid + product, d = y - target, dy = bf16(escale d), 4 consecutive
    // columns per lane; resid and target of the next 16-row step are in flight
    // while this one is computed. Rows and columns beyond
    // the problem are clamped for the loads and skipped for the stores.
    struct Row {
      uint2 t[TJ];
      float4 r[TJ];
    };
    auto load_row = [&](int i, Row& r) {
      const int row = min(m0 + wm0 + i * 16 + rl, a.M - 1);
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int64_t at = (int64_t)row * a.ldc + min(n0 + wn0 + j * 16 + cq, a.N - 4);
        r.t[j] = *(const uint2*)(a.target + at);
        r.r[j] = *(const float4*)(a.resid + at);
      }
    };
    float sq = 0.f;                                      // this lane's sum of d^2
    Row cur, nxt;
    load_row(0, cur);
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      if (i + 1 < TI) load_row(i + 1, nxt);
      const int row = m0 + wm0 + i * 16 + rl;
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int col = n0 + wn0 + j * 16 + cq;
        if (row >= a.M || col >= a.N) continue;
        const int64_t at = (int64_t)row * a.ldc + col;
        const uint2 tb = cur.t[j];
        const float4 rv = cur.r[j];
        const float t[4] = {__builtin_bit_cast(float, tb.x << 16), __builtin_bit_cast(float, tb.x & 0xFFFF0000u),
                            __builtin_bit_cast(float, tb.y << 16), __builtin_bit_cast(float, tb.y & 0xFFFF0000u)};
        const float y[4] = {rv.x + acc[j][i][0], rv.y + acc[j][i][1], rv.z + acc[j][i][2], rv.w + acc[j][i][3]};
        float dd[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dd[e] = y[e] - t[e];
          sq += dd[e] * dd[e];
        }
        if (a.Cf) *(float4*)(a.Cf + at) = make_float4(y[0], y[1], y[2], y[3]);
        *(uint2*)(a.C + at) = make_uint2(pack_bf16x2(a.escale * dd[0], a.escale * dd[1]),
                                         pack_bf16x2(a.escale * dd[2], a.escale * dd[3]));
      }
      cur = nxt;
    }
    // the tile's sum over lanes (shuffles), then over the waves in wave order
    // (LDS): the same partial from run to run
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o);
    const int wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
    if (lane == 0) red[wave] = sq;
    __syncthreads();
    if (threadIdx.x == 0) {
      float t = 0.f;
      for (int w = 0; w < nwave; ++w) t += red[w];
      a.partial[blockIdx.x] = t;
    }
  } else if constexpr (EP == kStoreF32) {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int row = m0 + wm0 + i * 16 + rl;
      if (row >= a.M) continue;
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int col = n0 + wn0 + j * 16 + cq;
        if (col < a.N)
          *(float4*)(a.Cf + (int64_t)row * a.ldc + col) = make_float4(acc[j][i][0], acc[j][i][1], acc[j][i][2], acc[j][i][3]);
      }
    }
  } else if constexpr (EP == kStoreBf16) {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int row = m0 + wm0 + i * 16 + rl;
      if (row >= a.M) continue;
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int col = n0 + wn0 + j * 16 + cq;
        if (col < a.N)
          *(uint2*)(a.C + (int64_t)row * a.ldc + col) =
              make_uint2(pack_bf16x2(acc[j][i][0], acc[j][i][1]), pack_bf16x2(acc[j][i][2], acc[j][i][3]));
      }
    }
  } else {
    static_assert(EP == kSteGrads || EP == kE2eScaleGrad, "every other epilogue has its own branch");
    // Rows are weight rows o (A = dY^T), columns inputs c (B = X^T). Steps
    // t = (i, g) walk the lane's rows and 64-column chunks; the loads of step
    // t + 1 are issued before step t is computed.
    constexpr int NG = WN / 64;
    constexpr int NT = TI * NG;
    constexpr int NH = GM == 1 ? 2 : 1;                  // groups per chunk
    const FastDiv gdiv = FastDiv::make((uint32_t)a.group);
    auto row_of = [&](int t) { return m0 + wm0 + (t / NG) * 16 + rl; };
    auto col_of = [&](int t) { return n0 + wn0 + (t % NG) * 64; };
    auto group_of = [&](int o, int cg) -> int64_t {     // first group of the chunk at column cg
      if constexpr (GM == 0) return (int64_t)o * a.G + cg / 64;
      else if constexpr (GM == 1) return (int64_t)o * a.G + cg / 32;
      else return (int64_t)o * a.G + gdiv.div((uint32_t)cg);
    };
    auto load = [&](int t, EpiIn<EP>& in) {
      const int o = row_of(t), cg = col_of(t);
      if (o < a.M && cg < a.N) {
        const int64_t gi = group_of(o, cg);
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          in.s[h] = a.s[gi + h];
          in.z[h] = a.z[gi + h];
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          if constexpr (EP == kSteGrads) in.w[jj] = *(const float4*)(a.W + (int64_t)o * a.ldw + cg + jj * 16 + cq);
          else in.c[jj] = codes4<NB>(a.Wq + (int64_t)o * a.ldq, cg + jj * 16 + cq);
        }
      }
    };
    EpiIn<EP> cur, nxt;
    load(0, cur);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t + 1 < NT) load(t + 1, nxt);
      const int i = t / NG, g = t % NG;
      const int o = row_of(t), cg = col_of(t);
      const bool ok = o < a.M && cg < a.N;
      const int64_t gi = ok ? group_of(o, cg) : 0;
      float ps[NH], pz[NH];
#pragma unroll
      for (int h = 0; h < NH; ++h) ps[h] = pz[h] = 0.f;
      if (ok) {
        if constexpr (EP == kSteGrads) {
          float zr[NH], rcp[NH];
#pragma unroll
          for (int h = 0; h < NH; ++h) {
            zr[h] = round_clamp_zero(cur.z[h], a.Kq);
            rcp[h] = 1.0f / cur.s[h];
          }
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int h = NH == 2 ? (jj >> 1) : 0;
            const f32x4 gw = acc[g * 4 + jj][i];
            const float wv[4] = {cur.w[jj].x, cur.w[jj].y, cur.w[jj].z, cur.w[jj].w};
            float dw[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const QElem e = quant_elem_rcp(wv[r], cur.s[h], rcp[h], zr[h], a.Kq);
              dw[r] = e.m ? gw[r] : 0.0f;
              ps[h] += gw[r] * (e.m ? (__builtin_rintf(e.u) - e.u) : (e.q - zr[h]));
              pz[h] += e.m ? 0.0f : gw[r];
            }
            const int64_t wi = (int64_t)o * a.ldw + cg + jj * 16 + cq;
            if (a.dW) *(float4*)(a.dW + wi) = make_float4(dw[0], dw[1], dw[2], dw[3]);
          }
        } else {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int h = NH == 2 ? (jj >> 1) : 0;
            const f32x4 gw = acc[g * 4 + jj][i];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float qv = (float)((cur.c[jj] >> (NB * r)) & ((1u << NB) - 1));
              ps[h] += gw[r] * (qv - cur.z[h]);
              pz[h] += gw[r];
            }
          }
        }
      }
      // the 4 lanes with the same (lane & 15) hold the 4 column quarters of the chunk
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        ps[h] += __shfl_xor(ps[h], 16);
        ps[h] += __shfl_xor(ps[h], 32);
        pz[h] += __shfl_xor(pz[h], 16);
        pz[h] += __shfl_xor(pz[h], 32);
      }
      if constexpr (GM >= 2) {
        // every (chunk, row) slot of the tile is written, zeros outside the problem
        if (lane < 16) {
          const int c = wn0 / 64 + g, r = wm0 + i * 16 + rl;
          red[c * BM + r] = ps[0];
          red[(BN / 64 + c) * BM + r] = pz[0];
        }
      } else if (ok && lane < 16 && a.ds) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          a.ds[gi + h] = ps[h];
          if (a.dz) a.dz[gi + h] = -cur.s[h] * pz[h];
        }
      }
      cur = nxt;
    }
    if constexpr (GM >= 2) {
      __syncthreads();
      constexpr int NC = BN / 64;
      const int cpg = GM == 2 ? a.group / 64 : NC;       // chunks per output
      const int n_out = BM * (NC / cpg);
      for (int idx = threadIdx.x; idx < n_out; idx += (int)blockDim.x) {
        const int r = idx % BM, c0 = (idx / BM) * cpg;
        const int o = m0 + r, col = n0 + c0 * 64;
        if (o >= a.M || col >= a.N || !a.ds) continue;
        float S = 0.f, Z = 0.f;
        for (int c = c0; c < c0 + cpg; ++c) {
          S += red[c * BM + r];
          Z += red[(NC + c) * BM + r];
        }
        const int64_t gi = (int64_t)o * a.G + gdiv.div((uint32_t)col);
        const float dz = -a.s[gi] * Z;
        if constexpr (GM == 2) {
          a.ds[gi] = S;
          if (a.dz) a.dz[gi] = dz;
        } else {
          atomicAdd(a.ds + gi, S);
          if (a.dz) atomicAdd(a.dz + gi, dz);
        }
      }
    }
  }
}

// Nontemporal 16-byte accesses: the AdamW stream (W, its moments and dW) is
// touched once per step, so it bypasses the caches' retention and leaves L2
// and the MALL to the operands of the products around it (measured: the
// Block-AP step 5.86 -> 5.61 ms, the gradient products 2.48 -> 2.35 ms).
__device__ __forceinline__ float4 nt_load4(const float* p) {
  const f32x4 t = __builtin_nontemporal_load((const f32x4*)p);
  return make_float4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void nt_store4(float* p, const float (&v)[4]) {
  __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, (f32x4*)p);
}

// ---------------------------------------------------------------------------
// kSteAdam epilogue, row by row. Once the main loop has drained, the LDS is
// free: the accumulators of one wave-row of the tile (WM rows x 256 columns,
// fp32, 128 KiB at 256x256) are written there, then every wave takes whole
// rows, one 16-byte column quad per lane, so that each access to W, m, v (and
// dW) is one contiguous KiB of the row and PF rows of loads are in flight per
// wave. A group of 32, 64, 128 or 256 columns is 8, 16, 32 or 64 lanes, whose
// s and z sums meet by lane shuffles. Column quad c of staged row r sits at
// quad c ^ 4 (r & 3): the 16 rows x 4 quads of one accumulator write then
// cover every bank four times, and a row read is a permutation of one row.
// ---------------------------------------------------------------------------
template <int BM, int BN, int TI, int TJ, int WN>
__device__ __forceinline__ void ste_adam_rows(const GemmArgs& a, const f32x4 (&acc)[TJ][TI], int m0, int n0,
                                              int wm0, int wn0, int lane, float* lds) {
  static_assert(BN == 256, "a row of the tile is one 16-byte quad per lane");
  constexpr int WM = TI * 16, WGM = BM / WM, NWAVE = WGM * (BN / WN), RPW = WM / NWAVE;
  constexpr int PF = 3;                                  // rows of loads in flight per wave
  static_assert(RPW * NWAVE == WM && RPW >= PF, "the staged rows split evenly over the waves");
  const int wave = threadIdx.x >> 6;
  const int col = n0 + 4 * lane;
  const bool col_ok = col < a.N;
  const int gl = a.group >> 2;                           // lanes per group
  const int64_t gcol = col_ok ? (int64_t)FastDiv::make((uint32_t)a.group).div((uint32_t)col) : 0;
  struct RowIn {
    float4 w, m, v;
    float s, z;
  };
#pragma unroll
  for (int h = 0; h < WGM; ++h) {
    const int row0 = m0 + h * WM;
    auto load = [&](int k, RowIn& in) {
      const int o = row0 + k * NWAVE + wave;
      if (o < a.M && col_ok) {
        const int64_t wi = (int64_t)o * a.ldw + col, gi = (int64_t)o * a.G + gcol;
        in.w = nt_load4(a.W + wi);
        in.m = nt_load4(a.mW + wi);
        in.v = nt_load4(a.vW + wi);
        in.s = a.s[gi];
        in.z = a.z[gi];
      }
    };
    RowIn buf[PF];                                       // the first rows' loads fly during the staging
#pragma unroll
    for (int k = 0; k < PF; ++k) load(k, buf[k]);
    __syncthreads();                                     // every read of the previous phase's rows is done
    if (wm0 == h * WM) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int r = 16 * i + (lane & 15), c = (wn0 >> 2) + 4 * j + (lane >> 4);
          *(f32x4*)&lds[r * BN + ((c ^ ((r & 3) << 2)) << 2)] = acc[j][i];
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
      const RowIn cur = buf[k % PF];
      if (k + PF < RPW) load(k + PF, buf[k % PF]);
      const int r = k * NWAVE + wave, o = row0 + r;
      const bool ok = o < a.M && col_ok;
      const f32x4 gw = *(const f32x4*)&lds[r * BN + ((lane ^ ((r & 3) << 2)) << 2)];
      float ps = 0.f, pz = 0.f;
      if (ok) {
        const float zr = round_clamp_zero(cur.z, a.Kq), rcp = 1.0f / cur.s;
        const float wv[4] = {cur.w.x, cur.w.y, cur.w.z, cur.w.w};
        float mv[4] = {cur.m.x, cur.m.y, cur.m.z, cur.m.w};
        float vv[4] = {cur.v.x, cur.v.y, cur.v.z, cur.v.w};
        float dw[4], pv[4];
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const QElem e = quant_elem_rcp(wv[e4], cur.s, rcp, zr, a.Kq);
          dw[e4] = e.m ? gw[e4] : 0.0f;
          ps += gw[e4] * (e.m ? (__builtin_rintf(e.u) - e.u) : (e.q - zr));
          pz += e.m ? 0.0f : gw[e4];
          // AdamW (the multi-tensor kernel's arithmetic) on the masked gradient
          const float pe = wv[e4] * a.adam_decay;
          mv[e4] = a.adam_b1 * mv[e4] + (1.0f - a.adam_b1) * dw[e4];
          vv[e4] = a.adam_b2 * vv[e4] + (1.0f - a.adam_b2) * dw[e4] * dw[e4];
          const float den = sqrtf(vv[e4]) * a.adam_isbc2 + a.adam_eps;
          pv[e4] = pe - a.adam_step * (mv[e4] / den);
        }
        const int64_t wi = (int64_t)o * a.ldw + col;
        if (a.dW) nt_store4(a.dW + wi, dw);
        nt_store4(a.Wupd + wi, pv);
        nt_store4(a.mW + wi, mv);
        nt_store4(a.vW + wi, vv);
      }
      for (int off = 1; off < gl; off <<= 1) {
        ps += __shfl_xor(ps, off);
        pz += __shfl_xor(pz, off);
      }
      if (ok && (lane & (gl - 1)) == 0 && a.ds) {
        const int64_t gi = (int64_t)o * a.G + gcol;
        a.ds[gi] = ps;
        if (a.dz) a.dz[gi] = -cur.s * pz;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The GEMM kernel for bf16 operands. A workgroup of WGM x WGN wave64s owns a
// BM x BN tile (4 waves: one per SIMD; 8 waves: two per SIMD, which hide each
// other's LDS and barrier waits); K advances in slabs of BK = 64, two
// k-steps of 32 each. Operand tiles reach LDS by DMA (AMN / BMN select the
// K- or MN-contiguous loader).
//
// Stage discipline: slab m lives in stage m % STAGES. Barrier B_kt sits
// between slab kt's two k-steps; before it each wave waits for its own DMA of
// slab kt + 1, so B_kt certifies slab kt + 1 for everyone. By B_kt every wave
// has also read all of slab kt's fragments into registers (k-step 0 during
// slab kt - 1, k-step 1 during slab kt's first k-step), so after B_kt the DMA
// for slab kt + STAGES may overwrite slab kt's stage: STAGES - 1 slabs of
// latency cover every load, and two stages already suffice. Slabs beyond the
// last re-load the last slab into free stages, keeping the vmcnt arithmetic
// uniform; nothing reads those copies.
//
// Schedule: every MFMA is followed by (at most) one fragment read for the next
// k-step and a share of the slab's DMA instructions, fenced so the compiler
// keeps that order: LDS reads run a full k-step ahead of their MFMAs and the
// DMA issue is spread over the k-step.
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, int STAGES, int WGM, int WGN, int GM, int AMN, int BMN, int EP, int NB>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void k_gemm(const GemmArgs a0) {
  int tile_id, prob;
  bool grouped;
  work_of(a0, tile_id, prob, grouped);
  const GemmArgs a = batch_view(a0, prob);
  constexpr int NW = WGM * WGN;
  using LA = typename DmaTileOf<BM, BK, AMN, NW>::T;
  using LB = typename DmaTileOf<BN, BK, BMN, NW>::T;
  static_assert(BK == 64, "two k-steps per slab");
  static_assert(STAGES >= 2, "two stages at least");
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TI = WM / 16, TJ = WN / 16;
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int NM = TI * TJ, NR = TI + TJ;
  constexpr int NLA = LA::NI, NL = LA::NI + LB::NI;      // DMA instructions per wave per slab
  // the slab's DMA instructions spread over a k-step's MFMAs: one after every
  // GAP-th MFMA, or DPM after each when there are more than MFMAs (4-byte DMA)
  constexpr int DPM = (NL + NM - 1) / NM;
  constexpr int GAP = DPM > 1 ? 1 : NM / NL;
  static_assert(NR <= NM && NL <= NM * DPM && (DPM == 1 || GAP == 1), "one k-step must cover the reads and the DMA");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE];
  static_assert(GM < 2 || 2 * (BN / 64) * BM * 4 <= STAGES * STAGE, "LDS holds the chunk sums");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm0 = (wave / WGN) * WM, wn0 = (wave % WGN) * WN;
  const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  int tm, tn;
  if (a.causal == kCausalNone) tile_of(tile_id, tiles_m, tiles_n, tm, tn);
  else causal_tile_of(tile_id, grouped, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const uint32_t lds0 = lds_addr_of(smem);

  // Slabs [0, nk) of the contraction (all of it, or up to the row tile's end).
  int nk = (a.K + BK - 1) / BK;
  if (a.causal == kCausalLower) nk = min(nk, (m0 + BM + BK - 1) / BK);

  LA la;
  LB lb;
  la.init(a.A, a.lda, m0, a.M, a.K);
  lb.init((const uint16_t*)a.B, a.ldb, n0, a.N, a.K);

  // DMA instruction q of slab `slab` into the stage at byte offset soff
  auto dma_q = [&](int slab, int q, int soff) {
    const uint32_t st = lds0 + (uint32_t)soff;
    const int k0 = (slab < nk ? slab : nk - 1) * BK;
    if (q < NLA) la.issue_q(st, k0, q);
    else lb.issue_q(st + A_BYTES, k0, q - NLA);
  };

  // Fragment reads. K-contiguous tiles: lane base per k-step + immediate
  // offsets; MN-contiguous tiles: transpose reads at a lane offset per
  // fragment, computed once, + the stage and k-step as immediates.
  int a_base[2] = {0, 0}, b_base[2] = {0, 0};
  int a_off[k_contig(AMN) ? 1 : TI], b_off[k_contig(BMN) ? 1 : TJ];
  if constexpr (!k_contig(AMN)) {
#pragma unroll
    for (int i = 0; i < TI; ++i) a_off[i] = LA::frag_off(wm0 + i * 16, lane);
  }
  if constexpr (!k_contig(BMN)) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) b_off[j] = A_BYTES + LB::frag_off(wn0 + j * 16, lane);
  }
  if constexpr (k_contig(AMN)) {
    a_base[0] = LA::frag_base(wm0, 0, lane);
    a_base[1] = LA::frag_base(wm0, 1, lane);
  }
  if constexpr (k_contig(BMN)) {
    b_base[0] = A_BYTES + LB::frag_base(wn0, 0, lane);
    b_base[1] = A_BYTES + LB::frag_base(wn0, 1, lane);
  }
  auto read_a = [&](int st, int ks, int i) -> bf16x8 {
    if constexpr (k_contig(AMN)) return *(const bf16x8*)&smem[st + a_base[ks] + i * LA::FRAG_STRIDE];
    else return LA::frag_at(&smem[st + a_off[i] + ks * 32 * LA::PITCH]);
  };
  auto read_b = [&](int st, int ks, int j) -> bf16x8 {
    if constexpr (k_contig(BMN)) return *(const bf16x8*)&smem[st + b_base[ks] + j * LB::FRAG_STRIDE];
    else return LB::frag_at(&smem[st + b_off[j] + ks * 32 * LB::PITCH]);
  };
  // read r of a k-step, in the order the MFMAs consume them: b0, a0 .. a(TI-1), b1 .. b(TJ-1)
  auto read_r = [&](int st, int ks, int r, Frags<TI, TJ>& f) {
    if (r == 0) f.b[0] = read_b(st, ks, 0);
    else if (r <= TI) f.a[r - 1] = read_a(st, ks, r - 1);
    else f.b[r - TI] = read_b(st, ks, r - TI);
  };

  f32x4 acc[TJ][TI];
#pragma unroll
  for (int j = 0; j < TJ; ++j)
#pragma unroll
    for (int i = 0; i < TI; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One k-step: MFMA t on `cur`, then read t of the next k-step (stage nst,
  // k-step nks) into `nxt` and, every GAP MFMAs, DPM DMA instructions of slab
  // dslab into the stage at dsoff (none if dslab < 0).
  auto kstep = [&](const Frags<TI, TJ>& cur, int nst, int nks, Frags<TI, TJ>& nxt, int dslab, int dsoff) {
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      const int j = t / TI, i = t % TI;
      mfma_acc(acc[j][i], cur.b[j], cur.a[i]);
      if (t < NR) read_r(nst, nks, t, nxt);
      if (dslab >= 0 && t % GAP == GAP - 1) {
#pragma unroll
        for (int d = 0; d < DPM; ++d)
          if ((t / GAP) * DPM + d < NL) dma_q(dslab, (t / GAP) * DPM + d, dsoff);
      }
      sched_fence();
    }
  };

  // prologue: slabs 0 .. STAGES-1 in flight; slab 0 visible; F0 = slab 0, k-step 0
#pragma unroll
  for (int sl = 0; sl < STAGES; ++sl)
#pragma unroll
    for (int q = 0; q < NL; ++q) dma_q(sl, q, sl * STAGE);
  wait_vmcnt<(STAGES - 1) * NL>();
  __syncthreads();
  Frags<TI, TJ> F0, F1;
#pragma unroll
  for (int r = 0; r < NR; ++r) read_r(0, 0, r, F0);
  sched_fence();

  // No unrolling or peeling: a peeled copy of the last iteration (the one
  // with the drain) lets the register allocator copy accumulators between
  // AGPRs right after their MFMAs, which the hazard recogniser cannot see.
  // The stage offsets of slabs kt and kt + 1 rotate from one iteration to
  // the next (no modulo in the loop); slab kt + STAGES reuses slab kt's.
  int st = 0, nx = STAGE % (STAGES * STAGE);
#pragma clang loop unroll(disable)
  for (int kt = 0; kt < nk; ++kt) {
    kstep(F0, st, 1, F1, -1, 0);                         // k-step 0; read k-step 1
    wait_vmcnt<(STAGES - 2) * NL>();
    __syncthreads();                                     // B_kt
    sched_fence();
    kstep(F1, nx, 0, F0, kt + STAGES, st);               // k-step 1; read slab kt+1; DMA
    st = nx;
    nx = nx + STAGE == STAGES * STAGE ? 0 : nx + STAGE;
    // The last iteration waits out the MFMA latency before leaving the loop,
    // so nothing placed after the loop (the epilogue, or spill code for an
    // accumulator) can read an accumulator before its result is written.
    if (kt == nk - 1) mfma_drain();
  }
  wait_vmcnt<0>();                                       // drain the trailing re-loads
  __syncthreads();
  mfma_drain();
  if constexpr (EP == kSteAdam) {
    static_assert(BM / WGM * BN * 4 <= STAGES * STAGE, "LDS holds one wave-row of accumulators");
    ste_adam_rows<BM, BN, TI, TJ, WN>(a, acc, m0, n0, wm0, wn0, lane, (float*)smem);
  } else {
    gemm_epilogue<EP, NB, GM, BM, BN, TI, TJ, WN>(a, acc, m0, n0, wm0, wn0, lane, (float*)smem);
  }
}

// ---------------------------------------------------------------------------
// The forward with a fused B operand (Y = X W_hat^T, no workspace): W_hat is
// made in LDS from the fp32 master weight (Eq. 1-2) or from packed codes,
// never stored. Slabs of BK = 32; 8 waves, one of each role per SIMD:
// - waves 0-3 (2 x 2 over a 256 x 128 or 128 x 128 tile, or 4 x 1 over a
//   512 x 64 tile: 128 x 64 or 64 x 64 per wave) load A themselves (D stages
//   by DMA, slab i + D issued during slab i's MFMAs) and run the MFMAs of
//   slab i interleaved with the fragment reads of slab i + 1;
// - waves 4-7 (converters) keep their WPT weights of every slab (16 for
//   128-row B tiles, 8 for 64-row ones) in a queue of U = 4 register slabs
//   (WRowLoader), load slab i + 2 + U while slab i + 2 is converted into B
//   stage (i + 2) % 3, and DMA the rows' s and z in chunks of four groups
//   (SzChunks). The 512 x 64 tile halves the weights converted per MFMA.
// One barrier per slab. The raw weights never pass through LDS (the LDS moves
// A's DMA and fragment reads, the bf16 B stage and its reads only), and A has
// up to six stages.
// Waits: the MFMA waves allow the last D - 2 slabs' A DMAs in flight at each
// barrier; the converters' register loads are waited for by the compiler
// before their conversion, and at each barrier a converter allows the last
// U - 1 slabs' loads in flight, so the chunk DMA of the slab after the next
// one (issued before its weights) has landed when its s and z are read.
// Slabs past the end re-load the last one; nothing reads what they make.
// ---------------------------------------------------------------------------
template <int BM, int BN, int BL, int NB>
struct FusedFwdShape {
  static constexpr int BK = 32, U = 4;
  static constexpr int WGN = BN == 64 ? 1 : 2, WGM = 4 / WGN;   // MFMA-wave grid
  static constexpr int WPT = BN * 32 / 256;             // weights per converter thread and slab
  using L = LdsLayout<BK, kLdsSlots>;
  using LA = DmaTileK<BM, BK, kLdsSlots, 4, 0>;
  using SZ = SzChunks<BN>;
  static constexpr int A_BYTES = BM * L::PITCH, B_BYTES = BN * L::PITCH;
  static constexpr int SZ_ALL = SZ::SZ_BYTES * SZ::ENTRIES;
  static constexpr int LDS_MAX = 160 * 1024;
  static constexpr int D_FIT = (LDS_MAX - 3 * B_BYTES - SZ_ALL) / A_BYTES;
  static constexpr int D_CNT = 2 + 63 / LA::NI;
  static constexpr int D_MIN = D_FIT < D_CNT ? D_FIT : D_CNT;
  static constexpr int D = D_MIN < 6 ? D_MIN : 6;
  static_assert(D >= 3, "three A stages at least");
  static constexpr int LDS = D * A_BYTES + 3 * B_BYTES + SZ_ALL;
};

template <int BM, int BN, int BL, int NB>
__global__ __launch_bounds__(512, 1) void k_gemm_fused_fwd(const GemmArgs a) {
  using Sh = FusedFwdShape<BM, BN, BL, NB>;
  constexpr int BK = Sh::BK, D = Sh::D, SB = 3, U = Sh::U;
  using LA = typename Sh::LA;
  using FB = DmaTileK<BN, BK, kLdsSlots>;
  static_assert(BL == kFp32Quant || BL == kPacked, "fused B operands only");
  static_assert(BN == 128 || BN == 64, "two or four converter threads per weight row");
  constexpr int WGN = Sh::WGN, WPT = Sh::WPT, TPR = 32 / WPT;
  constexpr int WM = BM / Sh::WGM, WN = BN / WGN;
  constexpr int TI = WM / 16, TJ = WN / 16, NM = TI * TJ, NR = TI + TJ;
  static_assert(NR <= NM, "a slab's MFMAs cover the next slab's reads");
  constexpr int A_BYTES = Sh::A_BYTES, B_BYTES = Sh::B_BYTES;
  constexpr int A0 = 0, B0 = D * A_BYTES, SZ0 = B0 + SB * B_BYTES;
  static_assert(SZ0 + Sh::SZ_ALL == Sh::LDS, "LDS map");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Sh::LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk = (a.K + BK - 1) / BK;
  const uint32_t lds0 = lds_addr_of(smem);
  auto clamp_slab = [&](int slab) { return slab < nk ? slab : nk - 1; };

  if (wave < 4) {
    // ---- MFMA waves: A by DMA, fragment reads, MFMAs
    LA la;
    la.init(a.A, a.lda, m0, a.M, a.K, wave);
    const int wm0 = (wave / WGN) * WM, wn0 = (wave % WGN) * WN;
    auto read_r = [&](int aoff, int boff, int r, Frags<TI, TJ>& f) {
      const uint8_t* at = &smem[A0 + aoff];
      const uint8_t* bt = &smem[B0 + boff];
      if (r < TI) f.a[r] = LA::frag(at, wm0 + r * 16 + (lane & 15), 0, lane);
      else f.b[r - TI] = FB::frag(bt, wn0 + (r - TI) * 16 + (lane & 15), 0, lane);
    };
    f32x4 acc[TJ][TI];
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int i = 0; i < TI; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int GAP = NM / LA::NI;                     // MFMAs per A DMA instruction
    static_assert(GAP >= 1 && GAP * LA::NI <= NM, "one slab's MFMAs cover its DMA");
    // MFMAs on `cur`, each followed by (at most) one read of the next slab
    // (A at aoff, B at boff) into `nxt`, and A's DMA of slab dslab into the
    // stage at doff spread over them
    auto step = [&](const Frags<TI, TJ>& cur, int aoff, int boff, Frags<TI, TJ>& nxt, int dslab, int doff) {
#pragma unroll
      for (int t = 0; t < NM; ++t) {
        const int j = t / TI, i = t % TI;
        acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.b[j], cur.a[i], acc[j][i], 0, 0, 0);
        if (t < NR) read_r(aoff, boff, t, nxt);
        if (t % GAP == GAP - 1 && t / GAP < LA::NI) la.issue_so_q(lds0 + A0 + doff, clamp_slab(dslab) * BK, t / GAP);
        sched_fence();
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);                // lgkmcnt(0): the next slab's reads are in
      wait_vmcnt<(D - 2) * LA::NI>();                    // A of the slab after next landed (own DMAs)
      __syncthreads();
    };
#pragma unroll
    for (int sl = 0; sl < D; ++sl) la.issue_so(lds0 + A0 + sl * A_BYTES, clamp_slab(sl) * BK);
    wait_vmcnt<(D - 2) * LA::NI>();                      // A slabs 0 and 1 landed (own)
    Frags<TI, TJ> F0, F1;
    __syncthreads();                                     // P0: everyone's A 0, 1 and (s, z) chunk 0
    __syncthreads();                                     // P1: B stages 0 and 1 converted
#pragma unroll
    for (int r = 0; r < NR; ++r) read_r(0, 0, r, F0);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __syncthreads();                                     // P2: slab 0 read; its A stage may be refilled
    int aoff = A_BYTES, boff = B_BYTES, doff = 0;        // slab i + 1's stages; A stage of slab i + D
    auto next = [&]() {
      aoff = aoff + A_BYTES == D * A_BYTES ? 0 : aoff + A_BYTES;
      boff = boff + B_BYTES == SB * B_BYTES ? 0 : boff + B_BYTES;
      doff = doff + A_BYTES == D * A_BYTES ? 0 : doff + A_BYTES;
    };
    for (int kt = 0; kt < nk; kt += 2) {
      step(F0, aoff, boff, F1, kt + D, doff);
      next();
      if (kt + 1 < nk) {
        step(F1, aoff, boff, F0, kt + 1 + D, doff);
        next();
      }
    }
    wait_vmcnt<0>();                                     // drain the trailing re-loads
    gemm_epilogue<kStoreBf16, NB, 0, BM, BN, TI, TJ, WN>(a, acc, m0, n0, wm0, wn0, lane, nullptr);
  } else {
    // ---- converter waves: raw weights to registers, (s, z) chunks, B stages
    const int cw = wave - 4, tid = threadIdx.x - 256;
    const int row = tid / TPR;
    WRowLoader<BL, NB, WPT> wl;
    wl.init(a.B, BL == kFp32Quant ? a.ldb * 4 : a.ldb, n0, a.N, tid);
    typename Sh::SZ sz;
    sz.init(a.s, a.z, n0, a.N, a.G, a.group, a.Kq, cw);
    constexpr int NLW = WRowLoader<BL, NB, WPT>::NL;
    const uint32_t lds_sz = lds0 + SZ0;
    auto fetch = [&](WSlab<BL, NB, WPT>& w, int slab) { // (s, z) chunk first, then the weights
      const int k0 = clamp_slab(slab) * BK;
      sz.issue(lds_sz, k0);
      wl.load(w, k0);
    };
    // this thread's row's s and z for a slab, read one slab before its
    // conversion (the LDS read's latency then hides behind a conversion)
    auto sz_read = [&](int slab, float& sv, float& zv) {
      const int c = sz.at(SZ0, row, clamp_slab(slab) * BK);
      sv = *(const float*)&smem[c];
      zv = *(const float*)&smem[c + BN * Sh::SZ::CG * 4];
    };
    auto convert = [&](const WSlab<BL, NB, WPT>& w, float sv, float zv, int boff) {
      convert_slab<BL, NB, WPT>(w, sv, zv, sz.K, smem, B0 + boff, tid);
    };
    WSlab<BL, NB, WPT> R0, R1, R2, R3;                   // slab j in R[j % 4]
    static_assert(U == 4, "four named register slabs");
    fetch(R0, 0);
    fetch(R1, 1);
    fetch(R2, 2);
    fetch(R3, 3);
    wait_vmcnt<U * NLW>();                               // chunk 0 (slabs 0-3 at least) landed (for this wave)
    __syncthreads();                                     // P0
    float sv, zv, sn, zn;                                // s, z of the slab converted now, and of the next
    sz_read(0, sv, zv);
    sz_read(1, sn, zn);
    convert(R0, sv, zv, 0);
    fetch(R0, U);
    sz_read(2, sv, zv);
    convert(R1, sn, zn, B_BYTES);
    fetch(R1, U + 1);
    __syncthreads();                                     // P1
    __syncthreads();                                     // P2
    int boff = 2 * B_BYTES;                              // B stage of slab i + 2
    // Iteration i converts slab i + 2 with the s, z read in the iteration
    // before and reads those of slab i + 3, whose chunk landed before the
    // last barrier: each wave issues the chunk DMA of a slab before the slab's
    // weights, and waits at a barrier until at most the weights of the next
    // U - 1 slabs (and chunk DMAs among them) are in flight.
    auto iter = [&](WSlab<BL, NB, WPT>& R, int kt) {
      sz_read(kt + 3, sn, zn);
      convert(R, sv, zv, boff);
      fetch(R, kt + 2 + U);
      sv = sn, zv = zn;
      boff = boff + B_BYTES == SB * B_BYTES ? 0 : boff + B_BYTES;
      wait_vmcnt<(U - 1) * NLW>();
      __syncthreads();
    };
    // Whole groups of four slabs in a loop without guards, the rest straight
    // after it: the compiler places the waits for the register loads, and
    // guards inside the loop body let it branch from one slab to a later one
    // of the same trip, after which it must assume fewer loads in flight and
    // waits for up to three slabs' loads that the conversion does not need.
    int kt = 0;
    for (; kt + 4 <= nk; kt += 4) {
      iter(R2, kt);
      iter(R3, kt + 1);
      iter(R0, kt + 2);
      iter(R1, kt + 3);
    }
    if (kt < nk) {
      iter(R2, kt);
      if (kt + 1 < nk) {
        iter(R3, kt + 1);
        if (kt + 2 < nk) iter(R0, kt + 2);
      }
    }
    wait_vmcnt<0>();                                     // drain the trailing re-loads
  }
}

// ---------------------------------------------------------------------------
// dX = dY W_hat with a fused B operand (no workspace): W_hat^T made in LDS from
// the fp32 master weight (Eq. 1-2) or from packed codes, never stored. The
// same two roles as the forward: waves 0-3 load dY themselves (D stages by
// DMA, 4-byte DMA with the contraction's tail masked when ADW) and run the
// MFMAs of slab i with the transpose reads of slab i + 1; waves 4-7 keep their
// 16 weights of every slab (and the row's s, z) in a queue of U = 4 register
// slabs (WColLoader), load slab i + 2 + U while slab i + 2 is converted into
// the MN-contiguous B stage (i + 2) % 3. One barrier per slab; the
// converters' loads land in their own registers, so their barrier waits for
// nothing but their B-stage writes.
// ---------------------------------------------------------------------------
template <int BM, int BN, int BL, int NB, int ADW>
struct FusedDxShape {
  static constexpr int BK = 32, U = 4, SB = 3;
  using L = LdsLayout<BK, kLdsSlots>;
  using LA = DmaTileK<BM, BK, kLdsSlots, 4, ADW>;
  using LT = DmaTileMN<BN, BK, 4>;
  static constexpr int A_BYTES = BM * L::PITCH, B_BYTES = BK * LT::PITCH;
  static constexpr int LDS_MAX = 160 * 1024;
  static constexpr int D_FIT = (LDS_MAX - SB * B_BYTES) / A_BYTES;
  static constexpr int D_CNT = 2 + 63 / LA::NI;
  static constexpr int D_MIN = D_FIT < D_CNT ? D_FIT : D_CNT;
  static constexpr int D = D_MIN < 6 ? D_MIN : 6;
  static_assert(D >= 3, "three A stages at least");
  static constexpr int LDS = D * A_BYTES + SB * B_BYTES;
};

template <int BM, int BN, int BL, int NB, int ADW>
__global__ __launch_bounds__(512, 1) void k_gemm_fused_dx(const GemmArgs a) {
  using Sh = FusedDxShape<BM, BN, BL, NB, ADW>;
  constexpr int BK = Sh::BK, D = Sh::D, SB = Sh::SB, U = Sh::U;
  using LA = typename Sh::LA;
  using LT = typename Sh::LT;
  static_assert(BL == kFp32Quant || BL == kPacked, "fused B operands only");
  static_assert(BN == 128, "eight converter threads per weight row, 16 columns each");
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TI = WM / 16, TJ = WN / 16, NM = TI * TJ, NR = TI + TJ;
  static_assert(NR <= NM, "a slab's MFMAs cover the next slab's reads");
  constexpr int A_BYTES = Sh::A_BYTES, B_BYTES = Sh::B_BYTES;
  constexpr int A0 = 0, B0 = D * A_BYTES;
  static_assert(B0 + SB * B_BYTES == Sh::LDS, "LDS map");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Sh::LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk = (a.K + BK - 1) / BK;
  const uint32_t lds0 = lds_addr_of(smem);
  auto clamp_slab = [&](int slab) { return slab < nk ? slab : nk - 1; };

  if (wave < 4) {
    // ---- MFMA waves: dY by DMA, fragment reads (B by transpose reads), MFMAs
    LA la;
    la.init(a.A, a.lda, m0, a.M, a.K, wave);
    const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
    auto read_r = [&](int aoff, int boff, int r, Frags<TI, TJ>& f) {
      const uint8_t* at = &smem[A0 + aoff];
      const uint8_t* bt = &smem[B0 + boff];
      if (r < TI) f.a[r] = LA::frag(at, wm0 + r * 16 + (lane & 15), 0, lane);
      else f.b[r - TI] = LT::frag(bt, wn0 + (r - TI) * 16 + (lane & 15), 0, lane);
    };
    f32x4 acc[TJ][TI];
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int i = 0; i < TI; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int GAP = NM / LA::NI > 0 ? NM / LA::NI : 1;   // MFMAs per dY DMA instruction
    constexpr int DPM = (LA::NI + NM - 1) / NM;            // DMA instructions per MFMA
    static_assert(DPM * NM >= LA::NI, "one slab's MFMAs cover its DMA");
    auto step = [&](const Frags<TI, TJ>& cur, int aoff, int boff, Frags<TI, TJ>& nxt, int dslab, int doff) {
#pragma unroll
      for (int t = 0; t < NM; ++t) {
        const int j = t / TI, i = t % TI;
        acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.b[j], cur.a[i], acc[j][i], 0, 0, 0);
        if (t < NR) read_r(aoff, boff, t, nxt);
#pragma unroll
        for (int u = 0; u < DPM; ++u) {
          const int q = DPM > 1 ? t * DPM + u : t / GAP;
          if ((DPM > 1 || t % GAP == GAP - 1) && q < LA::NI)
            la.issue_so_q(lds0 + A0 + doff, clamp_slab(dslab) * BK, q);
        }
        sched_fence();
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);                // lgkmcnt(0): the next slab's reads are in
      wait_vmcnt<(D - 2) * LA::NI>();                    // dY of the slab after next landed (own DMAs)
      __syncthreads();
    };
#pragma unroll
    for (int sl = 0; sl < D; ++sl) la.issue_so(lds0 + A0 + sl * A_BYTES, clamp_slab(sl) * BK);
    wait_vmcnt<(D - 2) * LA::NI>();                      // dY slabs 0 and 1 landed (own)
    Frags<TI, TJ> F0, F1;
    __syncthreads();                                     // P0: everyone's dY 0 and 1
    __syncthreads();                                     // P1: B stages 0 and 1 converted
#pragma unroll
    for (int r = 0; r < NR; ++r) read_r(0, 0, r, F0);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __syncthreads();                                     // P2: slab 0 read; its dY stage may be refilled
    int aoff = A_BYTES, boff = B_BYTES, doff = 0;        // slab i + 1's stages; dY stage of slab i + D
    auto next = [&]() {
      aoff = aoff + A_BYTES == D * A_BYTES ? 0 : aoff + A_BYTES;
      boff = boff + B_BYTES == SB * B_BYTES ? 0 : boff + B_BYTES;
      doff = doff + A_BYTES == D * A_BYTES ? 0 : doff + A_BYTES;
    };
    for (int kt = 0; kt < nk; kt += 2) {
      step(F0, aoff, boff, F1, kt + D, doff);
      next();
      if (kt + 1 < nk) {
        step(F1, aoff, boff, F0, kt + 1 + D, doff);
        next();
      }
    }
    wait_vmcnt<0>();                                     // drain the trailing re-loads
    gemm_epilogue<kStoreBf16, NB, 0, BM, BN, TI, TJ, WN>(a, acc, m0, n0, wm0, wn0, lane, nullptr);
  } else {
    // ---- converter waves: weight rows to registers, B stages (W_hat^T)
    const int tid = threadIdx.x - 256;
    const int row = tid / 8, c16 = tid % 8;
    WColLoader<BL, NB> wl;
    wl.init(a.B, BL == kFp32Quant ? a.ldb * 4 : a.ldb, n0, a.K, a.s, a.z, a.G, a.group, tid);
    uint4 pk[2];
    auto fetch = [&](WColSlab<BL, NB>& w, int slab) { wl.load(w, clamp_slab(slab) * BK); };
    auto convert = [&](const WColSlab<BL, NB>& w, int slab, int boff) {
      convert_cols<BL, NB>(w, a.Kq, slab * BK + row < a.K, wl.sh, pk);
#pragma unroll
      for (int m = 0; m < 2; ++m) *(uint4*)&smem[B0 + boff + LT::off(row, 2 * c16 + m)] = pk[m];
    };
    WColSlab<BL, NB> R0, R1, R2, R3;                     // slab j in R[j % 4]
    static_assert(U == 4, "four named register slabs");
    fetch(R0, 0);
    fetch(R1, 1);
    fetch(R2, 2);
    fetch(R3, 3);
    __syncthreads();                                     // P0
    convert(R0, 0, 0);
    fetch(R0, U);
    convert(R1, 1, B_BYTES);
    fetch(R1, U + 1);
    __syncthreads();                                     // P1
    __syncthreads();                                     // P2
    int boff = 2 * B_BYTES;                              // B stage of slab i + 2
    // The scheduling fence keeps each conversion after the barrier before
    // it: the conversions are register work, and the compiler otherwise
    // hoists a whole trip's of them to its start, where they wait for every
    // weight load in flight.
    auto iter = [&](WColSlab<BL, NB>& R, int kt) {
      sched_fence();
      convert(R, kt + 2, boff);
      fetch(R, kt + 2 + U);
      boff = boff + B_BYTES == SB * B_BYTES ? 0 : boff + B_BYTES;
      __syncthreads();
    };
    // Whole groups of four slabs in a loop without guards, the rest straight
    // after it: with guards inside the loop body the compiler may branch from
    // one slab to a later one of the same trip and then waits for register
    // loads the conversion does not need.
    int kt = 0;
    for (; kt + 4 <= nk; kt += 4) {
      iter(R2, kt);
      iter(R3, kt + 1);
      iter(R0, kt + 2);
      iter(R1, kt + 3);
    }
    if (kt < nk) {
      iter(R2, kt);
      if (kt + 1 < nk) {
        iter(R3, kt + 1);
        if (kt + 2 < nk) iter(R0, kt + 2);
      }
    }
    wait_vmcnt<0>();                                     // drain the trailing re-loads
  }
}

}  // namespace qat
