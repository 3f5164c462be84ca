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
template <int ROWS, int BK, int SLOTS, int NW = 4>
struct DmaTileK {
  using L = LdsLayout<BK, SLOTS>;
  static constexpr int RPI = 1024 / L::PITCH;            // rows per DMA instruction
  static constexpr int NI = ROWS / RPI / NW;             // instructions per wave per slab
  static_assert(NI * RPI * NW == ROWS, "tile rows must split over the waves");
  i32x4 rs;
  uint32_t voff[NI];
  uint32_t lrow[NI];                                     // wave-uniform LDS byte offsets
  // src is [rows][ld] with K contiguous; rows >= nrows read as zero. The
  // range ends with the last row's kdim-th element, so a view into a wider
  // tensor (one head's columns) reads nothing past that tensor.
  __device__ __forceinline__ void init(const uint16_t* src, int64_t ld, int row0, int nrows, int kdim) {
    rs = buffer_rsrc(src + (int64_t)row0 * ld, ((int64_t)(nrows - 1 - row0) * ld + kdim) * 2);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int r0 = (wave * NI + q) * RPI;
      const int row = r0 + lane / L::CH;
      const int pos = lane % L::CH;
      const int chunk = pos ^ ((row / L::RPL) & (L::CH - 1));
      voff[q] = (uint32_t)(row * ld * 2 + chunk * 16);
      lrow[q] = (uint32_t)(r0 * L::PITCH);
    }
  }
  __device__ __forceinline__ void issue(uint32_t lds_tile, int k0) const {
#pragma unroll
    for (int q = 0; q < NI; ++q) dma16(rs, lds_tile + lrow[q], voff[q] + (uint32_t)k0 * 2);
  }
  __device__ __forceinline__ void issue_q(uint32_t lds_tile, int k0, int q) const {
    dma16(rs, lds_tile + lrow[q], voff[q] + (uint32_t)k0 * 2);
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
template <int ROWS, int BK, int NW = 4>
struct DmaTileMN {
  static constexpr int CHR = ROWS / 8;                   // 16-byte chunks per k-row
  static constexpr int PITCH = ROWS * 2;
  static constexpr int KPI = 1024 / PITCH;               // k-rows per DMA instruction
  static constexpr int NI = BK / KPI / NW;               // instructions per wave per slab
  static_assert(CHR >= 16 && NI * KPI * NW == BK, "tile shape");
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
      const int k0 = (wave * NI + q) * KPI;
      const int kr = k0 + lane / CHR;
      const int pos = lane % CHR;
      const int chunk = pos ^ swz(kr);
      voff[q] = (uint32_t)(kr * ld * 2 + chunk * 16);
      lrow[q] = (uint32_t)(k0 * PITCH);
    }
  }
  __device__ __forceinline__ void issue(uint32_t lds_tile, int k0) const {
#pragma unroll
    for (int q = 0; q < NI; ++q) dma16(rs, lds_tile + lrow[q], voff[q] + (uint32_t)k0 * kstride);
  }
  __device__ __forceinline__ void issue_q(uint32_t lds_tile, int k0, int q) const {
    dma16(rs, lds_tile + lrow[q], voff[q] + (uint32_t)k0 * kstride);
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
struct DmaTileOf<ROWS, BK, 1, NW> { using T = DmaTileMN<ROWS, BK, NW>; };

// Quantised-weight operands through an LDS ring. Per slab, the raw weight
// bytes of ROWS rows (packed N-bit codes, BK*N/8 bytes per row; or the fp32
// master weight, BK*4 bytes per row) and the rows' s and z reach a ring entry
// by dword DMA, one slab ahead of the A operand. Every thread then converts
// its share into the K-contiguous bf16 B stage two slabs ahead of the MFMAs:
//   packed (E2E-QP):  W_hat = (q - z) * s, z as stored;
//   fp32 (Block-AP):  Eq. 1 then Eq. 2 with zr = clamp(rint(z), 0, K). u is
//     w * fl32(1/s), within 3 ulp of fl32(w/s); where that interval could
//     hold a half-integer the element is redone with the correctly rounded
//     division, so the codes are exactly the fp32 quantiser's.
// With BK = 32 a slab lies inside one quantisation group (groups of 32, 64,
// 128 or a whole row), so one (s, z) pair per row and slab.
template <int ROWS, int BK, int KIND, int NB>
struct DmaRing {
  using L = LdsLayout<BK, kLdsSlots>;
  static constexpr int DW = KIND == kPacked ? BK * NB / 32 : BK;   // weight dwords per row per slab
  static constexpr int NI_Q = ROWS * DW / 64 / 4;                  // weight DMA instructions per wave
  static constexpr int NI_S = 2 * ROWS / 64 / 4;                   // s and z, [2][ROWS] dwords
  static constexpr int NI = NI_Q + NI_S;
  static constexpr int P_BYTES = ROWS * DW * 4 + 2 * ROWS * 4;
  static_assert(NI_Q * 256 == ROWS * DW && NI_S * 256 == 2 * ROWS, "ring tile shape");
  i32x4 rq, rsz[2];
  uint32_t vq[NI_Q], vs[NI_S];
  int wave;
  float K;
  FastDiv gdiv;                                                    // k -> group index
  __device__ __forceinline__ void init(const void* Wsrc, int64_t row_bytes, int row0, int nrows, const float* s,
                                       const float* z, int64_t G, int group, float K_) {
    K = K_;
    gdiv = FastDiv::make((uint32_t)group);
    rq = buffer_rsrc((const uint8_t*)Wsrc + (int64_t)row0 * row_bytes, (int64_t)(nrows - row0) * row_bytes);
    rsz[0] = buffer_rsrc(s + (int64_t)row0 * G, (int64_t)(nrows - row0) * G * 4);
    rsz[1] = buffer_rsrc(z + (int64_t)row0 * G, (int64_t)(nrows - row0) * G * 4);
    const int lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int q = 0; q < NI_Q; ++q) {
      const int idx = (wave * NI_Q + q) * 64 + lane;       // flat dword of the [ROWS][DW] slab
      vq[q] = (uint32_t)((idx / DW) * row_bytes + (idx % DW) * 4);
    }
#pragma unroll
    for (int q = 0; q < NI_S; ++q) {
      const int idx = (wave * NI_S + q) * 64 + lane;       // flat dword of [2][ROWS]
      vs[q] = (uint32_t)((idx % ROWS) * G * 4);
    }
  }
  // lds_p: this slab's ring entry: [ROWS][DW] weight dwords, then s[ROWS], z[ROWS].
  __device__ __forceinline__ void issue(uint32_t lds_p, int k0) const {
    const uint32_t cb = KIND == kPacked ? (uint32_t)(k0 * NB / 8) : (uint32_t)(k0 * 4);
    const uint32_t gb = gdiv.div((uint32_t)k0) * 4;               // the slab lies inside one group
#pragma unroll
    for (int q = 0; q < NI_Q; ++q) dma4(rq, lds_p + (uint32_t)((wave * NI_Q + q) * 256), vq[q] + cb);
#pragma unroll
    for (int q = 0; q < NI_S; ++q) {
      const int which = ((wave * NI_S + q) * 64) / ROWS;    // 0: s, 1: z (uniform per instruction)
      i32x4 r = which ? rsz[1] : rsz[0];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = __builtin_amdgcn_readfirstlane(r[e]);
      dma4(r, lds_p + ROWS * DW * 4 + (uint32_t)((wave * NI_S + q) * 256), vs[q] + gb);
    }
  }
  // Convert one slab from the ring entry at byte p into the B stage at byte b.
  // IL > 0: the caller's IL MFMAs of the same slab precede this in the same
  // basic block; the conversion's VALU work is interleaved with them (all
  // fast paths first, near-ties redone behind one branch, then the stores).
  template <int IL = 0>
  __device__ __forceinline__ void commit(uint8_t* smem, int p, int b) const {
    constexpr int PARTS = 256 / ROWS;                      // threads per row
    constexpr int CPT = (BK / 8) / PARTS;                  // 8-element chunks per thread
    const int row = threadIdx.x / PARTS, part = threadIdx.x % PARTS;
    // fp32 rows are 128 bytes: odd row pairs take their two chunks in the
    // other order, so that the 16-byte reads of 8 neighbouring lanes fall on
    // distinct banks
    const int cx = (KIND != kPacked && PARTS == 2 && CPT == 2) ? (row >> 1) & 1 : 0;
    auto chunk = [&](int cc) { return (part * CPT + cc) ^ cx; };
    const uint32_t* q = (const uint32_t*)&smem[p + row * DW * 4];
    const float sv = *(const float*)&smem[p + ROWS * DW * 4 + row * 4];
    const float zv = *(const float*)&smem[p + ROWS * DW * 4 + ROWS * 4 + row * 4];
    float h[CPT][8];
    uint32_t tie = 0;                                      // fp32: elements near a rounding tie
    const float zr = round_clamp_zero(zv, K);
    const float rcp = 1.0f / sv;
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      const int c = chunk(cc);                             // chunk of this row's slab
      if constexpr (KIND == kPacked) {
        const int bit = c * 8 * NB;
        uint64_t w = q[bit >> 5];
        if (NB == 3 && (bit & 31) > 8) w |= (uint64_t)q[(bit >> 5) + 1] << 32;
        const uint32_t word = (uint32_t)(w >> (bit & 31));
#pragma unroll
        for (int k = 0; k < 8; ++k) h[cc][k] = ((float)((word >> (NB * k)) & ((1u << NB) - 1)) - zv) * sv;
      } else {
        const uint4 w0 = *(const uint4*)&q[c * 8], w1 = *(const uint4*)&q[c * 8 + 4];
        const uint32_t wb[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float w = __builtin_bit_cast(float, wb[k]);
          const float u = w * rcp;
          const float ru = __builtin_rintf(u);
          // distance to the nearest half-integer: 0.5 - |u - rint(u)|, exact
          // wherever it can fall under the threshold
          if (0.5f - fabsf(u - ru) <= fabsf(u) * 0x1p-20f + 0x1p-60f) tie |= 1u << (cc * 8 + k);
          const float qv = fminf(fmaxf(ru + zr, 0.0f), K);
          h[cc][k] = (qv - zr) * sv;
        }
      }
    }
    if constexpr (IL > 0) {
      // VALU instructions placed after each MFMA: NV per converted element,
      // spread over the IL MFMAs (NV measured best on the 2048- and 4096-token
      // shapes; the rest of the conversion follows the last MFMA).
      constexpr int NV = KIND == kPacked ? 2 : 6;
      constexpr int PER = (CPT * 8 * NV + IL - 1) / IL;
#pragma unroll
      for (int i = 0; i < IL; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, PER, 0); // then VALU
      }
    }
    if constexpr (KIND != kPacked) {
      if (tie) {                                           // near a rounding tie: exact division
#pragma unroll
        for (int cc = 0; cc < CPT; ++cc) {
          const uint32_t* qc = q + chunk(cc) * 8;
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (tie & (1u << (cc * 8 + k))) {
              float wt = __builtin_bit_cast(float, qc[k]);
              rare_branch(wt);
              h[cc][k] = quant_elem(wt, sv, zr, K).w_hat;
            }
        }
      }
    }
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      const int c = chunk(cc);
      *(uint4*)&smem[b + L::off(row, c)] = make_uint4(pack_bf16x2(h[cc][0], h[cc][1]), pack_bf16x2(h[cc][2], h[cc][3]),
                                                       pack_bf16x2(h[cc][4], h[cc][5]), pack_bf16x2(h[cc][6], h[cc][7]));
    }
  }
};

template <int BL, class Ld>
__device__ __forceinline__ void init_b(Ld& l, const GemmArgs& a, int n0) {
  if constexpr (BL == kFp32Quant) l.init(a.B, a.ldb * 4, n0, a.N, a.s, a.z, a.G, a.group, a.Kq);
  else l.init(a.B, a.ldb, n0, a.N, a.s, a.z, a.G, a.group, a.Kq);
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
  constexpr int GAP = NM / NL > 0 ? NM / NL : 1;
  static_assert(NR <= NM && NL * GAP <= NM, "one k-step must cover the reads and the DMA");
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
  int a_off[AMN == kKContig ? 1 : TI], b_off[BMN == kKContig ? 1 : TJ];
  if constexpr (AMN != kKContig) {
#pragma unroll
    for (int i = 0; i < TI; ++i) a_off[i] = LA::frag_off(wm0 + i * 16, lane);
  }
  if constexpr (BMN != kKContig) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) b_off[j] = A_BYTES + LB::frag_off(wn0 + j * 16, lane);
  }
  if constexpr (AMN == kKContig) {
    a_base[0] = LA::frag_base(wm0, 0, lane);
    a_base[1] = LA::frag_base(wm0, 1, lane);
  }
  if constexpr (BMN == kKContig) {
    b_base[0] = A_BYTES + LB::frag_base(wn0, 0, lane);
    b_base[1] = A_BYTES + LB::frag_base(wn0, 1, lane);
  }
  auto read_a = [&](int st, int ks, int i) -> bf16x8 {
    if constexpr (AMN == kKContig) return *(const bf16x8*)&smem[st + a_base[ks] + i * LA::FRAG_STRIDE];
    else return LA::frag_at(&smem[st + a_off[i] + ks * 32 * LA::PITCH]);
  };
  auto read_b = [&](int st, int ks, int j) -> bf16x8 {
    if constexpr (BMN == kKContig) return *(const bf16x8*)&smem[st + b_base[ks] + j * LB::FRAG_STRIDE];
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
  // k-step nks) into `nxt` and, every GAP MFMAs, one DMA instruction of slab
  // dslab into the stage at dsoff (none if dslab < 0).
  auto kstep = [&](const Frags<TI, TJ>& cur, int nst, int nks, Frags<TI, TJ>& nxt, int dslab, int dsoff) {
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      const int j = t / TI, i = t % TI;
      mfma_acc(acc[j][i], cur.b[j], cur.a[i]);
      if (t < NR) read_r(nst, nks, t, nxt);
      if (dslab >= 0 && t % GAP == GAP - 1 && t / GAP < NL) dma_q(dslab, t / GAP, dsoff);
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
// GEMM with a fused B operand (packed codes or the fp32 master weight through
// an LDS ring, see DmaRing) and a K-contiguous bf16 A; bf16 output. STAGES
// LDS stages (>= 3). With one k-step per slab (BK = 32) U2 = 1 unrolls slabs
// in pairs so the two fragment sets alternate; U2 = 0 copies the next slab's
// fragments instead (fewer live registers).
// Invariant at the top of slab kt: slabs <= kt are visible to every wave and
// F[0] holds the first k-step's fragments of slab kt. The barrier in slab kt
// certifies slab kt + 1, so the fragments of the next slab are read while the
// current slab's MFMAs run, and the DMA for slab kt + STAGES - 1 goes into the
// stage slab kt - 1 has just released. The ring runs one slab ahead of A and
// is converted into the bf16 B stage two slabs ahead of the MFMAs.
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, int STAGES, int U2, int BL, int NB>
__global__ __launch_bounds__(256, 1) void k_gemm_fused(const GemmArgs a) {
  using L = LdsLayout<BK, kLdsSlots>;
  using LA = DmaTileK<BM, BK, kLdsSlots>;
  using LB = DmaRing<BN, BK, BL, NB>;
  using FB = DmaTileK<BN, BK, kLdsSlots>;                 // B fragment reader
  static_assert(BL == kFp32Quant || BL == kPacked, "fused B operands only");
  static_assert(STAGES >= 3, "the shifted pipeline needs three stages");
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TI = WM / 16, TJ = WN / 16;
  constexpr int KS = BK / 32;                              // k-steps per slab
  constexpr int A_BYTES = BM * L::PITCH, B_BYTES = BN * L::PITCH;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int P_STAGE = LB::P_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE + STAGES * P_STAGE];
  constexpr int P0 = STAGES * STAGE;                       // byte offset of the ring

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
  const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const uint32_t lds0 = lds_addr_of(smem);

  LA la;
  LB lb;
  la.init(a.A, a.lda, m0, a.M, a.K);
  init_b<BL>(lb, a, n0);
  constexpr int NL = LA::NI + LB::NI;                     // DMA instructions per wave per slab

  const int nk = (a.K + BK - 1) / BK;
  auto clamp_slab = [&](int slab) { return slab < nk ? slab : nk - 1; };
  // All DMA of one iteration: A of slab `slab`, ring weights of slab + 1.
  auto issue = [&](int slab) {
    const uint32_t st = lds0 + (uint32_t)((slab % STAGES) * STAGE);
    la.issue(st, clamp_slab(slab) * BK);
    lb.issue(lds0 + P0 + (uint32_t)(((slab + 1) % STAGES) * P_STAGE), clamp_slab(slab + 1) * BK);
  };
  auto b_commit = [&](int slab) {
    lb.commit(smem, P0 + (slab % STAGES) * P_STAGE, (slab % STAGES) * STAGE + A_BYTES);
  };
  auto b_commit_il = [&](int slab) {
    lb.template commit<KS == 1 ? TI * TJ : 0>(smem, P0 + (slab % STAGES) * P_STAGE, (slab % STAGES) * STAGE + A_BYTES);
  };

  // Fragment reads index the __shared__ array directly (stage given as a byte
  // offset) so that they stay ds_read instructions.
  auto read_frags = [&](int st, int ks, Frags<TI, TJ>& f) {
#pragma unroll
    for (int i = 0; i < TI; ++i) f.a[i] = LA::frag(&smem[st], wm0 + i * 16 + (lane & 15), ks, lane);
#pragma unroll
    for (int j = 0; j < TJ; ++j) f.b[j] = FB::frag(&smem[st + A_BYTES], wn0 + j * 16 + (lane & 15), ks, lane);
  };

  f32x4 acc[TJ][TI];
#pragma unroll
  for (int j = 0; j < TJ; ++j)
#pragma unroll
    for (int i = 0; i < TI; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mfmas = [&](const Frags<TI, TJ>& f) {
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int i = 0; i < TI; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[j], f.a[i], acc[j][i], 0, 0, 0);
  };

  // prologue: ring slabs 0, 1 converted, A slabs 0 .. STAGES-2 in flight, F[0] loaded.
  lb.issue(lds0 + P0, 0);                     // ring slab 0; issue(sl) brings slab sl + 1
#pragma unroll
  for (int sl = 0; sl < STAGES - 1; ++sl) issue(sl);
  wait_vmcnt<0>();
  __syncthreads();                            // ring slabs 0, 1 visible
  b_commit(0);
  b_commit(1);
  __syncthreads();                            // their bf16 tiles visible
  Frags<TI, TJ> F[2];
  read_frags(0, 0, F[0]);

  // One slab: CUR holds its first k-step's fragments on entry, and the next
  // slab's first fragments are in CUR (two k-steps) or NXT (one k-step) on exit.
#define QAT_SLAB(KT, CUR, NXT)                                              \
  do {                                                                      \
    wait_vmcnt<(STAGES - 3) * NL>(); /* my DMAs for slabs <= KT+1 landed */ \
    __syncthreads();                 /* everyone's: slab KT+1 is visible */ \
    issue((KT) + STAGES - 1);                                               \
    const int st_ = ((KT) % STAGES) * STAGE;                                \
    const int nx_ = (((KT) + 1) % STAGES) * STAGE;                          \
    if constexpr (KS == 1) {                                                \
      read_frags(nx_, 0, NXT);                                              \
      mfmas(CUR);                                                           \
    } else {                                                                \
      read_frags(st_, 1, NXT);                                              \
      mfmas(CUR);                                                           \
      read_frags(nx_, 0, CUR);                                              \
      mfmas(NXT);                                                           \
    }                                                                       \
    b_commit_il((KT) + 2);                                                  \
  } while (0)

  for (int kt = 0; kt < nk; kt += (KS == 1 && U2) ? 2 : 1) {
    QAT_SLAB(kt, F[0], F[1]);
    if constexpr (KS == 1) {
      if constexpr (U2) {
        if (kt + 1 < nk) QAT_SLAB(kt + 1, F[1], F[0]);
      } else {
        F[0] = F[1];
      }
    }
  }
#undef QAT_SLAB
  wait_vmcnt<0>();                            // drain the trailing re-issued DMAs
  __syncthreads();
  gemm_epilogue<kStoreBf16, NB, 0, BM, BN, TI, TJ, WN>(a, acc, m0, n0, wm0, wn0, lane, nullptr);
}

}  // namespace qat
