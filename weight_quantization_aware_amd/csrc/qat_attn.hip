// Causal attention of the Block-AP step, fused (gfx950).
// Forward: for one (sequence, head) problem and a block of 128 queries, the
// scores of each 64-key block are formed by MFMA, folded into a running
// softmax (row max and sum in registers) and multiplied into the output by
// MFMA without leaving registers; only O (bf16) and the log-sum-exp of every
// row (fp32, base 2) reach memory. Backward (k_flash_bwd_kv, below): per block
// of 128 keys, the probabilities are recomputed from that log-sum-exp.
//
// Sources: the block is Llama-2's (causal softmax attention scaled by
// 1/sqrt(128)); see qat_block.hip.
//
// Layout. 256 threads = 4 waves; wave w owns queries q0 + 32 w .. + 31 as two
// 16-row tiles. MFMA v_mfma_f32_16x16x32_bf16 with the B operand first, so a
// lane holds 4 consecutive columns of one row (16-row tile row lane & 15,
// columns 4 (lane >> 4) + 0..3 of a 16-column tile).
//   S = Q K^T: Q fragments (row, 8 consecutive d) from global, kept for the
//   whole loop; K fragments from the LDS key block.
//   O += P V: the probabilities of key tiles 2 ks and 2 ks + 1 form the A
//   fragment of k-step ks as they sit in registers (the lane's keys 32 ks + 4 g
//   + 0..3 and 32 ks + 16 + 4 g + 0..3, g = lane >> 4); the V fragment takes
//   the same keys by two transposing LDS reads (ds_read_b64_tr_b16).
// LDS: two buffers of the K and V blocks [64 keys][128 d] bf16 (256-byte
// rows); 16-byte chunk c of key row k sits at c ^ (k & 15), so both the K
// fragment reads and the V transposing reads use every bank equally.
#include <type_traits>

#include "qat_device.h"
#include "qat_dma.h"
#include "qat_internal.h"

namespace qat {
namespace {

constexpr int kHD = 128;             // head size
constexpr int kBQ = 128;             // queries per workgroup
constexpr int kBK = 64;              // keys per block
constexpr int kRowBytes = kHD * 2;   // 256
constexpr int kTileBytes = kBK * kRowBytes;               // 16 KiB per K or V block

__device__ __forceinline__ int swz(int k, int c) { return (c ^ (k & 15)) << 4; }

struct AttnArgs {
  const uint16_t* q;                 // [B*T][H] bf16 (after RoPE)
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;                       // [B*T][H] bf16
  float* lse;                        // [B*nh][T] fp32, log2 units
  int T, H, nh, batches;
  float scale_log2;                  // log2(e) / sqrt(128)
};

__global__ __launch_bounds__(256, 2) void k_flash_fwd(const AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * 2 * kTileBytes];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  // (query block, problem), all blocks of one problem on one XCD when the
  // problem count is a multiple of 8, longest (last) query blocks first
  const int nqb = (int)gridDim.x;
  int qb = blockIdx.x, prob = blockIdx.y;
  if ((a.batches & 7) == 0) {
    const int w = blockIdx.x + blockIdx.y * nqb;
    const int r = w % (8 * nqb);
    prob = 8 * (w / (8 * nqb)) + (r & 7);
    qb = nqb - 1 - (r >> 3);
  }
  const int b = prob / a.nh, h = prob - b * a.nh;
  const int64_t tok0 = (int64_t)b * a.T;
  const int q0 = qb * kBQ;
  // key blocks up to the diagonal (T is a multiple of 64; a ragged last query
  // block has rows past T, whose loads re-read row T - 1 and which are not stored)
  const int nkb = min((q0 + kBQ - 1) / kBK + 1, a.T / kBK);

  // K and V blocks by DMA: instruction j of a wave moves 4 rows (1 KiB); lane
  // l lands at row 4 (4 w + j) + l / 16, position l % 16, and fetches the
  // logical chunk that position holds
  const i32x4 rk = buffer_rsrc(a.k + tok0 * a.H + h * kHD, ((int64_t)(a.T - 1) * a.H + kHD) * 2);
  const i32x4 rv = buffer_rsrc(a.v + tok0 * a.H + h * kHD, ((int64_t)(a.T - 1) * a.H + kHD) * 2);
  const uint32_t lds0 = lds_addr_of(smem);
  uint32_t voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 4 * (4 * wave + j) + (lane >> 4);
    const int chunk = (lane & 15) ^ (row & 15);
    voff[j] = (uint32_t)(row * a.H * 2 + chunk * 16);
  }
  auto issue = [&](int kb, int buf) {
    kb = min(kb, nkb - 1);                               // past the last block: re-load it (uniform counts)
    const uint32_t base = lds0 + (uint32_t)(buf * 2 * kTileBytes);
    const uint32_t koff = (uint32_t)(kb * kBK * a.H * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t dst = (uint32_t)__builtin_amdgcn_readfirstlane((int)(base + (uint32_t)((4 * wave + j) * 1024)));
      dma16(rk, dst, voff[j] + koff);
      dma16(rv, dst + kTileBytes, voff[j] + koff);
    }
  };

  // Q fragments: rows q0 + 32 w + 16 i + r16, d = 32 ks + 8 g .. + 7
  bf16x8 qf[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint16_t* qr = a.q + (tok0 + min(q0 + 32 * wave + 16 * i + r16, a.T - 1)) * a.H + h * kHD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[i][ks] = *(const bf16x8*)(qr + 32 * ks);
  }
  issue(0, 0);
  issue(1, 1);

  f32x4 o[8][2];
#pragma unroll
  for (int jd = 0; jd < 8; ++jd)
#pragma unroll
    for (int i = 0; i < 2; ++i) o[jd][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Running softmax per row, base 2: m is the subtracted maximum and moves
  // only when a block's maximum exceeds it by more than kLazy (a wave-uniform
  // test), so the 64 output accumulators per lane are rescaled rarely; the
  // probabilities exp2(s - m) then stay below 2^kLazy, and O / l and the
  // log-sum-exp m + log2(l) do not depend on which m was subtracted.
  // exp2 is the hardware's v_exp_f32: results below 2^-126 flush to zero,
  // which no probability that matters reaches.
  constexpr float kLazy = 8.0f;
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  const int qrow0 = q0 + 32 * wave + r16;                // query of this lane in tile i: qrow0 + 16 i

  // One 64-key block; DIAG: the block crosses the diagonal of this query block
  // (keys beyond a row's query are masked), which only the last two do.
  auto key_block = [&](int kb, auto diag_c) {
    constexpr bool DIAG = decltype(diag_c)::value;
    wait_vmcnt<8>();                                     // this wave's DMA of block kb has landed
    __syncthreads();                                     // ... and everyone's
    const uint8_t* kt = smem + (kb & 1) * 2 * kTileBytes;
    const uint8_t* vt = kt + kTileBytes;
    // S = Q K^T for 64 keys: s[jt][i][r] = S[q of tile i][key 16 jt + 4 g + r]
    f32x4 s[4][2];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int i = 0; i < 2; ++i) s[jt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int key = 16 * jt + r16;
        const bf16x8 kf = *(const bf16x8*)(kt + key * kRowBytes + swz(key, 4 * ks + g));
#pragma unroll
        for (int i = 0; i < 2; ++i) s[jt][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[i][ks], s[jt][i], 0, 0, 0);
      }
    }
    // scaled scores and each row's block maximum (rows of tile i: query qrow0 + 16 i)
    float mx[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = qrow0 + 16 * i;
      float x = -INFINITY;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = s[jt][i][r] * a.scale_log2;
          if constexpr (DIAG) {
            if (kb * kBK + 16 * jt + 4 * g + r > q) v = -INFINITY;
          }
          s[jt][i][r] = v;
          x = fmaxf(x, v);
        }
      x = fmaxf(x, __shfl_xor(x, 16));
      mx[i] = fmaxf(x, __shfl_xor(x, 32));
    }
    // a row with every key masked has mx = -inf and never moves m; key 0 of
    // block 0 is valid for every row, so m is finite from block 0 on
    if (__any(mx[0] > m[0] + kLazy || mx[1] > m[1] + kLazy)) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float mn = fmaxf(m[i], mx[i]);
        const float alpha = __builtin_amdgcn_exp2f(m[i] - mn);
        l[i] *= alpha;
        m[i] = mn;
#pragma unroll
        for (int jd = 0; jd < 8; ++jd)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[jd][i][r] *= alpha;
      }
    }
    bf16x8 pf[2][2];                                      // [i][ks]
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float sum = 0.f;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(s[jt][i][r] - m[i]);
          s[jt][i][r] = p;
          sum += p;
        }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      l[i] += sum;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const f32x4 lo = s[2 * ks][i], hi = s[2 * ks + 1][i];
        pf[i][ks] = bf16x8{(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                           (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
      }
    }
    // O += P V: V fragment of d-tile jd and k-step ks = keys 32 ks + 4 g + 0..3
    // and 32 ks + 16 + 4 g + 0..3 at d = 16 jd + r16 (two transposing reads;
    // lane j of the 16-lane group addresses key k0 + j / 4, d 16 jd + 4 (j % 4))
    typedef short i16x4_ __attribute__((ext_vector_type(4)));
    const __attribute__((address_space(3))) uint8_t* vl = (const __attribute__((address_space(3))) uint8_t*)vt;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int jd = 0; jd < 8; ++jd) {
        const int d0 = 16 * jd + 4 * (r16 & 3);
        const int ka = 32 * ks + 4 * g + (r16 >> 2), kc = ka + 16;
        const i16x4_ lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_*)(vl + ka * kRowBytes + swz(ka, d0 >> 3) + (d0 & 7) * 2));
        const i16x4_ hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_*)(vl + kc * kRowBytes + swz(kc, d0 >> 3) + (d0 & 7) * 2));
        typedef short i16x8_ __attribute__((ext_vector_type(8)));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, (i16x8_)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int i = 0; i < 2; ++i) o[jd][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[i][ks], o[jd][i], 0, 0, 0);
      }
    }
    __syncthreads();                                     // every wave is done with this buffer
    issue(kb + 2, kb & 1);
  };
  // blocks kb < q0 / 64 lie wholly below the diagonal of every row here
  const int kd = min(q0 / kBK, nkb);
  int kb = 0;
  for (; kb < kd; ++kb) key_block(kb, std::false_type{});
  for (; kb < nkb; ++kb) key_block(kb, std::true_type{});
  wait_vmcnt<0>();                                       // drain the trailing re-loads

  // O / l to bf16; the log-sum-exp (base 2) of each row
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = qrow0 + 16 * i;
    if (q >= a.T) continue;
    const float inv = 1.0f / l[i];
    uint16_t* orow = a.o + (tok0 + q) * a.H + h * kHD + 4 * g;
#pragma unroll
    for (int jd = 0; jd < 8; ++jd)
      *(uint2*)(orow + 16 * jd) = make_uint2(pack_bf16x2(o[jd][i][0] * inv, o[jd][i][1] * inv),
                                             pack_bf16x2(o[jd][i][2] * inv, o[jd][i][3] * inv));
    if (g == 0) a.lse[(int64_t)prob * a.T + q] = m[i] + __log2f(l[i]);
  }
}

// ---------------------------------------------------------------------------
// Causal attention backward for dK and dV, fused: one workgroup per 128 keys
// of one (sequence, head) visits every 64-query block at or below the
// diagonal once. S^T = K Q^T and dP^T = V dO^T are recomputed by MFMA from the
// keys' K and V fragments held in registers; P^T = exp2(log2(e)/sqrt(128) S^T
// - lse) from the forward's row log-sum-exp, 0 where the query precedes the
// key; dS^T = P^T (dP^T - D) / sqrt(128) with D = rowsum(dO O); dV += P^T dO
// and dK += dS^T Q accumulate in registers, the P^T and dS^T fragments taken
// from registers as in the forward's P V; dS^T is also stored ([key][query]
// bf16) for the dQ product. Query blocks start at the key block's first key,
// so every (key, query) pair of the 128-row query tiles that product reads
// below a row's end is written (zero above the diagonal).
// Wave w owns keys k0 + 32 w .. + 31 as two 16-key tiles; a lane holds 4
// consecutive queries (S^T, dP^T) or 4 consecutive d (dK, dV) of one key.
// LDS, two buffers of: the Q and dO blocks [64 queries][128 d] (same swizzle
// as the forward's K and V blocks), lse and D of the 64 queries.
// ---------------------------------------------------------------------------
constexpr int kBKV = 128;            // keys per workgroup
constexpr int kBQB = 64;             // queries per block
constexpr int kRowTermBytes = kBQB * 4;
constexpr int kBwdBuf = 2 * kTileBytes + 2 * kRowTermBytes;

struct AttnBwdArgs {
  const uint16_t* q;                 // [B*T][H] bf16 (after RoPE)
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dO;                // the attention output's gradient
  const float* lse;                  // [B*nh][T], log2 units
  const float* D;                    // [B*nh][T], rowsum(dO O)
  uint16_t* dk;                      // [B*T][H] bf16
  uint16_t* dv;
  uint16_t* dsT;                     // [B*nh][T][T] bf16, dS^T[key][query]
  int T, H, nh, batches;
  float scale, scale_log2;           // 1/sqrt(128), log2(e)/sqrt(128)
};

__global__ __launch_bounds__(256) void k_flash_bwd_kv(const AttnBwdArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kBwdBuf];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  // (key block, problem): all blocks of one problem on one XCD when the
  // problem count is a multiple of 8; the first key blocks (most query
  // blocks) first
  const int nkb = (int)gridDim.x;
  int kbi = blockIdx.x, prob = blockIdx.y;
  if ((a.batches & 7) == 0) {
    const int w = blockIdx.x + blockIdx.y * nkb;
    const int r = w % (8 * nkb);
    prob = 8 * (w / (8 * nkb)) + (r & 7);
    kbi = r >> 3;
  }
  const int b = prob / a.nh, h = prob - b * a.nh;
  const int64_t tok0 = (int64_t)b * a.T;
  const int k0 = kbi * kBKV;
  const int qb0 = k0 / kBQB, nblk = a.T / kBQB - qb0;     // query blocks qb0 .. T/64 - 1

  // Q, dO blocks by DMA as the forward's K and V blocks; lse and D of the
  // block's queries by one dword DMA each (every wave issues the same two, so
  // the per-wave load counts stay uniform)
  const int64_t span = ((int64_t)(a.T - 1) * a.H + kHD) * 2;
  const i32x4 rq = buffer_rsrc(a.q + tok0 * a.H + h * kHD, span);
  const i32x4 rdo = buffer_rsrc(a.dO + tok0 * a.H + h * kHD, span);
  const i32x4 rl = buffer_rsrc(a.lse + (int64_t)prob * a.T, (int64_t)a.T * 4);
  const i32x4 rd = buffer_rsrc(a.D + (int64_t)prob * a.T, (int64_t)a.T * 4);
  const uint32_t lds0 = lds_addr_of(smem);
  uint32_t voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 4 * (4 * wave + j) + (lane >> 4);
    const int chunk = (lane & 15) ^ (row & 15);
    voff[j] = (uint32_t)(row * a.H * 2 + chunk * 16);
  }
  auto issue = [&](int jb, int buf) {
    jb = min(jb, nblk - 1);                              // past the last block: re-load it (uniform counts)
    const uint32_t base = lds0 + (uint32_t)(buf * kBwdBuf);
    const int q0 = (qb0 + jb) * kBQB;
    const uint32_t qoff = (uint32_t)(q0 * a.H * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t dst = (uint32_t)__builtin_amdgcn_readfirstlane((int)(base + (uint32_t)((4 * wave + j) * 1024)));
      dma16(rq, dst, voff[j] + qoff);
      dma16(rdo, dst + kTileBytes, voff[j] + qoff);
    }
    const uint32_t tb = (uint32_t)__builtin_amdgcn_readfirstlane((int)(base + 2 * kTileBytes));
    dma4(rl, tb, (uint32_t)((q0 + lane) * 4));
    dma4(rd, tb + kRowTermBytes, (uint32_t)((q0 + lane) * 4));
  };

  // K and V fragments of this wave's keys: key k0 + 32 w + 16 t + r16, d = 32 ks + 8 g .. + 7
  bf16x8 kf[2][4], vf[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int64_t row = tok0 + min(k0 + 32 * wave + 16 * t + r16, a.T - 1);
    const uint16_t* kr = a.k + row * a.H + h * kHD + 8 * g;
    const uint16_t* vr = a.v + row * a.H + h * kHD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      kf[t][ks] = *(const bf16x8*)(kr + 32 * ks);
      vf[t][ks] = *(const bf16x8*)(vr + 32 * ks);
    }
  }
  issue(0, 0);
  issue(1, 1);

  f32x4 dk[8][2], dv[8][2];
#pragma unroll
  for (int jd = 0; jd < 8; ++jd)
#pragma unroll
    for (int t = 0; t < 2; ++t) dk[jd][t] = dv[jd][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int key0 = k0 + 32 * wave + r16;                 // key of this lane in tile t: key0 + 16 t
  uint16_t* dsp = a.dsT + (int64_t)prob * a.T * a.T;

  // One 64-query block; DIAG: it meets the key block's diagonal (the first two do)
  auto query_block = [&](int jb, auto diag_c) {
    constexpr bool DIAG = decltype(diag_c)::value;
    const int q0 = (qb0 + jb) * kBQB;
    wait_vmcnt<10>();                                    // this wave's DMA of block jb has landed
    __syncthreads();                                     // ... and everyone's
    const uint8_t* qt = smem + (jb & 1) * kBwdBuf;
    const uint8_t* dot = qt + kTileBytes;
    const float* lse_l = (const float*)(qt + 2 * kTileBytes);
    const float* d_l = lse_l + kBQB;
    // S^T and dP^T: s[t][jq][r] = S^T[key0 + 16 t][q0 + 16 jq + 4 g + r]
    f32x4 s[2][4], dp[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) s[t][jq] = dp[t][jq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int qr = 16 * jq + r16;
        const bf16x8 qfr = *(const bf16x8*)(qt + qr * kRowBytes + swz(qr, 4 * ks + g));
        const bf16x8 dfr = *(const bf16x8*)(dot + qr * kRowBytes + swz(qr, 4 * ks + g));
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          s[t][jq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qfr, kf[t][ks], s[t][jq], 0, 0, 0);
          dp[t][jq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dfr, vf[t][ks], dp[t][jq], 0, 0, 0);
        }
      }
    }
    // P^T, dS^T (in place of s, dp); dS^T to memory
    f32x4 lq[4], dq[4];
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      lq[jq] = *(const f32x4*)(lse_l + 16 * jq + 4 * g);
      dq[jq] = *(const f32x4*)(d_l + 16 * jq + 4 * g);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = key0 + 16 * t;
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float p = __builtin_amdgcn_exp2f(s[t][jq][r] * a.scale_log2 - lq[jq][r]);
          if constexpr (DIAG) {
            if (q0 + 16 * jq + 4 * g + r < key) p = 0.0f;
          }
          s[t][jq][r] = p;
          dp[t][jq][r] = p * (dp[t][jq][r] - dq[jq][r]) * a.scale;
        }
        if (key < a.T)
          *(uint2*)(dsp + (int64_t)key * a.T + q0 + 16 * jq + 4 * g) =
              make_uint2(pack_bf16x2(dp[t][jq][0], dp[t][jq][1]), pack_bf16x2(dp[t][jq][2], dp[t][jq][3]));
      }
    }
    // A fragments of k-step kq (queries 32 kq + 4 g + 0..3 and 32 kq + 16 + 4 g + 0..3)
    bf16x8 pf[2][2], df[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        const f32x4 plo = s[t][2 * kq], phi = s[t][2 * kq + 1];
        const f32x4 dlo = dp[t][2 * kq], dhi = dp[t][2 * kq + 1];
        pf[t][kq] = bf16x8{(__bf16)plo[0], (__bf16)plo[1], (__bf16)plo[2], (__bf16)plo[3],
                           (__bf16)phi[0], (__bf16)phi[1], (__bf16)phi[2], (__bf16)phi[3]};
        df[t][kq] = bf16x8{(__bf16)dlo[0], (__bf16)dlo[1], (__bf16)dlo[2], (__bf16)dlo[3],
                           (__bf16)dhi[0], (__bf16)dhi[1], (__bf16)dhi[2], (__bf16)dhi[3]};
      }
    // dV += P^T dO, dK += dS^T Q: B fragments of d-tile jd (dO^T, Q^T) by two
    // transposing reads each, with the queries in the A fragments' order
    typedef short i16x4_ __attribute__((ext_vector_type(4)));
    typedef short i16x8_ __attribute__((ext_vector_type(8)));
    const __attribute__((address_space(3))) uint8_t* ql = (const __attribute__((address_space(3))) uint8_t*)qt;
    const __attribute__((address_space(3))) uint8_t* dl = (const __attribute__((address_space(3))) uint8_t*)dot;
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
#pragma unroll
      for (int jd = 0; jd < 8; ++jd) {
        const int d0 = 16 * jd + 4 * (r16 & 3);
        const int qa = 32 * kq + 4 * g + (r16 >> 2), qc = qa + 16;
        const int oa = qa * kRowBytes + swz(qa, d0 >> 3) + (d0 & 7) * 2;
        const int oc = qc * kRowBytes + swz(qc, d0 >> 3) + (d0 & 7) * 2;
        const i16x4_ dlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_*)(dl + oa));
        const i16x4_ dhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_*)(dl + oc));
        const i16x4_ qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_*)(ql + oa));
        const i16x4_ qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_*)(ql + oc));
        const bf16x8 dob = __builtin_bit_cast(bf16x8, (i16x8_)__builtin_shufflevector(dlo, dhi, 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8 qb = __builtin_bit_cast(bf16x8, (i16x8_)__builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          dv[jd][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dob, pf[t][kq], dv[jd][t], 0, 0, 0);
          dk[jd][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb, df[t][kq], dk[jd][t], 0, 0, 0);
        }
      }
    }
    __syncthreads();                                     // every wave is done with this buffer
    issue(jb + 2, jb & 1);
  };
  const int ndiag = min(2, nblk);
  int jb = 0;
  for (; jb < ndiag; ++jb) query_block(jb, std::true_type{});
  for (; jb < nblk; ++jb) query_block(jb, std::false_type{});
  wait_vmcnt<0>();                                       // drain the trailing re-loads

  // dK, dV: lane holds d = 16 jd + 4 g + 0..3 of key key0 + 16 t
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = key0 + 16 * t;
    if (key >= a.T) continue;
    uint16_t* kro = a.dk + (tok0 + key) * a.H + h * kHD + 4 * g;
    uint16_t* vro = a.dv + (tok0 + key) * a.H + h * kHD + 4 * g;
#pragma unroll
    for (int jd = 0; jd < 8; ++jd) {
      *(uint2*)(kro + 16 * jd) = make_uint2(pack_bf16x2(dk[jd][t][0], dk[jd][t][1]), pack_bf16x2(dk[jd][t][2], dk[jd][t][3]));
      *(uint2*)(vro + 16 * jd) = make_uint2(pack_bf16x2(dv[jd][t][0], dv[jd][t][1]), pack_bf16x2(dv[jd][t][2], dv[jd][t][3]));
    }
  }
}

}  // namespace

void launch_flash_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse, int B, int T,
                      int H, hipStream_t st) {
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.T = T;
  a.H = H;
  a.nh = H / kHD;
  a.batches = B * a.nh;
  a.scale_log2 = 1.4426950408889634f / sqrtf((float)kHD);
  LaunchTimer t("attn_fwd", st);
  QAT_LAUNCH(k_flash_fwd, dim3((unsigned)((T + kBQ - 1) / kBQ), (unsigned)a.batches), dim3(256), 0, st, a);
}

void launch_flash_bwd_kv(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dO,
                         const float* lse, const float* D, uint16_t* dk, uint16_t* dv, uint16_t* dsT, int B, int T,
                         int H, hipStream_t st) {
  AttnBwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dO = dO;
  a.lse = lse;
  a.D = D;
  a.dk = dk;
  a.dv = dv;
  a.dsT = dsT;
  a.T = T;
  a.H = H;
  a.nh = H / kHD;
  a.batches = B * a.nh;
  a.scale = 1.0f / sqrtf((float)kHD);
  a.scale_log2 = 1.4426950408889634f / sqrtf((float)kHD);
  LaunchTimer t("attn_bwd_kv", st);
  QAT_LAUNCH(k_flash_bwd_kv, dim3((unsigned)((T + kBKV - 1) / kBKV), (unsigned)a.batches), dim3(256), 0, st,
                     a);
}

}  // namespace qat
