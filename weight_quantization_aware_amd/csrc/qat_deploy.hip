// Deployment format and the inference linear of a quantised model (gfx950,
// wave64). paperlayer.ai summary of EfficientQAT, Appendix D: each group of g
// weights shares an FP16 step size and an N-bit zero point; Appendix A and
// section 4: the INT2 model's linear-layer matrix-vector product, measured
// against the FP16 linear.
//
// Format: the packed codes of qat_pack ([out][in*N/8], LSB-first per row),
// s16 = fp16(s) [out][G], and zq, the N-bit zero points clamp(rint(z), 0, K)
// as an LSB-first bitstream per row, row stride ceil(G*N/8) bytes.
//
// The linear: Y[M][out] = fp16(sum_k X[m][k] W_hat[o][k]), fp16 X and Y, with
// W_hat = fp16((q - z) * s16) and fp32 accumulation, for M = 1..16 tokens.
#include "qat_device.h"
#include "qat_dma.h"
#include "qat_internal.h"

namespace qat {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// s16 and zq from the fp32 step sizes and zero points. Thread i writes s16[i]
// (i < out*G) and zq byte i (i < out*ldz): the byte gathers the bits of the
// zero points that overlap it.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_deploy_qparams(const float* __restrict__ s, const float* __restrict__ z,
                                                        int64_t out, int64_t G, int N, float Kq, int64_t ldz,
                                                        uint16_t* __restrict__ s16, uint8_t* __restrict__ zq) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < out * G) s16[i] = __builtin_bit_cast(uint16_t, (_Float16)s[i]);
  if (i < out * ldz) {
    const int64_t o = i / ldz, b = i - o * ldz;
    const int64_t g0 = 8 * b / N, g1 = min<int64_t>(G - 1, (8 * b + 7) / N);
    uint32_t v = 0;
    for (int64_t g = g0; g <= g1; ++g) {
      const uint32_t c = (uint32_t)fminf(fmaxf(__builtin_rintf(z[o * G + g]), 0.0f), Kq);
      const int64_t sh = N * g - 8 * b;
      v |= sh >= 0 ? (c << sh) : (c >> -sh);
    }
    zq[i] = (uint8_t)v;
  }
}

// ---------------------------------------------------------------------------
// The inference linear. MFMA v_mfma_f32_16x16x32_f16: A = W_hat (16 weight
// rows), B = X^T (16 token columns, zero beyond M). A workgroup owns 16 rows;
// its 8 waves split `in` into super-steps of 256 (wave w takes super-steps
// w, w + 8, ...). In a super-step lane l (row / token l & 15, quarter
// kq = l >> 4) owns the 64 consecutive inputs k0 = 256 ss + 64 kq .. + 63, and
// MFMA step t (0..7) puts inputs k0 + 8t .. k0 + 8t + 7 in the lane's 8
// k-slots, for A and B alike. So a lane reads its row's 8N bytes of codes, its
// token's 128 bytes of X and one (s16, zq) group (two for groups of 32) per
// super-step; the next super-step's loads are issued before this one's math.
//
// Dequantisation of a pair of codes (a, b) into two fp16 lanes: the codes go
// into the low mantissa bits under the exponent of 1024 (bits 0x6400), so the
// pair reads (1024 + a, 1024 + b) exactly; a packed add of -(1024 + z) gives
// a - z, b - z exactly, and a packed multiply by s16 rounds once: fp16((q - z)
// s16). Accumulation is fp32 in the MFMA; the 8 waves' partial sums meet in
// LDS and are rounded once to fp16.
// ---------------------------------------------------------------------------
// One lane's share of a 64-input chunk of one weight row: the codes and the
// raw step size / zero-point bits of the chunk's group (two groups of 32).
template <int N>
struct RowChunk {
  uint32_t c[2 * N];     // 64 codes, N * 8 bytes
  uint32_t sb[2], zb[2]; // raw s16 bits and zq bytes of the chunk's (first, second) group
};

// A chunk of the X-in-registers kernel: the row part plus the token's X.
template <int N>
struct Chunk {
  RowChunk<N> w;
  h8 x[8];               // X[tok][k0 + 8t .. + 7], t = 0..7
  int kl;                // first input of the chunk (clamped into range)
  bool live;             // false: the chunk lies beyond `in` (ragged last super-step)
};

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

// Codes 2a and 2a + 1 of step t (the step's 8 codes are k0 + 8t .. + 7) at
// bits 0.. and 16.. of a dword; other bits are garbage, removed by the mask.
template <int N>
__device__ __forceinline__ uint32_t code_pair(const uint32_t (&c)[2 * N], int t, int a) {
  if constexpr (N == 2) {
    const uint32_t h = (c[t >> 1] >> (16 * (t & 1))) & 0xFFFFu;
    const u16x2 v = u16x2{(uint16_t)h, (uint16_t)h} >> u16x2{(uint16_t)(4 * a), (uint16_t)(4 * a + 2)};
    return __builtin_bit_cast(uint32_t, v);
  } else if constexpr (N == 4) {
    const uint32_t h = (c[t] >> (16 * (a >> 1))) & 0xFFFFu;
    const uint16_t s0 = (uint16_t)(8 * (a & 1));
    const u16x2 v = u16x2{(uint16_t)h, (uint16_t)h} >> u16x2{s0, (uint16_t)(s0 + 4)};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    const int bit = 24 * t, w = bit >> 5, sh = bit & 31;
    uint32_t x = c[w] >> sh;
    if (sh > 8) x |= c[w + 1] << (32 - sh);
    const uint32_t u = (x >> (6 * a)) & 63u;    // the two codes, nothing above them
    return u | (u << 13);
  }
}

// Loop-invariant constants in registers: VOP3 instructions (v_and_or_b32)
// take no literal operands on gfx950, so the code mask sits in an SGPR and the
// exponent bits of 1024 in a VGPR. The asm makes the values opaque, so the
// compiler cannot turn them back into literals of separate v_and / v_or.
struct DqConst {
  uint32_t mask, magic;
};

template <int N>
__device__ __forceinline__ DqConst dq_const() {
  DqConst k;
  asm volatile("s_mov_b32 %0, %1" : "=s"(k.mask) : "i"(((1u << N) - 1) * 0x00010001u));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(k.magic));
  return k;
}

template <int N>
__device__ __forceinline__ h8 dequant_step(const uint32_t (&c)[2 * N], int t, const DqConst& k,
                                           const uint32_t (&zc)[2], const uint32_t (&sc)[2]) {
  uint32_t p[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) p[a] = code_pair<N>(c, t, a);
#pragma unroll
  for (int a = 0; a < 4; ++a) p[a] = (p[a] & k.mask) | k.magic;
  h2 w[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) w[a] = as_h2(p[a]) + as_h2(zc[t >> 2]);
#pragma unroll
  for (int a = 0; a < 4; ++a) w[a] = w[a] * as_h2(sc[t >> 2]);
  return __builtin_bit_cast(h8, w);
}

struct GemvArgs {
  const uint16_t* X;
  const uint8_t* Wq;
  const uint16_t* s16;
  const uint8_t* zq;
  int M, out, K;
  int64_t G, ldq, ldz;
  int group;
  uint16_t* Y;
};

// Loads of one chunk (issue only: nothing here waits for them). Rows beyond
// `out` and tokens beyond M read the last row / token instead: they only feed
// output rows and columns that are never stored. In the ragged last
// super-step a lane whose k0 lies beyond `in` reads the last chunk and is
// zeroed when it is used.
template <int N>
__device__ __forceinline__ void load_row_chunk(const GemvArgs& a, const FastDiv& gdiv, int row, int kl,
                                               RowChunk<N>& w) {
  const uint8_t* src = a.Wq + (int64_t)row * a.ldq + (int64_t)(kl / 64) * (8 * N);
  if constexpr (N == 2) {
    const uint4 v = *(const uint4*)src;
    w.c[0] = v.x, w.c[1] = v.y, w.c[2] = v.z, w.c[3] = v.w;
  } else if constexpr (N == 4) {
    const uint4 v0 = *(const uint4*)src, v1 = *(const uint4*)(src + 16);
    w.c[0] = v0.x, w.c[1] = v0.y, w.c[2] = v0.z, w.c[3] = v0.w;
    w.c[4] = v1.x, w.c[5] = v1.y, w.c[6] = v1.z, w.c[7] = v1.w;
  } else {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const uint2 v = *(const uint2*)(src + 8 * i);
      w.c[2 * i] = v.x, w.c[2 * i + 1] = v.y;
    }
  }
  const int64_t g0 = gdiv.div((uint32_t)kl);
  const int64_t g1 = a.group == 32 ? g0 + 1 : g0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t g = h ? g1 : g0;
    w.sb[h] = a.s16[(int64_t)row * a.G + g];
    const int64_t bit = g * N;
    const uint8_t* zr = a.zq + (int64_t)row * a.ldz + (bit >> 3);
    // the byte after the field's first byte (the same byte again at the row's
    // end); its bits are used only when the field straddles the two
    w.zb[h] = zr[0] | (uint32_t)zr[(bit >> 3) + 1 < a.ldz ? 1 : 0] << 8;
  }
}

// Loads of one chunk (issue only: nothing here waits for them). Rows beyond
// `out` and tokens beyond M read the last row / token instead: they only feed
// output rows and columns that are never stored. In the ragged last
// super-step a lane whose k0 lies beyond `in` reads the last chunk and is
// zeroed when it is used.
template <int N>
__device__ __forceinline__ void load_chunk(const GemvArgs& a, const FastDiv& gdiv, int row, int tok, int k0,
                                           Chunk<N>& ch) {
  ch.live = k0 < a.K;
  ch.kl = ch.live ? k0 : a.K - 64;
  load_row_chunk<N>(a, gdiv, row, ch.kl, ch.w);
  const h8* xs = (const h8*)(a.X + (int64_t)tok * a.K + ch.kl);
#pragma unroll
  for (int t = 0; t < 8; ++t) ch.x[t] = xs[t];
}

// -(1024 + z) and s16 fp16 pairs of the chunk's two group slots; zero step
// sizes for a dead chunk make its dequantised weights exactly 0.
template <int N>
__device__ __forceinline__ void decode_qparams(const RowChunk<N>& w, const GemvArgs& a, const FastDiv& gdiv, int kl,
                                               bool live, uint32_t (&zc)[2], uint32_t (&sc)[2]) {
  const int64_t g0 = gdiv.div((uint32_t)kl);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int sh = (int)(((h && a.group == 32 ? g0 + 1 : g0) * N) & 7);
    const uint32_t zv = (w.zb[h] >> sh) & ((1u << N) - 1);
    zc[h] = (0xE400u | zv) * 0x00010001u;
    sc[h] = live ? w.sb[h] * 0x00010001u : 0u;
  }
}

// The 8 MFMA steps of a chunk, alternating between two accumulators; the
// next step's operand is dequantised before this step's MFMA is issued.
template <int N>
__device__ __forceinline__ void gemv_steps(Chunk<N>& ch, const GemvArgs& a, const FastDiv& gdiv, bool tail,
                                           const DqConst& k, f32x4 (&acc)[2]) {
  uint32_t zc[2], sc[2];
  decode_qparams<N>(ch.w, a, gdiv, ch.kl, ch.live, zc, sc);
  if (tail) {                                    // wave-uniform: only the ragged last super-step
    if (!ch.live) {
#pragma unroll
      for (int t = 0; t < 8; ++t) ch.x[t] = h8{};
    }
  }
  h8 A = dequant_step<N>(ch.w.c, 0, k, zc, sc);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const h8 An = dequant_step<N>(ch.w.c, t < 7 ? t + 1 : t, k, zc, sc);
    acc[t & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, ch.x[t], acc[t & 1], 0, 0, 0);
    A = An;
  }
}

template <int N>
__global__ __launch_bounds__(512, 2) void k_deploy_gemv(const GemvArgs a) {
  __shared__ float red[8][4 * 64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int kq = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int row = min(row0 + (lane & 15), a.out - 1), tok = min(lane & 15, a.M - 1);
  const FastDiv gdiv = FastDiv::make((uint32_t)a.group);
  const int nfull = a.K / 256, nss = (a.K + 255) / 256;
  auto load = [&](int ss, Chunk<N>& ch) {
    load_chunk<N>(a, gdiv, row, tok, ss * 256 + 64 * kq, ch);
    asm volatile("" ::: "memory");                       // keep the prefetch ahead of the math
  };

  const DqConst k = dq_const<N>();
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  int ss = wave;
  if (ss < nss) {                            // wave-uniform
    // Two buffers, no register copies. The prefetch is unconditional (past
    // the end it re-reads the last super-step), so no branch separates a
    // load from its use and the compiler waits for exactly the loads needed.
    Chunk<N> c0, c1;
    load(ss, c0);
    for (;;) {
      load(min(ss + 8, nss - 1), c1);
      gemv_steps<N>(c0, a, gdiv, ss >= nfull, k, acc);
      ss += 8;
      if (ss >= nss) break;
      load(min(ss + 8, nss - 1), c0);
      gemv_steps<N>(c1, a, gdiv, ss >= nfull, k, acc);
      ss += 8;
      if (ss >= nss) break;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][i * 64 + lane] = acc[0][i] + acc[1][i];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int l = threadIdx.x & 63, i = threadIdx.x >> 6;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) sum += red[w][i * 64 + l];
    const int t = l & 15, o = row0 + 4 * (l >> 4) + i;
    if (t < a.M && o < a.out) a.Y[(int64_t)t * a.out + o] = __builtin_bit_cast(uint16_t, (_Float16)sum);
  }
}

// ---------------------------------------------------------------------------
// The inference linear with X staged in LDS (used whenever X [M][in] fp16 fits
// in LDS): a persistent workgroup of 16 waves per CU. Workgroup b takes the
// row blocks b, b + grid, ... of 16 RW weight rows (RW row tiles); in each,
// its waves split `in` into chunks of 256 inputs (wave w takes chunks w,
// w + 16, ...) and run all RW tiles on them, so one X fragment read from LDS
// feeds RW MFMAs. The in-chunk mapping is that of the kernel above.
//
// X reaches LDS once per workgroup, by direct-to-LDS loads issued after the
// wave's first code loads so that both are in flight together. Each token's
// row takes lds_x_stride(in) halves, whole KiB with at least 192 inputs of
// zeros after the row, and rows are 16 bytes further apart than that
// (lds_x_pitch: the tokens of one fragment read on distinct banks): a lane whose chunk lies beyond `in` (the
// ragged last chunk) reads those zeros as X and the last valid chunk as codes,
// so it adds exactly 0 without any masking.
//
// A wave's chunks over all its row blocks form one sequence of jobs, and the
// codes of the next NB - 1 jobs are in flight while it computes the current
// one (NB register buffers; loads past the last job re-read it, so no branch
// separates a load from its use), also across row-block ends. A job's step
// sizes and zero points come by one 16-byte load per lane (qp_load) rather
// than as per-lane 1- and 2-byte loads, whose instruction count, not their
// bytes, limited the first version of this kernel. At the end of a
// row block a wave writes its partial sums to LDS (one fp32 per row and token
// < M, a slot per row block) and adds one to the row block's LDS counter; the
// wave that brings the counter to the number of busy waves adds the partials
// and rounds them once to fp16, into an LDS copy of the workgroup's outputs
// that goes to HBM after the last row block. No wave waits for another
// before the end (a global store inside the loop would also make later waits
// for code loads wait for it: one counter covers both).
// ---------------------------------------------------------------------------
__host__ __device__ inline int lds_x_stride(int K) { return ((K * 2 + 384 + 1023) / 1024) * 512; }
// Halves between two token rows in LDS: the row plus 16 bytes, so that the
// tokens of one fragment read (lane & 15) fall on distinct banks.
__host__ __device__ inline int lds_x_pitch(int K) { return lds_x_stride(K) + 8; }

// LDS layout of the kernel below (byte offsets; the same on host and device).
struct DeployLds {
  int part, cnt, ybuf, qp, total;
  __host__ __device__ static DeployLds of(int M, int K, int my_rb, int RW, int NB = 3) {
    DeployLds l;
    auto up = [](int v) { return (v + 1023) / 1024 * 1024; };
    l.part = M * lds_x_pitch(K) * 2;
    l.cnt = l.part + up(my_rb * 16 * RW * 16 * M * 4);
    l.ybuf = l.cnt + up(my_rb * 4);
    l.qp = l.ybuf + up(my_rb * M * RW * 16 * 2);
    l.total = l.qp + 16 * NB * 2 * RW * 16 * 16;
    return l;
  }
};

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The codes of one chunk of RW row tiles and this lane's piece of its step
// sizes or zero points (see qp_load).
template <int N, int RW>
struct CodeChunks {
  uint4 q;               // this lane's 16-byte piece of step sizes or zero points (qp_load)
  uint32_t c[RW][2 * N]; // (q first: no padding, which keeps the 3-bit case out of scratch memory)
};

template <int N>
__device__ __forceinline__ void load_codes(const GemvArgs& a, int row, int kl, uint32_t (&c)[2 * N]) {
  const uint8_t* src = a.Wq + (int64_t)row * a.ldq + (int64_t)(kl / 64) * (8 * N);
  if constexpr (N == 2) {
    const uint4 v = *(const uint4*)src;
    c[0] = v.x, c[1] = v.y, c[2] = v.z, c[3] = v.w;
  } else if constexpr (N == 4) {
    const uint4 v0 = *(const uint4*)src, v1 = *(const uint4*)(src + 16);
    c[0] = v0.x, c[1] = v0.y, c[2] = v0.z, c[3] = v0.w;
    c[4] = v1.x, c[5] = v1.y, c[6] = v1.z, c[7] = v1.w;
  } else {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const uint2 v = *(const uint2*)(src + 8 * i);
      c[2 * i] = v.x, c[2 * i + 1] = v.y;
    }
  }
}

template <int N, int RW, int NB>
__global__ __launch_bounds__(1024) void k_deploy_gemv_lds(const GemvArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t dsm[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int kq = lane >> 4, r16 = lane & 15;
  const int tok = min(r16, a.M - 1);
  const FastDiv gdiv = FastDiv::make((uint32_t)a.group);
  const int nch = (a.K + 255) / 256;
  const int nbusy = min(nch, 16);                        // waves with chunks
  const int xs = lds_x_stride(a.K);                      // halves of a token row in LDS (data and zeros)
  const int xp = lds_x_pitch(a.K);                       // halves from one token row to the next
  const _Float16* xl = (const _Float16*)dsm;
  const int nrb = (a.out + 16 * RW - 1) / (16 * RW);
  const int my_rb = (nrb - 1 - (int)blockIdx.x) / (int)gridDim.x + 1;   // grid <= nrb
  // LDS after X: partial sums [my_rb][16][RW * 16][M] fp32, arrival counters
  // [my_rb], the workgroup's outputs [my_rb][M][RW * 16] fp16, and per wave
  // and code buffer 2 RW * 16 16-byte pieces of step sizes and zero points
  // (qp_load)
  const DeployLds L = DeployLds::of(a.M, a.K, my_rb, RW, NB);
  float* part = (float*)(dsm + L.part);
  uint32_t* cnt = (uint32_t*)(dsm + L.cnt);
  uint16_t* ybuf = (uint16_t*)(dsm + L.ybuf);
  uint8_t* qp = dsm + L.qp;
  const int cpw = wave < nch ? (nch - 1 - wave) / 16 + 1 : 0;         // chunks per row block
  const int njobs = cpw * my_rb;

  // Step sizes and zero points of a chunk, for all RW * 16 rows, by one
  // 16-byte load per lane: lane L < RW * 16 fetches 16 bytes of s16 holding
  // row L's step sizes for the chunk's groups, lane RW * 16 + L 16 bytes of zq
  // holding the row's zero-point bits for them. Each piece starts at the
  // 4-byte aligned address at or below the first needed byte, moved back if
  // needed so that it ends inside its buffer (both buffers hold at least 16
  // bytes); piece_start() gives the start on both sides. At use time the wave
  // passes the pieces through its LDS slot, so that each lane can read the
  // values of its own rows and groups.
  const uint32_t s_size = (uint32_t)(a.out * a.G * 2), z_size = (uint32_t)(a.out * a.ldz);
  auto piece_start = [&](uint32_t first, uint32_t size) __attribute__((always_inline)) { return min(first & ~3u, size - 16u); };
  auto qp_load = [&](int rb, int c, uint4& q) __attribute__((always_inline)) {
    const int g_first = (int)gdiv.div((uint32_t)(c * 256));
    const int L = lane & (RW * 16 - 1);
    const int row = min(rb * 16 * RW + L, a.out - 1);
    const bool sp = lane < RW * 16;
    const uint32_t src = sp ? piece_start((uint32_t)(row * a.G + g_first) * 2u, s_size)
                            : piece_start((uint32_t)(row * a.ldz) + ((uint32_t)g_first * N >> 3), z_size);
    q = *(const uint4*)((sp ? (const uint8_t*)a.s16 : a.zq) + src);
  };

  // loads walk the job sequence with their own (row block, chunk) counters
  int l_rb = 0, l_cc = 0, l_j = 0;
  auto load = [&](CodeChunks<N, RW>& b, int jb) __attribute__((always_inline)) {
    const int rb = (int)blockIdx.x + l_rb * (int)gridDim.x;
    const int c = wave + 16 * l_cc;
    qp_load(rb, c, b.q);
    const int k0 = c * 256 + 64 * kq;
    const int kl = k0 < a.K ? k0 : a.K - 64;
#pragma unroll
    for (int i = 0; i < RW; ++i) load_codes<N>(a, min(rb * 16 * RW + 16 * i + r16, a.out - 1), kl, b.c[i]);
    asm volatile("" ::: "memory");                       // keep the prefetch ahead of the math
    if (l_j + 1 < njobs) {
      ++l_j;
      if (++l_cc == cpw) {
        l_cc = 0;
        ++l_rb;
      }
    }
  };
  // named buffers (an array of them ends up in scratch memory when the
  // compiler keeps a loop over it)
  CodeChunks<N, RW> b0, b1, b2;
  if (cpw > 0) {
    load(b0, 0);
    load(b1, 1);
    if constexpr (NB == 3) load(b2, 2);
  }
  {
    // token m's row: xs * 2 / 1024 instructions of 1 KiB; source bytes past the
    // row's end are moved out of the buffer's range, so they land as zeros
    const i32x4 rsrc = buffer_rsrc(a.X, (int64_t)a.M * a.K * 2);
    const uint32_t base = lds_addr_of(dsm);
    const int per_row = xs * 2 / 1024;
    for (int i = wave; i < a.M * per_row; i += 16) {
      const int m = i / per_row, j = i - m * per_row;
      const int col = j * 1024 + 16 * lane;              // byte within the row
      const uint32_t src = col < a.K * 2 ? (uint32_t)(m * a.K * 2 + col) : 0x7FFFFFF0u;
      dma16(rsrc, (uint32_t)__builtin_amdgcn_readfirstlane((int)(base + (uint32_t)(m * xp * 2 + j * 1024))), src);
    }
  }
  for (int i = threadIdx.x; i < my_rb; i += 1024) cnt[i] = 0;
  wait_vmcnt<0>();
  __syncthreads();

  const DqConst k = dq_const<N>();
  f32x4 acc[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const CodeChunks<N, RW>& bc, int cc, int jb, int rbi) __attribute__((always_inline)) {
    const int c = wave + 16 * cc;
    const int k0 = c * 256 + 64 * kq;
    const int kl = k0 < a.K ? k0 : a.K - 64;
    const int g_first = (int)gdiv.div((uint32_t)(c * 256));
    const int g0 = (int)gdiv.div((uint32_t)kl);
    uint8_t* slot = qp + (wave * NB + jb) * (2 * RW * 16 * 16);
    if (lane < 2 * RW * 16) *(uint4*)(slot + 16 * lane) = bc.q;   // read back below by this wave only
    uint32_t zc[RW][2], sc[RW][2];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int row = min(((int)blockIdx.x + rbi * (int)gridDim.x) * 16 * RW + 16 * i + r16, a.out - 1);
      const uint32_t s0 = piece_start((uint32_t)(row * a.G + g_first) * 2u, s_size);
      const uint32_t z0 = piece_start((uint32_t)(row * a.ldz) + ((uint32_t)g_first * N >> 3), z_size);
      const uint8_t* sp = slot + (16 * i + r16) * 16;
      const uint32_t* zp = (const uint32_t*)(slot + (RW * 16 + 16 * i + r16) * 16);
      auto decode = [&](int g, uint32_t& zcv, uint32_t& scv) __attribute__((always_inline)) {
        const uint32_t sbits = *(const uint16_t*)(sp + ((uint32_t)(row * a.G + g) * 2u - s0));
        const int bit = (int)(((uint32_t)(row * a.ldz) - z0) * 8u + (uint32_t)(g * N));
        const int w = bit >> 5;
        const uint64_t zw = (uint64_t)zp[w] | ((uint64_t)zp[min(w + 1, 3)] << 32);
        const uint32_t zv = (uint32_t)(zw >> (bit & 31)) & ((1u << N) - 1);
        zcv = (0xE400u | zv) * 0x00010001u;
        scv = sbits * 0x00010001u;
      };
      decode(g0, zc[i][0], sc[i][0]);
      if (a.group == 32) {                               // wave-uniform: the chunk's second group
        decode(g0 + 1, zc[i][1], sc[i][1]);
      } else {
        zc[i][1] = zc[i][0];
        sc[i][1] = sc[i][0];
      }
    }
    const _Float16* xr = xl + tok * xp + k0;             // zeros past `in`
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const h8 B = *(const h8*)(xr + 8 * t);
#pragma unroll
      for (int i = 0; i < RW; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant_step<N>(bc.c[i], t, k, zc[i], sc[i]), B, acc[i], 0,
                                                        0, 0);
    }
  };
  // end of row block rbi: this wave's partial sums to LDS; the last of the
  // busy waves to arrive reduces them into ybuf
  auto flush = [&](int rbi) __attribute__((always_inline)) {
    float* pp = part + rbi * (16 * RW * 16 * a.M);
    if (r16 < a.M) {
#pragma unroll
      for (int i = 0; i < RW; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) pp[((wave * RW + i) * 16 + 4 * kq + r) * a.M + r16] = acc[i][r];
      }
    }
#pragma unroll
    for (int i = 0; i < RW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // LDS operations of a wave are performed in order: the partials are in
    // place before the increment, and every wave counted before ours has
    // written its own
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");    // partials written before the count
    uint32_t prev = 0;
    if (lane == 0) prev = atomicAdd(cnt + rbi, 1u);
    prev = __builtin_amdgcn_readfirstlane(prev);
    asm volatile("" ::: "memory");                        // no partial is read before the count
    if (prev == (uint32_t)nbusy - 1) {
      for (int e = lane; e < RW * 16 * a.M; e += 64) {
        const int m = e % a.M, rr = e / a.M;             // rr: row within the row block
        float sum = 0.f;
        for (int w = 0; w < nbusy; ++w) sum += pp[(w * RW * 16 + rr) * a.M + m];
        ybuf[(rbi * a.M + m) * (RW * 16) + rr] = __builtin_bit_cast(uint16_t, (_Float16)sum);
      }
    }
  };
  if (cpw > 0) {
    // the loads are unconditional (past the last job they re-read it), so no
    // branch separates a load from its use and the compiler's waits count
    // exactly the loads still needed
    int cc = 0, rbi = 0;
    auto step = [&](CodeChunks<N, RW>& bc, int j, int jb) __attribute__((always_inline)) {
      if (j < njobs) {                                   // wave-uniform
        compute(bc, cc, jb, rbi);
        if (++cc == cpw) {
          flush(rbi);
          cc = 0;
          ++rbi;
        }
      }
      load(bc, jb);
    };
    for (int j0 = 0; j0 < njobs; j0 += NB) {
      step(b0, j0, 0);
      step(b1, j0 + 1, 1);
      if constexpr (NB == 3) step(b2, j0 + 2, 2);
    }
  }
  lds_barrier();
  for (int e = threadIdx.x; e < my_rb * a.M * RW * 16; e += 1024) {
    const int rr = e % (RW * 16), m = (e / (RW * 16)) % a.M, rbi = e / (RW * 16 * a.M);
    const int o = ((int)blockIdx.x + rbi * (int)gridDim.x) * 16 * RW + rr;
    if (o < a.out) a.Y[(int64_t)m * a.out + o] = ybuf[e];
  }
}

// ---------------------------------------------------------------------------
// The inference linear when X [M][in] is too large for LDS (several tokens on
// a wide input, e.g. M = 16 at in = 8192): persistent workgroups of 16 waves
// stage X one chunk of 4096 inputs at a time, and a workgroup takes every
// chunk for all of its row blocks (row blocks b, b + grid, ...), so X crosses
// L2 once per workgroup rather than once per 16 rows. In a chunk, wave w takes
// the 256 inputs w * 256 .. + 255 (in-chunk lane mapping of the kernels
// above) for 16 rows; the 16 waves' partial sums of a row block meet in LDS
// behind a barrier and are added, in wave order, to the row block's fp32
// accumulator; after the last chunk the accumulators are rounded once to
// fp16. Each token's row of the X chunk sits at a stride of 4096 + 8 halves:
// the 16 tokens of a fragment read fall on distinct banks. Inputs beyond `in`
// are staged as zeros and multiply the last valid codes (adds exactly 0).
// Code loads run two jobs ahead of the math, across row blocks and chunks.
// ---------------------------------------------------------------------------
constexpr int kXC = 4096;                                // inputs per X chunk: 16 waves x 256
constexpr int kXStride = kXC + 8;                        // halves per token row in LDS

struct XChunkLds {
  int part, yacc, qp, total;
  __host__ __device__ static XChunkLds of(int M, int my_rb) {
    XChunkLds l;
    l.part = M * kXStride * 2;                           // X chunk [M][kXStride] fp16 at 0
    l.yacc = l.part + 16 * 16 * M * 4;                   // partials [16 waves][16 rows][M] fp32
    l.qp = l.yacc + my_rb * 16 * M * 4;                  // accumulators [my_rb][16 rows][M] fp32
    l.total = l.qp + 16 * 2 * 16 * 16;                   // step-size / zero-point pieces [16 waves][32][16 B]
    return l;
  }
};

template <int N>
__global__ __launch_bounds__(1024) void k_deploy_gemv_xchunk(const GemvArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t dsm[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int kq = lane >> 4, r16 = lane & 15;
  const int tok = min(r16, a.M - 1);
  const FastDiv gdiv = FastDiv::make((uint32_t)a.group);
  const int nch = (a.K + 255) / 256;                     // 256-input chunks
  const int nxc = (a.K + kXC - 1) / kXC;                 // X chunks
  const int nrb = (a.out + 15) / 16;
  const int my_rb = (nrb - 1 - (int)blockIdx.x) / (int)gridDim.x + 1;   // grid <= nrb
  const int njobs = nxc * my_rb;                         // the same sequence for every wave
  const XChunkLds L = XChunkLds::of(a.M, my_rb);
  const _Float16* xl = (const _Float16*)dsm;
  float* part = (float*)(dsm + L.part);
  float* yacc = (float*)(dsm + L.yacc);
  uint8_t* slot = dsm + L.qp + wave * (2 * 16 * 16);

  // job j: X chunk j / my_rb, row block (j % my_rb); chunk c of 256 inputs
  auto job_rb = [&](int j) __attribute__((always_inline)) { return (int)blockIdx.x + (j % my_rb) * (int)gridDim.x; };
  auto job_c = [&](int j) __attribute__((always_inline)) { return (j / my_rb) * 16 + wave; };

  // step sizes and zero points of a chunk by one 16-byte piece per lane (as in
  // the kernel above, one row tile)
  const uint32_t s_size = (uint32_t)(a.out * a.G * 2), z_size = (uint32_t)(a.out * a.ldz);
  auto piece_start = [&](uint32_t first, uint32_t size) __attribute__((always_inline)) { return min(first & ~3u, size - 16u); };
  auto load = [&](CodeChunks<N, 1>& b, int j) __attribute__((always_inline)) {
    j = min(j, njobs - 1);                               // past the last job: re-read it
    const int rb = job_rb(j), c = min(job_c(j), nch - 1);
    const int g_first = (int)gdiv.div((uint32_t)(c * 256));
    const int row = min(rb * 16 + r16, a.out - 1);
    const bool sp = lane < 16;
    const uint32_t src = sp ? piece_start((uint32_t)(row * a.G + g_first) * 2u, s_size)
                            : piece_start((uint32_t)(row * a.ldz) + ((uint32_t)g_first * N >> 3), z_size);
    b.q = *(const uint4*)((sp ? (const uint8_t*)a.s16 : a.zq) + src);
    const int k0 = c * 256 + 64 * kq;
    load_codes<N>(a, row, k0 < a.K ? k0 : a.K - 64, b.c[0]);
    asm volatile("" ::: "memory");                       // keep the prefetch ahead of the math
  };
  const DqConst k = dq_const<N>();
  auto compute = [&](const CodeChunks<N, 1>& bc, int j, f32x4& acc) __attribute__((always_inline)) {
    const int rb = job_rb(j), c = job_c(j);
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (c >= nch) return;                                // wave-uniform: no chunk for this wave here
    const int k0 = c * 256 + 64 * kq;
    const int kl = k0 < a.K ? k0 : a.K - 64;
    const int g_first = (int)gdiv.div((uint32_t)(c * 256));
    const int g0 = (int)gdiv.div((uint32_t)kl);
    if (lane < 32) *(uint4*)(slot + 16 * lane) = bc.q;   // read back below by this wave only
    const int row = min(rb * 16 + r16, a.out - 1);
    const uint32_t s0 = piece_start((uint32_t)(row * a.G + g_first) * 2u, s_size);
    const uint32_t z0 = piece_start((uint32_t)(row * a.ldz) + ((uint32_t)g_first * N >> 3), z_size);
    const uint8_t* sp = slot + r16 * 16;
    const uint32_t* zp = (const uint32_t*)(slot + (16 + r16) * 16);
    uint32_t zc[2], sc[2];
    auto decode = [&](int g, uint32_t& zcv, uint32_t& scv) __attribute__((always_inline)) {
      const uint32_t sbits = *(const uint16_t*)(sp + ((uint32_t)(row * a.G + g) * 2u - s0));
      const int bit = (int)(((uint32_t)(row * a.ldz) - z0) * 8u + (uint32_t)(g * N));
      const int w = bit >> 5;
      const uint64_t zw = (uint64_t)zp[w] | ((uint64_t)zp[min(w + 1, 3)] << 32);
      const uint32_t zv = (uint32_t)(zw >> (bit & 31)) & ((1u << N) - 1);
      zcv = (0xE400u | zv) * 0x00010001u;
      scv = sbits * 0x00010001u;
    };
    decode(g0, zc[0], sc[0]);
    if (a.group == 32) {                                 // wave-uniform: the chunk's second group
      decode(g0 + 1, zc[1], sc[1]);
    } else {
      zc[1] = zc[0];
      sc[1] = sc[0];
    }
    const _Float16* xr = xl + tok * kXStride + (k0 - (j / my_rb) * kXC);   // zeros past `in`
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const h8 B = *(const h8*)(xr + 8 * t);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant_step<N>(bc.c[0], t, k, zc, sc), B, acc, 0, 0, 0);
    }
  };

  CodeChunks<N, 1> b0, b1;
  load(b0, 0);
  load(b1, 1);
  for (int e = threadIdx.x; e < my_rb * 16 * a.M; e += 1024) yacc[e] = 0.f;
  const i32x4 rsrc = buffer_rsrc(a.X, (int64_t)a.M * a.K * 2);
  const uint32_t xbase = lds_addr_of(dsm);
  // one row block of job j (buffer bc): partials, sum in wave order, prefetch
  auto step = [&](CodeChunks<N, 1>& bc, int j) __attribute__((always_inline)) {
    f32x4 acc;
    compute(bc, j, acc);
    load(bc, j + 2);
    if (r16 < a.M) {
#pragma unroll
      for (int r = 0; r < 4; ++r) part[(wave * 16 + 4 * kq + r) * a.M + r16] = acc[r];
    }
    lds_barrier();
    float* ya = yacc + (j % my_rb) * 16 * a.M;
    for (int e = threadIdx.x; e < 16 * a.M; e += 1024) {
      float sum = ya[e];
      for (int w = 0; w < 16; ++w) sum += part[w * 16 * a.M + e];
      ya[e] = sum;
    }
    lds_barrier();                                       // partials free again
  };
  for (int xc = 0; xc < nxc; ++xc) {
    // stage X chunk xc: token m's row in 8 instructions of 1 KiB; inputs past
    // `in` are moved out of the buffer's range and land as zeros
    for (int i = wave; i < a.M * 8; i += 16) {
      const int m = i >> 3, q = i & 7;
      const int col = xc * kXC + q * 512 + 8 * lane;     // input index (multiples of 8)
      const uint32_t src = col < a.K ? (uint32_t)((m * a.K + col) * 2) : 0x7FFFFFF0u;
      dma16(rsrc, (uint32_t)__builtin_amdgcn_readfirstlane((int)(xbase + (uint32_t)(m * kXStride * 2 + q * 1024))),
            src);
    }
    wait_vmcnt<0>();
    __syncthreads();
    const int j0 = xc * my_rb;
    int i = 0;
    for (; i + 1 < my_rb; i += 2) {                      // buffers alternate with the job index
      if (((j0 + i) & 1) == 0) {
        step(b0, j0 + i);
        step(b1, j0 + i + 1);
      } else {
        step(b1, j0 + i);
        step(b0, j0 + i + 1);
      }
    }
    if (i < my_rb) {
      if (((j0 + i) & 1) == 0) step(b0, j0 + i);
      else step(b1, j0 + i);
    }
  }
  for (int e = threadIdx.x; e < my_rb * 16 * a.M; e += 1024) {
    const int rbi = e / (16 * a.M), rem = e - rbi * 16 * a.M;
    const int r = rem / a.M, m = rem - r * a.M;
    const int o = ((int)blockIdx.x + rbi * (int)gridDim.x) * 16 + r;
    if (o < a.out) a.Y[(int64_t)m * a.out + o] = __builtin_bit_cast(uint16_t, (_Float16)yacc[e]);
  }
}

}  // namespace

void launch_deploy_qparams(const float* s, const float* z, int64_t out, int64_t in, int group, int bits,
                           uint16_t* s16, uint8_t* zq, hipStream_t st) {
  const int64_t G = in / group, ldz = (G * bits + 7) / 8;
  const int64_t n = out * (G > ldz ? G : ldz);
  LaunchTimer t("deploy_qparams", st);
  QAT_LAUNCH(k_deploy_qparams, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, s, z, out, G, bits,
                     (float)((1 << bits) - 1), ldz, s16, zq);
}

namespace {

constexpr int64_t kLdsLimit = 160 * 1024;                // LDS per workgroup on gfx950

// Compute units of the current device (one persistent workgroup each).
int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// One persistent workgroup per resident slot: as many per CU as registers and
// LDS allow (the grid is capped by the row blocks).
template <int N, int RW, int NB>
void launch_lds(const GemvArgs& a, int64_t nrb, int lds, hipStream_t st) {
  static bool raised = false;                            // allow more than 64 KiB of dynamic LDS, once
  if (!raised) {
    (void)hipFuncSetAttribute((const void*)k_deploy_gemv_lds<N, RW, NB>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kLdsLimit);
    raised = true;
  }
  int per_cu = 1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_deploy_gemv_lds<N, RW, NB>, 1024, (size_t)lds) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const int64_t slots = (int64_t)num_cus() * per_cu;
  const dim3 grid((unsigned)(nrb < slots ? nrb : slots));
  QAT_LAUNCH((k_deploy_gemv_lds<N, RW, NB>), grid, dim3(1024), (size_t)lds, st, a);
}

template <int N>
void launch_xchunk(const GemvArgs& a, int64_t grid, int lds, hipStream_t st) {
  static bool raised = false;                            // allow more than 64 KiB of dynamic LDS, once
  if (!raised) {
    (void)hipFuncSetAttribute((const void*)k_deploy_gemv_xchunk<N>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kLdsLimit);
    raised = true;
  }
  QAT_LAUNCH((k_deploy_gemv_xchunk<N>), dim3((unsigned)grid), dim3(1024), (size_t)lds, st, a);
}

}  // namespace

void launch_deploy_gemv(const uint16_t* X, const uint8_t* Wq, const uint16_t* s16, const uint8_t* zq, int64_t M,
                        int64_t out, int64_t in, int group, int bits, uint16_t* Y, hipStream_t st) {
  GemvArgs a;
  a.X = X;
  a.Wq = Wq;
  a.s16 = s16;
  a.zq = zq;
  a.M = (int)M;
  a.out = (int)out;
  a.K = (int)in;
  a.G = in / group;
  a.ldq = in * bits / 8;
  a.ldz = (a.G * bits + 7) / 8;
  a.group = group;
  a.Y = Y;
  LaunchTimer t("deploy_gemv", st);
  // X in LDS when it fits beside the partial sums (16 waves x 16 rows x M fp32
  // per row block), the workgroup's fp16 outputs and the step-size / zero-point
  // slots: persistent workgroups (the LDS size assumes one per CU, the largest
  // share of row blocks). Two code buffers: the loads of one job are in
  // flight during the previous one; deeper buffering measured slower (it adds
  // redundant loads past a wave's last job and LDS slots).
  constexpr int kRW = 1;
  const int64_t nrb = (out + 16 * kRW - 1) / (16 * kRW);
  const int64_t grid1 = nrb < num_cus() ? nrb : num_cus();
  const int64_t my_rb = (nrb + grid1 - 1) / grid1;
  constexpr int nb = 2;
  const int64_t xbytes = M * (int64_t)lds_x_pitch((int)in) * 2;
  const int64_t lds = xbytes > kLdsLimit ? xbytes : DeployLds::of((int)M, (int)in, (int)my_rb, kRW, nb).total;
  const bool qp_fits = out * (in / group) * 2 >= 16 && out * a.ldz >= 16;   // one 16-byte piece per buffer
  if (lds <= kLdsLimit && qp_fits) {
    if (bits == 2) launch_lds<2, kRW, nb>(a, nrb, (int)lds, st);
    else if (bits == 3) launch_lds<3, kRW, nb>(a, nrb, (int)lds, st);
    else launch_lds<4, kRW, nb>(a, nrb, (int)lds, st);
    return;
  }
  // X too large for LDS: stage it chunk by chunk when the accumulators of one
  // workgroup's row blocks fit beside a chunk; otherwise X stays in registers.
  const int64_t rb16 = (out + 15) / 16;
  const int64_t gx = rb16 < num_cus() ? rb16 : num_cus();
  const int64_t xlds = XChunkLds::of((int)M, (int)((rb16 + gx - 1) / gx)).total;
  if (xlds <= kLdsLimit && qp_fits) {
    if (bits == 2) launch_xchunk<2>(a, gx, (int)xlds, st);
    else if (bits == 3) launch_xchunk<3>(a, gx, (int)xlds, st);
    else launch_xchunk<4>(a, gx, (int)xlds, st);
    return;
  }
  const dim3 grid((unsigned)((out + 15) / 16));
  if (bits == 2) QAT_LAUNCH(k_deploy_gemv<2>, grid, dim3(512), 0, st, a);
  else if (bits == 3) QAT_LAUNCH(k_deploy_gemv<3>, grid, dim3(512), 0, st, a);
  else QAT_LAUNCH(k_deploy_gemv<4>, grid, dim3(512), 0, st, a);
}

}  // namespace qat
