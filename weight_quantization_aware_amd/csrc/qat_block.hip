// One Block-AP training step on a Llama-2 decoder block with seven
// fake-quantised linears (gfx950): the row kernels of the block (RMSNorm,
// rotary embedding, the softmax-gradient row term, SiLU-gated product, the
// loss sum), the multi-tensor AdamW, and the launch sequence of the forward,
// the straight-through backward and the update. The output, the loss and its
// gradient come from the epilogue of the down product (kResidMse).
//
// Sources: "EfficientQAT, low-bit training on a single GPU"
// (modelfoundations.com), Phase 1 (Block-AP: block-wise MSE to the
// full-precision outputs, W with s and z trained together, AdamW with two
// learning rates on cosine schedules); paperlayer.ai summary of arXiv
// 2407.11062v3, Appendix A (straight-through gradients of W, s, z). The block
// itself is Llama-2's (the pages name the model family, not its layers).
//
// Memory-bound row kernels: one workgroup per token row for the norms (a row
// of H <= 8192 values stays in registers between the reduction and the
// write), 16-byte vector accesses throughout. Attention (qat_attn.hip): the
// forward is one fused kernel; the backward is one fused pass per key block
// for dK and dV (P and dS recomputed in registers from the forward's
// log-sum-exp and a per-query row term), which also leaves dS^T for the dQ
// product.
#include <math.h>
#include <string.h>

#include "../../include/qat_block.h"
#include "qat_device.h"
#include "qat_internal.h"

namespace qat {
namespace {

constexpr float kRmsEps = 1e-5f;
constexpr double kRopeBase = 10000.0;
constexpr int kHeadDim = 128;

__device__ __forceinline__ void unpack8(uint4 u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Sum over a 256-thread workgroup; every thread gets the result.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();                        // red may still be read by a previous call
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// ---------------------------------------------------------------------------
// RMSNorm forward: h = bf16(x r g), r = 1 / sqrt(mean(x^2) + eps) per row.
// RES = 1 forms the residual x = x_in + o (bf16 + fp32) first and stores it
// as fp32 (the block's x2). A thread owns chunks of 8 columns t, t + 256, ...
// (at most 4: H <= 8192).
// ---------------------------------------------------------------------------
template <int RES>
__global__ __launch_bounds__(256) void k_rmsnorm_fwd(const uint16_t* __restrict__ x, const float* __restrict__ o,
                                                      float* __restrict__ xres, const float* __restrict__ g,
                                                      uint16_t* __restrict__ h, float* __restrict__ r, int H) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int nc = H / 8;
  float v[4][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = threadIdx.x + 256 * j;
    if (c < nc) {
      unpack8(*(const uint4*)(x + row * H + 8 * c), v[j]);
      if constexpr (RES) {
        const float4 a = *(const float4*)(o + row * H + 8 * c), b = *(const float4*)(o + row * H + 8 * c + 4);
        const float ov[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[j][e] += ov[e];
        *(float4*)(xres + row * H + 8 * c) = make_float4(v[j][0], v[j][1], v[j][2], v[j][3]);
        *(float4*)(xres + row * H + 8 * c + 4) = make_float4(v[j][4], v[j][5], v[j][6], v[j][7]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[j][e] * v[j][e];
    }
  }
  const float tot = block_sum(ss, red);
  const float rr = 1.0f / sqrtf(tot / (float)H + kRmsEps);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = threadIdx.x + 256 * j;
    if (c < nc) {
      const float4 a = *(const float4*)(g + 8 * c), b = *(const float4*)(g + 8 * c + 4);
      const float gv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      float out[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = v[j][e] * rr * gv[e];
      *(uint4*)(h + row * H + 8 * c) = pack8(out);
    }
  }
  if (threadIdx.x == 0) r[row] = rr;
}

// RMSNorm backward with the residual: dx = dres + r (g dh) - r^3 x mean(x g dh),
// dh = dh_a + dh_b (the two linears fed by the normed row), out bf16.
__global__ __launch_bounds__(256) void k_rmsnorm_bwd(const uint16_t* __restrict__ dha,
                                                      const uint16_t* __restrict__ dhb,
                                                      const float* __restrict__ x, const float* __restrict__ r,
                                                      const float* __restrict__ g, const uint16_t* __restrict__ dres,
                                                      uint16_t* __restrict__ dx, int H) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int nc = H / 8;
  float gd[4][8], xv[4][8];
  float dot = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = threadIdx.x + 256 * j;
    if (c < nc) {
      float a[8], b[8];
      unpack8(*(const uint4*)(dha + row * H + 8 * c), a);
      unpack8(*(const uint4*)(dhb + row * H + 8 * c), b);
      const float4 g0 = *(const float4*)(g + 8 * c), g1 = *(const float4*)(g + 8 * c + 4);
      const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const float4 x0 = *(const float4*)(x + row * H + 8 * c), x1 = *(const float4*)(x + row * H + 8 * c + 4);
      const float xx[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        gd[j][e] = (a[e] + b[e]) * gv[e];
        xv[j][e] = xx[e];
        dot += xx[e] * gd[j][e];
      }
    }
  }
  const float mean = block_sum(dot, red) / (float)H;
  const float rr = r[row];
  const float r3m = rr * rr * rr * mean;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = threadIdx.x + 256 * j;
    if (c < nc) {
      float d[8], out[8];
      unpack8(*(const uint4*)(dres + row * H + 8 * c), d);
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = d[e] + (rr * gd[j][e] - r3m * xv[j][e]);
      *(uint4*)(dx + row * H + 8 * c) = pack8(out);
    }
  }
}

// ---------------------------------------------------------------------------
// Rotary embedding. cs[t][i] = (cos, sin) of t * 10000^(-2 i / 128), from
// double-precision angles. A thread rotates 8 pairs (i, i + 64) of one head
// in place: a' = a c - b s, b' = b c + a s (s negated for the gradient,
// which is the inverse rotation).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rope_table(float2* __restrict__ cs, int T) {
  constexpr int half = kHeadDim / 2;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * half) return;
  const int t = idx / half, i = idx % half;
  const double ang = (double)t * pow(kRopeBase, -2.0 * i / kHeadDim);
  cs[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

__global__ __launch_bounds__(256) void k_rope(uint16_t* __restrict__ q, uint16_t* __restrict__ k,
                                              const float2* __restrict__ cs, int64_t rows, int T, int H,
                                              float sgn) {
  constexpr int half = kHeadDim / 2, TPH = half / 8;   // threads per head
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per = rows * (H / 16);                  // threads per tensor
  if (idx >= 2 * per) return;
  uint16_t* x = idx < per ? q : k;
  const int64_t rem = idx < per ? idx : idx - per;
  const int64_t row = rem / (H / 16);
  const int j = (int)(rem % (H / 16));
  const int head = j / TPH, i0 = (j % TPH) * 8;
  const int t = (int)(row % T);
  uint16_t* base = x + row * H + head * kHeadDim + i0;
  float a[8], b[8], oa[8], ob[8];
  unpack8(*(const uint4*)base, a);
  unpack8(*(const uint4*)(base + half), b);
  const float2* c = cs + (int64_t)t * half + i0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float2 v = c[e];
    const float sn = sgn * v.y;
    oa[e] = a[e] * v.x - b[e] * sn;
    ob[e] = b[e] * v.x + a[e] * sn;
  }
  *(uint4*)base = pack8(oa);
  *(uint4*)(base + half) = pack8(ob);
}

// ---------------------------------------------------------------------------
// Row term of the softmax backward: D[problem][q] = sum_k P[q][k] dP[q][k],
// which equals dO[q] . O[q] (sum over k of P dP = dO . sum_k P v_k = dO . O),
// from the attention output and its gradient (bf16 [B*T][H]). One thread per
// (token, head), 128 products in fp32.
__global__ __launch_bounds__(256) void k_attn_rowdot(const uint16_t* __restrict__ dO, const uint16_t* __restrict__ O,
                                                      float* __restrict__ D, int64_t rows, int T, int H, int nh) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * nh) return;
  const int64_t tok = idx / nh;
  const int head = (int)(idx % nh);
  const uint4* a = (const uint4*)(dO + tok * H + head * kHeadDim);
  const uint4* o = (const uint4*)(O + tok * H + head * kHeadDim);
  float acc = 0.f;
#pragma unroll 4
  for (int c = 0; c < kHeadDim / 8; ++c) {
    float x[8], y[8];
    unpack8(a[c], x);
    unpack8(o[c], y);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += x[e] * y[e];
  }
  const int64_t b = tok / T, t = tok % T;
  D[(b * nh + head) * T + t] = acc;
}

// ---------------------------------------------------------------------------
// SiLU-gated product: a = bf16(silu(gate) up); backward in place:
// gate <- da up silu'(gate), up <- da silu(gate), with
// silu'(x) = sg (1 + x (1 - sg)), sg = 1 / (1 + e^-x).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_swiglu_fwd(const uint16_t* __restrict__ gate, const uint16_t* __restrict__ up,
                                                     uint16_t* __restrict__ a, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  float g[8], u[8], o[8];
  unpack8(((const uint4*)gate)[i], g);
  unpack8(((const uint4*)up)[i], u);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = g[e] / (1.0f + __expf(-g[e])) * u[e];
  ((uint4*)a)[i] = pack8(o);
}

__global__ __launch_bounds__(256) void k_swiglu_bwd(uint16_t* __restrict__ gate, uint16_t* __restrict__ up,
                                                     const uint16_t* __restrict__ da, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  float g[8], u[8], d[8], dg[8], du[8];
  unpack8(((const uint4*)gate)[i], g);
  unpack8(((const uint4*)up)[i], u);
  unpack8(((const uint4*)da)[i], d);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float sg = 1.0f / (1.0f + __expf(-g[e]));
    dg[e] = d[e] * u[e] * (sg * (1.0f + g[e] * (1.0f - sg)));
    du[e] = d[e] * (g[e] * sg);
  }
  ((uint4*)gate)[i] = pack8(dg);
  ((uint4*)up)[i] = pack8(du);
}

// ---------------------------------------------------------------------------
// The loss: the down product's epilogue (kResidMse) leaves one fp32 partial
// of sum (y - target)^2 per workgroup; one workgroup sums them in double.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_loss_final(const float* __restrict__ partial, int nblk, double inv_n,
                                                     float* __restrict__ loss) {
  __shared__ double red[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < nblk; i += 256) s += (double)partial[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = (float)(red[0] * inv_n);
}

// ---------------------------------------------------------------------------
// AdamW over up to 14 tensors in one launch (the seven linears' s and z; each W
// is updated in its gradient epilogue). Segment i covers blocks
// [start[i], start[i + 1]); a thread updates 4 consecutive parameters of 16
// per thread (4 float4 steps), all in fp32:
//   p <- p decay; m <- b1 m + (1 - b1) g; v <- b2 v + (1 - b2) g^2;
//   p <- p - step_size m / (sqrt(v) inv_sqrt_bc2 + eps).
// ---------------------------------------------------------------------------
constexpr int kAdamSegs = 2 * QAT_BLOCK_LINEARS;
constexpr int kAdamPerBlock = 256 * 16;

struct AdamSeg {
  float* p;
  const float* g;
  float* m;
  float* v;
  int64_t n4;              // float4 count
  float step_size;         // lr / (1 - b1^t)
  float decay;             // 1 - lr wd
};

struct AdamArgs {
  AdamSeg seg[kAdamSegs];
  int start[kAdamSegs + 1];
  int nseg;
  float b1, b2, inv_sqrt_bc2, eps;
};

__global__ __launch_bounds__(256) void k_adamw(const AdamArgs a) {
  int si = 0;
  while (si + 1 < a.nseg && (int)blockIdx.x >= a.start[si + 1]) ++si;
  const AdamSeg sg = a.seg[si];
  const int64_t base = (int64_t)(blockIdx.x - a.start[si]) * (kAdamPerBlock / 4) + threadIdx.x;
  // every load of the thread's 16 parameters is issued before any arithmetic
  float4 p[4], m[4], v[4], g[4];
  bool ok[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t i = base + r * 256;
    ok[r] = i < sg.n4;
    if (ok[r]) {
      p[r] = ((const float4*)sg.p)[i];
      m[r] = ((const float4*)sg.m)[i];
      v[r] = ((const float4*)sg.v)[i];
      g[r] = ((const float4*)sg.g)[i];
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (!ok[r]) continue;
    float* pp = &p[r].x;
    float* mm = &m[r].x;
    float* vv = &v[r].x;
    const float* gg = &g[r].x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float pe = pp[e] * sg.decay;
      mm[e] = a.b1 * mm[e] + (1.0f - a.b1) * gg[e];
      vv[e] = a.b2 * vv[e] + (1.0f - a.b2) * gg[e] * gg[e];
      const float den = sqrtf(vv[e]) * a.inv_sqrt_bc2 + a.eps;
      pp[e] = pe - sg.step_size * (mm[e] / den);
    }
    const int64_t i = base + r * 256;
    ((float4*)sg.p)[i] = p[r];
    ((float4*)sg.m)[i] = m[r];
    ((float4*)sg.v)[i] = v[r];
  }
}

// ---------------------------------------------------------------------------
// Host side: shapes, workspace layout, launch sequence.
// ---------------------------------------------------------------------------
int blocks_of(int64_t n, int per) { return (int)((n + per - 1) / per); }

struct Dims {
  int64_t H, nh, I, T, B, BT;
  int bits, group;
  int64_t out[QAT_BLOCK_LINEARS], in[QAT_BLOCK_LINEARS];
};

Dims dims_of(const qat_block_shape& s) {
  Dims d;
  d.H = s.hidden;
  d.nh = s.heads;
  d.I = s.inter;
  d.T = s.seq;
  d.B = s.batch;
  d.BT = s.batch * s.seq;
  d.bits = s.bits;
  d.group = s.group;
  for (int i = 0; i < QAT_BLOCK_LINEARS; ++i) {
    d.out[i] = (i == QAT_BLOCK_GATE || i == QAT_BLOCK_UP) ? d.I : d.H;
    d.in[i] = i == QAT_BLOCK_DOWN ? d.I : d.H;
  }
  return d;
}

int32_t check_shape(const qat_block_shape* s) {
  if (!s) return QAT_ERR_NULL;
  if (s->bits < 2 || s->bits > 4) return QAT_ERR_BITS;
  const int64_t H = s->hidden, I = s->inter, T = s->seq, B = s->batch, nh = s->heads;
  if (H <= 0 || I <= 0 || T <= 0 || B <= 0 || nh <= 0) return QAT_ERR_SHAPE;
  if (H % 128 != 0 || H > 8192 || H != nh * kHeadDim) return QAT_ERR_SHAPE;
  if (I % 64 != 0 || I > (int64_t(1) << 20)) return QAT_ERR_SHAPE;
  if (T % 64 != 0 || T > 4096 || B > (int64_t(1) << 16)) return QAT_ERR_SHAPE;
  const int64_t BT = B * T;
  if (BT * I * 2 > 0x7FFFFFF0 || BT * H * 4 > 0x7FFFFFF0 || H * I * 4 > 0x7FFFFFF0) return QAT_ERR_SHAPE;
  if (!(s->group == 32 || s->group == 64 || s->group == 128) || H % s->group || I % s->group) return QAT_ERR_GROUP;
  return QAT_OK;
}

// Workspace regions (each 256-byte aligned).
struct Ws {
  float2* rope;          // [T][64]
  uint16_t *h1, *q, *k, *v, *attn, *h2, *gate, *up, *a, *dy, *wh, *da, *dxg, *dxu, *dx2, *dattn, *dq, *dk, *dv;
  uint16_t* whk[QAT_BLOCK_LINEARS];   // W_hat kept from the forward for the dX products (o, gate, up, down)
  float *lse, *o, *x2, *r1, *r2, *partial, *D;
  uint16_t* P;
  size_t bytes;
};

Ws ws_layout(const Dims& d, uint8_t* base) {
  Ws w;
  size_t off = 0;
  auto take = [&](int64_t bytes) {
    void* p = base ? (void*)(base + off) : nullptr;
    off += (size_t)((bytes + 255) / 256 * 256);
    return p;
  };
  const int64_t th = d.BT * d.H, ti = d.BT * d.I, sc = d.B * d.nh * d.T * d.T;
  int64_t wmax = 0;                                      // the staging buffer of q, k and v
  for (int i = QAT_BLOCK_Q; i <= QAT_BLOCK_V; ++i) wmax = d.out[i] * d.in[i] > wmax ? d.out[i] * d.in[i] : wmax;
  w.rope = (float2*)take(d.T * (kHeadDim / 2) * 8);
  w.h1 = (uint16_t*)take(th * 2);
  w.q = (uint16_t*)take(th * 2);
  w.k = (uint16_t*)take(th * 2);
  w.v = (uint16_t*)take(th * 2);
  w.lse = (float*)take(d.B * d.nh * d.T * 4);
  w.P = (uint16_t*)take(sc * 2);
  w.attn = (uint16_t*)take(th * 2);
  w.o = (float*)take(th * 4);
  w.x2 = (float*)take(th * 4);
  w.r1 = (float*)take(d.BT * 4);
  w.r2 = (float*)take(d.BT * 4);
  w.h2 = (uint16_t*)take(th * 2);
  w.gate = (uint16_t*)take(ti * 2);
  w.up = (uint16_t*)take(ti * 2);
  w.a = (uint16_t*)take(ti * 2);
  w.dy = (uint16_t*)take(th * 2);
  w.partial = (float*)take(gemm_fwd_max_workgroups(d.BT, d.H) * 4);
  w.wh = (uint16_t*)take(wmax * 2);
  for (int i = 0; i < QAT_BLOCK_LINEARS; ++i)
    w.whk[i] = i >= QAT_BLOCK_O ? (uint16_t*)take(d.out[i] * d.in[i] * 2) : nullptr;
  w.da = (uint16_t*)take(ti * 2);
  w.dxg = (uint16_t*)take(th * 2);
  w.dxu = (uint16_t*)take(th * 2);
  w.dx2 = (uint16_t*)take(th * 2);
  w.dattn = (uint16_t*)take(th * 2);
  w.dq = (uint16_t*)take(th * 2);
  w.dk = (uint16_t*)take(th * 2);
  w.dv = (uint16_t*)take(th * 2);
  w.D = (float*)take(d.B * d.nh * d.T * 4);
  w.bytes = off;
  return w;
}

GemmArgs zero_args() {
  GemmArgs a;
  memset(&a, 0, sizeof a);
  return a;
}

// The forward product of linear li on X: W_hat staged as bf16 [out][in] (kept
// for the backward's dX product where the linear has one, else in the shared
// ws.wh), and the GEMM arguments of Y = X W_hat^T with the output left to the
// caller.
GemmArgs fq_forward_args(const Dims& d, const qat_block_linear& L, int li, const uint16_t* X, const Ws& w,
                         hipStream_t st) {
  const int64_t out = d.out[li], in = d.in[li];
  uint16_t* wh = w.whk[li] ? w.whk[li] : w.wh;
  launch_quant_codes(L.W, L.s, L.z, out, in, d.group, d.bits, nullptr, wh, st);
  GemmArgs a = zero_args();
  a.A = X;
  a.lda = in;
  a.B = wh;
  a.ldb = in;
  a.M = (int)d.BT;
  a.N = (int)out;
  a.K = (int)in;
  a.ldc = out;
  return a;
}

// Y = X W_hat^T, bf16 (Y) or fp32 (Yf) out.
void fq_forward(const Dims& d, const qat_block_linear& L, int li, const uint16_t* X, uint16_t* Y, float* Yf,
                const Ws& w, hipStream_t st) {
  GemmArgs a = fq_forward_args(d, L, li, X, w, st);
  if (Yf) {
    a.Cf = Yf;
    launch_gemm_fwd_f32(a, st);
  } else {
    a.C = Y;
    launch_gemm_fwd(a, kBf16, d.bits, st);
  }
}

// One optimizer step's constants (host, double precision): learning rates
// after the cosine schedule and the bias corrections of step t = k + 1. W's
// update runs in its gradient epilogue; s and z go through the multi-tensor
// kernel.
struct AdamConst {
  double lr_w, lr_q, bc1, bc2;
  const qat_block_adamw* o;
};

AdamConst adam_const(const qat_block_adamw& o) {
  const double pi = 3.14159265358979323846;
  const double c = (1.0 + cos(pi * (double)o.step / (double)o.total_steps)) / 2.0;
  const double t = (double)(o.step + 1);
  return AdamConst{o.lr_weight * c, o.lr_quant * c, 1.0 - pow(o.beta1, t), 1.0 - pow(o.beta2, t), &o};
}

// Straight-through backward of linear li: dX (if requested; q, k and v need
// none) from the W_hat its forward staged, read in place, and dW, ds, dz from
// the gradient GEMM's epilogue. With an optimizer step (ac), the same epilogue
// also applies AdamW to W and its moments (W_hat is already staged, so the dX
// product does not depend on the update's order); s and z are updated
// afterwards by k_adamw.
void fq_backward(const Dims& d, const qat_block_linear& L, int li, const uint16_t* dY, const uint16_t* X,
                 uint16_t* dX, const Ws& w, const AdamConst* ac, hipStream_t st) {
  const int64_t out = d.out[li], in = d.in[li];
  if (dX) {
    GemmArgs a = zero_args();
    a.A = dY;
    a.lda = out;
    a.B = w.whk[li];
    a.ldb = in;
    a.M = (int)d.BT;
    a.N = (int)in;
    a.K = (int)out;
    a.C = dX;
    a.ldc = in;
    launch_gemm_dx_mn(a, st);
  }
  GemmArgs a = linear_grads_args(dY, X, L.s, L.z, d.BT, out, in, d.group, d.bits);
  a.W = L.W;
  a.ldw = in;
  a.dW = L.dW;
  a.ds = L.ds;
  a.dz = L.dz;
  const bool fuse = ac != nullptr;
  if (fuse) {
    a.Wupd = L.W;
    a.mW = L.m_W;
    a.vW = L.v_W;
    a.adam_b1 = (float)ac->o->beta1;
    a.adam_b2 = (float)ac->o->beta2;
    a.adam_isbc2 = (float)(1.0 / sqrt(ac->bc2));
    a.adam_eps = (float)ac->o->eps;
    a.adam_step = (float)(ac->lr_w / ac->bc1);
    a.adam_decay = (float)(1.0 - ac->lr_w * ac->o->weight_decay);
  }
  launch_gemm_grads(a, fuse ? kSteAdam : kSteGrads, d.bits, st);
}

// Per-(sequence, head) views for the attention products: the operand that
// lives in a token-major [B*T][H] tensor advances by T*H per sequence and 128
// per head; one that lives in a [B*nh][T][T] score tensor by nh*T*T and T*T.
enum View { kTok = 0, kScore = 1 };
void set_batch(GemmArgs& a, const Dims& d, View va, View vb, View vc) {
  auto sb = [&](View v) { return v == kTok ? d.T * d.H : d.nh * d.T * d.T; };
  auto sh = [&](View v) { return v == kTok ? (int64_t)kHeadDim : d.T * d.T; };
  a.batch_h = (int)d.nh;
  a.batches = (int)(d.B * d.nh);
  a.sa_b = sb(va);
  a.sa_h = sh(va);
  a.sb_b = sb(vb);
  a.sb_h = sh(vb);
  a.sc_b = sb(vc);
  a.sc_h = sh(vc);
}

void rope(const Dims& d, uint16_t* q, uint16_t* k, const Ws& w, float sgn, hipStream_t st) {
  LaunchTimer t("rope", st);
  const int64_t n = 2 * d.BT * (d.H / 16);
  QAT_LAUNCH(k_rope, dim3((unsigned)blocks_of(n, 256)), dim3(256), 0, st, q, k, w.rope, d.BT, (int)d.T,
                     (int)d.H, sgn);
}

// The forward through the loss; leaves in the workspace everything the
// backward reads.
void block_forward(const Dims& d, const qat_block_linear* L, const float* g1, const float* g2, const uint16_t* x,
                   const uint16_t* target, float* y, float* loss, const Ws& w, hipStream_t st) {
  {
    LaunchTimer t("rope_table", st);
    QAT_LAUNCH(k_rope_table, dim3((unsigned)blocks_of(d.T * (kHeadDim / 2), 256)), dim3(256), 0, st,
                       w.rope, (int)d.T);
  }
  {
    LaunchTimer t("rmsnorm_fwd", st);
    QAT_LAUNCH(k_rmsnorm_fwd<0>, dim3((unsigned)d.BT), dim3(256), 0, st, x, nullptr, nullptr, g1, w.h1,
                       w.r1, (int)d.H);
  }
  fq_forward(d, L[QAT_BLOCK_Q], QAT_BLOCK_Q, w.h1, w.q, nullptr, w, st);
  fq_forward(d, L[QAT_BLOCK_K], QAT_BLOCK_K, w.h1, w.k, nullptr, w, st);
  fq_forward(d, L[QAT_BLOCK_V], QAT_BLOCK_V, w.h1, w.v, nullptr, w, st);
  rope(d, w.q, w.k, w, 1.0f, st);
  // causal attention, fused: attn and the rows' log-sum-exp (P is rebuilt in the backward)
  launch_flash_fwd(w.q, w.k, w.v, w.attn, w.lse, (int)d.B, (int)d.T, (int)d.H, st);
  fq_forward(d, L[QAT_BLOCK_O], QAT_BLOCK_O, w.attn, nullptr, w.o, w, st);
  {
    LaunchTimer t("rmsnorm_fwd", st);
    QAT_LAUNCH(k_rmsnorm_fwd<1>, dim3((unsigned)d.BT), dim3(256), 0, st, x, w.o, w.x2, g2, w.h2, w.r2,
                       (int)d.H);
  }
  fq_forward(d, L[QAT_BLOCK_GATE], QAT_BLOCK_GATE, w.h2, w.gate, nullptr, w, st);
  fq_forward(d, L[QAT_BLOCK_UP], QAT_BLOCK_UP, w.h2, w.up, nullptr, w, st);
  {
    LaunchTimer t("swiglu_fwd", st);
    const int64_t n8 = d.BT * d.I / 8;
    QAT_LAUNCH(k_swiglu_fwd, dim3((unsigned)blocks_of(n8, 256)), dim3(256), 0, st, w.gate, w.up, w.a, n8);
  }
  {
    // down, with y = x2 + down, dy = 2 (y - target) / n and the loss partials in its epilogue
    const int64_t n = d.BT * d.H;
    GemmArgs a = fq_forward_args(d, L[QAT_BLOCK_DOWN], QAT_BLOCK_DOWN, w.a, w, st);
    a.Cf = y;
    a.C = w.dy;
    a.resid = w.x2;
    a.target = target;
    a.partial = w.partial;
    a.escale = (float)(2.0 / (double)n);
    const int64_t nb = launch_gemm_fwd_mse(a, st);
    LaunchTimer t("loss", st);
    QAT_LAUNCH(k_loss_final, dim3(1), dim3(256), 0, st, w.partial, (int)nb, 1.0 / (double)n, loss);
  }
}

void block_backward(const Dims& d, const qat_block_linear* L, const float* g2, const Ws& w, const AdamConst* ac,
                    hipStream_t st) {
  const float scale = 1.0f / sqrtf((float)kHeadDim);
  fq_backward(d, L[QAT_BLOCK_DOWN], QAT_BLOCK_DOWN, w.dy, w.a, w.da, w, ac, st);
  {
    LaunchTimer t("swiglu_bwd", st);
    const int64_t n8 = d.BT * d.I / 8;
    QAT_LAUNCH(k_swiglu_bwd, dim3((unsigned)blocks_of(n8, 256)), dim3(256), 0, st, w.gate, w.up, w.da, n8);
  }
  // gate and up now hold their output gradients
  fq_backward(d, L[QAT_BLOCK_GATE], QAT_BLOCK_GATE, w.gate, w.h2, w.dxg, w, ac, st);
  fq_backward(d, L[QAT_BLOCK_UP], QAT_BLOCK_UP, w.up, w.h2, w.dxu, w, ac, st);
  {
    LaunchTimer t("rmsnorm_bwd", st);
    QAT_LAUNCH(k_rmsnorm_bwd, dim3((unsigned)d.BT), dim3(256), 0, st, w.dxg, w.dxu, w.x2, w.r2, g2, w.dy,
                       w.dx2, (int)d.H);
  }
  fq_backward(d, L[QAT_BLOCK_O], QAT_BLOCK_O, w.dx2, w.attn, w.dattn, w, ac, st);
  {
    // D = rowsum(P dP) = dO . O per query
    LaunchTimer t("attn_rowdot", st);
    const int64_t n = d.BT * d.nh;
    QAT_LAUNCH(k_attn_rowdot, dim3((unsigned)blocks_of(n, 256)), dim3(256), 0, st, w.dattn, w.attn, w.D,
                       d.BT, (int)d.T, (int)d.H, (int)d.nh);
  }
  // dk, dv and dS^T (into the P buffer) in one pass over the causal pairs
  launch_flash_bwd_kv(w.q, w.k, w.v, w.dattn, w.lse, w.D, w.dk, w.dv, w.P, (int)d.B, (int)d.T, (int)d.H, st);
  {
    // dq = dS k: A[m = query][k = key] = dS^T[key][query], both MN-contiguous
    GemmArgs a = zero_args();
    a.A = w.P;
    a.lda = d.T;
    a.B = w.k;
    a.ldb = d.H;
    a.M = (int)d.T;
    a.N = kHeadDim;
    a.K = (int)d.T;
    a.C = w.dq;
    a.ldc = d.H;
    a.causal = kCausalLower;
    set_batch(a, d, kScore, kTok, kTok);
    launch_gemm_attn(a, st);
  }
  rope(d, w.dq, w.dk, w, -1.0f, st);
  // q, k, v: gradients of W, s, z only (the block input's gradient is not needed)
  fq_backward(d, L[QAT_BLOCK_Q], QAT_BLOCK_Q, w.dq, w.h1, nullptr, w, ac, st);
  fq_backward(d, L[QAT_BLOCK_K], QAT_BLOCK_K, w.dk, w.h1, nullptr, w, ac, st);
  fq_backward(d, L[QAT_BLOCK_V], QAT_BLOCK_V, w.dv, w.h1, nullptr, w, ac, st);
}

// AdamW on every linear's s and z (W was updated in its gradient epilogue).
void adamw_rest(const Dims& d, const qat_block_linear* L, const AdamConst& ac, hipStream_t st) {
  const qat_block_adamw& o = *ac.o;
  AdamArgs a;
  memset(&a, 0, sizeof a);
  a.b1 = (float)o.beta1;
  a.b2 = (float)o.beta2;
  a.inv_sqrt_bc2 = (float)(1.0 / sqrt(ac.bc2));
  a.eps = (float)o.eps;
  int nseg = 0, blk = 0;
  for (int i = 0; i < QAT_BLOCK_LINEARS; ++i) {
    const int64_t ng = d.out[i] * (d.in[i] / d.group);
    struct {
      float *p, *g, *m, *v;
      int64_t n;
      double lr;
    } t2[2] = {{L[i].s, L[i].ds, L[i].m_s, L[i].v_s, ng, ac.lr_q}, {L[i].z, L[i].dz, L[i].m_z, L[i].v_z, ng, ac.lr_q}};
    for (auto& e : t2) {
      AdamSeg& sg = a.seg[nseg];
      sg.p = e.p;
      sg.g = e.g;
      sg.m = e.m;
      sg.v = e.v;
      sg.n4 = e.n / 4;
      sg.step_size = (float)(e.lr / ac.bc1);
      sg.decay = (float)(1.0 - e.lr * o.weight_decay);
      a.start[nseg] = blk;
      blk += blocks_of(e.n, kAdamPerBlock);
      ++nseg;
    }
  }
  a.start[nseg] = blk;
  a.nseg = nseg;
  LaunchTimer tm("adamw", st);
  QAT_LAUNCH(k_adamw, dim3((unsigned)blk), dim3(256), 0, st, a);
}

// ---- validation ----
struct Span {
  const void* p;
  size_t n;
};

bool spans_overlap(const Span& a, const Span& b) {
  if (!a.p || !b.p || !a.n || !b.n) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Every pointer present and aligned; no written region overlaps any other region.
int32_t check_args(const Dims& d, const qat_block_linear* L, const float* g1, const float* g2, const uint16_t* x,
                   const uint16_t* target, float* y, float* loss, void* ws, bool step) {
  if (!L || !g1 || !g2 || !x || !target || !loss || !ws) return QAT_ERR_NULL;
  const size_t th = (size_t)(d.BT * d.H);
  Span rd[4 + 3 * QAT_BLOCK_LINEARS];
  Span wr[3 + 12 * QAT_BLOCK_LINEARS];   // W, s, z, 3 gradients, 6 moments per linear
  int nr = 0, nw = 0;
  rd[nr++] = {g1, (size_t)d.H * 4};
  rd[nr++] = {g2, (size_t)d.H * 4};
  rd[nr++] = {x, th * 2};
  rd[nr++] = {target, th * 2};
  wr[nw++] = {y, y ? th * 4 : 0};
  wr[nw++] = {loss, 4};
  wr[nw++] = {ws, ws_layout(d, nullptr).bytes};
  for (int i = 0; i < QAT_BLOCK_LINEARS; ++i) {
    const qat_block_linear& l = L[i];
    const size_t nwt = (size_t)(d.out[i] * d.in[i]) * 4, ng = (size_t)(d.out[i] * (d.in[i] / d.group)) * 4;
    if (!l.W || !l.s || !l.z) return QAT_ERR_NULL;
    if (step && (!l.ds || !l.dz || !l.m_W || !l.v_W || !l.m_s || !l.v_s || !l.m_z || !l.v_z))
      return QAT_ERR_NULL;
    const void* all[] = {l.W, l.s, l.z, l.dW, l.ds, l.dz, l.m_W, l.v_W, l.m_s, l.v_s, l.m_z, l.v_z};
    for (const void* p : all)
      if (p && !al16(p)) return QAT_ERR_ALIGN;
    Span* dst = step ? wr : rd;
    int& nd = step ? nw : nr;
    dst[nd++] = {l.W, nwt};
    dst[nd++] = {l.s, ng};
    dst[nd++] = {l.z, ng};
    if (step) {
      const Span more[] = {{l.dW, nwt}, {l.ds, ng}, {l.dz, ng}, {l.m_W, nwt}, {l.v_W, nwt},
                           {l.m_s, ng}, {l.v_s, ng}, {l.m_z, ng}, {l.v_z, ng}};
      for (const Span& s : more) wr[nw++] = s;
    }
  }
  const void* top[] = {g1, g2, x, target, y, loss, ws};
  for (const void* p : top)
    if (p && !al16(p)) return QAT_ERR_ALIGN;
  for (int i = 0; i < nw; ++i) {
    for (int j = i + 1; j < nw; ++j)
      if (spans_overlap(wr[i], wr[j])) return QAT_ERR_ALIAS;
    for (int j = 0; j < nr; ++j)
      if (spans_overlap(wr[i], rd[j])) return QAT_ERR_ALIAS;
  }
  return QAT_OK;
}

}  // namespace
}  // namespace qat

#define QAT_API extern "C" __attribute__((visibility("default")))

QAT_API size_t qat_block_ws_bytes(const qat_block_shape* shape) {
  if (qat::check_shape(shape) != QAT_OK) return 0;
  return qat::ws_layout(qat::dims_of(*shape), nullptr).bytes;
}

QAT_API int32_t qat_block_forward(const qat_block_shape* shape, const qat_block_linear* lin, const float* g1,
                                  const float* g2, const uint16_t* x, const uint16_t* target, float* y, float* loss,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
  using namespace qat;
  const int32_t sc = check_shape(shape);
  if (sc != QAT_OK) return sc;
  const Dims d = dims_of(*shape);
  const int32_t ac = check_args(d, lin, g1, g2, x, target, y, loss, ws, false);
  if (ac != QAT_OK) return ac;
  if (ws_bytes < ws_layout(d, nullptr).bytes) return QAT_ERR_WORKSPACE;
  const Ws w = ws_layout(d, (uint8_t*)ws);
  block_forward(d, lin, g1, g2, x, target, y, loss, w, stream);
  return finish_call();
}

QAT_API int32_t qat_block_ap_step(const qat_block_shape* shape, const qat_block_linear* lin, const float* g1,
                                  const float* g2, const uint16_t* x, const uint16_t* target,
                                  const qat_block_adamw* opt, float* y, float* loss, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  using namespace qat;
  const int32_t sc = check_shape(shape);
  if (sc != QAT_OK) return sc;
  if (!opt) return QAT_ERR_NULL;
  if (opt->total_steps <= 0 || opt->step < 0 || !(opt->beta1 >= 0 && opt->beta1 < 1) ||
      !(opt->beta2 >= 0 && opt->beta2 < 1) || !(opt->eps > 0))
    return QAT_ERR_SHAPE;
  const Dims d = dims_of(*shape);
  const int32_t st = check_args(d, lin, g1, g2, x, target, y, loss, ws, true);
  if (st != QAT_OK) return st;
  if (ws_bytes < ws_layout(d, nullptr).bytes) return QAT_ERR_WORKSPACE;
  const Ws w = ws_layout(d, (uint8_t*)ws);
  const AdamConst ac = adam_const(*opt);
  block_forward(d, lin, g1, g2, x, target, y, loss, w, stream);
  block_backward(d, lin, g2, w, &ac, stream);
  adamw_rest(d, lin, ac, stream);
  return finish_call();
}
