// C ABI of the group-wise fake-quant linear: argument validation, workspace
// layout and the launch sequence of each call. Everything is validated on the
// host before the first launch; on error nothing is enqueued.
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/qat.h"
#include "qat_internal.h"

#define QAT_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512] = "";

constexpr int64_t kMaxDim = int64_t(1) << 30;      // GEMM indices are 32-bit
constexpr int64_t kMaxBytes = 0x7FFFFFF0;          // kernels address each operand with 32-bit offsets

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
size_t region(int64_t bytes) { return (size_t)round_up(bytes, 256); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

struct Range {
  const void* p;
  size_t n;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Outputs must not overlap inputs or each other.
int32_t check_alias(const Range* outs, int nout, const Range* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j])) return QAT_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return QAT_ERR_ALIAS;
  }
  return QAT_OK;
}

// Elementwise calls accept any row count; the GEMM calls (gemm = true) need
// out % 4 == 0: bf16 rows of `out` elements (Y, dY) are then 8-byte aligned,
// which the 8-byte stores of Y and the 4-byte DMAs that read such dY (out not
// a multiple of 64) rely on. Groups: 32, 64 or 128 elements along `in`, or the
// whole row (group == in, channel-wise).
int32_t check_common(int64_t out, int64_t in, int32_t group, int32_t bits, bool gemm = false) {
  if (bits < 2 || bits > 4) return QAT_ERR_BITS;
  if (out <= 0 || in <= 0 || in % 64 != 0 || (gemm && out % 4 != 0)) return QAT_ERR_SHAPE;
  if (out > kMaxDim || in > kMaxDim || out * in * 4 > kMaxBytes) return QAT_ERR_SHAPE;
  if (!(group == 32 || group == 64 || group == 128 || group == in) || in % group != 0) return QAT_ERR_GROUP;
  return QAT_OK;
}

// Bytes of one [out][in / group] fp32 parameter (s, z, ds, dz).
size_t gbytes(int64_t out, int64_t in, int32_t group) { return (size_t)(out * (in / group) * 4); }

int32_t check_m(int64_t M, int64_t out, int64_t in) {
  if (M <= 0 || M > kMaxDim) return QAT_ERR_SHAPE;
  if (M * out * 2 > kMaxBytes || M * in * 2 > kMaxBytes) return QAT_ERR_SHAPE;
  return QAT_OK;
}

int32_t check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!aligned16(p)) return QAT_ERR_ALIGN;
  return QAT_OK;
}

int32_t finish() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(g_last_error, sizeof g_last_error, "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
    return QAT_ERR_HIP;
  }
  return QAT_OK;
}

#define QAT_CHECK(x)               \
  do {                             \
    int32_t _st = (x);             \
    if (_st != QAT_OK) return _st; \
  } while (0)

// Workspace: the bf16 W_hat [out][in] that the forward and backward GEMMs read.
size_t ws_bytes_for(int64_t out, int64_t in) { return region(out * in * 2); }

qat::GemmArgs gemm_args() {
  qat::GemmArgs a;
  memset(&a, 0, sizeof a);
  return a;
}

}  // namespace

QAT_API const char* qat_status_string(int32_t st) {
  switch (st) {
    case QAT_OK: return "ok";
    case QAT_ERR_NULL: return "a required pointer is NULL";
    case QAT_ERR_SHAPE: return "invalid shape (dimension <= 0, in not a multiple of 64, out not a multiple of 4 for the GEMM calls, or an operand of 2 GiB or more)";
    case QAT_ERR_BITS: return "bits must be 2, 3 or 4";
    case QAT_ERR_GROUP: return "group must be 32, 64, 128 or in (channel-wise), dividing in";
    case QAT_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case QAT_ERR_WORKSPACE: return "workspace missing or too small";
    case QAT_ERR_HIP: return "HIP launch failed (see qat_last_error)";
    case QAT_ERR_ALIAS: return "an output overlaps an input or another output";
    case QAT_ERR_SCRATCH: return "out * in exceeds the static scratch of the no-allocation entry point (qat_noalloc_max_weights)";
    default: return "unknown status";
  }
}

QAT_API const char* qat_last_error(void) { return g_last_error; }

QAT_API size_t qat_fakequant_ws_bytes(int64_t out, int64_t in, int32_t bits) {
  if (bits < 2 || bits > 4 || out <= 0 || in <= 0 || out > kMaxDim || in > kMaxDim) return 0;
  return ws_bytes_for(out, in);
}

QAT_API size_t qat_dequant_ws_bytes(int64_t out, int64_t in, int32_t bits) {
  return qat_fakequant_ws_bytes(out, in, bits);
}

QAT_API int32_t qat_init_minmax(const float* W, int64_t out, int64_t in, int32_t group, int32_t bits,
                                float* s, float* z, hipStream_t stream) {
  QAT_CHECK(check_common(out, in, group, bits));
  if (!W || !s || !z) return QAT_ERR_NULL;
  QAT_CHECK(check_ptrs({W, s, z}));
  const size_t nw = out * in * 4, ng = gbytes(out, in, group);
  Range outs[] = {{s, ng}, {z, ng}};
  Range ins[] = {{W, nw}};
  QAT_CHECK(check_alias(outs, 2, ins, 1));
  qat::launch_init_minmax(W, out, in, group, bits, s, z, stream);
  return finish();
}

QAT_API int32_t qat_quant_codes(const float* W, const float* s, const float* z, int64_t out, int64_t in,
                                int32_t group, int32_t bits, uint8_t* codes, uint16_t* W_hat,
                                hipStream_t stream) {
  QAT_CHECK(check_common(out, in, group, bits));
  if (!W || !s || !z || (!codes && !W_hat)) return QAT_ERR_NULL;
  QAT_CHECK(check_ptrs({W, s, z, codes, W_hat}));
  const size_t n = out * in, ng = gbytes(out, in, group);
  Range outs[] = {{codes, n}, {W_hat, n * 2}};
  Range ins[] = {{W, n * 4}, {s, ng}, {z, ng}};
  QAT_CHECK(check_alias(outs, 2, ins, 3));
  qat::launch_quant_codes(W, s, z, out, in, group, bits, codes, W_hat, stream);
  return finish();
}

QAT_API int32_t qat_pack(const float* W, const float* s, const float* z, int64_t out, int64_t in,
                         int32_t group, int32_t bits, uint8_t* Wq, float* z_round, hipStream_t stream) {
  QAT_CHECK(check_common(out, in, group, bits));
  if (!W || !s || !z || !Wq) return QAT_ERR_NULL;
  QAT_CHECK(check_ptrs({W, s, z, Wq, z_round}));
  const size_t n = out * in, ng = gbytes(out, in, group);
  Range outs[] = {{Wq, n * bits / 8}, {z_round, ng}};
  Range ins[] = {{W, n * 4}, {s, ng}, {z, ng}};
  QAT_CHECK(check_alias(outs, 2, ins, 3));
  qat::launch_pack(W, s, z, out, in, group, bits, Wq, z_round, stream);
  return finish();
}

namespace {

// Validation shared by the fake-quant forwards (Y over the inputs; the
// workspace `ws` of `need` bytes, if any, over neither).
int32_t check_fq_fwd(const uint16_t* X, const float* W, const float* s, const float* z, int64_t M, int64_t out,
                     int64_t in, int32_t group, int32_t bits, const uint16_t* Y, const void* ws, size_t need) {
  QAT_CHECK(check_common(out, in, group, bits, true));
  QAT_CHECK(check_m(M, out, in));
  if (!X || !W || !s || !z || !Y) return QAT_ERR_NULL;
  QAT_CHECK(check_ptrs({X, W, s, z, Y, ws}));
  const size_t ng = gbytes(out, in, group);
  Range outs[] = {{Y, (size_t)(M * out * 2)}, {ws, ws ? need : 0}};
  Range ins[] = {{X, (size_t)(M * in * 2)}, {W, (size_t)(out * in * 4)}, {s, ng}, {z, ng}};
  return check_alias(outs, 2, ins, 4);
}

// Y = X W_hat^T: with w_hat (device memory of out * in bf16) the quantiser
// stages W_hat there and the GEMM reads it; without, the fused kernel
// quantises fp32 W tiles into LDS.
void launch_fq_fwd(const uint16_t* X, const float* W, const float* s, const float* z, int64_t M, int64_t out,
                   int64_t in, int32_t group, int32_t bits, uint16_t* Y, uint16_t* w_hat, hipStream_t stream) {
  qat::GemmArgs a = gemm_args();
  a.A = X;
  a.lda = in;
  a.M = (int)M;
  a.N = (int)out;
  a.K = (int)in;
  a.C = Y;
  a.ldc = out;
  a.s = s;
  a.z = z;
  a.G = in / group;
  a.group = group;
  a.Kq = (float)((1 << bits) - 1);
  a.ldb = in;
  if (w_hat) {
    qat::launch_quant_codes(W, s, z, out, in, group, bits, nullptr, w_hat, stream);
    a.B = w_hat;
    qat::launch_gemm_fwd(a, qat::kBf16, bits, stream);
  } else {
    a.B = W;
    qat::launch_gemm_fwd(a, qat::kFp32Quant, bits, stream);
  }
}

}  // namespace

QAT_API int32_t qat_fakequant_linear_fwd(const uint16_t* X, const float* W, const float* s,
                                         const float* z, int64_t M, int64_t out, int64_t in,
                                         int32_t group, int32_t bits, uint16_t* Y, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
  const size_t need = ws_bytes_for(out, in);
  QAT_CHECK(check_fq_fwd(X, W, s, z, M, out, in, group, bits, Y, ws, need));
  if (ws && ws_bytes < need) return QAT_ERR_WORKSPACE;
  launch_fq_fwd(X, W, s, z, M, out, in, group, bits, Y, (uint16_t*)ws, stream);
  return finish();
}

// ---------------------------------------------------------------------------
// The staged forward for callers that cannot allocate device memory. Its
// W_hat lives in `scratch`, a file-scope device array of kScratchWeights bf16
// values of which each GPU that runs the library holds one copy until the
// process ends. Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address of each
// GPU's copy is looked up once per device, with that device current, and
// kept in g_scratch. The array has external linkage (in a namespace of its
// own): the runtime resolves a device variable through the code object's
// dynamic symbol table, which lists a namespace-scope __device__ variable
// (GLOBAL, PROTECTED, like the kernels) but not a `static` one (LOCAL only),
// and its lookup of a static one aborts the process.
// ---------------------------------------------------------------------------
constexpr int64_t kScratchWeights = int64_t(48) << 20;   // 96 MiB of bf16: out * in <= 48 Mi

namespace qat {
namespace noalloc {
__device__ __align__(256) uint16_t scratch[kScratchWeights];
}  // namespace noalloc
}  // namespace qat

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint16_t* g_scratch[kMaxDevices] = {};

int32_t hip_error(hipError_t e) {
  snprintf(g_last_error, sizeof g_last_error, "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return QAT_ERR_HIP;
}

// The device address of the scratch copy on the device that runs `stream`.
int32_t scratch_for(hipStream_t stream, uint16_t** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_error(e);
  if (dev < 0 || dev >= kMaxDevices) return hip_error(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_error(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_error(e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(qat::noalloc::scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_error(e);
    if (!p) return hip_error(hipErrorInvalidSymbol);
    g_scratch[dev] = (uint16_t*)p;
  }
  *out = g_scratch[dev];
  return QAT_OK;
}

}  // namespace

QAT_API int64_t qat_noalloc_max_weights(void) { return kScratchWeights; }

QAT_API int32_t qat_fakequant_linear_fwd_noalloc(const uint16_t* X, const float* W, const float* s, const float* z,
                                                 int64_t M, int64_t out, int64_t in, int32_t group, int32_t bits,
                                                 uint16_t* Y, hipStream_t stream) {
  QAT_CHECK(check_fq_fwd(X, W, s, z, M, out, in, group, bits, Y, nullptr, 0));
  if (out * in > kScratchWeights) return QAT_ERR_SCRATCH;
  uint16_t* w_hat = nullptr;
  QAT_CHECK(scratch_for(stream, &w_hat));
  launch_fq_fwd(X, W, s, z, M, out, in, group, bits, Y, w_hat, stream);
  return finish();
}

namespace qat {

// dX = dY W_hat with W_hat^T [in][out] bf16 staged in the workspace: both
// operands K-contiguous (K = out).
void launch_linear_dx(const uint16_t* dY, const uint16_t* w_hat_t, int64_t M, int64_t out, int64_t in,
                      uint16_t* dX, hipStream_t stream) {
  qat::GemmArgs a = gemm_args();
  a.A = dY;
  a.lda = out;
  a.B = w_hat_t;
  a.ldb = out;
  a.M = (int)M;
  a.N = (int)in;
  a.K = (int)out;
  a.C = dX;
  a.ldc = in;
  qat::launch_gemm_dx(a, stream);
}

// dX = dY W_hat with W_hat made in LDS from B (the fp32 master weight,
// ldb elements per row, or packed codes, ldb bytes per row) inside the GEMM.
void launch_linear_dx_fused(const uint16_t* dY, const void* B, int64_t ldb, const float* s, const float* z, int64_t M,
                            int64_t out, int64_t in, int group, int bits, uint16_t* dX, int bload, hipStream_t stream) {
  qat::GemmArgs a = gemm_args();
  a.A = dY;
  a.lda = out;
  a.B = B;
  a.ldb = ldb;
  a.M = (int)M;
  a.N = (int)in;
  a.K = (int)out;
  a.C = dX;
  a.ldc = in;
  a.s = s;
  a.z = z;
  a.G = in / group;
  a.group = group;
  a.Kq = (float)((1 << bits) - 1);
  qat::launch_gemm_dx_fused(a, bload, bits, stream);
}

// Gw = dY^T X over the M tokens, both read in place, reduced by the epilogue.
qat::GemmArgs linear_grads_args(const uint16_t* dY, const uint16_t* X, const float* s, const float* z,
                                int64_t M, int64_t out, int64_t in, int group, int bits) {
  qat::GemmArgs a = gemm_args();
  a.A = dY;
  a.lda = out;
  a.B = X;
  a.ldb = in;
  a.M = (int)out;
  a.N = (int)in;
  a.K = (int)M;
  a.s = s;
  a.z = z;
  a.G = in / group;
  a.group = group;
  a.Kq = (float)((1 << bits) - 1);
  return a;
}

// QAT_OK, or QAT_ERR_HIP with the launch error kept for qat_last_error.
int32_t finish_call() { return finish(); }

}  // namespace qat

QAT_API int32_t qat_fakequant_linear_bwd(const uint16_t* dY, const uint16_t* X, const float* W,
                                         const float* s, const float* z, int64_t M, int64_t out,
                                         int64_t in, int32_t group, int32_t bits, uint16_t* dX,
                                         float* dW, float* ds, float* dz, void* ws, size_t ws_bytes,
                                         hipStream_t stream) {
  QAT_CHECK(check_common(out, in, group, bits, true));
  QAT_CHECK(check_m(M, out, in));
  if (!dY || !X || !W || !s || !z) return QAT_ERR_NULL;
  if ((ds == nullptr) != (dz == nullptr)) return QAT_ERR_NULL;
  QAT_CHECK(check_ptrs({dY, X, W, s, z, dX, dW, ds, dz, ws}));
  const size_t need = ws_bytes_for(out, in);
  if (dX && ws && ws_bytes < need) return QAT_ERR_WORKSPACE;
  const size_t ng = gbytes(out, in, group);
  Range outs[] = {{dX, (size_t)(M * in * 2)}, {dW, (size_t)(out * in * 4)}, {ds, ng}, {dz, ng},
                  {dX ? ws : nullptr, need}};
  Range ins[] = {{dY, (size_t)(M * out * 2)}, {X, (size_t)(M * in * 2)}, {W, (size_t)(out * in * 4)},
                 {s, ng}, {z, ng}};
  QAT_CHECK(check_alias(outs, 5, ins, 5));

  if (dX && ws) {
    uint16_t* w_hat = (uint16_t*)ws;
    if (out % 64 == 0) {                     // W_hat^T: both dX operands K-contiguous
      qat::launch_w_hat_t(W, s, z, out, in, group, bits, w_hat, stream);
      qat::launch_linear_dx(dY, w_hat, M, out, in, dX, stream);
    } else {                                 // W_hat [out][in], read MN-contiguous
      qat::launch_quant_codes(W, s, z, out, in, group, bits, nullptr, w_hat, stream);
      qat::launch_linear_dx_saved(dY, w_hat, M, out, in, dX, stream);
    }
  } else if (dX) {
    qat::launch_linear_dx_fused(dY, W, in, s, z, M, out, in, group, bits, dX, qat::kFp32Quant, stream);
  }
  if (dW || ds) {
    qat::GemmArgs a = qat::linear_grads_args(dY, X, s, z, M, out, in, group, bits);
    a.W = W;
    a.ldw = in;
    a.dW = dW;
    a.ds = ds;
    a.dz = dz;
    qat::launch_gemm_grads(a, qat::kSteGrads, bits, stream);
  }
  return finish();
}

// dX = dY W_hat on a W_hat [out][in] staged by a forward call, read in place.
void qat::launch_linear_dx_saved(const uint16_t* dY, const uint16_t* w_hat, int64_t M, int64_t out, int64_t in,
                                 uint16_t* dX, hipStream_t stream) {
  qat::GemmArgs a = gemm_args();
  a.A = dY;
  a.lda = out;
  a.B = w_hat;
  a.ldb = in;
  a.M = (int)M;
  a.N = (int)in;
  a.K = (int)out;
  a.C = dX;
  a.ldc = in;
  qat::launch_gemm_dx_mn(a, stream);
}

QAT_API int32_t qat_fakequant_linear_bwd_saved(const uint16_t* dY, const uint16_t* X, const float* W,
                                               const float* s, const float* z, const uint16_t* w_hat,
                                               int64_t M, int64_t out, int64_t in, int32_t group, int32_t bits,
                                               uint16_t* dX, float* dW, float* ds, float* dz,
                                               hipStream_t stream) {
  QAT_CHECK(check_common(out, in, group, bits, true));
  QAT_CHECK(check_m(M, out, in));
  if (!dY || !X || !W || !s || !z || (dX && !w_hat)) return QAT_ERR_NULL;
  if ((ds == nullptr) != (dz == nullptr)) return QAT_ERR_NULL;
  QAT_CHECK(check_ptrs({dY, X, W, s, z, w_hat, dX, dW, ds, dz}));
  const size_t ng = gbytes(out, in, group);
  Range outs[] = {{dX, (size_t)(M * in * 2)}, {dW, (size_t)(out * in * 4)}, {ds, ng}, {dz, ng}};
  Range ins[] = {{dY, (size_t)(M * out * 2)}, {X, (size_t)(M * in * 2)}, {W, (size_t)(out * in * 4)},
                 {s, ng}, {z, ng}, {dX ? w_hat : nullptr, (size_t)(out * in * 2)}};
  QAT_CHECK(check_alias(outs, 4, ins, 6));

  if (dX) qat::launch_linear_dx_saved(dY, w_hat, M, out, in, dX, stream);
  if (dW || ds) {
    qat::GemmArgs a = qat::linear_grads_args(dY, X, s, z, M, out, in, group, bits);
    a.W = W;
    a.ldw = in;
    a.dW = dW;
    a.ds = ds;
    a.dz = dz;
    qat::launch_gemm_grads(a, qat::kSteGrads, bits, stream);
  }
  return finish();
}

QAT_API int32_t qat_dequant_gemm_fwd(const uint16_t* X, const uint8_t* Wq, const float* s,
                                     const float* z, int64_t M, int64_t out, int64_t in, int32_t group,
                                     int32_t bits, uint16_t* Y, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  QAT_CHECK(check_common(out, in, group, bits, true));
  QAT_CHECK(check_m(M, out, in));
  if (!X || !Wq || !s || !z || !Y) return QAT_ERR_NULL;
  QAT_CHECK(check_ptrs({X, Wq, s, z, Y, ws}));
  const size_t need = ws_bytes_for(out, in);
  if (ws && ws_bytes < need) return QAT_ERR_WORKSPACE;
  const size_t ng = gbytes(out, in, group);
  Range outs[] = {{Y, (size_t)(M * out * 2)}, {ws, ws ? need : 0}};
  Range ins[] = {{X, (size_t)(M * in * 2)}, {Wq, (size_t)(out * in * bits / 8)}, {s, ng}, {z, ng}};
  QAT_CHECK(check_alias(outs, 2, ins, 4));
  qat::GemmArgs a = gemm_args();
  a.A = X;
  a.lda = in;
  a.M = (int)M;
  a.N = (int)out;
  a.K = (int)in;
  a.C = Y;
  a.ldc = out;
  a.s = s;
  a.z = z;
  a.G = in / group;
  a.group = group;
  a.Kq = (float)((1 << bits) - 1);
  if (ws) {
    uint16_t* w_hat = (uint16_t*)ws;
    qat::launch_dequant(Wq, s, z, out, in, group, bits, w_hat, stream);
    a.B = w_hat;
    a.ldb = in;
    qat::launch_gemm_fwd(a, qat::kBf16, bits, stream);
  } else {
    a.B = Wq;
    a.ldb = in * bits / 8;
    qat::launch_gemm_fwd(a, qat::kPacked, bits, stream);
  }
  return finish();
}

QAT_API int32_t qat_dequant_gemm_bwd_s(const uint16_t* dY, const uint16_t* X, const uint8_t* Wq,
                                       const float* s, const float* z, int64_t M, int64_t out,
                                       int64_t in, int32_t group, int32_t bits, uint16_t* dX,
                                       float* ds, float* dz, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
  QAT_CHECK(check_common(out, in, group, bits, true));
  QAT_CHECK(check_m(M, out, in));
  if (!dY || !X || !Wq || !s || !z || !ds) return QAT_ERR_NULL;
  QAT_CHECK(check_ptrs({dY, X, Wq, s, z, dX, ds, dz, ws}));
  const size_t need = ws_bytes_for(out, in);
  if (dX && ws && ws_bytes < need) return QAT_ERR_WORKSPACE;
  const size_t ng = gbytes(out, in, group);
  Range outs[] = {{dX, (size_t)(M * in * 2)}, {ds, ng}, {dz, ng}, {dX ? ws : nullptr, need}};
  Range ins[] = {{dY, (size_t)(M * out * 2)}, {X, (size_t)(M * in * 2)},
                 {Wq, (size_t)(out * in * bits / 8)}, {s, ng}, {z, ng}};
  QAT_CHECK(check_alias(outs, 4, ins, 5));

  if (dX && ws) {
    uint16_t* w_hat = (uint16_t*)ws;
    if (out % 64 == 0) {
      qat::launch_dequant_t(Wq, s, z, out, in, group, bits, w_hat, stream);
      qat::launch_linear_dx(dY, w_hat, M, out, in, dX, stream);
    } else {
      qat::launch_dequant(Wq, s, z, out, in, group, bits, w_hat, stream);
      qat::launch_linear_dx_saved(dY, w_hat, M, out, in, dX, stream);
    }
  } else if (dX) {
    qat::launch_linear_dx_fused(dY, Wq, in * bits / 8, s, z, M, out, in, group, bits, dX, qat::kPacked, stream);
  }
  qat::GemmArgs a = qat::linear_grads_args(dY, X, s, z, M, out, in, group, bits);
  a.Wq = Wq;
  a.ldq = in * bits / 8;
  a.ds = ds;
  a.dz = dz;
  qat::launch_gemm_grads(a, qat::kE2eScaleGrad, bits, stream);
  return finish();
}

QAT_API int32_t qat_dequant_gemm_bwd_s_saved(const uint16_t* dY, const uint16_t* X, const uint8_t* Wq,
                                             const float* s, const float* z, const uint16_t* w_hat, int64_t M,
                                             int64_t out, int64_t in, int32_t group, int32_t bits,
                                             uint16_t* dX, float* ds, float* dz, hipStream_t stream) {
  QAT_CHECK(check_common(out, in, group, bits, true));
  QAT_CHECK(check_m(M, out, in));
  if (!dY || !X || !Wq || !s || !z || !ds || (dX && !w_hat)) return QAT_ERR_NULL;
  QAT_CHECK(check_ptrs({dY, X, Wq, s, z, w_hat, dX, ds, dz}));
  const size_t ng = gbytes(out, in, group);
  Range outs[] = {{dX, (size_t)(M * in * 2)}, {ds, ng}, {dz, ng}};
  Range ins[] = {{dY, (size_t)(M * out * 2)}, {X, (size_t)(M * in * 2)},
                 {Wq, (size_t)(out * in * bits / 8)}, {s, ng}, {z, ng}, {dX ? w_hat : nullptr, (size_t)(out * in * 2)}};
  QAT_CHECK(check_alias(outs, 3, ins, 6));

  if (dX) qat::launch_linear_dx_saved(dY, w_hat, M, out, in, dX, stream);
  qat::GemmArgs a = qat::linear_grads_args(dY, X, s, z, M, out, in, group, bits);
  a.Wq = Wq;
  a.ldq = in * bits / 8;
  a.ds = ds;
  a.dz = dz;
  qat::launch_gemm_grads(a, qat::kE2eScaleGrad, bits, stream);
  return finish();
}

// ---------------------------------------------------------------------------
// Deployment format and the inference linear
// ---------------------------------------------------------------------------

static int64_t zq_stride(int64_t in, int32_t group, int32_t bits) { return ((in / group) * bits + 7) / 8; }

QAT_API int64_t qat_deploy_zq_stride(int64_t in, int32_t group, int32_t bits) {
  if (check_common(1, in, group, bits) != QAT_OK) return 0;
  return zq_stride(in, group, bits);
}

QAT_API int32_t qat_deploy_qparams(const float* s, const float* z, int64_t out, int64_t in, int32_t group,
                                   int32_t bits, uint16_t* s16, uint8_t* zq, hipStream_t stream) {
  QAT_CHECK(check_common(out, in, group, bits));
  if (!s || !z || !s16 || !zq) return QAT_ERR_NULL;
  QAT_CHECK(check_ptrs({s, z, s16, zq}));
  const size_t ng = gbytes(out, in, group);
  Range outs[] = {{s16, ng / 2}, {zq, (size_t)(out * zq_stride(in, group, bits))}};
  Range ins[] = {{s, ng}, {z, ng}};
  QAT_CHECK(check_alias(outs, 2, ins, 2));
  qat::launch_deploy_qparams(s, z, out, in, group, bits, s16, zq, stream);
  return finish();
}

QAT_API int32_t qat_deploy_gemv(const uint16_t* X, const uint8_t* Wq, const uint16_t* s16, const uint8_t* zq,
                                int64_t M, int64_t out, int64_t in, int32_t group, int32_t bits, uint16_t* Y,
                                hipStream_t stream) {
  QAT_CHECK(check_common(out, in, group, bits));
  if (M < 1 || M > 16) return QAT_ERR_SHAPE;
  if (!X || !Wq || !s16 || !zq || !Y) return QAT_ERR_NULL;
  QAT_CHECK(check_ptrs({X, Wq, s16, zq, Y}));
  Range outs[] = {{Y, (size_t)(M * out * 2)}};
  Range ins[] = {{X, (size_t)(M * in * 2)},
                 {Wq, (size_t)(out * in * bits / 8)},
                 {s16, gbytes(out, in, group) / 2},
                 {zq, (size_t)(out * zq_stride(in, group, bits))}};
  QAT_CHECK(check_alias(outs, 1, ins, 4));
  qat::launch_deploy_gemv(X, Wq, s16, zq, M, out, in, group, bits, Y, stream);
  return finish();
}
