// Practical-peak probes for the roofline: a register-resident MFMA loop (the
// bf16 matrix-core ceiling at the running clock) and read- and write-stream
// kernels (the HBM read and write ceilings for buffers larger than the
// 256 MiB MALL). Measurement utilities beside the method's calls; they
// compute nothing of the method.
#include <hip/hip_runtime.h>

#include "../../include/qat_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Eight independent accumulator chains per wave, accumulators pinned to AGPRs.
__global__ __launch_bounds__(512) void k_mfma_loop(int iters, float* out) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)(threadIdx.x + i));
    b[i] = (__bf16)(1e-3f * (float)i);
  }
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[j]) : "v"(a), "v"(b));
  }
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);                                  // reads stay after the wait
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Grid-stride read of n float4, one partial sum per thread.
__global__ __launch_bounds__(256) void k_read_stream(const float4* __restrict__ p, int64_t n, float* out) {
  float acc = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float4 v = p[i];
    acc += (v.x + v.y) + (v.z + v.w);
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// Grid-stride store of n float4 (each the index as a float, so every store
// writes data the kernel computed).
__global__ __launch_bounds__(256) void k_write_stream(float4* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float f = (float)i;
    p[i] = make_float4(f, f, f, f);
  }
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int64_t qat_peak_mfma_flops(int32_t blocks, int32_t iters) {
  if (blocks <= 0 || iters <= 0) return -1;
  return (int64_t)blocks * 8 /* waves */ * 8 /* chains */ * iters * (16LL * 16 * 32 * 2);
}

extern "C" __attribute__((visibility("default"))) size_t qat_peak_scratch_bytes(int32_t blocks) {
  return blocks > 0 ? (size_t)blocks * 512 * sizeof(float) : 0;
}

extern "C" __attribute__((visibility("default"))) int32_t qat_peak_mfma(int32_t blocks, int32_t iters, float* scratch,
                                                                        hipStream_t stream) {
  if (blocks <= 0 || iters <= 0 || !scratch) return 1;
  hipLaunchKernelGGL(k_mfma_loop, dim3((unsigned)blocks), dim3(512), 0, stream, iters, scratch);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

extern "C" __attribute__((visibility("default"))) int32_t qat_peak_read(const void* buf, size_t bytes, int32_t blocks,
                                                                        float* scratch, hipStream_t stream) {
  if (!buf || !scratch || blocks <= 0 || bytes < 16 || ((uintptr_t)buf & 15)) return 1;
  hipLaunchKernelGGL(k_read_stream, dim3((unsigned)blocks), dim3(256), 0, stream, (const float4*)buf,
                     (int64_t)(bytes / 16), scratch);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

extern "C" __attribute__((visibility("default"))) int32_t qat_peak_write(void* buf, size_t bytes, int32_t blocks,
                                                                         hipStream_t stream) {
  if (!buf || blocks <= 0 || bytes < 16 || ((uintptr_t)buf & 15)) return 1;
  hipLaunchKernelGGL(k_write_stream, dim3((unsigned)blocks), dim3(256), 0, stream, (float4*)buf,
                     (int64_t)(bytes / 16));
  return hipGetLastError() == hipSuccess ? 0 : 7;
}
