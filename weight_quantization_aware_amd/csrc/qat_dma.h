// Direct-to-LDS loads (buffer_load ... lds) and the waits that go with them,
// shared by the MFMA GEMMs and the inference linear (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qat {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// buffer_load_dwordx4 ... lds writes 64 lanes x 16 B = 1 KiB of LDS starting
// at M0 (lane l at byte 16 l). The loads are issued from inline asm because
// the compiler's own LDS-DMA tracking waits for every outstanding DMA before
// any LDS read; the kernels wait on vmcnt themselves. Bytes beyond the buffer
// resource's range read as zero.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

__device__ __forceinline__ void dma4(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// The same with a wave-uniform byte offset added in the scalar offset field
// (no per-lane add). Only for accesses whose out-of-range lanes are already
// out of range by their per-lane offset: whether the range check counts the
// scalar offset is not relied on.
__device__ __forceinline__ void dma16s(i32x4 rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

__device__ __forceinline__ void dma4s(i32x4 rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int64_t nbytes) {
  if (nbytes < 0) nbytes = 0;
  if (nbytes > 0x7FFFFFF0) nbytes = 0x7FFFFFF0;
  const uint64_t b = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)((b >> 32) & 0xFFFF));
  r[2] = __builtin_amdgcn_readfirstlane((int)nbytes);
  r[3] = 0x00020000;
  return r;
}

}  // namespace qat
