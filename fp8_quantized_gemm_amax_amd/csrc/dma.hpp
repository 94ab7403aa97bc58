// dma.hpp - LDS DMA (buffer_load ... lds) helpers shared by the GEMM and GEMV kernels, gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8amax {

constexpr uint32_t kRsrcWord3 = 0x00020000u;

typedef int v4i __attribute__((ext_vector_type(4)));
#define FP8_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Buffer resource for a raw byte range: 48-bit base, stride 0, `bytes` records (offsets at
// or past it read as zero), gfx9 data-format word.  All inputs are wave-uniform.
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a)));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffff));
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = static_cast<int>(kRsrcWord3);
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(FP8_LDS(p)));
}

// LDS DMA: every lane's 16 (or 4) bytes at `voff` in the buffer go to LDS at
// m0 + lane * 16 (or 4).  Written as inline asm so the compiler does not treat the LDS as
// written by an outstanding load and wait for every DMA in flight before each LDS read;
// the kernel orders them itself (wait_vmcnt + barrier).  The instruction has no
// destination registers, and its address operands are read when it issues.
__device__ __forceinline__ void dma16(const v4i& rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const v4i& rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the memory fence __syncthreads() adds (that fence would wait
// for every LDS DMA still in flight, i.e. for the slabs being prefetched).  The empty asm
// statements keep the compiler from moving memory accesses across it; the caller waits
// for the DMA it needs with wait_vmcnt first.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace fp8amax
