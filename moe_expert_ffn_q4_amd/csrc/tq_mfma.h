// tq_mfma.h -- helpers shared by the matrix-core kernels (internal to libtq, gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_device.h"

namespace tq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));


__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// s_waitcnt that waits until at most n vector-memory operations of this wave are outstanding
// (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Byte address of a __shared__ location in the LDS aperture.
__device__ __forceinline__ uint32_t lds_address(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// 16 bytes from global memory straight into LDS: lane l's bytes land at lds_base + 16 l
// (lds_base must be the same for the whole wave). The LDS address comes from M0, and an LDS-DMA
// load needs one wait state after a scalar write of M0 (the compiler's hazard pass does not look
// inside inline asm, hence the explicit s_nop).
__device__ __forceinline__ void load_lds16(const void *g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory", "m0");
}

// An empty use of a loaded value. The pipelined kernels issue the same loads on every step (past
// the end they repeat the last block) because their hand-counted vmcnt waits depend on it; the
// results of the last such loads are never read, and without a use the compiler would drop them,
// which would shrink the number of loads in flight below what a wait count assumes (a barrier
// would then pass before the last tile had landed). Every register set a pipeline loads into must
// get a keep_alive after the pipeline's last step.
template <typename T>
__device__ __forceinline__ void keep_alive(const T &v) {
  asm volatile("" : : "v"(v));
}

// Workgroup barrier once at most N vector-memory operations and no LDS operation of this wave
// are outstanding. Written as one asm statement with a memory clobber: the compiler keeps memory
// accesses on their side of it and adds no waits of its own.
template <int N>
__device__ __forceinline__ void barrier_after_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "i"(N) : "memory");
}

}  // namespace tq
