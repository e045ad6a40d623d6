// Direct HBM -> LDS loads on gfx950 and the small helpers around them, shared
// by the matrix-core kernels (grouped GEMM, router).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace moe {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

// dword 3 of a raw buffer descriptor on gfx9-family GPUs (32-bit data format, no swizzle)
constexpr int kBufferFlags = 0x00020000;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: base address, stride 0, byte range `bytes` (loads at
// or past it return zero), made wave-uniform.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = kBufferFlags;
  return r;
}

// 16 bytes per lane from buffer offset voff + soff straight into LDS: lane i
// writes bytes [16 i, 16 i + 16) after the wave-uniform LDS address lds.
// Issued as inline assembly so that the compiler does not wait on it before
// unrelated LDS reads; the caller waits (vmcnt) before the barrier that
// publishes the data.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void buffer_load_lds16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a shared-memory pointer, made wave-uniform
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(lds_void*)p);
}

// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace moe
