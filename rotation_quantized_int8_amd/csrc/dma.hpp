// Helpers of the one-launch kernels that stream weights with direct
// global->LDS loads and wait for them with explicit counts (gfx950).
#pragma once

#include "common.hpp"

namespace convrot {

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Workgroup barrier; the wave's LDS operations complete first.  It does not
// wait for outstanding global loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  compiler_fence();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 0xF) | ((N >> 4) << 14));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One direct global->LDS load: 64 lanes x 16 bytes land contiguously at LDS
// byte offset `lds` (wave-uniform); M0 holds the base, one wait state later.
// The compiler does not count these loads: callers wait with wait_vmcnt.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gptr), "s"(lds) : "memory", "m0");
}

// Eight fp16 additions, each rounded once (fp32 sum, then fp16).
__device__ __forceinline__ v4i add_f16x8(v4i a, v4i b) {
  const __half* x = reinterpret_cast<const __half*>(&a);
  const __half* y = reinterpret_cast<const __half*>(&b);
  __half z[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = __float2half_rn(__half2float(x[e]) + __half2float(y[e]));
  return *reinterpret_cast<const v4i*>(z);
}

}  // namespace convrot
