// Shared device helpers of the INT8ConvRot HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace convrot {

constexpr int kGroup = 256;          // rotation group along K
constexpr int kKMax = 131072;        // 127 * 127 * K < 2^31

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

// Orders LDS traffic between the lanes of one wavefront (no workgroup barrier):
// earlier LDS writes of the wave are visible to its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// x as a finished fp32 value in a register: the compiler can no longer fuse
// the operation that produced x with the next one.  An fp32 product followed
// by a conversion to fp16 would otherwise be folded into one mixed-precision
// FMA (v_fma_mixlo_f16), which rounds the exact product once to fp16 instead
// of first to fp32 -- a different result in rare cases (-ffp-contract=off
// does not prevent it).
__device__ __forceinline__ float as_fp32(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Two finished fp32 values to fp16, each rounded once to nearest even as
// __float2half_rn does, packed low then high: one v_cvt_pk_f16_f32 (checked
// bit for bit against the scalar conversion over every fp32 bit pattern,
// NaNs compared as NaNs).
__device__ __forceinline__ uint32_t pack_f16x2_rn(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 h = __builtin_convertvector((f2){as_fp32(a), as_fp32(b)}, h2);
  return __builtin_bit_cast(uint32_t, h);
}

// fp64 -> fp16 with a single round-to-nearest-even.  The fp32 intermediate is
// taken with round-to-odd (truncate, then force the last bit when inexact):
// 24 >= 11 + 2 significand bits make the second rounding exact in effect.
__device__ __forceinline__ __half f64_to_f16_rn(double d) {
  float f = (float)d;
  double back = (double)f;
  if (back != d) {
    uint32_t u = __float_as_uint(f);
    if (fabs(back) > fabs(d)) u -= 1u;   // step one ulp toward zero
    u |= 1u;                             // sticky bit: round-to-odd
    f = __uint_as_float(u);
  }
  return __float2half_rn(f);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN), and back.
__device__ __forceinline__ uint16_t f32_to_bf16_rn(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// One DPP lane permutation of a float inside each 16-lane row of the wave.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float warp_max16(float v) {
  // max over the 16 lanes of an aligned 16-lane segment (a DPP row), by
  // register-to-register lane permutations: swap neighbours (quad_perm
  // [1,0,3,2]), swap pairs ([2,3,0,1]), mirror each 8-lane half, mirror the row
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return v;
}

// The same maximum for non-negative finite floats, on their bit patterns
// (which order like unsigned integers): integer maxima need no NaN
// canonicalisation, and with bound_ctrl each permutation folds into the max.
__device__ __forceinline__ uint32_t seg_max16_bits(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true));
  return v;
}

__device__ __forceinline__ float wave_max64(float v) {
  v = warp_max16(v);
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

}  // namespace convrot
