// Offline weight preparation: W_rot = W H^T per 256-group, s_W, Q_W.
//
// Page "INT8ConvRot GEMM vs fp16 on M1 Max with Metal, MPSMatrix, and MLX
// (fp16 Wins)", section "What changed in the computation", weight equation:
// once at model creation the weights are rotated and quantised with one scale
// per output channel, s_W[n] = max_k |W_rot[n,k]| / 127, Q_W = round(W_rot/s_W),
// clamped to [-128, 127].
//
// The rotation must be the exact product rounded once to fp32, for any fp32
// input.  Every fp32 value is an integer multiple of 2^-149 below 2^128, so
// each weight is turned into a 288-bit two's-complement fixed-point integer
// (least significant bit 2^-149), the unnormalised Walsh-Hadamard transform
// (entries +-1) runs on those integers with exact multi-limb adds, and the
// result t represents t * 2^-153 (the extra 2^-4 is the 1/16 normalisation).
// A 256-term sum is below 2^136, so 9 limbs of 32 bits never overflow.
//
// This runs once per model, so it favours plain exactness over speed: one
// workgroup of 256 threads per output row, one thread per group column, the
// butterflies exchanged through LDS, the row visited twice (max, quantise).

#include "launch.hpp"

namespace convrot {
namespace {

constexpr int kLimbs = 9;

__device__ __forceinline__ void fx_from_f32(float w, uint32_t (&t)[kLimbs]) {
  const uint32_t bits = __float_as_uint(w);
  const uint32_t ex = (bits >> 23) & 0xffu;
  const uint32_t man = ex ? ((bits & 0x7fffffu) | 0x800000u) : (bits & 0x7fffffu);
  // value = man * 2^(ex - 150) (normal) or man * 2^-149 (subnormal);
  // in units of 2^-149 that is man << (ex - 1) or man << 0.
  const int shift = ex ? (int)ex - 1 : 0;  // 0 .. 254
  const int limb = shift >> 5;
  const int off = shift & 31;
  const uint32_t lo = man << off;
  const uint32_t hi = off ? (man >> (32 - off)) : 0u;
#pragma unroll
  for (int l = 0; l < kLimbs; ++l) t[l] = (l == limb) ? lo : ((l == limb + 1) ? hi : 0u);
  if (bits >> 31) {  // two's-complement negation
    uint32_t carry = 1u;
#pragma unroll
    for (int l = 0; l < kLimbs; ++l) {
      const uint64_t v = (uint64_t)(~t[l]) + carry;
      t[l] = (uint32_t)v;
      carry = (uint32_t)(v >> 32);
    }
  }
}

__device__ __forceinline__ void fx_add(const uint32_t (&a)[kLimbs], const uint32_t (&b)[kLimbs],
                                       uint32_t (&r)[kLimbs]) {
  uint32_t carry = 0u;
#pragma unroll
  for (int l = 0; l < kLimbs; ++l) {
    const uint64_t v = (uint64_t)a[l] + b[l] + carry;
    r[l] = (uint32_t)v;
    carry = (uint32_t)(v >> 32);
  }
}

// r = a - b
__device__ __forceinline__ void fx_sub(const uint32_t (&a)[kLimbs], const uint32_t (&b)[kLimbs],
                                       uint32_t (&r)[kLimbs]) {
  uint32_t carry = 1u;
#pragma unroll
  for (int l = 0; l < kLimbs; ++l) {
    const uint64_t v = (uint64_t)a[l] + (uint32_t)(~b[l]) + carry;
    r[l] = (uint32_t)v;
    carry = (uint32_t)(v >> 32);
  }
}

// Bit `pos` (may be negative or past the top: then 0) of the magnitude.
__device__ __forceinline__ uint32_t fx_bit(const uint32_t (&t)[kLimbs], int pos) {
  uint32_t r = 0u;
#pragma unroll
  for (int l = 0; l < kLimbs; ++l) {
    const int o = pos - 32 * l;
    r |= (o >= 0 && o < 32) ? ((t[l] >> o) & 1u) : 0u;
  }
  return r;
}

// Any bit strictly below `pos` set?
__device__ __forceinline__ bool fx_any_below(const uint32_t (&t)[kLimbs], int pos) {
  uint32_t r = 0u;
#pragma unroll
  for (int l = 0; l < kLimbs; ++l) {
    const int o = pos - 32 * l;  // number of bits of limb l below pos
    const uint32_t mask = (o >= 32) ? 0xffffffffu : ((o <= 0) ? 0u : ((1u << o) - 1u));
    r |= t[l] & mask;
  }
  return r != 0u;
}

// 24 bits starting at `pos` (pos >= 0).
__device__ __forceinline__ uint32_t fx_bits24(const uint32_t (&t)[kLimbs], int pos) {
  uint32_t r = 0u;
#pragma unroll
  for (int l = 0; l < kLimbs; ++l) {
    const int o = 32 * l - pos;  // where limb l's bit 0 lands in the result
    uint32_t c = 0u;
    if (o >= 0 && o < 32) c = t[l] << o;
    else if (o < 0 && o > -32) c = t[l] >> (-o);
    r |= c;
  }
  return r & 0xffffffu;
}

// Round t * 2^-153 (t two's complement) to the nearest fp32, ties to even.
__device__ __forceinline__ float fx_to_f32(const uint32_t (&tin)[kLimbs]) {
  uint32_t t[kLimbs];
  const bool neg = (tin[kLimbs - 1] >> 31) != 0u;
  if (neg) {
    uint32_t carry = 1u;
#pragma unroll
    for (int l = 0; l < kLimbs; ++l) {
      const uint64_t v = (uint64_t)(~tin[l]) + carry;
      t[l] = (uint32_t)v;
      carry = (uint32_t)(v >> 32);
    }
  } else {
#pragma unroll
    for (int l = 0; l < kLimbs; ++l) t[l] = tin[l];
  }
  int top = -1;
#pragma unroll
  for (int l = 0; l < kLimbs; ++l)
    if (t[l]) top = 32 * l + 31 - __clz(t[l]);
  if (top < 0) return 0.0f;
  int e = top - 153;                       // weight of the leading bit: 2^e
  const int q = (e >= -126) ? top - 23 : 4; // position of the last kept bit (2^-149 -> 4)
  uint32_t mant = fx_bits24(t, q);
  const uint32_t guard = fx_bit(t, q - 1);
  const bool sticky = fx_any_below(t, q - 1);
  if (guard && (sticky || (mant & 1u))) mant += 1u;
  uint32_t bits;
  if (e >= -126) {
    if (mant == (1u << 24)) { mant >>= 1; e += 1; }
    bits = (e > 127) ? 0x7f800000u : (((uint32_t)(e + 127) << 23) | (mant & 0x7fffffu));
  } else {
    bits = mant;  // subnormal; mant == 2^23 is exactly the smallest normal
  }
  return __uint_as_float(bits | (neg ? 0x80000000u : 0u));
}

// One group: exact Walsh-Hadamard of 256 fixed-point values, column `c` is
// this thread's output.  `buf` holds two [kLimbs][256] LDS planes.
__device__ float rotate_group_exact(const float* __restrict__ wrow, int c,
                                    uint32_t (*buf)[kLimbs][kGroup]) {
  uint32_t own[kLimbs], other[kLimbs], res[kLimbs];
  fx_from_f32(wrow[c], own);
#pragma unroll 1
  for (int s = 0; s < 8; ++s) {
    const int h = 1 << s;
    uint32_t(*plane)[kGroup] = buf[s & 1];
#pragma unroll
    for (int l = 0; l < kLimbs; ++l) plane[l][c] = own[l];
    __syncthreads();
#pragma unroll
    for (int l = 0; l < kLimbs; ++l) other[l] = plane[l][c ^ h];
    if (c & h) fx_sub(other, own, res);   // upper butterfly output: x[c^h] - x[c]
    else fx_add(own, other, res);         // lower: x[c] + x[c^h]
#pragma unroll
    for (int l = 0; l < kLimbs; ++l) own[l] = res[l];
  }
  // the next call writes plane 0 first; everyone must be done reading plane 1
  __syncthreads();
  return fx_to_f32(own);
}

__global__ void __launch_bounds__(kGroup)
quantize_weights_kernel(const float* __restrict__ W, int64_t K, int8_t* __restrict__ QW,
                        float* __restrict__ sW) {
  __shared__ uint32_t buf[2][kLimbs][kGroup];
  __shared__ float red[kGroup / 64];
  const int c = threadIdx.x;
  const int64_t row = blockIdx.x;
  const float* wrow = W + row * K;
  const int64_t groups = K / kGroup;

  float amax = 0.0f;
  for (int64_t g = 0; g < groups; ++g)
    amax = fmaxf(amax, fabsf(rotate_group_exact(wrow + g * kGroup, c, buf)));
  amax = wave_max64(amax);
  if ((c & 63) == 0) red[c >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax / 127.0f;  // IEEE fp32 division
  if (c == 0) sW[row] = s;

  int8_t* qrow = QW + row * K;
  for (int64_t g = 0; g < groups; ++g) {
    const float v = rotate_group_exact(wrow + g * kGroup, c, buf);
    float q = 0.0f;
    if (s != 0.0f) q = fminf(fmaxf(rintf(v / s), -128.0f), 127.0f);
    qrow[g * kGroup + c] = (int8_t)(int)q;
  }
}

}  // namespace

hipError_t launch_quantize_weights(const float* W, int64_t N, int64_t K, int8_t* QW, float* sW,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(quantize_weights_kernel, dim3((unsigned)N), dim3(kGroup), 0, stream, W, K,
                     QW, sW);
  return hipGetLastError();
}

}  // namespace convrot
