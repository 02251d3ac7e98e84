// Exact 256-point rotation and per-row quantisation of fp16 activations, as
// device functions shared by the stand-alone prologue kernel and the fused
// W8A8 launch.
//
// Page "INT8ConvRot GEMM vs fp16 on M1 Max with Metal, MPSMatrix, and MLX
// (fp16 Wins)", section "What changed in the computation": X_rot = X H in
// groups of 256 along K, s_X = max |X_rot| / 127 over the row,
// Q_X = round(X_rot / s_X).
//
// Exactness.  An fp16 value is a multiple of 2^-24 below 2^16, so every
// partial sum of the 256-point transform is a multiple of 2^-24 below 2^24:
// 48 significand bits.  The butterflies therefore run in fp64, where they are
// exact, and the result is rounded once (to fp32, or to fp16 through
// round-to-odd).  gfx950 issues fp64 adds at the full vector rate, so this
// costs the same number of VALU operations as an inexact fp32 transform.
//
// Layout.  A 256-group is viewed as a 16x16 matrix G[a][b] (element 16a + b)
// and H = H16 (x) H16 (up to the 1/16), so the transform is a 16-point
// transform along a followed by one along b.  Each group is owned by 16
// consecutive lanes of one wavefront (a "segment") and a private LDS slot:
//   1. lane a holds row a (32 contiguous bytes) and parks its two 16-byte
//      halves in two regions of the slot (the first halves of the 16 rows,
//      then the second halves: each parking store covers all banks once,
//      where 32-byte rows put lanes a and a + 8 on the same banks);
//   2. lane b reads column b back, transforms along a in registers (fp64);
//   3. the columns go through an XOR-swizzled fp64 transpose in the slot;
//   4. lane c holds row c, transforms along b in registers -> 16 contiguous
//      outputs, which become one 16-byte int8 store (or two for fp16).
// All exchanges stay inside a wavefront.
#pragma once

#include "common.hpp"

namespace convrot {

constexpr int kSlotBytes = 2048 + 64;  // one group: 256 doubles + bank-offset pad
constexpr int kParkHi = 272;           // byte offset of the second-half region (256 + a 16-byte bank offset)

// Step 1: row `lane` of the group, as its halves r0 (elements 16 lane .. +7)
// and r1 (+8 .. +15), into the slot's two parking regions.
__device__ __forceinline__ void park_row(char* slot, int lane, v4i r0, v4i r1) {
  *reinterpret_cast<v4i*>(slot + 16 * lane) = r0;
  *reinterpret_cast<v4i*>(slot + kParkHi + 16 * lane) = r1;
}

__device__ __forceinline__ void fwht16(double (&v)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const double a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// One 16-bit input value as a double: fp16, or bf16 (the upper half of an fp32).
template <bool kBF16>
__device__ __forceinline__ double in16_to_f64(uint16_t bits) {
  if constexpr (kBF16) return (double)__uint_as_float((uint32_t)bits << 16);
  else return (double)__half2float(__ushort_as_half(bits));
}

// Steps 2-4 for a group of 16-bit values (fp16, or bf16 with kBF16) already
// parked in `slot` by park_row (written by lanes of this wavefront).  On return y[] holds 16 * x_rot of row `lane`
// of the group: exact for fp16 inputs, and for bf16 inputs whenever the
// group's values span at most 45 binades (every partial sum then fits 53
// bits).  `slot` is the segment's private LDS slot (kSlotBytes); it is free
// again on return.
template <bool kBF16 = false>
__device__ __forceinline__ void rotate_staged(char* slot, int lane, double (&y)[16]) {
  wave_lds_sync();
  // column `lane`: element (a, lane) for a = 0..15, from its column's half region
  const uint16_t* sh = reinterpret_cast<const uint16_t*>(slot + (lane < 8 ? 0 : kParkHi));
  double v[16];
#pragma unroll
  for (int a = 0; a < 16; ++a) v[a] = in16_to_f64<kBF16>(sh[8 * a + (lane & 7)]);
  wave_lds_sync();  // all staging reads done before the slot is reused below
  fwht16(v);        // along a: v[c] = Z[c][lane]
  // transpose: Z[c][b] at row c, 16-byte chunk (b >> 1) ^ (c & 7)
  double* sd = reinterpret_cast<double*>(slot);
#pragma unroll
  for (int c = 0; c < 16; ++c) sd[16 * c + 2 * ((lane >> 1) ^ (c & 7)) + (lane & 1)] = v[c];
  wave_lds_sync();
  const double2* rowp = reinterpret_cast<const double2*>(slot + 128 * lane);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const double2 d = rowp[q ^ (lane & 7)];
    y[2 * q] = d.x;
    y[2 * q + 1] = d.y;
  }
  wave_lds_sync();  // reads done before the slot's next use
  fwht16(y);        // along b
}

// Steps 1-4: this lane holds row `lane` (elements 16 lane .. 16 lane + 15)
// of the group as two 16-byte halves r0, r1 and parks it in the slot first.
template <bool kBF16 = false>
__device__ __forceinline__ void rotate_loaded(v4i r0, v4i r1, char* slot, int lane, double (&y)[16]) {
  park_row(slot, lane, r0, r1);
  rotate_staged<kBF16>(slot, lane, y);
}

// Loads row `lane` of the group at `src` and rotates it (see rotate_loaded).
template <bool kBF16 = false>
__device__ __forceinline__ void rotate_group(const uint16_t* __restrict__ src, char* slot, int lane,
                                             double (&y)[16]) {
  const v4i* s4 = reinterpret_cast<const v4i*>(src + 16 * lane);
  const v4i r0 = __builtin_nontemporal_load(s4);
  const v4i r1 = __builtin_nontemporal_load(s4 + 1);
  rotate_loaded<kBF16>(r0, r1, slot, lane, y);
}
__device__ __forceinline__ void rotate_group(const __half* __restrict__ src, char* slot, int lane,
                                             double (&y)[16]) {
  rotate_group<false>(reinterpret_cast<const uint16_t*>(src), slot, lane, y);
}

// Exact-definition quantisation of 16 fp32 values with scale s (> 0, or 0
// for an all-zero row, whose codes are 0):
// q = round_half_even(fp32(v / s)).  The fast path rounds the exact product
// v r, with r the hardware reciprocal of s (within one ulp of 1 / s), to an
// integer in one step: m = fma(v, r, 1.5 * 2^23) rounds v r + 1.5 * 2^23 once,
// and for |v r| < 2^22 the units place of that sum is where v r gets rounded,
// half to even; the integer k = m - 1.5 * 2^23 sits, two's complement, in the
// low mantissa bits of m, so the low byte of m's bits is the int8 code.  For
// finite inputs |v / s| <= 127 (1 + 2^-23), so v r is within 1.6e-5 of v / s
// and fp32(v / s) within 3.9e-6: whenever v r lies more than 3e-5 from a
// half-integer, both round to the same integer.  d = fma(v, r, -k), the
// distance v r - k rounded once, detects the rest: when any |d| > 0.49997 the
// lane falls back to IEEE division for its 16 values.  No clamp is needed.
// With s = 0 the reciprocal is taken as 0, so every product is 0 and the
// codes are 0 without a separate path.
__device__ __forceinline__ uint4 quantize16(const float (&v)[16], float s) {
  constexpr float kMagic = 12582912.0f;   // 1.5 * 2^23
  const float rcp = s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s);
  uint32_t b[16];
  float dmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float m = __fmaf_rn(v[i], rcp, kMagic);
    const float k = __fsub_rn(m, kMagic);   // exact: an integer of at most 8 bits
    dmax = fmaxf(dmax, fabsf(__fmaf_rn(v[i], rcp, -k)));
    b[i] = __float_as_uint(m);
  }
  if (dmax > 0.49997f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) b[i] = __float_as_uint(__fadd_rn(v[i] / s, kMagic));
  }
  // low bytes of four words -> one word: bytes (b0, b1) and (b2, b3) by byte
  // permutes, then the two halves side by side
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = __builtin_amdgcn_perm(b[4 * j + 1], b[4 * j], 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(b[4 * j + 3], b[4 * j + 2], 0x0c0c0400u);
    w[j] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace convrot
