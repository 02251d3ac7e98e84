// Activation prologue: X_rot = X H per 256-group, s_X = row max / 127,
// Q_X = round(X_rot / s_X) -- or, for the weight-only path, X16 = fp16(X H).
//
// Page "INT8ConvRot GEMM vs fp16 on M1 Max with Metal, MPSMatrix, and MLX
// (fp16 Wins)", section "What changed in the computation": activation
// equation (every call) and the weight-only listing (x_rot kept in fp16).
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
// consecutive lanes of one wavefront:
//   1. lane a loads row a (32 contiguous bytes) and parks it in LDS;
//   2. lane b reads column b back, transforms along a in registers (fp64);
//   3. the columns go through an XOR-swizzled fp64 LDS transpose;
//   4. lane c holds row c, transforms along b in registers -> 16 contiguous
//      outputs, which become one 16-byte int8 store (or two for fp16).
// All exchanges stay inside a wavefront; only the row maximum crosses waves.
//
// Work split.  G = K/256 groups per row.  K <= 4096: a 256-thread workgroup
// holds floor(16/G) rows.  K <= 16384: one row, 16*G threads.  Longer rows:
// 1024 threads walk the row in chunks of 64 groups twice (maximum, then
// quantise), recomputing the transform instead of holding the row.

#include "launch.hpp"

namespace convrot {
namespace {

constexpr int kSlotBytes = 2048 + 64;  // one group: 256 doubles + bank-offset pad

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

// Transform one group owned by this lane's 16-lane segment.  On return y[]
// holds the fp64-exact outputs (16 * x_rot, i.e. before the 1/16) of row
// `lane` of the group: elements 16*lane .. 16*lane + 15.
__device__ __forceinline__ void rotate_group(const __half* __restrict__ src, char* slot, int lane,
                                             double (&y)[16]) {
  // 1. row `lane` (16 halves, 32 bytes) -> LDS staging (first 512 B of the slot)
  const v4i* s4 = reinterpret_cast<const v4i*>(src + 16 * lane);
  const v4i r0 = __builtin_nontemporal_load(s4);
  const v4i r1 = __builtin_nontemporal_load(s4 + 1);
  v4i* st = reinterpret_cast<v4i*>(slot + 32 * lane);
  st[0] = r0;
  st[1] = r1;
  wave_lds_sync();
  // 2. column `lane`: element (a, lane) for a = 0..15
  const __half* sh = reinterpret_cast<const __half*>(slot);
  double v[16];
#pragma unroll
  for (int a = 0; a < 16; ++a) v[a] = (double)__half2float(sh[16 * a + lane]);
  wave_lds_sync();  // all staging reads done before the slot is reused below
  fwht16(v);        // along a: v[c] = Z[c][lane]
  // 3. transpose through LDS: Z[c][b] at row c, 16-byte chunk (b>>1)^(c&7)
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
  wave_lds_sync();  // reads done before the next group's staging writes
  // 4. along b
  fwht16(y);
}

struct Split {
  int rows_per_wg;   // rows handled by one workgroup
  int gpc;           // groups per chunk (groups of one row handled at once)
  int chunks;        // chunks per row
};

// Exact-definition quantisation of 16 fp32 values with scale s (> 0):
// q = round_half_even(fp32(v / s)).  The fast path multiplies by the
// reciprocal; when any product lies within 3e-5 of a half-integer -- closer
// than its possible deviation from the correctly rounded quotient -- the
// lane falls back to IEEE division for its 16 values.
__device__ __forceinline__ uint4 quantize16(const float (&v)[16], float s) {
  float q[16];
  if (s == 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = 0.0f;
  } else {
    const float rcp = 1.0f / s;
    bool near_tie = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float t = v[i] * rcp;
      q[i] = rintf(t);
      near_tie |= fabsf(t - q[i]) > 0.49997f;
    }
    if (near_tie) {
#pragma unroll
      for (int i = 0; i < 16; ++i) q[i] = rintf(v[i] / s);
    }
  }
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t b0 = (uint32_t)(int)fminf(fmaxf(q[4 * j + 0], -128.f), 127.f) & 0xffu;
    uint32_t b1 = (uint32_t)(int)fminf(fmaxf(q[4 * j + 1], -128.f), 127.f) & 0xffu;
    uint32_t b2 = (uint32_t)(int)fminf(fmaxf(q[4 * j + 2], -128.f), 127.f) & 0xffu;
    uint32_t b3 = (uint32_t)(int)fminf(fmaxf(q[4 * j + 3], -128.f), 127.f) & 0xffu;
    w[j] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <bool kInt8>
__global__ void __launch_bounds__(1024)
prologue_kernel(const __half* __restrict__ X, int64_t M, int64_t K, Split sp,
                int8_t* __restrict__ QX, float* __restrict__ sX, __half* __restrict__ X16) {
  extern __shared__ __align__(16) char smem[];
  __shared__ float gmax[64];
  __shared__ float rowmax[16];

  const int tid = threadIdx.x;
  const int slot_id = tid >> 4;     // group slot in the workgroup
  const int lane = tid & 15;        // lane within the group
  const int G = (int)(K / kGroup);
  const int row_in_wg = slot_id / sp.gpc;
  const int gi = slot_id - row_in_wg * sp.gpc;       // group index inside a chunk
  const int64_t row = (int64_t)blockIdx.x * sp.rows_per_wg + row_in_wg;
  const bool active = row_in_wg < sp.rows_per_wg && row < M;
  char* slot = smem + slot_id * kSlotBytes;

  const __half* xrow = X + row * K;
  double y[16];
  float f[16];

  if (!kInt8) {
    // Weight-only path: no row scale, just fp16(X H) per group.
    if (active) {
      for (int c = 0; c < sp.chunks; ++c) {
        const int g = c * sp.gpc + gi;
        if (g >= G) break;
        rotate_group(xrow + (int64_t)g * kGroup, slot, lane, y);
        __half h[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) h[i] = f64_to_f16_rn(y[i] * 0.0625);
        uint4* dst = reinterpret_cast<uint4*>(X16 + row * K + (int64_t)g * kGroup + 16 * lane);
        dst[0] = *reinterpret_cast<const uint4*>(&h[0]);
        dst[1] = *reinterpret_cast<const uint4*>(&h[8]);
      }
    }
    return;
  }

  // pass 1: transform, keep the values when the row fits in one chunk, take max
  float amax = 0.0f;
  if (active) {
    for (int c = 0; c < sp.chunks; ++c) {
      const int g = c * sp.gpc + gi;
      if (g >= G) break;
      rotate_group(xrow + (int64_t)g * kGroup, slot, lane, y);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        f[i] = (float)(y[i] * 0.0625);  // exact scaling, single rounding to fp32
        amax = fmaxf(amax, fabsf(f[i]));
      }
    }
  }
  amax = warp_max16(amax);
  if (lane == 0) gmax[slot_id] = amax;
  __syncthreads();
  if (sp.rows_per_wg > 1 || sp.gpc <= 16) {
    if (lane == 0 && gi == 0 && row_in_wg < sp.rows_per_wg) {
      float m = 0.0f;
      for (int j = 0; j < sp.gpc; ++j) m = fmaxf(m, gmax[row_in_wg * sp.gpc + j]);
      rowmax[row_in_wg] = m;
    }
  } else if (tid < 64) {
    float m = (tid < sp.gpc) ? gmax[tid] : 0.0f;
    m = wave_max64(m);
    if (tid == 0) rowmax[0] = m;
  }
  __syncthreads();
  if (!active) return;
  const float s = rowmax[row_in_wg] / 127.0f;  // IEEE fp32 division
  if (slot_id == row_in_wg * sp.gpc && lane == 0) sX[row] = s;

  // pass 2: quantise and store
  for (int c = 0; c < sp.chunks; ++c) {
    const int g = c * sp.gpc + gi;
    if (g >= G) break;
    if (sp.chunks > 1) {
      rotate_group(xrow + (int64_t)g * kGroup, slot, lane, y);
#pragma unroll
      for (int i = 0; i < 16; ++i) f[i] = (float)(y[i] * 0.0625);
    }
    const uint4 packed = quantize16(f, s);
    *reinterpret_cast<uint4*>(QX + row * K + (int64_t)g * kGroup + 16 * lane) = packed;
  }
}

Split choose_split(int64_t K) {
  const int G = (int)(K / kGroup);
  Split sp;
  if (G <= 16) {
    sp.rows_per_wg = 16 / G;
    sp.gpc = G;
    sp.chunks = 1;
  } else if (G <= 64) {
    sp.rows_per_wg = 1;
    sp.gpc = G;
    sp.chunks = 1;
  } else {
    sp.rows_per_wg = 1;
    sp.gpc = 64;
    sp.chunks = (G + 63) / 64;
  }
  return sp;
}

template <bool kInt8>
hipError_t launch(const __half* X, int64_t M, int64_t K, int8_t* QX, float* sX, __half* X16,
                  hipStream_t stream) {
  const Split sp = choose_split(K);
  const int slots = sp.rows_per_wg * sp.gpc;
  const int threads = ((slots * 16 + 63) / 64) * 64;
  const int64_t blocks = (M + sp.rows_per_wg - 1) / sp.rows_per_wg;
  const size_t lds = (size_t)(threads / 16) * kSlotBytes;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prologue_kernel<kInt8>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(prologue_kernel<kInt8>, dim3((unsigned)blocks), dim3(threads), lds, stream,
                     X, M, K, sp, QX, sX, X16);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_act_quant(const void* X, int64_t M, int64_t K, int8_t* QX, float* sX,
                            hipStream_t stream) {
  return launch<true>(reinterpret_cast<const __half*>(X), M, K, QX, sX, nullptr, stream);
}

hipError_t launch_act_rotate_f16(const void* X, int64_t M, int64_t K, void* X16,
                                 hipStream_t stream) {
  return launch<false>(reinterpret_cast<const __half*>(X), M, K, nullptr, nullptr,
                       reinterpret_cast<__half*>(X16), stream);
}

}  // namespace convrot
