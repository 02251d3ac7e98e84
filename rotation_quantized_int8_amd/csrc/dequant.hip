// Dequantise-every-call baseline: W_deq = fp16((Q_W (.) s_W) H) per 256-group.
//
// Page "INT8ConvRot GEMM vs fp16 on M1 Max with Metal, MPSMatrix, and MLX
// (fp16 Wins)", section "What changed in the computation": the earlier
// workaround turned the int8 weights and their per-channel scale back into
// fp16 and un-rotated them on every call before a plain fp16 X W^T; the
// three-way table of that section times it against fp16 and the weight-only
// path.  H is symmetric and orthogonal, so un-rotating is one more
// multiplication by H.
//
// Exactness.  The int8 codes are exact in fp16, and the 256-point transform
// of integers (|sum| <= 2^15) is exact in the fp64 butterflies of
// rotate.hpp; times s_W / 16 (an fp32 value and a power of two) it stays
// exact in fp64 (at most 15 + 24 significand bits), and one rounding to fp16
// (through round-to-odd fp32) gives the correctly rounded result.
//
// Work split: one 16-lane segment per 256-group, 16 groups per 256-thread
// workgroup; lane c writes elements 16c .. 16c + 15 of its group (two
// 16-byte stores).

#include "launch.hpp"
#include "rotate.hpp"

namespace convrot {
namespace {

__global__ void __launch_bounds__(256)
dequant_kernel(const int8_t* __restrict__ QW, const float* __restrict__ sW, int64_t N, int64_t K,
               __half* __restrict__ W16) {
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x;
  const int seg = tid >> 4, lane = tid & 15;
  const int64_t groups = K / kGroup;
  const int64_t gi = (int64_t)blockIdx.x * 16 + seg;
  if (gi >= N * groups) return;        // whole segments only: no workgroup barrier below
  const int64_t n = gi / groups, g = gi - n * groups;
  const int64_t off = n * K + g * kGroup + 16 * lane;

  const uint4 raw = *reinterpret_cast<const uint4*>(QW + off);
  const int8_t* b = reinterpret_cast<const int8_t*>(&raw);
  __half h[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) h[i] = __int2half_rn((int)b[i]);   // exact for int8
  double y[16];
  rotate_loaded(*reinterpret_cast<const v4i*>(&h[0]), *reinterpret_cast<const v4i*>(&h[8]),
                smem + seg * kSlotBytes, lane, y);
  const double sc = (double)sW[n] * 0.0625;
  __half o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = f64_to_f16_rn(y[i] * sc);
  uint4* dst = reinterpret_cast<uint4*>(W16 + off);
  dst[0] = *reinterpret_cast<const uint4*>(&o[0]);
  dst[1] = *reinterpret_cast<const uint4*>(&o[8]);
}

}  // namespace

hipError_t launch_dequantize(const int8_t* QW, const float* sW, int64_t N, int64_t K, void* W16,
                             hipStream_t stream) {
  const int64_t groups = N * (K / kGroup);
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((groups + 15) / 16)), dim3(256), 16 * kSlotBytes,
                     stream, QW, sW, N, K, reinterpret_cast<__half*>(W16));
  return hipGetLastError();
}

}  // namespace convrot
