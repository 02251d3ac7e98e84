// GEMM dispatch: which tile configuration of the direct-to-LDS kernel
// (gemm_dma.hip) serves a problem size, for every product of the library:
// the int8 W8A8 product with or without its scale epilogue, the weight-only
// product with s_W, bias and LoRA, and the fp16 baseline.

#include "launch.hpp"

namespace convrot {

// 256x128 tiles read half the operand bytes per output of 128x64 tiles,
// which pays once they still give most of the 256 CUs a tile; otherwise
// 128x64 tiles spread the work wider, and when even those would leave half
// the CUs idle, 64x64 or 32x64 tiles do.  The 256x128 tile runs as 8 waves
// of 64x64 (two per SIMD, so one wave's waits overlap the other's MFMAs).
// With few rows (M <= 128) the product streams the weights, and 32x64 tiles
// keep the activation loads from being mostly padding while giving four
// times as many workgroups.
int choose_gemm_cfg(GemmMode mode, int64_t M, int64_t N, int64_t K) {
  (void)mode; (void)K;
  if (M <= 128) return 9;
  const auto tiles = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (tiles(256, 128) >= 160) return 13;
  if (tiles(128, 64) >= 128) return 8;
  if (tiles(64, 64) >= 128) return 10;
  return 9;
}

// W8A8 with few rows: when the 32x64 tile grid is too small to occupy the
// chip (fewer than 64 tiles), K is split so that tiles x splits reaches about
// 256 workgroups with at least 512 K values each.  The int32 partial sums are
// exact, so the split result is bit-identical to the unsplit one.
int64_t w8a8_splits(int64_t M, int64_t N, int64_t K) {
  if (M > 128) return 1;
  const int64_t tiles = ((M + 31) / 32) * ((N + 63) / 64);
  if (tiles >= 64) return 1;
  int64_t s = 1;
  while (tiles * s * 2 <= 256 && K % (s * 2 * 256) == 0 && K / (s * 2) >= 512) s *= 2;
  return s;
}

namespace {

constexpr int kEpiRows = 4;   // rows per thread of the split-K epilogue

// One thread per output column n and kEpiRows rows (the loads of all its
// rows go out together, and the column's s_W, bias and LoRA up values are
// fetched once for them):
//   y = fp32(sum_z A_z) * fp32(s_X * s_W) [+ bias]   (the GEMM epilogue's
//       fp32 operations in the same order),
//   [+ LoRA term sum_r T[m, r] U'[n, r] accumulated in fp32],
//   Y = fp16(y) [then one fp16 addition of the residual].
__global__ void __launch_bounds__(64)
splitk_epilogue_kernel(const int32_t* __restrict__ parts, int64_t splits, GemmArgs p) {
  const int64_t n = (int64_t)blockIdx.x * 64 + threadIdx.x;
  const int64_t M = p.M, N = p.N, total = M * N;
  if (n >= N) return;
  const int64_t m0 = (int64_t)blockIdx.y * kEpiRows;
  int32_t a[kEpiRows];
  float l[kEpiRows];
#pragma unroll
  for (int i = 0; i < kEpiRows; ++i) {
    a[i] = 0;
    l[i] = 0.0f;
  }
  for (int64_t z = 0; z < splits; ++z) {
#pragma unroll
    for (int i = 0; i < kEpiRows; ++i)
      if (m0 + i < M) a[i] += parts[z * total + (m0 + i) * N + n];
  }
  for (int r = 0; r < p.t_ld; ++r) {
    const float u = __half2float(p.U[n * p.t_ld + r]);
#pragma unroll
    for (int i = 0; i < kEpiRows; ++i)
      if (m0 + i < M) l[i] = fmaf(__half2float(p.T[(m0 + i) * p.t_ld + r]), u, l[i]);
  }
  __half* Y = reinterpret_cast<__half*>(p.out);
  const float sw = p.sW[n];
  const float b = p.bias ? p.bias[n] : 0.0f;
#pragma unroll
  for (int i = 0; i < kEpiRows; ++i) {
    const int64_t m = m0 + i;
    if (m >= M) break;
    const int64_t e = m * N + n;
    float y = __fmul_rn((float)a[i], __fmul_rn(p.sX[m], sw));
    if (p.bias) y = __fadd_rn(y, b);
    if (p.t_ld > 0) y = __fadd_rn(y, l[i]);
    __half h = __float2half_rn(y);
    if (p.R) h = __float2half_rn(__half2float(h) + __half2float(p.R[e]));
    Y[e] = h;
  }
}

}  // namespace

hipError_t launch_splitk_epilogue(const int32_t* parts, int64_t splits, const GemmArgs& a,
                                  hipStream_t stream) {
  const dim3 grid((unsigned)((a.N + 63) / 64), (unsigned)((a.M + kEpiRows - 1) / kEpiRows));
  hipLaunchKernelGGL(splitk_epilogue_kernel, grid, dim3(64), 0, stream, parts, splits, a);
  return hipGetLastError();
}

template <GemmMode MODE>
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  return launch_gemm_dma_cfg<MODE>(a, choose_gemm_cfg(MODE, a.M, a.N, a.K), stream);
}

template hipError_t launch_gemm<GemmMode::kI8toI32>(const GemmArgs&, hipStream_t);
template hipError_t launch_gemm<GemmMode::kI8toF16>(const GemmArgs&, hipStream_t);
template hipError_t launch_gemm<GemmMode::kF16>(const GemmArgs&, hipStream_t);
template hipError_t launch_gemm<GemmMode::kW8A16>(const GemmArgs&, hipStream_t);

}  // namespace convrot
