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

// One thread per output: Y = fp16( fp32(sum_z A_z) * fp32(s_X * s_W) [+ bias] ),
// the same fp32 operations in the same order as the GEMM epilogue.
__global__ void __launch_bounds__(256)
splitk_epilogue_kernel(const int32_t* __restrict__ parts, int64_t splits, const float* __restrict__ sX,
                       const float* __restrict__ sW, const float* __restrict__ bias, int64_t M,
                       int64_t N, __half* __restrict__ Y) {
  const int64_t total = M * N;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t m = e / N, n = e - m * N;
    int32_t a = 0;
    for (int64_t z = 0; z < splits; ++z) a += parts[z * total + e];
    const float sc = __fmul_rn(sX[m], sW[n]);
    float y = __fmul_rn((float)a, sc);
    if (bias) y = __fadd_rn(y, bias[n]);
    Y[e] = __float2half_rn(y);
  }
}

}  // namespace

hipError_t launch_splitk_epilogue(const int32_t* parts, int64_t splits, const float* sX,
                                  const float* sW, const float* bias, int64_t M, int64_t N,
                                  void* Y, hipStream_t stream) {
  const int64_t total = M * N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(splitk_epilogue_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, parts,
                     splits, sX, sW, bias, M, N, reinterpret_cast<__half*>(Y));
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
