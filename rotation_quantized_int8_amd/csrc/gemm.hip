// GEMM dispatch: which tile configuration of the direct-to-LDS kernel
// (gemm_dma.hip) serves a problem size, for every product of the library:
// the int8 W8A8 product with or without its scale epilogue, the weight-only
// product with s_W, bias and LoRA, and the fp16 baseline.

#include "launch.hpp"

namespace convrot {

// 256x128 tiles read half the operand bytes per output of 128x64 tiles,
// which pays once they still give most of the 256 CUs a tile; otherwise
// 128x64 tiles spread the work wider.  With few rows (M <= 128) the product
// streams the weights, and 32x64 tiles keep the activation loads from being
// mostly padding while giving four times as many workgroups.
int choose_gemm_cfg(GemmMode mode, int64_t M, int64_t N, int64_t K) {
  (void)mode; (void)K;
  if (M <= 128) return 9;
  const int64_t big = ((M + 255) / 256) * ((N + 127) / 128);
  return big >= 160 ? 2 : 8;
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
