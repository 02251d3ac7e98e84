// Empty contractions (K = 0).
//
// Page "[PR #249] Add an mps backend: weight-only INT8 and W4A8/W6A8 linears
// for Apple GPUs", commit list: empty contractions return early instead of
// reaching the kernels.  With K = 0 every sum over k is empty: A = 0, a row
// maximum is 0 (so s = 0 and the range-safe exponent is 0, as for a zero
// row), the LoRA term is 0, and a linear's output is its bias rounded to the
// output type (+0 without a bias), plus the residual as one addition.  The
// arithmetic is the epilogue's: +0 + bias in fp32 (a -0 bias gives +0), one
// rounding, then the residual sum in fp32 and one rounding (fp32 holds more
// than twice the significand bits of fp16 and bf16, so that is the correctly
// rounded sum).
//
// Plain elementwise fills: one thread per output element, grid-stride.

#include "launch.hpp"

namespace convrot {
namespace {

constexpr int64_t kMaxBlocks = 65536;

__global__ void __launch_bounds__(256)
empty_linear_kernel(int64_t M, int64_t N, const float* __restrict__ bias, const void* R, int out,
                    void* Y) {
  const int64_t total = M * N;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    if (out == kEmptyI32) {
      reinterpret_cast<int32_t*>(Y)[e] = 0;
      continue;
    }
    const int64_t n = e % N;
    const float y = bias ? __fadd_rn(0.0f, bias[n]) : 0.0f;
    if (out == kEmptyF16) {
      __half h = __float2half_rn(y);
      if (R) h = __float2half_rn(__half2float(h) + __half2float(reinterpret_cast<const __half*>(R)[e]));
      reinterpret_cast<__half*>(Y)[e] = h;
    } else {
      uint16_t b = f32_to_bf16_rn(y);
      if (R) b = f32_to_bf16_rn(bf16_to_f32(b) + bf16_to_f32(reinterpret_cast<const uint16_t*>(R)[e]));
      reinterpret_cast<uint16_t*>(Y)[e] = b;
    }
  }
}

__global__ void __launch_bounds__(256) fill32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) p[e] = v;
}

unsigned blocks_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)(b < kMaxBlocks ? b : kMaxBlocks);
}

}  // namespace

hipError_t launch_empty_linear(int64_t M, int64_t N, const float* bias, const void* R, EmptyOut out, void* Y,
                               hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  hipLaunchKernelGGL(empty_linear_kernel, dim3(blocks_for(M * N)), dim3(256), 0, stream, M, N, bias, R,
                     (int)out, Y);
  return hipGetLastError();
}

hipError_t launch_fill32(void* p, int64_t n, uint32_t value, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill32_kernel, dim3(blocks_for(n)), dim3(256), 0, stream, reinterpret_cast<uint32_t*>(p),
                     n, value);
  return hipGetLastError();
}

}  // namespace convrot
