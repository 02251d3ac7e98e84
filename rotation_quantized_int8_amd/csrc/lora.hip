// Operands of the unmerged LoRA: the low-rank activation
// T[m, r] = sum_k X[m, k] down[r, k] and the scaled up weight
// U'[n, r] = fp16(scale * up[n, r]), both fp16 with row stride t_ld.
//
// Page "[PR #249] Add an mps backend: weight-only INT8 and W4A8/W6A8 linears
// for Apple GPUs", sections "What" and "Design": the int8 linears take
// lora_down [R, K], lora_up [N, R] and lora_scale and add
// scale * (X down^T) up^T; the up product is applied in the GEMM epilogue.
//
// Since H is orthogonal and symmetric, (XH)(down H)^T = X down^T, so the
// unrotated activation and down weight are used directly.  Products are fp16
// x fp16 on v_mfma_f32_16x16x32_f16 with fp32 accumulation; `down` is rounded
// to fp16 on the fly.
//
// Work split.  The product is tiny (2 M K R operations); what costs is the
// latency of bringing X and down into the CUs, so K is split until each
// workgroup has one or two 256-column chunks: a workgroup of 4 wavefronts
// owns 32 activation rows and one K range, stages each chunk of X and down
// through LDS with coalesced 16-byte loads (every wavefront load reads whole
// 512-byte row segments), and each wavefront multiplies 16 rows by all rank
// columns over half of the chunk's K steps.  The two halves are added through
// LDS.  With one K range the workgroup writes T; otherwise it writes fp32
// partial sums and a second kernel adds the ranges in order, so the result
// does not depend on the order in which workgroups ran.  T has row stride
// t_ld = rank rounded up to 32; its padding columns are zero.  The
// workgroup's body is lora_down_block (lora_body.hpp): this file's kernel
// runs it alone, and where the activation prologue runs 256-thread
// workgroups the prologue's launch runs it beside the prologue
// (prologue_lora_kernel, prologue.hip), since both read only X.

#include "launch.hpp"
#include "lora_body.hpp"

namespace convrot {
namespace {

// The down projection as its own launch: (row blocks + up blocks) x splits
// workgroups of lora_down_block.
template <int NFR>
__global__ void __launch_bounds__(256)
lora_down_kernel(const __half* __restrict__ X, const float* __restrict__ D, const float* __restrict__ up,
                 float scale, int64_t M, int64_t N, int64_t K, int rank, int64_t kc,
                 float* __restrict__ P, __half* __restrict__ T, __half* __restrict__ U) {
  extern __shared__ __align__(16) char smem[];
  lora_down_block<NFR>(X, D, up, scale, M, N, K, rank, kc, P, T, U, blockIdx.x, blockIdx.y, gridDim.y, smem);
}

// T[m, r..r+3] = fp16(sum over K ranges z in order of P[z, m, r..r+3]).
// The ranges' pieces are loaded kBatch at a time, all in flight together,
// and then added in range order.
__global__ void __launch_bounds__(256)
lora_sum_kernel(const float* __restrict__ P, int64_t splits, int64_t M, int t_ld, int rank,
                __half* __restrict__ T) {
  constexpr int kBatch = 8;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q = t_ld / 4;
  if (e >= M * q) return;
  const int64_t m = e / q;
  const int r = 4 * (int)(e - m * q);
  v4f s = v4f{0.f, 0.f, 0.f, 0.f};
  for (int64_t z0 = 0; z0 < splits; z0 += kBatch) {
    v4f v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      v[u] = z0 + u < splits ? *reinterpret_cast<const v4f*>(P + ((z0 + u) * M + m) * t_ld + r) : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kBatch; ++u) s += v[u];
  }
  v4h h;
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = (_Float16)(r + i < rank ? s[i] : 0.0f);
  *reinterpret_cast<v4h*>(T + m * t_ld + r) = h;
}

}  // namespace

// K ranges: a power of two dividing K / 256, at most 32.
int64_t lora_splits(int64_t K) {
  const int64_t chunks = K / kLoraChunk;
  int64_t s = 1;
  while (s * 2 <= kLoraMaxSplits && chunks % (s * 2) == 0) s *= 2;
  return s;
}

hipError_t launch_lora_prep(const void* X, const float* down, const float* up, float scale, int64_t M,
                            int64_t N, int64_t K, int rank, int t_ld, float* P, __half* T, __half* U,
                            hipStream_t stream) {
  const int64_t splits = lora_splits(K);
  const int64_t blocks = (M + kLoraRows - 1) / kLoraRows + (N + 31) / 32;
  auto fn = t_ld > 32 ? &lora_down_kernel<4> : &lora_down_kernel<2>;
  const int lds = lora_lds_bytes(t_ld > 32 ? 4 : 2);
  if (const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(fn), lds); e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks, (unsigned)splits), dim3(256), lds, stream,
                     reinterpret_cast<const __half*>(X), down, up, scale, M, N, K, rank, K / splits, P, T, U);
  if (splits == 1) return hipGetLastError();
  if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  return launch_lora_sum(P, splits, M, t_ld, rank, T, stream);
}

hipError_t launch_lora_sum(const float* P, int64_t splits, int64_t M, int t_ld, int rank, __half* T,
                           hipStream_t stream) {
  const int64_t threads = M * (t_ld / 4);
  hipLaunchKernelGGL(lora_sum_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, P,
                     splits, M, t_ld, rank, T);
  return hipGetLastError();
}

}  // namespace convrot
