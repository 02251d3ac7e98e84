// Low-rank activation of the unmerged LoRA: T[m, r] = sum_k X[m, k] down[r, k].
//
// Page "[PR #249] Add an mps backend: weight-only INT8 and W4A8/W6A8 linears
// for Apple GPUs", sections "What" and "Design": the weight-only linear takes
// lora_down [R, K], lora_up [N, R] and lora_scale and adds
// scale * (X down^T) up^T; the up product is applied in the GEMM epilogue.
//
// Since H is orthogonal and symmetric, (XH)(down H)^T = X down^T, so the
// unrotated activation and down weight are used directly.  Products are fp16
// x fp16 on v_mfma_f32_16x16x32_f16 with fp32 accumulation; `down` is rounded
// to fp16 on the fly.  A workgroup owns 16 activation rows; its 8 wavefronts
// take interleaved K steps, each with kUnroll steps of loads in flight before
// their MFMAs (the product is tiny, so load latency is what costs), and the
// wavefronts' partial sums are added in a fixed order, so the result is
// deterministic.  T is written in fp16 with row stride t_ld = rank rounded up
// to 32 (padding columns are zero).

#include "launch.hpp"

namespace convrot {
namespace {

constexpr int kWaves = 8;
constexpr int kUnroll = 4;

// NFR = t_ld / 16 fragments of 16 rank columns (2 or 4: t_ld is 32 or 64)
template <int NFR>
__global__ void __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
lora_down_kernel(const __half* __restrict__ X, const float* __restrict__ D, int64_t M, int64_t K,
                 int rank, int t_ld, __half* __restrict__ T) {
  constexpr int kMaxRFrags = NFR;
  __shared__ v4f part[kWaves][kMaxRFrags][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int frow = lane & 15, fk = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  constexpr int nfr = NFR;
  const int64_t m = m0 + frow;

  v4f acc[kMaxRFrags];
#pragma unroll
  for (int f = 0; f < kMaxRFrags; ++f) acc[f] = v4f{0.f, 0.f, 0.f, 0.f};

  constexpr int64_t kStride = (int64_t)kWaves * 32;   // K between one wave's steps
  // Loads are unconditional (addresses clamped into the tensors) and padding
  // is zeroed at use, so the compiler keeps all of a batch's loads in flight.
  const int64_t mc = m < M ? m : M - 1;
  const bool mrow = m < M;
  for (int64_t k0 = (int64_t)wave * 32; k0 < K; k0 += kStride * kUnroll) {
    uint4 xv[kUnroll];
    float4 dv[kUnroll][kMaxRFrags][2];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t k = k0 + u * kStride;
      const int64_t kc = k < K ? k : K - 32;
      xv[u] = *reinterpret_cast<const uint4*>(X + mc * K + kc + 8 * fk);
#pragma unroll
      for (int f = 0; f < kMaxRFrags; ++f) {
        if (f < nfr) {
          int r = f * 16 + frow;
          r = r < rank ? r : rank - 1;
          const float4* dp = reinterpret_cast<const float4*>(D + (int64_t)r * K + kc + 8 * fk);
          dv[u][f][0] = dp[0];
          dv[u][f][1] = dp[1];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bool kin = k0 + u * kStride < K;
      uint4 xz = xv[u];
      if (!(kin && mrow)) xz = make_uint4(0, 0, 0, 0);
      const v8h xb = *reinterpret_cast<const v8h*>(&xz);
#pragma unroll
      for (int f = 0; f < kMaxRFrags; ++f) {
        if (f < nfr) {
          const bool live = kin && (f * 16 + frow < rank);
          const float4 d0 = dv[u][f][0], d1 = dv[u][f][1];
          v8h da;
          da[0] = (_Float16)d0.x; da[1] = (_Float16)d0.y; da[2] = (_Float16)d0.z; da[3] = (_Float16)d0.w;
          da[4] = (_Float16)d1.x; da[5] = (_Float16)d1.y; da[6] = (_Float16)d1.z; da[7] = (_Float16)d1.w;
          if (!live) da = v8h{0, 0, 0, 0, 0, 0, 0, 0};
          acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(da, xb, acc[f], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int f = 0; f < kMaxRFrags; ++f) part[wave][f][lane] = acc[f];
  __syncthreads();
  if (wave == 0) {
    // result register i of lane l: r = 16 f + 4 (l / 16) + i, m = m0 + l % 16
    for (int f = 0; f < nfr; ++f) {
      v4f s = part[0][f][lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) s += part[w][f][lane];
      if (m < M) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = f * 16 + 4 * fk + i;
          T[m * t_ld + r] = __float2half_rn(r < rank ? s[i] : 0.0f);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_lora_down(const void* X, const float* D, int64_t M, int64_t K, int rank,
                            int t_ld, void* T, hipStream_t stream) {
  const int64_t blocks = (M + 15) / 16;
  auto fn = t_ld > 32 ? &lora_down_kernel<4> : &lora_down_kernel<2>;
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(64 * kWaves), 0, stream,
                     reinterpret_cast<const __half*>(X), D, M, K, rank, t_ld,
                     reinterpret_cast<__half*>(T));
  return hipGetLastError();
}

}  // namespace convrot
