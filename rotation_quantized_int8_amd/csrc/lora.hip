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
// t_ld = rank rounded up to 32; its padding columns are zero.

#include "launch.hpp"

namespace convrot {
namespace {

constexpr int kRows = 32;                   // activation rows per workgroup
constexpr int kChunk = 256;                 // K columns per staged chunk
constexpr int kRowBytes = kChunk * 2 + 16;  // LDS bytes per staged fp16 row (+16: bank offset)
constexpr int kMaxSplits = 32;

// NFR = t_ld / 16 fragments of 16 rank columns (2 or 4: t_ld is 32 or 64).
// Workgroups past the row blocks (first K range only) write U' instead, 32
// rows of up each.
template <int NFR>
__global__ void __launch_bounds__(256)
lora_down_kernel(const __half* __restrict__ X, const float* __restrict__ D, const float* __restrict__ up,
                 float scale, int64_t M, int64_t N, int64_t K, int rank, int64_t kc,
                 float* __restrict__ P, __half* __restrict__ T, __half* __restrict__ U) {
  constexpr int t_ld = NFR * 16;
  __shared__ __align__(16) char xs[kRows * kRowBytes];
  __shared__ __align__(16) char ds[t_ld * kRowBytes];
  __shared__ v4f red[2][NFR][64];

  const int tid = threadIdx.x;
  const int64_t row_blocks = (M + kRows - 1) / kRows;
  if ((int64_t)blockIdx.x >= row_blocks) {
    if (blockIdx.y != 0) return;
    const int64_t n0 = ((int64_t)blockIdx.x - row_blocks) * 32;
    for (int e = tid; e < 32 * (t_ld / 4); e += 256) {
      const int64_t n = n0 + e / (t_ld / 4);
      const int r = 4 * (e % (t_ld / 4));
      if (n >= N) continue;
      v4h h;
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = (_Float16)as_fp32(r + i < rank ? __fmul_rn(up[n * rank + r + i], scale) : 0.0f);
      *reinterpret_cast<v4h*>(U + n * t_ld + r) = h;
    }
    return;
  }

  const int lane = tid & 63, wave = tid >> 6;
  const int frow = lane & 15, fk = lane >> 4;
  const int rb = wave & 1;    // 16-row block of this wave
  const int kh = wave >> 1;   // which half of each chunk's K steps
  const int64_t m0 = (int64_t)blockIdx.x * kRows;
  const int64_t z = blockIdx.y;

  v4f acc[NFR];
#pragma unroll
  for (int f = 0; f < NFR; ++f) acc[f] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = z * kc; k0 < (z + 1) * kc; k0 += kChunk) {
    // X chunk: 32 rows x 32 16-byte pieces (rows past M repeat row M - 1 and
    // are dropped at the end)
#pragma unroll
    for (int i = 0; i < kRows * 32 / 256; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 5, col = c & 31;
      int64_t m = m0 + row;
      m = m < M ? m : M - 1;
      const uint4 v = *reinterpret_cast<const uint4*>(X + m * K + k0 + 8 * col);
      *reinterpret_cast<uint4*>(xs + row * kRowBytes + 16 * col) = v;
    }
    // down chunk: t_ld rows x 64 float4 pieces, rounded to fp16; rows past
    // the rank are zero
#pragma unroll
    for (int i = 0; i < t_ld * 64 / 256; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 6, col = c & 63;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (row < rank) v = *reinterpret_cast<const float4*>(D + (int64_t)row * K + k0 + 4 * col);
      v4h h;
      h[0] = (_Float16)v.x; h[1] = (_Float16)v.y; h[2] = (_Float16)v.z; h[3] = (_Float16)v.w;
      *reinterpret_cast<v4h*>(ds + row * kRowBytes + 8 * col) = h;
    }
    __syncthreads();
    // K steps j of 32 (this wave: j = kh, kh + 2, ...): A = down rows (16 per
    // fragment), B = the wave's 16 X rows
#pragma unroll
    for (int j = kh; j < kChunk / 32; j += 2) {
      const v8h b = *reinterpret_cast<const v8h*>(xs + (16 * rb + frow) * kRowBytes + 64 * j + 16 * fk);
#pragma unroll
      for (int f = 0; f < NFR; ++f) {
        const v8h a = *reinterpret_cast<const v8h*>(ds + (16 * f + frow) * kRowBytes + 64 * j + 16 * fk);
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[f], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // add the second half's sums to the first's (fixed order)
  if (kh == 1) {
#pragma unroll
    for (int f = 0; f < NFR; ++f) red[rb][f][lane] = acc[f];
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int f = 0; f < NFR; ++f) acc[f] += red[rb][f][lane];

  // lane holds r = 16 f + 4 fk + i of row m
  const int64_t m = m0 + 16 * rb + frow;
  if (m >= M) return;
  if (gridDim.y == 1) {
#pragma unroll
    for (int f = 0; f < NFR; ++f) {
      v4h h;
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = (_Float16)(16 * f + 4 * fk + i < rank ? acc[f][i] : 0.0f);
      *reinterpret_cast<v4h*>(T + m * t_ld + 16 * f + 4 * fk) = h;
    }
  } else {
#pragma unroll
    for (int f = 0; f < NFR; ++f) *reinterpret_cast<v4f*>(P + (z * M + m) * t_ld + 16 * f + 4 * fk) = acc[f];
  }
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
  const int64_t chunks = K / kChunk;
  int64_t s = 1;
  while (s * 2 <= kMaxSplits && chunks % (s * 2) == 0) s *= 2;
  return s;
}

hipError_t launch_lora_prep(const void* X, const float* down, const float* up, float scale, int64_t M,
                            int64_t N, int64_t K, int rank, int t_ld, float* P, __half* T, __half* U,
                            hipStream_t stream) {
  const int64_t splits = lora_splits(K);
  const int64_t blocks = (M + kRows - 1) / kRows + (N + 31) / 32;
  auto fn = t_ld > 32 ? &lora_down_kernel<4> : &lora_down_kernel<2>;
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks, (unsigned)splits), dim3(256), 0, stream,
                     reinterpret_cast<const __half*>(X), down, up, scale, M, N, K, rank, K / splits, P, T, U);
  if (splits == 1) return hipGetLastError();
  if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int64_t threads = M * (t_ld / 4);
  hipLaunchKernelGGL(lora_sum_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, P,
                     splits, M, t_ld, rank, T);
  return hipGetLastError();
}

}  // namespace convrot
