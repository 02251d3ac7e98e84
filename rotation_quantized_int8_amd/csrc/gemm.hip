// GEMM dispatch: which tile configuration of the direct-to-LDS kernel
// (gemm_dma.hip) serves a problem size, for every product of the library:
// the int8 W8A8 product with or without its scale epilogue, the weight-only
// product with s_W, bias and LoRA, and the fp16 baseline.

#include "launch.hpp"

namespace convrot {

// 256x128 tiles read half the operand bytes per output of 128x64 tiles,
// which pays once they still give most of the 256 CUs a tile; otherwise
// 128x64 tiles spread the work wider (as 8 waves of 32x32: two waves per
// SIMD, 5 % faster than 4 waves of 64x32 for the int8 product on 2048x2048
// and 6-10 % for the fp16 one; the weight-only product, which widens its int8
// weights per wave, keeps 4 waves), and when even those would leave half the
// CUs idle, 64x64 or 32x64 tiles do.  The 8-wave 128x64 tile streams the
// int8 product in 128-byte K slices on a 4-stage ring (96 KiB): against 3
// stages of 256-byte slices (144 KiB) the first slice lands sooner, which
// measured 0.5-2.8 % faster per layer at 2048x2048 and 2048x1024 (M = 1024,
// each layer its own weights or the same ones) and level at 2048x8192; the
// fp16 product keeps the 256-byte slices (half the barriers for its longer
// rows).  The 256x128 tile runs as 8 waves
// of 64x64 (two per SIMD, so one wave's waits overlap the other's MFMAs).
// With at most two 128-byte K slices (K <= 256) an int8 tile is one
// serial fill, product, epilogue and store; 128x128 tiles on a two-stage
// ring (64 KiB of LDS) put two workgroups on a CU, so one tile's epilogue
// and stores overlap another's loads and products, and every CU gets work
// (1024x6144x256: 8.1 -> 7.45 us against 256x128 tiles, W8A8 sweep -0.5 %).
// Only the fp16-output product: an int32 tile does not fit the ring for the
// staged output.
// A narrow int8 product (32x64 tiles leaving CUs idle, e.g. N = 256 at
// M = 1024) takes 32x32 tiles with 256-byte K slices: one tile per CU and
// half as many slice barriers.
// With few rows (M <= 128) the int8 product streams the weights: 64x64
// tiles when they still give at least 192 workgroups, else 32x32 tiles with
// 256-byte K slices (measured ahead of 32x64, 16x64 and 64x32 tiles at every
// row count from 2 to 128 on the sweep's large shapes); the other products
// use 32x64.
int choose_gemm_cfg(GemmMode mode, int64_t M, int64_t N, int64_t K) {
  const auto tiles = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (M <= 128) {
    if (mode != GemmMode::kI8toF16 && mode != GemmMode::kI8toI32) return 9;
    if (tiles(64, 64) >= 192) return 10;
    return 19;
  }
  const bool int8 = mode == GemmMode::kI8toF16 || mode == GemmMode::kI8toI32;
  if (mode == GemmMode::kI8toF16 && K <= 256 && tiles(128, 128) >= 256) return 21;
  if (tiles(256, 128) >= 160) return 13;
  if (tiles(128, 64) >= 128) return mode == GemmMode::kW8A16 ? 8 : (int8 ? 22 : 20);
  if (tiles(64, 64) >= 128) return 10;
  if (int8 && tiles(32, 64) < 256) return 19;
  return 9;
}

// W8A8 through the tiled GEMM with few rows.  K is split only when a
// workgroup would stream at least 512 KiB of operands (32x32 tiles at
// K >= 8192) and the tiles fill at most a quarter of the CUs, so that four or
// more K ranges are possible: below that, the second launch (the split
// epilogue, about 3 us in a graph) costs more than the shorter ranges save.
// Splits double while tiles x splits stays within 256 workgroups and each
// range keeps at least 1024 K values.  The int32 partial sums are exact, so
// the split result is bit-identical to the unsplit one.
int64_t w8a8_splits(int64_t M, int64_t N, int64_t K) {
  if (M > 128) return 1;
  const int cfg = choose_gemm_cfg(GemmMode::kI8toI32, M, N, K);
  const int64_t bm = cfg == 10 ? 64 : 32, bn = cfg == 10 ? 64 : 32;
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  if (tiles > 64 || (bm + bn) * K < (512 << 10)) return 1;
  int64_t s = 1;
  while (tiles * s * 2 <= 256 && K % (s * 2 * 256) == 0 && K / (s * 2) >= 1024) s *= 2;
  return s;
}

// Few rows: one fused launch when every workgroup can quantise the rows
// itself; up to 8 rows and at most 4096 outputs per row, the few-row kernel
// (it re-reads the activation rows for every 8 weight rows, which stops
// paying beyond 8 rows: there the 32x32-tile GEMM is as fast or faster);
// otherwise the tiled GEMM.
W8A8Plan w8a8_plan(int64_t M, int64_t N, int64_t K, bool lora) {
  if (!lora && skinny_fusable(M, K)) return {W8A8Plan::kFused, 1, false};
  if (!lora && band_fusable(M, N, K)) return {W8A8Plan::kBand, 1, false};
  if (!lora && narrow_fusable(M, N, K)) return {W8A8Plan::kNarrow, 1, false};
  if (M <= 8 && N <= 4096) {
    const int64_t s = skinny_splits(M, N, K);
    return {W8A8Plan::kSkinny, s, lora || s > 1};
  }
  const int64_t s = w8a8_splits(M, N, K);
  return {W8A8Plan::kGemm, s, s > 1};
}

namespace {

constexpr int kSplitBatch = 8;   // K-range partials loaded together

// One thread per output row m and 4 consecutive columns n .. n + 3 (one
// 16-byte piece of every K range's int32 partial; all ranges' pieces are in
// flight together, kSplitBatch at a time):
//   y = fp32(sum_z A_z) * fp32(s_X * s_W) [+ bias]   (the GEMM epilogue's
//       fp32 operations in the same order),
//   [+ LoRA term sum_r T[m, r] U'[n, r] accumulated in fp32],
//   Y = fp16(y) [then one fp16 addition of the residual].
__global__ void __launch_bounds__(256)
splitk_epilogue_kernel(const int32_t* __restrict__ parts, int64_t splits, GemmArgs p) {
  const int64_t M = p.M, N = p.N, total = M * N;
  const int64_t q = (N + 3) / 4;                  // pieces per row
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= M * q) return;
  const int64_t m = e / q;
  const int64_t n0 = 4 * (e - m * q);
  const int cols = N - n0 < 4 ? (int)(N - n0) : 4;
  const bool vec = (N % 4) == 0;                  // 16-byte aligned pieces
  const int32_t* base = parts + m * N + n0;

  int32_t a[4] = {0, 0, 0, 0};
  for (int64_t z0 = 0; z0 < splits; z0 += kSplitBatch) {
    v4i v[kSplitBatch];
#pragma unroll
    for (int u = 0; u < kSplitBatch; ++u) {
      v[u] = v4i{0, 0, 0, 0};
      if (z0 + u < splits) {
        const int32_t* src = base + (z0 + u) * total;
        if (vec) {
          v[u] = *reinterpret_cast<const v4i*>(src);
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (c < cols) v[u][c] = src[c];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kSplitBatch; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) a[c] += v[u][c];
  }

  // Columns past N (a ragged tail) are computed on the last column and not
  // stored.  Every per-column array is indexed by unrolled constants only: a
  // data-dependent index would make the compiler move the array to LDS,
  // which made this kernel several times slower.
  float l[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int r = 0; r < p.t_ld; ++r) {
    const float t = __half2float(p.T[m * p.t_ld + r]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t n = n0 + c < N ? n0 + c : N - 1;
      l[c] = fmaf(t, __half2float(p.U[n * p.t_ld + r]), l[c]);
    }
  }
  __half* Y = reinterpret_cast<__half*>(p.out);
  const float sx = p.sX[m];
  uint32_t hb[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t n = n0 + c < N ? n0 + c : N - 1;
    float y = __fmul_rn((float)a[c], __fmul_rn(sx, p.sW[n]));
    if (p.bias) y = __fadd_rn(y, p.bias[n]);
    if (p.t_ld > 0) y = __fadd_rn(y, l[c]);
    __half h = __float2half_rn(as_fp32(y));
    if (p.R) h = __float2half_rn(__half2float(h) + __half2float(p.R[m * N + n]));
    hb[c] = __half_as_ushort(h);
  }
  if (vec) {
    uint2 o;
    o.x = hb[0] | (hb[1] << 16);
    o.y = hb[2] | (hb[3] << 16);
    *reinterpret_cast<uint2*>(Y + m * N + n0) = o;
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (c < cols) Y[m * N + n0 + c] = __ushort_as_half((uint16_t)hb[c]);
  }
}

}  // namespace

hipError_t launch_splitk_epilogue(const int32_t* parts, int64_t splits, const GemmArgs& a,
                                  hipStream_t stream) {
  const int64_t threads = a.M * ((a.N + 3) / 4);
  hipLaunchKernelGGL(splitk_epilogue_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     parts, splits, a);
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
