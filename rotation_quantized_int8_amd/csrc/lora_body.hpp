// Device body of the LoRA down projection T = X down^T (and of the scaled
// up weight U' = fp16(scale * up)), shared by its own kernel (lora.hip) and
// by the launch that also runs the activation prologue (prologue.hip).
// Page "[PR #249] Add an mps backend: weight-only INT8 and W4A8/W6A8 linears
// for Apple GPUs", sections "What" and "Design" (unmerged LoRA).
#pragma once

#include "common.hpp"

namespace convrot {

constexpr int kLoraRows = 32;                       // activation rows per workgroup
constexpr int kLoraChunk = 256;                     // K columns per staged chunk
constexpr int kLoraRowBytes = kLoraChunk * 2 + 16;  // LDS bytes per staged fp16 row (+16: bank offset)
constexpr int kLoraMaxSplits = 32;

// LDS of one workgroup: the X chunk, the down chunk and the halves' sums.
constexpr int lora_lds_bytes(int nfr) { return (kLoraRows + 16 * nfr) * kLoraRowBytes + 2 * nfr * 64 * 16; }

// One workgroup of the down projection, block (bx, by) of a (row blocks +
// up blocks) x gy grid.  NFR = t_ld / 16 fragments of 16 rank columns (2 or
// 4: t_ld is 32 or 64).  Blocks past the row blocks (first K range only)
// write U' instead, 32 rows of up each.  `smem` holds lora_lds_bytes(NFR)
// bytes, 16-byte aligned.
template <int NFR>
__device__ __forceinline__ void lora_down_block(const __half* __restrict__ X, const float* __restrict__ D,
                                                const float* __restrict__ up, float scale, int64_t M, int64_t N,
                                                int64_t K, int rank, int64_t kc, float* __restrict__ P,
                                                __half* __restrict__ T, __half* __restrict__ U, int64_t bx,
                                                int64_t by, int64_t gy, char* smem) {
  constexpr int t_ld = NFR * 16;
  char* xs = smem;
  char* ds = smem + kLoraRows * kLoraRowBytes;
  v4f* red = reinterpret_cast<v4f*>(smem + (kLoraRows + t_ld) * kLoraRowBytes);   // [2][NFR][64]

  const int tid = threadIdx.x;
  const int64_t row_blocks = (M + kLoraRows - 1) / kLoraRows;
  if (bx >= row_blocks) {
    if (by != 0) return;
    const int64_t n0 = (bx - row_blocks) * 32;
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
  const int64_t m0 = bx * kLoraRows;
  const int64_t z = by;

  v4f acc[NFR];
#pragma unroll
  for (int f = 0; f < NFR; ++f) acc[f] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = z * kc; k0 < (z + 1) * kc; k0 += kLoraChunk) {
    // X chunk: 32 rows x 32 16-byte pieces (rows past M repeat row M - 1 and
    // are dropped at the end)
#pragma unroll
    for (int i = 0; i < kLoraRows * 32 / 256; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 5, col = c & 31;
      int64_t m = m0 + row;
      m = m < M ? m : M - 1;
      const uint4 v = *reinterpret_cast<const uint4*>(X + m * K + k0 + 8 * col);
      *reinterpret_cast<uint4*>(xs + row * kLoraRowBytes + 16 * col) = v;
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
      *reinterpret_cast<v4h*>(ds + row * kLoraRowBytes + 8 * col) = h;
    }
    __syncthreads();
    // K steps j of 32 (this wave: j = kh, kh + 2, ...): A = down rows (16 per
    // fragment), B = the wave's 16 X rows
#pragma unroll
    for (int j = kh; j < kLoraChunk / 32; j += 2) {
      const v8h b = *reinterpret_cast<const v8h*>(xs + (16 * rb + frow) * kLoraRowBytes + 64 * j + 16 * fk);
#pragma unroll
      for (int f = 0; f < NFR; ++f) {
        const v8h a = *reinterpret_cast<const v8h*>(ds + (16 * f + frow) * kLoraRowBytes + 64 * j + 16 * fk);
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[f], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // add the second half's sums to the first's (fixed order)
  if (kh == 1) {
#pragma unroll
    for (int f = 0; f < NFR; ++f) red[(rb * NFR + f) * 64 + lane] = acc[f];
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int f = 0; f < NFR; ++f) acc[f] += red[(rb * NFR + f) * 64 + lane];

  // lane holds r = 16 f + 4 fk + i of row m
  const int64_t m = m0 + 16 * rb + frow;
  if (m >= M) return;
  if (gy == 1) {
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

}  // namespace convrot
