// The W8A8 layer in one launch for narrow layers: few output columns
// (N <= 256) and rows of 2 or 4 rotation groups (K = 512, 1024).
// Page "INT8ConvRot GEMM vs fp16 on M1 Max with Metal, MPSMatrix, and MLX
// (fp16 Wins)", section "What changed in the computation" (X_rot = X H,
// s_X = max |X_rot| / 127, Q_X = round(X_rot / s_X), A = Q_X Q_W^T in int32,
// Y = A (.) s_X s_W^T).
//
// A narrow layer's weights are small (256 x 1024 int8 is 256 KiB), so the
// cost of the usual two launches is mostly the prologue's own launch and the
// round trip of Q_X through memory.  Here a workgroup (8 wavefronts) owns a
// band of 8 activation rows and one group of 128 output columns; it
// quantises its band itself and multiplies it by its 128 weight rows, which
// stream through an LDS ring in K slices of 256 bytes while the band
// rotates.  With N = 256 each band is quantised twice (once per column
// group); at M = 1024 that is 256 workgroups.  Used while the grid is one
// workgroup per CU at most (ceil(M / 8) ceil(N / 128) <= 256): measured
// 15-40 % faster than the prologue and GEMM there (M = 64 ... 2048), level
// or slower beyond.  At K = 2048 it was no faster than the two launches
// (10.8 against 10.6 us at 1024 x 256): the fixed cost of the band loads and
// of one barrier-separated step per K slice, plus the second rotation pass
// and the weight stream after it, outweigh the saved launch.
//
// Per workgroup:
//   1. every segment (16 lanes) loads one rotation group of the band (row
//      j = group / G, G = K / 256) and parks it in its LDS slot; the direct
//      global->LDS loads of K slices 0 and 1 (128 weight rows x 256 bytes
//      each, in 1 KiB blocks, 16-byte chunks XOR-swizzled by row & 15) go
//      out once the first groups are parked;
//   2. the segments rotate their groups (exact fp64, rotate.hpp), take each
//      row's maximum through LDS, s = max / 127
//      (IEEE fp32 division), and write the codes to LDS (chunk c of row j's
//      group g at 256 g + 16 (c ^ (j & 15))) -- the functions and arithmetic
//      of the stand-alone prologue;
//   3. the rotation slots become two more ring stages; per slice: wait for
//      its blocks, one barrier, refill the stage freed by the previous
//      slice, 4 v_mfma_i32_16x16x64_i8 per wavefront (its 16 columns x the
//      band, padded to 16 rows) into int32 accumulators;
//   4. the scale epilogue (fp32(A) * fp32(s_X s_W) [+ bias], fp16) into an
//      LDS staging tile, then 16-byte stores [+ the residual, one fp16
//      addition].
//
// The direct loads are inline assembly (the compiler does not count them):
// a wavefront's loads of one slice form a group of 4 and the kernel waits
// for "at most k groups in flight" with explicit vmcnt values.  The weight
// scales, biases and activation rows are loaded first and have landed
// before the first direct load goes out.
//
// Workgroup b takes column group b % R and band b / R (R = ceil(N / 128)):
// with R = 2 the XCDs (b mod 8) split into two sets of four, each reading
// one half of the weight rows through its own L2.  Rows past M and columns
// past N are clamped for the loads and dropped at the stores.

#include "dma.hpp"
#include "launch.hpp"
#include "rotate.hpp"

namespace convrot {
namespace {

constexpr int kNRows = 8;                          // activation rows per workgroup
constexpr int kNWaves = 8;                         // 32 segments of 16 lanes
constexpr int kNSegs = 4 * kNWaves;
constexpr int kNCols = 128;                        // weight rows (output columns) per workgroup
constexpr int kSliceBytes = kNCols * kGroup;       // 32 KiB: one 256-byte K slice of the 128 rows
constexpr int kNMaxG = 4;                          // K <= 1024

// LDS map: F ring stages, the rotation slots (S - F more stages once the
// rotation is done, stage s at s * 32 KiB), the codes (8 rows of up to
// 1024 bytes), S = 16 s_X and the row maxima of the band, the output
// staging tile (8 rows x 256 bytes, 16-byte chunks XOR-swizzled by row).
struct NarrowLayout {
  static constexpr int F = 2;
  static constexpr int S = F + 2;                  // ring stages
  static constexpr int kSlots = F * kSliceBytes;
  static constexpr int kSlotsEnd = kSlots + kNSegs * kSlotBytes;
  static constexpr int kCodes = kSlotsEnd;
  static constexpr int kSx = kCodes + kNRows * kNMaxG * kGroup;
  static constexpr int kMax = kSx + kNRows * 4;
  static constexpr int kStage = kMax + kNRows * 4;
  static constexpr int kBytes = kStage + kNRows * kNCols * 2;
  static_assert(kSlots + 2 * kSliceBytes <= kSlotsEnd, "two stages fit in the rotation slots");
  static_assert(kBytes <= 160 * 1024, "LDS");
  static_assert(kCodes % 16 == 0 && kStage % 16 == 0, "alignment");
};

// Wait until at most `groups` slice groups (4 direct loads each) are in flight.
__device__ __forceinline__ void wait_slices(int groups) {
  switch (groups) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<4>(); break;
    case 2: wait_vmcnt<8>(); break;
    default: wait_vmcnt<12>(); break;
  }
}

// G = K / 256 rotation groups per row (2 or 4); R column groups.
template <int G, bool kBias>
__global__ void __launch_bounds__(64 * kNWaves)
narrow_kernel(GemmArgs p, const __half* X, int64_t R) {
  using L = NarrowLayout;
  constexpr int S = L::S;
  constexpr int K = G * kGroup;
  constexpr int Q = (kNRows * G + kNSegs - 1) / kNSegs;   // rotation passes
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in a scalar register
  const int frow = lane & 15, fk = lane >> 4;
  const int64_t M = p.M, N = p.N;
  const int n0 = (int)((int64_t)blockIdx.x % R) * kNCols;
  const int64_t m0 = (int64_t)blockIdx.x / R * kNRows;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
  uint32_t* rowmax = reinterpret_cast<uint32_t*>(smem + L::kMax);
  float* sxs = reinterpret_cast<float*>(smem + L::kSx);
  if (tid < kNRows) rowmax[tid] = 0u;

  // Epilogue operands of this lane's columns n0 + 16 wave + 4 fk + r
  // (quads past N repeat the last one: N is a multiple of 4).
  const int qcol = min(n0 + 16 * wave + 4 * fk, (int)N - 4);
  const v4f sw = *reinterpret_cast<const v4f*>(p.sW + qcol);
  v4f bs = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (kBias) bs = *reinterpret_cast<const v4f*>(p.bias + qcol);

  // Direct loads of K slice t into stage t % S: this wavefront's blocks
  // 4 w .. 4 w + 3 (weight rows 4 b .. 4 b + 3 of the column group; lane l
  // fetches row 4 b + l / 16, chunk (l % 16) ^ (row & 15) of the slice).
  // Rows past N repeat the last one.
  const int lrow = 16 * wave + (lane >> 4);              // row of block u: lrow + 4 u
  const char* wsrc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int tr = lrow + 4 * u;
    const int n = min(n0 + tr, (int)N - 1);
    wsrc[u] = reinterpret_cast<const char*>(p.W) + ((int64_t)n * K + (((lane & 15) ^ (tr & 15)) << 4));
  }
  auto issue = [&](int t) {
    const uint32_t sb = lds_base + (uint32_t)((t % S) * kSliceBytes);
#pragma unroll
    for (int u = 0; u < 4; ++u) dma16(wsrc[u] + t * kGroup, sb + (uint32_t)((4 * wave + u) * 1024));
  };

  // 1-2. the band's groups, 32 at a time: segment `seg` takes group
  // gi = 32 q + seg (row gi / G, group gi % G; rows past M repeat the last).
  const int seg = tid >> 4, l16 = tid & 15;
  char* slot = smem + L::kSlots + seg * kSlotBytes;
  v4i xr[Q][2];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int gi = kNSegs * q + seg < kNRows * G ? kNSegs * q + seg : kNRows * G - 1;
    const int64_t m = m0 + gi / G < M ? m0 + gi / G : M - 1;
    const v4i* src = reinterpret_cast<const v4i*>(X + m * K + (gi % G) * kGroup + 16 * l16);
    xr[q][0] = __builtin_nontemporal_load(src);
    xr[q][1] = __builtin_nontemporal_load(src + 1);
  }
  asm volatile("" :: "v"(sw), "v"(bs));
#pragma unroll
  for (int q = 0; q < Q; ++q) asm volatile("" :: "v"(xr[q][0]), "v"(xr[q][1]));   // all loads landed
  lds_barrier();   // the row maxima are cleared
  float f[Q][16];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    // segments without a group (G = 2: wavefronts 4-7) skip the rotation;
    // every wavefront issues its direct loads
    const int gi = kNSegs * q + seg;
    const bool has = gi < kNRows * G;
    if (has) park_row(slot, l16, xr[q][0], xr[q][1]);
    if (q == 0) {
      compiler_fence();
#pragma unroll
      for (int t = 0; t < L::F; ++t)
        if (t < G) issue(t);
    }
    if (has) {
      double y[16];
      rotate_staged(slot, l16, y);
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        f[q][i] = (float)y[i];   // fp32(16 X_rot): the single rounding
        amax = fmaxf(amax, fabsf(f[q][i]));
      }
      const uint32_t amax_bits = seg_max16_bits(__float_as_uint(amax));
      if (l16 == 0) atomicMax(&rowmax[gi / G], amax_bits);
    }
  }
  lds_barrier();   // row maxima complete; the rotation slots are free
#pragma unroll
  for (int t = L::F; t < S; ++t)
    if (t < G) issue(t);
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int gi = kNSegs * q + seg;
    if (gi < kNRows * G) {
      const int j = gi / G, g = gi % G;
      // S = fp32(max |16 X_rot|) / 127 = 16 s_X exactly, and round(F / S)
      // equals round(X_rot / s_X) (power-of-two scaling commutes with the
      // fp32 roundings of normal values)
      const float sc = __uint_as_float(rowmax[j]) / 127.0f;
      if (g == 0 && l16 == 0) sxs[j] = sc * 0.0625f;
      *reinterpret_cast<uint4*>(smem + L::kCodes + j * K + g * kGroup + ((l16 ^ (j & 15)) << 4)) = quantize16(f[q], sc);
    }
  }

  // 3. one barrier per slice: it publishes slice t's blocks (and, at t = 0,
  // the codes and s_X), and every wavefront has finished slice t - 1, whose
  // stage is refilled next.
  const int wr = 16 * wave + frow;      // this lane's weight row (MFMA operand)
  const int cr = frow & (kNRows - 1);   // this lane's band row (rows 8-15 repeat 0-7: dropped)
  v4i acc = v4i{0, 0, 0, 0};
#pragma unroll
  for (int t = 0; t < G; ++t) {
    // slice groups issued after slice t: t + 1 .. min(G - 1, S - 1) at t = 0,
    // t + 1 .. min(G - 1, t + S - 2) later
    const int after = t == 0 ? (G - 1 < S - 1 ? G - 1 : S - 1) : (G - 1 - t < S - 2 ? G - 1 - t : S - 2);
    wait_slices(after);
    lds_barrier();
    if (t >= 1 && t + S - 1 < G) issue(t + S - 1);   // into the stage slice t - 1 used
    const char* ws = smem + (t % S) * kSliceBytes;
    const char* cs = smem + L::kCodes + cr * K + t * kGroup;
    v4i wa[4], fa[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      wa[s] = *reinterpret_cast<const v4i*>(ws + wr * kGroup + (((4 * s + fk) ^ (wr & 15)) << 4));
      fa[s] = *reinterpret_cast<const v4i*>(cs + (((4 * s + fk) ^ cr) << 4));
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[s], fa[s], acc, 0, 0, 0);
  }

  // 4. lane holds A[m][n] for m = m0 + frow, n = n0 + 16 wave + 4 fk + r
  // (valid for frow < 8): 8 bytes at staging row frow, chunk 2 wave + fk / 2
  // (swizzled), half fk & 1.
  char* sbw = smem + L::kStage;
  if (frow < kNRows) {
    const float sx = sxs[frow];
    float y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      y[r] = __fmul_rn((float)acc[r], __fmul_rn(sx, sw[r]));
      if constexpr (kBias) y[r] = __fadd_rn(y[r], bs[r]);
    }
    uint2 v;
    v.x = pack_f16x2_rn(y[0], y[1]);
    v.y = pack_f16x2_rn(y[2], y[3]);
    *reinterpret_cast<uint2*>(sbw + frow * (2 * kNCols) + (((2 * wave + (fk >> 1)) ^ frow) << 4) + 8 * (fk & 1)) = v;
  }
  lds_barrier();
  // 8 rows x 16 pieces of 16 bytes, one per thread of the first 128
  if (tid < kNRows * 16) {
    const int rl = tid >> 4, pc = tid & 15;
    const int64_t m = m0 + rl, n = n0 + 8 * pc;
    if (m < M && n < N) {
      v4i v = *reinterpret_cast<const v4i*>(sbw + rl * (2 * kNCols) + ((pc ^ rl) << 4));
      __half* Y = reinterpret_cast<__half*>(p.out);
      __half* dst = Y + m * N + n;
      if ((N % 8) == 0 && n + 8 <= N) {
        if (p.R) v = add_f16x8(v, *reinterpret_cast<const v4i*>(p.R + m * N + n));
        __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(dst));
      } else {
        // N is a multiple of 4: rows start 8-byte aligned, and each 4-column
        // half of the piece is in range or wholly past N
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (n + 4 * h >= N) break;
          uint2 o = h == 0 ? make_uint2(v.x, v.y) : make_uint2(v.z, v.w);
          if (p.R) {
            const uint2 rr = *reinterpret_cast<const uint2*>(p.R + m * N + n + 4 * h);
            const __half* a = reinterpret_cast<const __half*>(&o);
            const __half* b = reinterpret_cast<const __half*>(&rr);
            __half z[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) z[e] = __float2half_rn(__half2float(a[e]) + __half2float(b[e]));
            o = *reinterpret_cast<const uint2*>(z);
          }
          *reinterpret_cast<uint2*>(dst + 4 * h) = o;
        }
      }
    }
  }
}

template <int G, bool kBias>
hipError_t launch_g(const GemmArgs& a, const void* X, hipStream_t stream) {
  auto fn = &narrow_kernel<G, kBias>;
  constexpr int lds = NarrowLayout::kBytes;
  if (const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(fn), lds); e != hipSuccess) return e;
  const int64_t R = (a.N + kNCols - 1) / kNCols;
  const int64_t bands = (a.M + kNRows - 1) / kNRows;
  hipLaunchKernelGGL(fn, dim3((unsigned)(bands * R)), dim3(64 * kNWaves), lds, stream, a,
                     reinterpret_cast<const __half*>(X), R);
  return hipGetLastError();
}

template <int G>
hipError_t launch_gb(const GemmArgs& a, const void* X, hipStream_t stream) {
  return a.bias ? launch_g<G, true>(a, X, stream) : launch_g<G, false>(a, X, stream);
}

}  // namespace

bool narrow_fusable(int64_t M, int64_t N, int64_t K) {
  if (!(K == 512 || K == 1024) || M <= 16 || N < 4 || N > 2 * kNCols || N % 4 != 0) return false;
  return ((M + kNRows - 1) / kNRows) * ((N + kNCols - 1) / kNCols) <= 256;
}

hipError_t launch_narrow(const GemmArgs& a, const void* X, hipStream_t stream) {
  if (!narrow_fusable(a.M, a.N, a.K)) return hipErrorInvalidValue;
  return a.K == 512 ? launch_gb<2>(a, X, stream) : launch_gb<4>(a, X, stream);
}

}  // namespace convrot
