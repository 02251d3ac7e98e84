// W8A8 product for few activation rows (M <= 16): the weight-streaming
// regime of the row-count sweep on the page "INT8ConvRot GEMM vs fp16 on M1
// Max with Metal, MPSMatrix, and MLX (fp16 Wins)" (section "What changed in
// the computation": A = Q_X Q_W^T in int32, Y = A (.) s_X s_W^T).
//
// With M <= 16 the int8 weights are almost all of the traffic (N K bytes
// against M K activation bytes), so the kernel is organised around streaming
// them: a workgroup of W wavefronts owns 16 weight rows and a K range, each
// wavefront a contiguous 1/W of that range (W grows with K so that a
// wavefront has about 8 steps of 64 K bytes).  A wavefront's loads go
// straight into registers in the MFMA operand layout (lane l: weight row
// l % 16, 16 consecutive K bytes at 16 (l / 16) within each 64-byte step) in
// batches of 8 steps, the next batch in flight while the current one is
// multiplied; with all of a workgroup's weight bytes requested at once there
// is a single dependent memory round trip for most shapes.
// v_mfma_i32_16x16x64_i8 accumulates 16 weight rows x 16 activation rows; the
// wavefronts' int32 sums are added through LDS in wavefront order (exact).
//
// Activations.  Unfused, Q_X comes from global memory (the prologue kernel
// wrote it) through the same register path.  Fused (M <= 16, M K <= 8192): every
// workgroup quantises the few activation rows itself, with the same device
// functions and arithmetic as the prologue kernel (exact fp64 rotation, row
// maximum, IEEE division by 127, round-half-even), into LDS, so the whole
// layer is one launch.  The activation loads are issued before the weight
// loads and the rotation runs while the weights are in flight.
//
// With one K range the workgroup applies the scale epilogue (fp32(A) *
// fp32(s_X s_W) [+ bias], fp16, [+ residual as one fp16 addition]) itself;
// otherwise it writes int32 partial sums [splits, M, N] for the K-split
// epilogue kernel.  The result is bit-identical either way.

#include "launch.hpp"
#include "rotate.hpp"

namespace convrot {
namespace {

constexpr int kBatch = 8;        // 64-byte K steps per load batch
constexpr int kSeg = 16;         // 16-lane segments that run the fused prologue (waves 0-3)
constexpr int kFusedJobs = 32;   // at most M * K / 256 rotation groups when fused
constexpr int kFusedBytes = kFusedJobs * kGroup;

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier that does not wait for outstanding global loads (the
// weight batch in flight); LDS traffic is ordered by lgkmcnt(0) before it.
__device__ __forceinline__ void lds_barrier() {
  wait_lgkm0();
  compiler_fence();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// CB activation column blocks of 16 rows, W wavefronts; with 16 wavefronts
// (4 per SIMD, at most 128 registers each) one register buffer of loads.
template <int CB, int W, bool FUSED>
__global__ void __launch_bounds__(64 * W)
skinny_kernel(GemmArgs p, const __half* __restrict__ Xf, int64_t kr, int rpb, int32_t* __restrict__ parts) {
  __shared__ v4i red[W - 1][CB][64];
  __shared__ __align__(16) char slots[FUSED ? kSeg * kSlotBytes : 16];
  __shared__ __align__(16) int8_t qx[FUSED ? kFusedBytes : 16];
  __shared__ float jmax[FUSED ? kFusedJobs : 1];
  __shared__ float srow[FUSED ? 16 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int frow = lane & 15, fk = lane >> 4;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t n0 = (int64_t)blockIdx.x * rpb;      // rpb = 16 or 8 weight rows per workgroup
  const int64_t z = blockIdx.y;
  const int64_t kw = kr / W;                          // K bytes of this wavefront (multiple of 64)
  const int64_t kbeg = z * kr + wave * kw;
  const int steps = (int)(kw / 64);

  // Fused prologue, part 1: the activation loads of this segment's groups
  // (job j = m G + g: group g of row m), before any weight load.
  const int G = (int)(K / kGroup);
  const int seg = tid >> 4, l16 = tid & 15;
  v4i xr[2][2];
  if constexpr (FUSED) {
    if (wave < 4) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int j = seg + kSeg * t;
        if (j < M * G) {
          const int m = j / G, g = j - m * G;
          const v4i* src = reinterpret_cast<const v4i*>(Xf + (int64_t)m * K + (int64_t)g * kGroup + 16 * l16);
          xr[t][0] = __builtin_nontemporal_load(src);
          xr[t][1] = __builtin_nontemporal_load(src + 1);
        }
      }
    }
  }

  // with 8 rows per workgroup, MFMA rows 8-15 repeat rows 0-7 (same
  // addresses in the same load, so no extra traffic) and are not stored
  int64_t wrow = n0 + (frow & (rpb - 1));
  wrow = wrow < N ? wrow : N - 1;
  const int8_t* wp = reinterpret_cast<const int8_t*>(p.W) + wrow * K + kbeg + 16 * fk;
  const int8_t* xp[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    int64_t xrow = 16 * c + frow;
    xrow = xrow < M ? xrow : M - 1;
    xp[c] = FUSED ? reinterpret_cast<const int8_t*>(qx) + xrow * K + kbeg + 16 * fk
                  : reinterpret_cast<const int8_t*>(p.X) + xrow * K + kbeg + 16 * fk;
  }

  v4i acc[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) acc[c] = v4i{0, 0, 0, 0};
  constexpr int NBUF = W >= 16 ? 1 : 2;
  v4i wa[NBUF][kBatch], xb[NBUF][CB][kBatch];
  auto load_w = [&](int buf, int s0) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int s = s0 + j < steps ? s0 + j : steps - 1;   // tail: repeat the last step, unused
      wa[buf][j] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wp + 64 * s));
    }
  };
  auto load_x = [&](int buf, int s0) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int s = s0 + j < steps ? s0 + j : steps - 1;
#pragma unroll
      for (int c = 0; c < CB; ++c) xb[buf][c][j] = *reinterpret_cast<const v4i*>(xp[c] + 64 * s);
    }
  };
  auto mma = [&](int buf, int s0) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (s0 + j < steps) {
#pragma unroll
        for (int c = 0; c < CB; ++c)
          acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[buf][j], xb[buf][c][j], acc[c], 0, 0, 0);
      }
    }
  };

  load_w(0, 0);
  if constexpr (!FUSED) load_x(0, 0);

  if constexpr (FUSED) {
    // part 2: rotate (exact), per-group maximum, row maximum over the groups
    // of the row, s = max / 127, quantise into LDS
    float f[2][16];
    if (wave < 4) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int j = seg + kSeg * t;
        if (j < M * G) {
          double y[16];
          rotate_loaded(xr[t][0], xr[t][1], slots + seg * kSlotBytes, l16, y);
          float amax = 0.0f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            f[t][i] = (float)y[i];   // fp32(16 X_rot): the single rounding
            amax = fmaxf(amax, fabsf(f[t][i]));
          }
          amax = __uint_as_float(seg_max16_bits(__float_as_uint(amax)));
          if (l16 == 0) jmax[j] = amax;
        }
      }
    }
    lds_barrier();
    if (wave < 4) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int j = seg + kSeg * t;
        if (j < M * G) {
          const int m = j / G, g = j - m * G;
          float rmax = 0.0f;
          for (int q = 0; q < G; ++q) rmax = fmaxf(rmax, jmax[m * G + q]);
          // S = fp32(max|16 X_rot|) / 127 = 16 s_X exactly (power-of-two
          // scaling commutes with the fp32 roundings of normal values) and
          // the codes round(F / S) equal round(X_rot / s_X)
          const float s = rmax / 127.0f;                    // IEEE fp32 division
          if (g == 0 && l16 == 0) srow[m] = s * 0.0625f;    // s_X, exact
          *reinterpret_cast<uint4*>(qx + (int64_t)m * K + (int64_t)g * kGroup + 16 * l16) = quantize16(f[t], s);
        }
      }
    }
    lds_barrier();
    load_x(0, 0);
  }

  if constexpr (NBUF == 2) {
    // two register buffers, alternating with compile-time indices
    for (int s0 = 0; s0 < steps; s0 += 2 * kBatch) {
      if (s0 + kBatch < steps) {
        load_w(1, s0 + kBatch);
        load_x(1, s0 + kBatch);
      }
      mma(0, s0);
      if (s0 + kBatch < steps) {
        if (s0 + 2 * kBatch < steps) {
          load_w(0, s0 + 2 * kBatch);
          load_x(0, s0 + 2 * kBatch);
        }
        mma(1, s0 + kBatch);
      }
    }
  } else {
    for (int s0 = 0; s0 < steps; s0 += kBatch) {
      if (s0 > 0) {
        load_w(0, s0);
        load_x(0, s0);
      }
      mma(0, s0);
    }
  }

  // add the wavefronts' sums (exact int32) in wavefront order
  if (wave > 0) {
#pragma unroll
    for (int c = 0; c < CB; ++c) red[wave - 1][c][lane] = acc[c];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < W - 1; ++w)
#pragma unroll
    for (int c = 0; c < CB; ++c) acc[c] += red[w][c][lane];

  // lane holds A[m][n] for n = n0 + 4 fk + i (i = 0..3), m = 16 c + frow
  if (4 * fk >= rpb) return;
  const int64_t nb = n0 + 4 * fk;
  const bool vec = (N % 4) == 0 && nb + 4 <= N;
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    const int64_t m = 16 * c + frow;
    if (m >= M) continue;
    if (gridDim.y > 1 || parts) {
      int32_t* dst = parts + (z * M + m) * N + nb;
      if (vec) {
        *reinterpret_cast<v4i*>(dst) = acc[c];
      } else {
        for (int i = 0; i < 4; ++i)
          if (nb + i < N) dst[i] = acc[c][i];
      }
      continue;
    }
    const float sx = FUSED ? srow[m] : p.sX[m];
    __half h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t n = nb + i < N ? nb + i : N - 1;
      float y = __fmul_rn((float)acc[c][i], __fmul_rn(sx, p.sW[n]));
      if (p.bias) y = __fadd_rn(y, p.bias[n]);
      h[i] = __float2half_rn(as_fp32(y));
      if (p.R) h[i] = __float2half_rn(__half2float(h[i]) + __half2float(p.R[m * N + n]));
    }
    __half* Y = reinterpret_cast<__half*>(p.out) + m * N + nb;
    if (vec) {
      uint2 o;
      o.x = (uint32_t)__half_as_ushort(h[0]) | ((uint32_t)__half_as_ushort(h[1]) << 16);
      o.y = (uint32_t)__half_as_ushort(h[2]) | ((uint32_t)__half_as_ushort(h[3]) << 16);
      *reinterpret_cast<uint2*>(Y) = o;
    } else {
      for (int i = 0; i < 4; ++i)
        if (nb + i < N) Y[i] = h[i];
    }
  }
}

// wavefronts per workgroup for a K range: about 8 steps of 64 bytes each
int waves_for(int64_t kr) {
  if (kr % 1024 == 0 && kr >= 8192) return 16;
  if (kr % 512 == 0 && kr >= 4096) return 8;
  return 4;
}

// 16 weight rows per workgroup, or 8 when 16-row blocks would leave CUs idle
int rows_per_block(int64_t N, int64_t splits) { return (N + 15) / 16 * splits < 256 ? 8 : 16; }

template <int CB, bool FUSED>
hipError_t launch_w(const GemmArgs& a, const __half* Xf, int64_t splits, int32_t* parts, hipStream_t stream) {
  const int rpb = rows_per_block(a.N, splits);
  const dim3 grid((unsigned)((a.N + rpb - 1) / rpb), (unsigned)splits);
  const int64_t kr = a.K / splits;
  switch (waves_for(kr)) {
    case 16: hipLaunchKernelGGL((skinny_kernel<CB, 16, FUSED>), grid, dim3(1024), 0, stream, a, Xf, kr, rpb, parts); break;
    case 8: hipLaunchKernelGGL((skinny_kernel<CB, 8, FUSED>), grid, dim3(512), 0, stream, a, Xf, kr, rpb, parts); break;
    default: hipLaunchKernelGGL((skinny_kernel<CB, 4, FUSED>), grid, dim3(256), 0, stream, a, Xf, kr, rpb, parts); break;
  }
  return hipGetLastError();
}

}  // namespace

bool skinny_fusable(int64_t M, int64_t K) { return M >= 1 && M <= 16 && M * (K / kGroup) <= kFusedJobs; }

// K ranges for the unfused few-row kernel: split only while the 8-row
// blocks cover fewer than 128 CUs and a workgroup would still stream more
// than 64 KiB of weight and activation bytes (below that the split's second
// launch costs more than it saves), each range a multiple of 256 K values
// and at least 1024 long.
int64_t skinny_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t blocks = (N + 7) / 8;
  int64_t s = 1;
  while (blocks * s < 128 && K % (s * 2 * 256) == 0 && K / (s * 2) >= 1024 && (8 + M) * (K / s) > 65536) s *= 2;
  return s;
}

hipError_t launch_skinny(const GemmArgs& a, int64_t splits, int32_t* parts, hipStream_t stream) {
  if (a.M > 16 || a.K % (splits * 256) != 0 || (splits > 1 && !parts)) return hipErrorInvalidValue;
  return launch_w<1, false>(a, nullptr, splits, parts, stream);
}

hipError_t launch_skinny_fused(const GemmArgs& a, const void* X, hipStream_t stream) {
  if (!skinny_fusable(a.M, a.K)) return hipErrorInvalidValue;
  return launch_w<1, true>(a, reinterpret_cast<const __half*>(X), 1, nullptr, stream);
}

}  // namespace convrot
