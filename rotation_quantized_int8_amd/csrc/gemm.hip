// MFMA GEMMs of the INT8ConvRot linear ("TN": both operands K-contiguous).
//
// Page "INT8ConvRot GEMM vs fp16 on M1 Max with Metal, MPSMatrix, and MLX
// (fp16 Wins)", section "What changed in the computation":
//   A = Q_X Q_W^T (int32),  Y = A (.) s_X s_W^T            -> kI8 modes
//   weight-only: x_rot fp16 times int8 weight and scale     -> kW8A16
//   and the plain fp16 product of the six-shape table        -> kF16
// plus the unmerged LoRA of page "[PR #249] Add an mps backend ...",
// sections "What" and "Design" (W8A16 only).
//
// One kernel template.  A workgroup of 256 threads (2x2 wavefronts) owns a
// BM x BN output tile and walks K in 128-byte slices (128 int8 or 64 fp16
// values per row), double-buffered in LDS through registers.  LDS rows are
// 128 bytes with their 16-byte chunks XOR-swizzled by (row & 7), which keeps
// both the staging writes and the MFMA operand reads free of bank conflicts.
// The weight tile is the MFMA "A" operand and the activation tile the "B"
// operand, so each lane's 4 accumulators are 4 consecutive output columns of
// one output row: the epilogue stores 8 (fp16) or 16 (int32) contiguous bytes.
//
// Instructions: v_mfma_i32_16x16x64_i8 (int8) and v_mfma_f32_16x16x32_f16.
// Lane l supplies operand row (l % 16) and the 16-byte K chunk (l / 16) of a
// 64-byte K step; result register r of lane l is output (4*(l/16) + r, l%16)
// in (A-row, B-row) coordinates.

#include <type_traits>

#include "launch.hpp"

namespace convrot {

namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;  // bytes of one K slice per tile row

template <GemmMode MODE>
struct Traits;
template <>
struct Traits<GemmMode::kI8toI32> {
  static constexpr int kXElem = 1, kWElem = 1;
};
template <>
struct Traits<GemmMode::kI8toF16> {
  static constexpr int kXElem = 1, kWElem = 1;
};
template <>
struct Traits<GemmMode::kF16> {
  static constexpr int kXElem = 2, kWElem = 2;
};
template <>
struct Traits<GemmMode::kW8A16> {
  static constexpr int kXElem = 2, kWElem = 1;  // int8 in HBM, fp16 in LDS
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 7)) << 4); }

// int8 x16 -> fp16 x16 (exact: |q| <= 128).
__device__ __forceinline__ void decode_i8x16(const uint4 q, uint4& lo, uint4& hi) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  uint32_t o[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int8_t b0 = (int8_t)((w[j] >> (16 * p)) & 0xff);
      const int8_t b1 = (int8_t)((w[j] >> (16 * p + 8)) & 0xff);
      const __half h0 = __int2half_rn((int)b0);
      const __half h1 = __int2half_rn((int)b1);
      o[2 * j + p] = (uint32_t)__half_as_ushort(h0) | ((uint32_t)__half_as_ushort(h1) << 16);
    }
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

template <GemmMode MODE, int BM, int BN>
__global__ void __launch_bounds__(kThreads)
gemm_kernel(GemmArgs p) {
  constexpr bool kInt = (MODE == GemmMode::kI8toI32 || MODE == GemmMode::kI8toF16);
  constexpr int WM = BM / 2, WN = BN / 2;        // wave tile (m, n)
  constexpr int FM = WM / 16, FN = WN / 16;       // 16x16 fragments per wave
  constexpr int XCH = BM * 8 / kThreads;          // 16-byte chunks per thread (X tile)
  constexpr int WCH = BN * 8 / kThreads;          // (W tile, in LDS bytes)
  static_assert(XCH >= 1 && WCH >= 1, "tile too small");
  constexpr int kTileBytes = (BM + BN) * kRowBytes;

  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int64_t tiles_n = (p.N + BN - 1) / BN;
  const int64_t tile_m = blockIdx.x / tiles_n;
  const int64_t tile_n = blockIdx.x - tile_m * tiles_n;
  const int64_t m0 = tile_m * BM, n0 = tile_n * BN;
  const int64_t M = p.M, N = p.N, K = p.K;

  const char* Xb = reinterpret_cast<const char*>(p.X);
  const char* Wb = reinterpret_cast<const char*>(p.W);
  const int64_t x_ld = K * Traits<MODE>::kXElem;   // bytes per row
  const int64_t w_ld = K * Traits<MODE>::kWElem;
  const int64_t nk = x_ld / kRowBytes;              // K slices (K % 256 == 0)

  // staging registers
  uint4 xr[XCH];
  uint4 wr[WCH];
  constexpr int kWLoad = (MODE == GemmMode::kW8A16) ? (WCH + 1) / 2 : WCH;  // 16-byte global loads

  auto load_tile = [&](int64_t kt) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid * XCH + i;
      const int r = c >> 3, ch = c & 7;
      const int64_t gm = m0 + r;
      xr[i] = make_uint4(0, 0, 0, 0);
      if (gm < M) xr[i] = *reinterpret_cast<const uint4*>(Xb + gm * x_ld + kt * kRowBytes + ch * 16);
    }
    if constexpr (MODE == GemmMode::kW8A16) {
      // 64 int8 per row per slice: 4 chunks of 16 values; each expands to 2 LDS chunks
#pragma unroll
      for (int i = 0; i < kWLoad; ++i) {
        const int c = tid * kWLoad + i;
        const int r = c >> 2, ch = c & 3;
        const int64_t gn = n0 + r;
        uint4 q = make_uint4(0, 0, 0, 0);
        if (r < BN && gn < N) q = *reinterpret_cast<const uint4*>(Wb + gn * w_ld + kt * (kRowBytes / 2) + ch * 16);
        decode_i8x16(q, wr[2 * i], wr[2 * i + 1]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < WCH; ++i) {
        const int c = tid * WCH + i;
        const int r = c >> 3, ch = c & 7;
        const int64_t gn = n0 + r;
        wr[i] = make_uint4(0, 0, 0, 0);
        if (gn < N) wr[i] = *reinterpret_cast<const uint4*>(Wb + gn * w_ld + kt * kRowBytes + ch * 16);
      }
    }
  };

  auto store_tile = [&](int buf) {
    char* xs = smem + buf * kTileBytes;
    char* ws = xs + BM * kRowBytes;
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid * XCH + i;
      *reinterpret_cast<uint4*>(xs + swz(c >> 3, c & 7)) = xr[i];
    }
    if constexpr (MODE == GemmMode::kW8A16) {
#pragma unroll
      for (int i = 0; i < kWLoad; ++i) {
        const int c = tid * kWLoad + i;
        const int r = c >> 2, ch = c & 3;
        if (r < BN) {
          *reinterpret_cast<uint4*>(ws + swz(r, 2 * ch)) = wr[2 * i];
          *reinterpret_cast<uint4*>(ws + swz(r, 2 * ch + 1)) = wr[2 * i + 1];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < WCH; ++i) {
        const int c = tid * WCH + i;
        *reinterpret_cast<uint4*>(ws + swz(c >> 3, c & 7)) = wr[i];
      }
    }
  };

  using Acc = typename std::conditional<kInt, v4i, v4f>::type;
  Acc acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = Acc{0, 0, 0, 0};

  const int frow = lane & 15;   // operand row within a fragment
  const int fk = lane >> 4;     // 16-byte K chunk within a 64-byte step

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    if (kt + 1 < nk) load_tile(kt + 1);
    const char* xs = smem + buf * kTileBytes;
    const char* ws = xs + BM * kRowBytes;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint4 af[FN], bf[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i)
        af[i] = *reinterpret_cast<const uint4*>(ws + swz(wn * WN + i * 16 + frow, kk * 4 + fk));
#pragma unroll
      for (int j = 0; j < FM; ++j)
        bf[j] = *reinterpret_cast<const uint4*>(xs + swz(wm * WM + j * 16 + frow, kk * 4 + fk));
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          if constexpr (kInt) {
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                *reinterpret_cast<const v4i*>(&af[i]), *reinterpret_cast<const v4i*>(&bf[j]),
                acc[i][j], 0, 0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                *reinterpret_cast<const v8h*>(&af[i]), *reinterpret_cast<const v8h*>(&bf[j]),
                acc[i][j], 0, 0, 0);
          }
        }
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  const int orow = lane & 15;        // output row (m) within a fragment
  const int ocol = (lane >> 4) * 4;  // first of 4 output columns (n) within a fragment

  if constexpr (MODE == GemmMode::kW8A16) {
    // scale by s_W, then the LoRA product T U'^T as extra K steps on the MFMA
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int64_t nb = n0 + wn * WN + i * 16 + ocol;
      float sw[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sw[r] = (nb + r < N) ? p.sW[nb + r] : 0.0f;
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] *= sw[r];
    }
    if (p.rank > 0) {
      for (int r0 = 0; r0 < p.t_ld; r0 += 32) {
        // A operand: U'[n][r0 + 8*fk .. +7] = fp16(scale * U), B operand: T[m][same]
        v8h ua[FN], tb[FM];
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const int64_t n = n0 + wn * WN + i * 16 + frow;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int rr = r0 + 8 * fk + e;
            float u = 0.0f;
            if (n < N && rr < p.rank) u = p.U[n * p.rank + rr] * p.lora_scale;
            ua[i][e] = (_Float16)u;
          }
        }
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          const int64_t m = m0 + wm * WM + j * 16 + frow;
          uint4 t = make_uint4(0, 0, 0, 0);
          if (m < M) t = *reinterpret_cast<const uint4*>(p.T + m * p.t_ld + r0 + 8 * fk);
          tb[j] = *reinterpret_cast<const v8h*>(&t);
        }
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
          for (int j = 0; j < FM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ua[i], tb[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  const bool vec_ok = (N % 4) == 0;
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int64_t nb = n0 + wn * WN + i * 16 + ocol;
    float sw[4] = {0.f, 0.f, 0.f, 0.f}, bs[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (MODE == GemmMode::kI8toF16) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sw[r] = (nb + r < N) ? p.sW[nb + r] : 0.0f;
    }
    if constexpr (MODE == GemmMode::kI8toF16 || MODE == GemmMode::kW8A16) {
      if (p.bias) {
#pragma unroll
        for (int r = 0; r < 4; ++r) bs[r] = (nb + r < N) ? p.bias[nb + r] : 0.0f;
      }
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int64_t m = m0 + wm * WM + j * 16 + orow;
      if (m >= M) continue;
      if constexpr (MODE == GemmMode::kI8toI32) {
        int32_t* o = reinterpret_cast<int32_t*>(p.out) + m * N + nb;
        if (vec_ok && nb + 3 < N) {
          *reinterpret_cast<v4i*>(o) = acc[i][j];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (nb + r < N) o[r] = acc[i][j][r];
        }
      } else {
        __half h[4];
        if constexpr (MODE == GemmMode::kI8toF16) {
          const float sx = p.sX[m];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // Y = fp16( fp32(A) * fp32(s_X * s_W) [+ bias] ), no contraction
            const float sc = __fmul_rn(sx, sw[r]);
            float y = __fmul_rn((float)acc[i][j][r], sc);
            if (p.bias) y = __fadd_rn(y, bs[r]);
            h[r] = __float2half_rn(y);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float y = acc[i][j][r];
            if (MODE == GemmMode::kW8A16 && p.bias) y = __fadd_rn(y, bs[r]);
            h[r] = __float2half_rn(y);
          }
        }
        __half* o = reinterpret_cast<__half*>(p.out) + m * N + nb;
        if (vec_ok && nb + 3 < N) {
          uint2 v;
          v.x = (uint32_t)__half_as_ushort(h[0]) | ((uint32_t)__half_as_ushort(h[1]) << 16);
          v.y = (uint32_t)__half_as_ushort(h[2]) | ((uint32_t)__half_as_ushort(h[3]) << 16);
          *reinterpret_cast<uint2*>(o) = v;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (nb + r < N) o[r] = h[r];
        }
      }
    }
  }
}

template <GemmMode MODE, int BM, int BN>
hipError_t launch_tile(const GemmArgs& a, hipStream_t stream) {
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const size_t lds = 2 * (size_t)(BM + BN) * kRowBytes;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<MODE, BM, BN>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((gemm_kernel<MODE, BM, BN>), dim3((unsigned)tiles), dim3(kThreads), lds,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

// Tile choice for the direct-to-LDS kernel.  256x128 tiles read half the
// operand bytes per output of 128x64 tiles, which pays once they still give
// most of the 256 CUs a tile; otherwise 128x64 tiles spread the work wider.
int choose_gemm_cfg(GemmMode mode, int64_t M, int64_t N, int64_t K) {
  (void)mode; (void)K;
  const int64_t big = ((M + 255) / 256) * ((N + 127) / 128);
  return big >= 160 ? 2 : 8;
}

template <GemmMode MODE>
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  if constexpr (MODE == GemmMode::kW8A16) {
    return launch_tile<MODE, 128, 128>(a, stream);
  } else {
    return launch_gemm_dma_cfg<MODE>(a, choose_gemm_cfg(MODE, a.M, a.N, a.K), stream);
  }
}

template hipError_t launch_gemm<GemmMode::kI8toI32>(const GemmArgs&, hipStream_t);
template hipError_t launch_gemm<GemmMode::kI8toF16>(const GemmArgs&, hipStream_t);
template hipError_t launch_gemm<GemmMode::kF16>(const GemmArgs&, hipStream_t);
template hipError_t launch_gemm<GemmMode::kW8A16>(const GemmArgs&, hipStream_t);

}  // namespace convrot
