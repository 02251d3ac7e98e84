// The W8A8 layer in one launch when every activation row is a single
// rotation group (K = 256): page "INT8ConvRot GEMM vs fp16 on M1 Max with
// Metal, MPSMatrix, and MLX (fp16 Wins)", section "What changed in the
// computation" (X_rot = X H, s_X = max |X_rot| / 127, Q_X = round(X_rot /
// s_X), A = Q_X Q_W^T in int32, Y = A (.) s_X s_W^T).
//
// With K = 256 a row's quantisation needs only that row, so a workgroup can
// quantise the rows it multiplies itself: the layer needs no second launch
// and no Q_X round trip through memory.  A workgroup (8 wavefronts) owns a
// band of 32 activation rows (16 when M <= 128) and a group of 128-column
// weight tiles; the column groups of a band each quantise the band again, so
// the grid is sized to about one workgroup per CU (bands x groups ~ 256) and
// a group is as wide as that allows (the repeated rotation is a fixed ~2.6 k
// vector cycles per workgroup, while narrower groups would re-read more
// weight bytes).
//
// Per workgroup (BR = 32 rows; with 16, segments 16-31 skip steps 1-2):
//   1. every lane loads its part of the band (16-lane segments, one row
//      each) and parks it in its segment's LDS slot; then the direct
//      global->LDS loads of weight tiles 0 and 1 go out (each tile 128 rows
//      x 256 bytes in 1 KiB blocks, 16-byte chunks XOR-swizzled by row & 15;
//      with the tile's 128 weight scales and biases in one more block), so
//      the weights stream in while the rows rotate;
//   2. the segments rotate their rows (exact fp64, rotate.hpp), take the row
//      maximum, s = max / 127 (IEEE fp32 division), s_X = s / 16, and write
//      the codes to LDS -- the same functions and arithmetic as the
//      stand-alone prologue;
//   3. after a barrier the rotation slots become two more ring stages (tiles
//      2 and 3 go out); every wavefront reads the band's codes as MFMA
//      operands once;
//   4. per tile: wait for its blocks, one barrier, refill the stage freed
//      by the previous tile, store the previous tile's output (whole 256-byte
//      rows as 16-byte stores [+ the residual, one fp16 addition]), then
//      (BR / 16) x 4 v_mfma_i32_16x16x64_i8 per wavefront (its 16 columns x
//      BR rows) and the scale epilogue (fp32(A) * fp32(s_X s_W) [+ bias],
//      fp16) into one of two LDS staging tiles.
//
// The direct loads are inline assembly (the compiler does not count them),
// so the kernel waits for them with explicit vmcnt values: a wavefront's
// loads of one tile form a group (4 weight blocks, plus the scale block for
// wavefront 0) and the groups go out in tile order; waiting for "at most k
// groups in flight" also covers the output stores issued in between, which
// only makes a wait longer, never shorter.  The activation loads complete
// (the parking store waits for them) before the first direct load is
// issued.
//
// Workgroup b takes column group b % groups and band b / groups, so with 8
// groups (M = 1024) the workgroups on one XCD (dispatched round-robin) all
// read the same weight rows through that XCD's L2.  Rows past M and columns
// past N are clamped for the loads and dropped at the stores.

#include "dma.hpp"
#include "launch.hpp"
#include "rotate.hpp"

namespace convrot {
namespace {

constexpr int kBandRows = 32;                      // activation rows per workgroup
constexpr int kWaves = 8;                          // 32 segments of 16 lanes
constexpr int kSegs = 4 * kWaves;
constexpr int kTileN = 128;                        // weight rows (output columns) per tile
constexpr int kTileBytes = kTileN * kGroup;        // 32 KiB
constexpr int kStageRow = 2 * kTileN;              // staged output row bytes (fp16)

// LDS map of a band of BR rows: F ring stages, then the rotation slots (two
// more stages once the rotation is done, so stage s sits at s * 32 KiB), the
// codes, s_X, two output staging tiles (16-byte chunks XOR-swizzled by
// row & 15) and the scale blocks of the stages.  Bands of 32 rows leave room
// for F = 2.  (64-row bands, which halve the weight bytes per output but
// double the rotation per workgroup and leave room for one stage during it,
// measured slower at M <= 1024 and within 2 % at M = 2048.)
template <int BR>
struct BandLayout {
  static constexpr int F = 2;
  static constexpr int S = F + 2;                  // ring stages
  static constexpr int kSlots = F * kTileBytes;
  static constexpr int kSlotsEnd = kSlots + kSegs * kSlotBytes;
  static constexpr int kCodes = kSlotsEnd;
  static constexpr int kSx = kCodes + BR * kGroup;
  static constexpr int kStage = kSx + BR * 4;
  static constexpr int kScales = kStage + 2 * BR * kStageRow;
  static constexpr int kBytes = kScales + S * 1024;
  static_assert(kSlots + 2 * kTileBytes <= kSlotsEnd, "two stages fit in the rotation slots");
  static_assert(kBytes <= 160 * 1024, "LDS");
  static_assert(kStage % 16 == 0 && kScales % 16 == 0 && kCodes % 16 == 0, "alignment");
};

// Wait until at most `groups` load groups of 4 (or 5) loads are in flight.
__device__ __forceinline__ void wait_groups(int groups, bool five) {
  if (five) {
    switch (groups) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<5>(); break;
      case 2: wait_vmcnt<10>(); break;
      default: wait_vmcnt<15>(); break;
    }
  } else {
    switch (groups) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<4>(); break;
      case 2: wait_vmcnt<8>(); break;
      default: wait_vmcnt<12>(); break;
    }
  }
}


// groups: column groups; tpg: 128-column tiles per group.
template <int BR, bool kBias>
__global__ void __launch_bounds__(64 * kWaves)
band_kernel(GemmArgs p, const __half* X, int64_t groups, int64_t tpg) {
  using L = BandLayout<BR>;
  constexpr int S = L::S;
  constexpr int FM = BR / 16;                      // 16-row MFMA blocks of the band
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in a scalar register
  const int frow = lane & 15, fk = lane >> 4;
  const int64_t M = p.M, N = p.N;
  const int64_t g = (int64_t)blockIdx.x % groups;
  const int64_t m0 = (int64_t)blockIdx.x / groups * BR;
  const int64_t tiles_n = (N + kTileN - 1) / kTileN;
  const int64_t t_first = g * tpg;
  const int T = (int)((t_first + tpg < tiles_n ? t_first + tpg : tiles_n) - t_first);
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
  const bool five = wave == 0;   // wavefront 0 also loads each tile's scale block

  // Direct loads of tile t (t < T) into stage t % S: this wavefront's blocks
  // 4 w .. 4 w + 3 (tile rows 4 b .. 4 b + 3; lane l fetches row 4 b + l / 16,
  // chunk (l % 16) ^ (row & 15)), and for wavefront 0 the scale block (lanes
  // 0-31: s_W of the tile's columns in quads, 32-63: the biases, or s_W
  // again without a bias; quads past N repeat the last one).
  // Per-lane parts of those addresses that do not depend on the tile (row
  // and column indices fit in 32 bits: N < 2^31, checked at launch): block
  // u's source in tile 0 of the group; tile t adds t whole tiles, unless the
  // tile reaches past N (then the rows are clamped one by one).
  const int n_last = (int)N - 1;
  const int lrow = 16 * wave + (lane >> 4);              // tile row of block u: lrow + 4 u
  const char* wbase = reinterpret_cast<const char*>(p.W);
  const float* sbase = (lane >= 32 && p.bias) ? p.bias : p.sW;
  const int squad = 4 * (lane & 31);
  const char* wsrc0[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int tr = lrow + 4 * u;
    wsrc0[u] = wbase + ((int64_t)(t_first * kTileN + tr) * kGroup + (((lane & 15) ^ (tr & 15)) << 4));
  }
  auto issue = [&](int t) {
    const int n0 = (int)((t_first + t) * kTileN);
    const int st = t % S;
    const uint32_t sb = lds_base + (uint32_t)(st * kTileBytes);
    if (n0 + kTileN <= N) {   // whole tile
#pragma unroll
      for (int u = 0; u < 4; ++u)
        dma16(wsrc0[u] + (int64_t)t * kTileBytes, sb + (uint32_t)((4 * wave + u) * 1024));
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int tr = lrow + 4 * u;
        const int n = min(n0 + tr, n_last);
        dma16(wbase + ((int64_t)n * kGroup + (((lane & 15) ^ (tr & 15)) << 4)), sb + (uint32_t)((4 * wave + u) * 1024));
      }
    }
    if (five) {
      const int q = min(n0 + squad, n_last - 3);
      dma16(sbase + q, lds_base + L::kScales + (uint32_t)(st * 1024));
    }
  };

  // 1-2. the band, 32 rows at a time: segment `seg` takes row m0 + 32 q +
  // seg (clamped to M - 1), parks it in its slot, rotates it and writes the
  // row's scale and codes (chunk c of row j at slot c ^ (j & 15)).  Every
  // activation load completes before the first direct load goes out (the
  // compiler's wait for them would otherwise cover the direct loads too);
  // the first F tiles' direct loads go out once the first rows are parked.
  const int seg = tid >> 4, l16 = tid & 15;
  char* slot = smem + L::kSlots + seg * kSlotBytes;
  float* sxs = reinterpret_cast<float*>(smem + L::kSx);
  constexpr int Q = (BR + kSegs - 1) / kSegs;        // segments past BR (BR = 16) idle
  v4i xr[Q][2];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int jl = BR >= kSegs || kSegs * q + seg < BR ? kSegs * q + seg : BR - 1;
    const int64_t m = m0 + jl < M ? m0 + jl : M - 1;
    const v4i* src = reinterpret_cast<const v4i*>(X + m * kGroup + 16 * l16);
    xr[q][0] = __builtin_nontemporal_load(src);
    xr[q][1] = __builtin_nontemporal_load(src + 1);
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) asm volatile("" :: "v"(xr[q][0]), "v"(xr[q][1]));   // all loads landed
  compiler_fence();
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int j = kSegs * q + seg;
    const bool idle = BR < kSegs && j >= BR;   // whole wavefronts (BR = 16: wavefronts 4-7)
    if (!idle) park_row(slot, l16, xr[q][0], xr[q][1]);
    if (q == 0) {
      compiler_fence();
#pragma unroll
      for (int t = 0; t < L::F; ++t)
        if (t < T) issue(t);
    }
    if (idle) continue;
    double y[16];
    rotate_staged(slot, l16, y);
    float f[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      f[i] = (float)y[i];   // fp32(16 X_rot): the single rounding
      amax = fmaxf(amax, fabsf(f[i]));
    }
    const float rmax = __uint_as_float(seg_max16_bits(__float_as_uint(amax)));
    // S = fp32(max |16 X_rot|) / 127 = 16 s_X exactly, and round(F / S)
    // equals round(X_rot / s_X) (power-of-two scaling commutes with the fp32
    // roundings of normal values)
    const float sc = rmax / 127.0f;
    if (l16 == 0) sxs[j] = sc * 0.0625f;
    *reinterpret_cast<uint4*>(smem + L::kCodes + j * kGroup + ((l16 ^ (j & 15)) << 4)) = quantize16(f, sc);
  }
  lds_barrier();   // codes and s_X visible; the rotation slots are free
#pragma unroll
  for (int t = L::F; t < S; ++t)
    if (t < T) issue(t);

  // 3. codes as MFMA operands (row 16 j + frow, chunk 4 s + fk) and s_X of
  // this lane's output rows, for every tile
  v4i fb[FM][4];
  float sxv[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int r = 16 * j + frow;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      fb[j][s] = *reinterpret_cast<const v4i*>(smem + L::kCodes + r * kGroup + (((4 * s + fk) ^ (r & 15)) << 4));
    sxv[j] = sxs[r];
  }

  const bool vec_rows = (N % 8) == 0;   // every output row starts 16-byte aligned
  __half* Y = reinterpret_cast<__half*>(p.out);
  // Tile u's output from staging tile u & 1: BR rows x 16 pieces of 16 bytes,
  // one per thread and 32 rows at a time (rows tid / 16 + 32 h, columns
  // n0 + 8 (tid % 16) ..), [+ the residual] to Y.
  auto store_tile = [&](int u) {
    const char* sb = smem + L::kStage + (u & 1) * BR * kStageRow;
#pragma unroll
    for (int h = 0; h < (BR + 31) / 32; ++h) {
      const int rl = (tid >> 4) + 32 * h, pc = tid & 15;
      const int64_t m = m0 + rl, n = (t_first + u) * kTileN + 8 * pc;
      if ((BR % 32 == 0 || rl < BR) && m < M && n < N) {
        v4i v = *reinterpret_cast<const v4i*>(sb + rl * kStageRow + ((pc ^ (rl & 15)) << 4));
        __half* dst = Y + m * N + n;
        if (vec_rows && n + 8 <= N) {
          if (p.R) v = add_f16x8(v, *reinterpret_cast<const v4i*>(p.R + m * N + n));
          __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(dst));
        } else {
          // N is a multiple of 4: rows start 8-byte aligned, and each 4-column
          // half of the piece is in range or wholly past N
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            if (n + 4 * q >= N) break;
            uint2 o = q == 0 ? make_uint2(v.x, v.y) : make_uint2(v.z, v.w);
            if (p.R) {
              const uint2 r = *reinterpret_cast<const uint2*>(p.R + m * N + n + 4 * q);
              const __half* a = reinterpret_cast<const __half*>(&o);
              const __half* b = reinterpret_cast<const __half*>(&r);
              __half z[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) z[e] = __float2half_rn(__half2float(a[e]) + __half2float(b[e]));
              o = *reinterpret_cast<const uint2*>(z);
            }
            *reinterpret_cast<uint2*>(dst + 4 * q) = o;
          }
        }
      }
    }
  };

  // One barrier per tile: it publishes tile t's blocks, and every
  // wavefront has finished tile t - 1 (its reads of the stage refilled next,
  // and its writes to staging tile (t - 1) & 1, stored right after).
  const int wr = 16 * wave + frow;      // this lane's weight row within a tile (MFMA operand)
  for (int t = 0; t < T; ++t) {
    // groups issued after tile t so far: tiles t + 1 .. min(T - 1, S - 1) at
    // t = 0, t + 1 .. min(T - 1, t + S - 2) later
    const int after = t == 0 ? (T - 1 < S - 1 ? T - 1 : S - 1) : (T - 1 - t < S - 2 ? T - 1 - t : S - 2);
    wait_groups(after, five);
    lds_barrier();
    if (t >= 1 && t + S - 1 < T) issue(t + S - 1);   // into the stage tile t - 1 used
    if (t >= 1) store_tile(t - 1);

    const int st = t % S;
    const char* ws = smem + st * kTileBytes;
    v4i wa[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      wa[s] = *reinterpret_cast<const v4i*>(ws + wr * kGroup + (((4 * s + fk) ^ (wr & 15)) << 4));
    v4i acc[FM];
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      acc[j] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[s], fb[j][s], acc[j], 0, 0, 0);
    }

    // 4. lane holds A[m][n] for m = m0 + 16 j + frow, n = n0 + 16 wave + 4 fk + r:
    // 8 bytes at row 16 j + frow, chunk 2 wave + fk / 2 (swizzled), half fk & 1
    const float* sc = reinterpret_cast<const float*>(smem + L::kScales + st * 1024);
    const v4f sw = *reinterpret_cast<const v4f*>(sc + 16 * wave + 4 * fk);
    const v4f bs = *reinterpret_cast<const v4f*>(sc + 128 + 16 * wave + 4 * fk);
    char* sbw = smem + L::kStage + (t & 1) * BR * kStageRow;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      float y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        y[r] = __fmul_rn((float)acc[j][r], __fmul_rn(sxv[j], sw[r]));
        if constexpr (kBias) y[r] = __fadd_rn(y[r], bs[r]);
      }
      uint2 v;
      v.x = pack_f16x2_rn(y[0], y[1]);
      v.y = pack_f16x2_rn(y[2], y[3]);
      const int row = 16 * j + frow;
      *reinterpret_cast<uint2*>(sbw + row * kStageRow + (((2 * wave + (fk >> 1)) ^ (row & 15)) << 4) + 8 * (fk & 1)) = v;
    }
  }
  lds_barrier();
  store_tile(T - 1);
}

struct BandPlan {
  int br;
  int64_t groups, tpg;
};

// About one workgroup per CU: groups = 256 / bands (at least 1, at most one
// per tile) and the tiles spread evenly over the groups.
BandPlan band_plan(int64_t M, int64_t N, int br) {
  const int64_t bands = (M + br - 1) / br;
  const int64_t tiles = (N + kTileN - 1) / kTileN;
  int64_t groups = 256 / bands;
  groups = groups < 1 ? 1 : groups > tiles ? tiles : groups;
  const int64_t tpg = (tiles + groups - 1) / groups;
  groups = (tiles + tpg - 1) / tpg;
  return {br, groups, tpg};
}

template <int BR, bool kBias>
hipError_t launch_br(const GemmArgs& a, const void* X, const BandPlan& bp, hipStream_t stream) {
  auto fn = &band_kernel<BR, kBias>;
  constexpr int lds = BandLayout<BR>::kBytes;
  if (const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(fn), lds); e != hipSuccess) return e;
  const int64_t bands = (a.M + BR - 1) / BR;
  hipLaunchKernelGGL(fn, dim3((unsigned)(bands * bp.groups)), dim3(64 * kWaves), lds, stream, a,
                     reinterpret_cast<const __half*>(X), bp.groups, bp.tpg);
  return hipGetLastError();
}

}  // namespace

bool band_fusable(int64_t M, int64_t N, int64_t K) {
  return K == kGroup && M > 16 && M <= 2048 && N >= 4 && N % 4 == 0 && N < ((int64_t)1 << 31);
}

// Bands of 32 rows; with at most 128 rows, bands of 16 (half the segments
// rotate, twice the bands share the CUs): 5-15 % faster there (17, 100 and
// 128 rows), 5-29 % slower from 512 rows on.
hipError_t launch_band(const GemmArgs& a, const void* X, hipStream_t stream) {
  if (!band_fusable(a.M, a.N, a.K)) return hipErrorInvalidValue;
  if (a.M <= 128) {
    const BandPlan bp = band_plan(a.M, a.N, 16);
    return a.bias ? launch_br<16, true>(a, X, bp, stream) : launch_br<16, false>(a, X, bp, stream);
  }
  const BandPlan bp = band_plan(a.M, a.N, kBandRows);
  return a.bias ? launch_br<kBandRows, true>(a, X, bp, stream) : launch_br<kBandRows, false>(a, X, bp, stream);
}

}  // namespace convrot
