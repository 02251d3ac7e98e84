// Pipelined MFMA GEMMs whose operands go to LDS by direct global->LDS loads:
// the int8 W8A8 product (A = Q_X Q_W^T, optionally with the scale epilogue),
// the weight-only product (fp16 activations times int8 weights; s_W, bias and
// the unmerged LoRA in the epilogue) and the fp16 baseline.  Page "INT8ConvRot
// GEMM vs fp16 on M1 Max with Metal, MPSMatrix, and MLX (fp16 Wins)", section
// "What changed in the computation" (A, Y and the weight-only listing) and
// the fp16 column of its six-shape table; page "[PR #249] Add an mps backend
// ...", sections "What" and "Design" (the LoRA term).
//
// Data flow (gfx950).  A workgroup of WAVES_M x WAVES_N wavefronts owns a
// (16 FM WAVES_M) x (16 FN WAVES_N) output tile; each wavefront an FM x FN
// block of 16x16 MFMA fragments.  K advances in slices of XS = 128 or 256
// activation bytes per row (int8 values, or half as many fp16) through a ring
// of STAGES LDS
// buffers filled by direct global->LDS loads (global_load_lds_dwordx4:
// 64 lanes x 16 B = one 1 KiB block per instruction, no register staging).
// STAGES-1 slices are in flight while one is consumed.  The ring holds the
// activation rows of every stage first, then the weight rows of every stage,
// and each wave loads the same number of activation blocks and of weight
// blocks per slice.  256- and 128-byte LDS rows have their 16-byte chunks
// XOR-swizzled by (row & 15) and (row & 7); the weight-only
// mode's int8 weight rows are 64 bytes per slice (16 rows per block) with
// their chunks swizzled by ((row >> 2) & 3).  Both make the fills and the
// fragment reads conflict-free; a direct load places a lane's chunk at its
// swizzled slot by choosing which global chunk that lane fetches.  In the
// weight-only mode each lane widens its 8-byte weight fragment to fp16 in
// registers (exact for int8) before the fp16 MFMA.
//
// Synchronisation per slice: every wave waits (s_waitcnt vmcnt) until its own
// loads of the next slice have landed and its LDS reads are done (lgkmcnt),
// then s_barrier publishes everyone's loads; the refill of the buffer just
// consumed is issued right after that barrier.  The direct loads are written
// as inline assembly so that the compiler does not treat them as LDS stores
// that every later fragment read must wait for.
//
// Epilogue: scale and bias operands are fetched at kernel entry; the finished
// tile is converted in registers, staged through the (now idle) LDS ring (each
// barrier waits for the wave's own LDS operations first) and
// written as whole 16-byte chunks of contiguous output rows with
// non-temporal stores.
//
// Tile order is XCD-aware: workgroups are dispatched round-robin over the 8
// XCDs, so the i-th workgroup on XCD x gets the i-th tile of a contiguous
// range of a grouped order (groups of group_m row tiles, N-major inside a
// group).  Each XCD then streams a few weight panels through its own L2 while
// its resident workgroups share the activation bands.  group_m is chosen on
// the host (choose_group_m below); when the prologue has written Q_X in
// eight row bands, band x from XCD x, XCD x takes exactly those rows.
//
// Rows past M or N are clamped to the last valid row for the loads (so every
// load is in bounds) and dropped in the epilogue.

#include <type_traits>

#include "launch.hpp"

namespace convrot {
namespace {

// LDS row layouts, by row bytes RB (the K slice of one tile row): 16-byte
// chunk c of row r sits at slot c ^ key(r), key = r & 15 (256-byte rows),
// r & 7 (128-byte rows) or (r >> 2) & 3 (64-byte rows: 16 rows per 1 KiB
// block).  In each case the 16 rows a fragment read touches at one chunk
// index land in distinct banks, and so do the lanes of one direct load.
template <int RB>
__device__ __forceinline__ int swz_key(int row) {
  if constexpr (RB == 64) return (row >> 2) & 3;
  else return row & (RB / 16 - 1);
}
template <int RB>
__device__ __forceinline__ int swz(int row, int chunk) { return row * RB + ((chunk ^ swz_key<RB>(row)) << 4); }

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt low bits 3:0,
// high bits 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 0xF) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One direct global->LDS load: 64 lanes x 16 bytes land contiguously at LDS
// byte offset `lds` (wave-uniform).  Issued as inline assembly so that the
// compiler does not treat it as a store that every later LDS read must wait
// for; the kernel orders it with explicit vmcnt waits and barriers instead.
// M0 holds the LDS base; one wait state separates its write from the load.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gptr), "s"(lds) : "memory", "m0");
}

// 8 int8 values (two dwords) -> 8 fp16, exactly: with the sign bit flipped a
// byte u = b + 128 sits under the fp16 pattern 0x64 (1024 + u), and
// subtracting 1152 leaves b.  All three steps are exact in fp16.
__device__ __forceinline__ v8h widen_i8x8(uint2 w) {
  typedef _Float16 v2h __attribute__((ext_vector_type(2)));
  const uint32_t x0 = w.x ^ 0x80808080u, x1 = w.y ^ 0x80808080u;
  uint32_t h[4];
  // v_perm_b32 selector bytes 0-3 pick from the second operand, 4-7 from the first
  h[0] = __builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u);  // bytes 0, 1
  h[1] = __builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u);  // bytes 2, 3
  h[2] = __builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u);
  h[3] = __builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u);
  v8h r;
  const v2h bias = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const v2h v = *reinterpret_cast<const v2h*>(&h[q]) - bias;
    r[2 * q] = v[0];
    r[2 * q + 1] = v[1];
  }
  return r;
}

// MFMA operand of a LoRA product: 8 fp16 values at columns r0 + 8 (lane / 16)
// of row `row` (clamped to rows - 1) of a [rows, t_ld] fp16 matrix.
__device__ __forceinline__ v8h lora_frag(const __half* __restrict__ base, int64_t row, int64_t rows,
                                         int t_ld, int r0, int lane) {
  row = row < rows ? row : rows - 1;
  const uint4 v = *reinterpret_cast<const uint4*>(base + row * t_ld + r0 + 8 * (lane >> 4));
  return *reinterpret_cast<const v8h*>(&v);
}

// Eight bf16 additions, each rounded once: a + b in fp32 (fp32 carries more
// than twice bf16's precision, so this is the correctly rounded bf16 sum).
__device__ __forceinline__ v4i add_bf16x8(v4i a, v4i b) {
  const uint16_t* x = reinterpret_cast<const uint16_t*>(&a);
  const uint16_t* y = reinterpret_cast<const uint16_t*>(&b);
  uint16_t z[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = f32_to_bf16_rn(bf16_to_f32(x[e]) + bf16_to_f32(y[e]));
  return *reinterpret_cast<const v4i*>(z);
}

// Eight fp16 additions, each rounded once: a + b in fp32, then to fp16.
__device__ __forceinline__ v4i add_f16x8(v4i a, v4i b) {
  const __half* x = reinterpret_cast<const __half*>(&a);
  const __half* y = reinterpret_cast<const __half*>(&b);
  __half z[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = __float2half_rn(__half2float(x[e]) + __half2float(y[e]));
  return *reinterpret_cast<const v4i*>(z);
}

template <GemmMode MODE, int WAVES_M, int WAVES_N, int FM, int FN, int STAGES, int XS, bool EXTRA>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
gemm_dma_kernel(GemmArgs p) {
  constexpr bool kInt = (MODE == GemmMode::kI8toI32 || MODE == GemmMode::kI8toF16);
  constexpr bool kW16 = (MODE == GemmMode::kW8A16);
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WM = 16 * FM, WN = 16 * FN;     // wave tile (m, n)
  constexpr int BM = WAVES_M * WM, BN = WAVES_N * WN;
  constexpr int kRowX = XS;                     // activation bytes of one K slice per row
  constexpr int kRowW = kW16 ? XS / 2 : XS;     // weight bytes of one K slice per row
  constexpr int NKK = XS / 64;                  // K steps (64 activation bytes) per slice
  constexpr int XROWS = 1024 / kRowX;           // activation rows per 1 KiB block
  constexpr int WROWS = 1024 / kRowW;           // weight rows per 1 KiB block
  constexpr int XBLK = BM / XROWS;              // activation blocks per slice
  constexpr int WBLK = BN / WROWS;              // weight blocks per slice
  constexpr int XL = XBLK / NW, WL = WBLK / NW; // per wave per slice
  constexpr int LPW = XL + WL;
  constexpr int XBYTES = BM * kRowX;            // one stage of activation rows
  constexpr int WBYTES = BN * kRowW;            // one stage of weight rows
  constexpr int WBASE = STAGES * XBYTES;        // LDS offset of the weight stages
  constexpr int kElemX = kInt ? 1 : 2;
  constexpr int kElemW = (MODE == GemmMode::kF16) ? 2 : 1;
  constexpr int kAhead = (STAGES - 2) * LPW;    // loads issued after the awaited slice
  static_assert(XBLK % NW == 0 && WBLK % NW == 0, "blocks must split evenly over waves");
  static_assert(BN % WROWS == 0 && BM % XROWS == 0, "whole blocks");
  static_assert(NKK % 2 == 0, "fragment buffers alternate per K step");
  // Two stages keep one slice in flight while one is consumed (the refill of
  // a buffer still waits for the barrier after its last reads).
  static_assert(STAGES >= 2 && kAhead < 64, "pipeline depth");

  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  const int64_t M = p.M, N = p.N;
  // Split K (grid y > 1, int32 output only): split z takes K values
  // [z kc, (z + 1) kc) of rows of stride p.K and writes its own partial A.
  const int64_t K = p.kc ? p.kc : p.K;
  const int64_t kz = (int64_t)blockIdx.y * K;
  const int64_t tiles_m = (M + BM - 1) / BM;
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t T = tiles_m * tiles_n;
  int64_t t;
  {
    const int64_t b = blockIdx.x;
    const int64_t x = b & 7, i = b >> 3;
    const int64_t per = T >> 3, rem = T & 7;
    t = x * per + (x < rem ? x : rem) + i;
  }
  // Grouped order: tiles run in groups of GM row tiles, N-major inside a
  // group (a bijection of [0, T) for any GM >= 1).
  const int64_t GM = p.group_m;
  const int64_t in_group = GM * tiles_n;
  const int64_t first_m = (t / in_group) * GM;
  const int64_t gsize = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int64_t tile_m = first_m + (t % in_group) % gsize;
  const int64_t tile_n = (t % in_group) / gsize;
  const int64_t m0 = tile_m * BM, n0 = tile_n * BN;
  const int64_t ldx = p.K * kElemX;              // row bytes of the activations
  const int64_t ldw = p.K * kElemW;              // row bytes of the weights
  const int64_t nk = K * kElemX / kRowX;

  // Epilogue operands are fetched first so that their latency hides behind the
  // main loop (issued before the first direct load, they also complete first).
  const int orow = lane & 15;        // output row within a fragment
  const int ocol = (lane >> 4) * 4;  // first of 4 output columns within a fragment
  float sxv[FM], swv[FN][4], bsv[FN][4];
  int rexp[FM];   // range-safe weight-only: per-row power of two to restore
  if constexpr (kW16 && EXTRA) {
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int64_t m = m0 + wm * WM + j * 16 + orow;
      rexp[j] = p.rowexp ? p.rowexp[m < M ? m : M - 1] : 0;
    }
  }
  if constexpr (MODE == GemmMode::kI8toF16) {
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int64_t m = m0 + wm * WM + j * 16 + orow;
      sxv[j] = p.sX[m < M ? m : M - 1];
    }
  }
  if constexpr (MODE == GemmMode::kI8toF16 || kW16) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t n = n0 + wn * WN + i * 16 + ocol + r;
        const int64_t nc = n < N ? n : N - 1;
        swv[i][r] = p.sW[nc];
        bsv[i][r] = p.bias ? p.bias[nc] : 0.0f;
      }
  } else if constexpr (MODE == GemmMode::kF16) {
    if (p.bias) {
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t n = n0 + wn * WN + i * 16 + ocol + r;
          bsv[i][r] = p.bias[n < N ? n : N - 1];
        }
    }
  }

  // LoRA operands of the first 32 rank columns (rows past M or N repeat the
  // last row; their results are dropped)
  constexpr bool kScaled = (MODE == GemmMode::kI8toF16 || kW16);
  constexpr bool kLora = kScaled && EXTRA;
  v8h lua[kLora ? FN : 1], ltb[kLora ? FM : 1];
  if constexpr (kLora) {
    if (p.t_ld > 0) {
#pragma unroll
      for (int i = 0; i < FN; ++i) lua[i] = lora_frag(p.U, n0 + wn * WN + i * 16 + (lane & 15), N, p.t_ld, 0, lane);
#pragma unroll
      for (int j = 0; j < FM; ++j) ltb[j] = lora_frag(p.T, m0 + wm * WM + j * 16 + (lane & 15), M, p.t_ld, 0, lane);
    }
  }

  // Per-lane direct-load sources of this wave's blocks: activation blocks
  // j = wave XL + i (XROWS rows each) and weight blocks j = wave WL + i
  // (WROWS rows each) of every slice.
  const char* srcx[XL];
  const char* srcw[WL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int j = wave * XL + i;
    const int rl = lane / (kRowX / 16);          // row within the block
    const int slot = lane % (kRowX / 16);
    const int trow = XROWS * j + rl;             // row within the tile
    const int chunk = slot ^ swz_key<kRowX>(trow);   // logical chunk landing at `slot`
    int64_t row = m0 + trow;
    row = row < M ? row : M - 1;
    srcx[i] = reinterpret_cast<const char*>(p.X) + row * ldx + kz * kElemX + chunk * 16;
  }
#pragma unroll
  for (int i = 0; i < WL; ++i) {
    const int j = wave * WL + i;
    const int rl = lane / (kRowW / 16);
    const int slot = lane % (kRowW / 16);
    const int trow = WROWS * j + rl;
    const int chunk = slot ^ swz_key<kRowW>(trow);
    int64_t row = n0 + trow;
    row = row < N ? row : N - 1;
    srcw[i] = reinterpret_cast<const char*>(p.W) + row * ldw + kz * kElemW + chunk * 16;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
  auto issue_x = [&](int64_t kt) {
    const uint32_t dst = lds_base + ((uint32_t)kt % STAGES) * XBYTES + wave * XL * 1024;
#pragma unroll
    for (int i = 0; i < XL; ++i)
      dma16(srcx[i] + kt * kRowX, __builtin_amdgcn_readfirstlane(dst + i * 1024));
  };
  auto issue_w = [&](int64_t kt) {
    const uint32_t dst = lds_base + WBASE + ((uint32_t)kt % STAGES) * WBYTES + wave * WL * 1024;
#pragma unroll
    for (int i = 0; i < WL; ++i)
      dma16(srcw[i] + kt * kRowW, __builtin_amdgcn_readfirstlane(dst + i * 1024));
  };
  auto issue = [&](int64_t kt) {
    issue_x(kt);
    issue_w(kt);
  };

  using Acc = typename std::conditional<kInt, v4i, v4f>::type;
  Acc acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = Acc{0, 0, 0, 0};

  const int frow = lane & 15;
  const int fk = lane >> 4;
  // Fragments of one K step (64 activation bytes), double-buffered in registers.
  using WFrag = typename std::conditional<kW16, uint2, uint4>::type;
  WFrag fa[2][FN];
  uint4 fb[2][FM];
  auto load_frags = [&](int buf, int64_t kt, int kk) {
    const char* xs = smem + (int)((uint32_t)kt % STAGES) * XBYTES;
    const char* ws = smem + WBASE + (int)((uint32_t)kt % STAGES) * WBYTES;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int row = wn * WN + i * 16 + frow;
      if constexpr (kW16) {   // K step kk: weight bytes [32 kk + 8 fk, + 8)
        const int c = 2 * kk + (fk >> 1);
        fa[buf][i] = *reinterpret_cast<const uint2*>(ws + swz<kRowW>(row, c) + 8 * (fk & 1));
      } else {
        fa[buf][i] = *reinterpret_cast<const uint4*>(ws + swz<kRowW>(row, kk * 4 + fk));
      }
    }
#pragma unroll
    for (int j = 0; j < FM; ++j)
      fb[buf][j] = *reinterpret_cast<const uint4*>(xs + swz<kRowX>(wm * WM + j * 16 + frow, kk * 4 + fk));
  };
  // Weight-only: the widened weight fragments of a K step are produced right
  // after the MFMAs of the previous step are issued, so the VALU work runs
  // while the matrix cores are busy instead of in front of them.
  v8h wa[2][kW16 ? FN : 1];
  auto widen = [&](int buf) {
    if constexpr (kW16) {
#pragma unroll
      for (int i = 0; i < FN; ++i) wa[buf][i] = widen_i8x8(fa[buf][i]);
    }
  };
  auto mma = [&](int buf) {
    if constexpr (kW16) {
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              wa[buf][i], *reinterpret_cast<const v8h*>(&fb[buf][j]), acc[i][j], 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          if constexpr (kInt) {
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                *reinterpret_cast<const v4i*>(&fa[buf][i]), *reinterpret_cast<const v4i*>(&fb[buf][j]),
                acc[i][j], 0, 0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                *reinterpret_cast<const v8h*>(&fa[buf][i]), *reinterpret_cast<const v8h*>(&fb[buf][j]),
                acc[i][j], 0, 0, 0);
          }
        }
    }
  };
  // Workgroup barrier.  The hardware barrier does not wait for the wave's
  // own LDS operations, so lgkmcnt(0) comes first: LDS writes made before
  // the barrier are visible to every wave after it, and LDS reads made
  // before it are done before any wave overwrites their addresses.
  auto barrier = [&]() {
    wait_lgkm0();
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
  };

  // Pipeline.  Slices 0 .. STAGES-2 are requested up front; slice s lives in
  // buffer s % STAGES.  Before the MFMAs of a slice's second K step run, the
  // wave already holds its fragments; the next slice's first-step fragments
  // are read right after the barrier that publishes it, and that barrier is
  // also where the buffer of the slice just finished gets refilled (every
  // wave has drained its reads of it: lgkmcnt(0) precedes the barrier).
  // Every slice's loads go out as one group, so the number of loads issued
  // after a given slice is fixed: kAhead once the pipeline is full; near the
  // end (fewer groups in flight) the waits fall back to 0.
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s);
  if (nk >= STAGES - 1) wait_vmcnt<kAhead>();
  else wait_vmcnt<0>();
  barrier();
  if (STAGES - 1 < nk) issue(STAGES - 1);
  load_frags(0, 0, 0);
  widen(0);

  // The last slice is peeled off so that the loop body has a single path into
  // its second MFMA group: the LDS-read counter then only waits for reads that
  // group actually consumes, not for the next slice's reads issued before it.
  // K steps alternate between the two fragment buffers (NKK is even).
  //
  // Int8 products: the MFMAs before the barrier run at raised wave priority,
  // and after it the refill is not issued as one burst but one or two loads
  // at a time between the MFMA groups of each weight fragment.  Issuing all
  // of a slice's loads at once left the waves stalled at issue while the
  // address unit drained them, with no MFMAs in flight (measured on the
  // 256x128 tile: 22.4 -> 21.3 us at 1024x8192x2048).  The scheduling
  // barriers keep the compiler from regrouping the loads.
  for (int64_t kt = 0; kt + 1 < nk; ++kt) {
#pragma unroll
    for (int kk = 0; kk + 1 < NKK; ++kk) {
      if constexpr (kInt) __builtin_amdgcn_s_setprio(1);
      load_frags((kk + 1) & 1, kt, kk + 1);
      mma(kk & 1);
      if constexpr (kInt) __builtin_amdgcn_s_setprio(0);
      widen((kk + 1) & 1);
    }
    if (kt + STAGES - 1 < nk) wait_vmcnt<kAhead>();
    else wait_vmcnt<0>();
    barrier();
    if constexpr (kInt) {
      const bool refill = kt + STAGES < nk;
      const int64_t kn = kt + STAGES;
      const uint32_t dx = lds_base + ((uint32_t)kn % STAGES) * XBYTES + wave * XL * 1024;
      const uint32_t dw = lds_base + WBASE + ((uint32_t)kn % STAGES) * WBYTES + wave * WL * 1024;
      load_frags(0, kt + 1, 0);
#pragma unroll
      for (int i = 0; i < FN; ++i) {
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(*reinterpret_cast<const v4i*>(&fa[1][i]),
                                                            *reinterpret_cast<const v4i*>(&fb[1][j]), acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        // loads u = i LPW / FN .. (i + 1) LPW / FN - 1 of the refill
#pragma unroll
        for (int u = i * LPW / FN; u < (i + 1) * LPW / FN; ++u) {
          if (refill) {
            if (u < XL) dma16(srcx[u] + kn * kRowX, __builtin_amdgcn_readfirstlane(dx + u * 1024));
            else dma16(srcw[u - XL] + kn * kRowW, __builtin_amdgcn_readfirstlane(dw + (u - XL) * 1024));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      if (kt + STAGES < nk) issue(kt + STAGES);
      load_frags(0, kt + 1, 0);
      mma(1);
      widen(0);
    }
  }
#pragma unroll
  for (int kk = 0; kk + 1 < NKK; ++kk) {
    load_frags((kk + 1) & 1, nk - 1, kk + 1);
    mma(kk & 1);
    widen((kk + 1) & 1);
  }
  mma(1);

  // Unmerged LoRA: the product T U'^T (T = fp16(X down^T) [M, t_ld],
  // U' = fp16(scale * up) [N, t_ld]) runs as extra fp16 MFMA K steps of 32
  // rank columns on fp32 accumulators in the fragment layout.  The operands
  // of the first step were fetched at kernel entry.
  auto lora_mma = [&](v4f (&y)[FN][FM]) {
    for (int r0 = 0; r0 < p.t_ld; r0 += 32) {
      v8h ua[FN], tb[FM];
      if (r0 == 0) {
#pragma unroll
        for (int i = 0; i < FN; ++i) ua[i] = lua[i];
#pragma unroll
        for (int j = 0; j < FM; ++j) tb[j] = ltb[j];
      } else {
#pragma unroll
        for (int i = 0; i < FN; ++i) ua[i] = lora_frag(p.U, n0 + wn * WN + i * 16 + frow, N, p.t_ld, r0, lane);
#pragma unroll
        for (int j = 0; j < FM; ++j) tb[j] = lora_frag(p.T, m0 + wm * WM + j * 16 + frow, M, p.t_ld, r0, lane);
      }
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          y[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ua[i], tb[j], y[i][j], 0, 0, 0);
    }
  };

  // Output geometry of the epilogue: 16-byte chunks, CPT per thread.
  using OutT = typename std::conditional<MODE == GemmMode::kI8toI32, int32_t, __half>::type;
  constexpr int kOut = sizeof(OutT);
  constexpr int CPR = BN * kOut / 16;             // 16-byte chunks per tile row
  constexpr int NTH = 64 * NW;
  constexpr int CPT = (BM * CPR + NTH - 1) / NTH; // chunks per thread
  const bool vec_rows = ((N * kOut) % 16) == 0;   // every output row starts 16-byte aligned

  // W8A8 residual: the whole-chunk parts this thread will add are fetched now,
  // so that their latency hides behind the epilogue arithmetic.
  constexpr bool kRes = (MODE == GemmMode::kI8toF16 || kW16) && EXTRA;
  const __half* res = kRes ? p.R : nullptr;
  v4i rres[kRes ? CPT : 1];
  if constexpr (kRes) {
    if (res && vec_rows) {
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int c = tid + q * NTH;
        const int rl = c / CPR, cc = c - rl * CPR;
        int64_t m = m0 + rl;
        m = m < M ? m : M - 1;
        const int64_t n = n0 + cc * 8;
        rres[q] = v4i{0, 0, 0, 0};
        if (n + 8 <= N) rres[q] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(res + m * N + n));
      }
    }
  }

  // fp32 output tile of the scaled modes, in the fragment layout.
  // W8A8: Y = fp32(A) * fp32(s_X * s_W) [+ bias], no contraction, then the
  // LoRA term.  Weight-only: s_W scales the accumulators, then the LoRA term;
  // the bias follows at the conversion to fp16.
  v4f yf[kScaled ? FN : 1][kScaled ? FM : 1];
  if constexpr (MODE == GemmMode::kI8toF16) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sc = __fmul_rn(sxv[j], swv[i][r]);
          float y = __fmul_rn((float)acc[i][j][r], sc);
          if (p.bias) y = __fadd_rn(y, bsv[i][r]);
          yf[i][j][r] = y;
        }
  } else if constexpr (kW16) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float y = __fmul_rn(acc[i][j][r], swv[i][r]);
          if constexpr (EXTRA) y = ldexpf(y, rexp[j]);   // exact power-of-two restore
          yf[i][j][r] = y;
        }
  }
  if constexpr (kLora) {
    if (p.t_ld > 0) lora_mma(yf);
  }

  // ---------------------------------------------------------------- epilogue
  // The finished tile goes through LDS (the ring is free now) so that global
  // stores are whole 16-byte chunks of contiguous output rows.
  constexpr int ROWB = BN * kOut + 16;            // staged row bytes (+16: bank offset per row)
  static_assert(BM * ROWB <= STAGES * (XBYTES + WBYTES), "staging tile must fit in the ring");
  barrier();                                      // every wave is done reading the ring
#pragma unroll
  for (int i = 0; i < FN; ++i) {
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int ml = wm * WM + j * 16 + orow;     // row within the tile
      const int nl = wn * WN + i * 16 + ocol;     // first of 4 columns within the tile
      char* d = smem + ml * ROWB + nl * kOut;
      if constexpr (MODE == GemmMode::kI8toI32) {
        *reinterpret_cast<v4i*>(d) = acc[i][j];
      } else {
        uint2 v;
        if constexpr (MODE == GemmMode::kI8toF16) {
          v.x = pack_f16x2_rn(yf[i][j][0], yf[i][j][1]);
          v.y = pack_f16x2_rn(yf[i][j][2], yf[i][j][3]);
        } else if constexpr (kW16) {
          __half h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float y = yf[i][j][r];
            if (p.bias) y = __fadd_rn(y, bsv[i][r]);
            h[r] = EXTRA && p.out_bf16 ? __ushort_as_half(f32_to_bf16_rn(y)) : __float2half_rn(as_fp32(y));
          }
          v.x = (uint32_t)__half_as_ushort(h[0]) | ((uint32_t)__half_as_ushort(h[1]) << 16);
          v.y = (uint32_t)__half_as_ushort(h[2]) | ((uint32_t)__half_as_ushort(h[3]) << 16);
        } else {
          float y[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = p.bias ? __fadd_rn(acc[i][j][r], bsv[i][r]) : acc[i][j][r];
          v.x = pack_f16x2_rn(y[0], y[1]);
          v.y = pack_f16x2_rn(y[2], y[3]);
        }
        *reinterpret_cast<uint2*>(d) = v;
      }
    }
  }
  barrier();
  char* outb = reinterpret_cast<char*>(p.out) + (int64_t)blockIdx.y * M * N * kOut;
  // The residual is one fp16 addition to the finished fp16 output (the fp32
  // sum of two fp16 values rounded to fp16 is their correctly rounded fp16
  // sum: fp32 carries more than twice fp16's precision).  Each element's
  // residual is read by the thread that writes that element, before the
  // write, so the residual may be the output buffer itself.
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int c = tid + q * NTH;
    if (c >= BM * CPR) break;
    const int rl = c / CPR, cc = c - rl * CPR;
    const int64_t m = m0 + rl;
    if (m >= M) continue;
    const int64_t n = n0 + cc * (16 / kOut);
    const char* sp = smem + rl * ROWB + cc * 16;
    char* gp = outb + (m * N + n) * kOut;
    if (vec_rows && n + 16 / kOut <= N) {
      v4i v = *reinterpret_cast<const v4i*>(sp);
      if constexpr (kRes) {
        if (res) v = p.out_bf16 ? add_bf16x8(v, rres[q]) : add_f16x8(v, rres[q]);
      }
      // streaming store: the output is not re-read by this kernel
      __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(gp));
    } else {
#pragma unroll
      for (int e = 0; e < 16 / kOut; ++e) {
        if (n + e >= N) continue;
        OutT o = reinterpret_cast<const OutT*>(sp)[e];
        if constexpr (kRes) {
          if (res) {
            if (p.out_bf16) {
              const float sum = bf16_to_f32(__half_as_ushort(o)) + bf16_to_f32(__half_as_ushort(res[m * N + n + e]));
              o = __ushort_as_half(f32_to_bf16_rn(sum));
            } else {
              o = __float2half_rn(__half2float(o) + __half2float(res[m * N + n + e]));
            }
          }
        }
        reinterpret_cast<OutT*>(gp)[e] = o;
      }
    }
  }
}

// Row tiles per group of the tile order.  With more tiles than CUs the
// groups cover 1024 rows, so the workgroups resident on one XCD at a time
// share a few activation bands and weight panels in its L2.  With at most one
// tile per CU every XCD holds its whole range at once, and the range is the
// block of a row tiles by ceil(T / 8 / a) column tiles; a minimises that
// block's operand rows with the activation rows weighted 4x.  The activation
// operand is usually written by the preceding launch (the prologue), so each
// XCD fetches it from beyond its L2, while every XCD's weight panel is read
// by that XCD alone.  Measured on the pages' six layer shapes at M = 1024
// (prologue then GEMM, graph-replayed): the dependent pair is 3.6 to 9.5 %
// faster than with the 1024-row groups on five shapes and unchanged on the
// sixth, and the weighting picks the best measured a on each.
int64_t choose_group_m(int64_t tiles_m, int64_t tiles_n, int BM, int BN) {
  const int64_t wide = BM >= 1024 ? 1 : 1024 / BM;
  const int64_t T = tiles_m * tiles_n;
  if (T > 256) return wide;
  const int64_t per = (T + 7) / 8;
  int64_t best = wide, best_cost = -1;
  for (int64_t a = 1; a <= tiles_m; a *= 2) {
    const int64_t cols = (per + a - 1) / a;
    if (cols > tiles_n) continue;
    const int64_t cost = 4 * a * BM + cols * BN;
    if (best_cost < 0 || cost < best_cost) { best = a; best_cost = cost; }
  }
  return best;
}

template <GemmMode MODE, int WAM, int WAN, int FM, int FN, int ST, bool EXTRA = false, int XS = 128>
hipError_t launch_cfg(const GemmArgs& args, hipStream_t stream) {
  constexpr int BM = 16 * FM * WAM, BN = 16 * FN * WAN;
  constexpr int kRowW = MODE == GemmMode::kW8A16 ? XS / 2 : XS;
  const int64_t tiles_m = (args.M + BM - 1) / BM, tiles_n = (args.N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  GemmArgs a = args;
  a.group_m = choose_group_m(tiles_m, tiles_n, BM, BN);
  // Rows banded by XCD (one tile per CU, M a whole number of row tiles): with
  // 8k row tiles XCD x takes one group of k of them, exactly the rows its own
  // L2 wrote; with 1, 2 or 4 it takes row tile floor(x tiles_m / 8), which
  // holds its band (N x K = 8192 x 2048 at M = 1024: 27.5 -> 27.1 us).
  if (args.xcd_row_bands && args.M % BM == 0 && tiles <= 256 && tiles % 8 == 0 && args.kc == 0) {
    if (tiles_m % 8 == 0) a.group_m = tiles_m / 8;
    else if (8 % tiles_m == 0) a.group_m = 1;
  }
  const size_t lds = (size_t)ST * ((size_t)BM * XS + (size_t)BN * kRowW);
  auto fn = &gemm_dma_kernel<MODE, WAM, WAN, FM, FN, ST, XS, EXTRA>;
  if (lds > 160 * 1024) return hipErrorInvalidValue;   // more than one CU's LDS
  if (const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(fn), lds); e != hipSuccess) return e;
  const unsigned splits = a.kc ? (unsigned)(a.K / a.kc) : 1u;
  hipLaunchKernelGGL(fn, dim3((unsigned)tiles, splits), dim3(64 * WAM * WAN), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

// Configuration table: id -> (wave grid, fragments per wave, pipeline depth,
// K slice bytes); output tile = (16 FM WAVES_M) x (16 FN WAVES_N) in (M, N).
// Only the configurations choose_gemm_cfg dispatches to are built (ids of
// configurations measured and dropped are not reused).  A residual, a LoRA,
// row exponents or a bf16 output select the kernels compiled with those
// epilogue steps, so the plain kernels carry none of their registers or code.
template <GemmMode MODE>
hipError_t launch_gemm_dma_cfg(const GemmArgs& a, int cfg, hipStream_t stream) {
  const bool extra = a.R || a.t_ld > 0 || a.rowexp || a.out_bf16;
  if constexpr (MODE == GemmMode::kI8toF16 || MODE == GemmMode::kW8A16) {
    if (extra) {
      switch (cfg) {
        case 8: return launch_cfg<MODE, 2, 2, 4, 2, 4, true>(a, stream);
        case 9: return launch_cfg<MODE, 2, 2, 1, 2, 4, true>(a, stream);
        case 10: return launch_cfg<MODE, 2, 2, 2, 2, 4, true>(a, stream);
        case 13: return launch_cfg<MODE, 4, 2, 4, 4, 3, true>(a, stream);
        case 21: return launch_cfg<MODE, 4, 2, 4, 4, 3, true>(a, stream);   // extras: the 256x128 tile
        case 19: return launch_cfg<MODE, 2, 2, 1, 1, 4, true, 256>(a, stream);
        case 22:
          if constexpr (MODE == GemmMode::kI8toF16) return launch_cfg<MODE, 4, 2, 2, 2, 4, true, 128>(a, stream);
          return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
      }
    }
  } else {
    if (extra) return hipErrorInvalidValue;
  }
  switch (cfg) {
    case 8: return launch_cfg<MODE, 2, 2, 4, 2, 4>(a, stream);   // 128x64, 4 waves of 64x32
    case 9: return launch_cfg<MODE, 2, 2, 1, 2, 4>(a, stream);   // 32x64
    case 10: return launch_cfg<MODE, 2, 2, 2, 2, 4>(a, stream);  // 64x64
    case 13: return launch_cfg<MODE, 4, 2, 4, 4, 3>(a, stream);  // 256x128, 8 waves of 64x64
    case 21:   // 128x128, 4 waves of 64x64, 2 stages (64 KiB: two workgroups per CU), fp16 output
      if constexpr (MODE == GemmMode::kI8toF16)
        return launch_cfg<MODE, 2, 2, 4, 4, 2>(a, stream);
      return hipErrorInvalidValue;
    case 19: return launch_cfg<MODE, 2, 2, 1, 1, 4, false, 256>(a, stream);  // 32x32, 256-byte K slices
    case 20:   // 128x64, 8 waves of 32x32, 256-byte K slices on 3 stages: fp16 product
      if constexpr (MODE == GemmMode::kF16) return launch_cfg<MODE, 4, 2, 2, 2, 3, false, 256>(a, stream);
      return hipErrorInvalidValue;
    case 22:   // 128x64, 8 waves of 32x32, 128-byte K slices on 4 stages: int8 products
      if constexpr (MODE == GemmMode::kI8toF16 || MODE == GemmMode::kI8toI32)
        return launch_cfg<MODE, 4, 2, 2, 2, 4, false, 128>(a, stream);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template hipError_t launch_gemm_dma_cfg<GemmMode::kI8toI32>(const GemmArgs&, int, hipStream_t);
template hipError_t launch_gemm_dma_cfg<GemmMode::kI8toF16>(const GemmArgs&, int, hipStream_t);
template hipError_t launch_gemm_dma_cfg<GemmMode::kF16>(const GemmArgs&, int, hipStream_t);
template hipError_t launch_gemm_dma_cfg<GemmMode::kW8A16>(const GemmArgs&, int, hipStream_t);

}  // namespace convrot
