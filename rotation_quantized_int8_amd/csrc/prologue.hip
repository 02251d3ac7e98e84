// Activation prologue: X_rot = X H per 256-group, s_X = row max / 127,
// Q_X = round(X_rot / s_X) -- or, for the weight-only path, X16 = fp16(X H),
// or, range-safe, X16 = fp16(X H 2^-e) with a power of two per row.
//
// Page "INT8ConvRot GEMM vs fp16 on M1 Max with Metal, MPSMatrix, and MLX
// (fp16 Wins)", section "What changed in the computation": activation
// equation (every call) and the weight-only listing (x_rot kept in fp16);
// page "[PR #249] Add an mps backend ...", section "Design": the range-safe
// prologue divides each row by an exact power of two so that its rotated
// maximum is at most 1.
//
// The rotation (exact fp64 butterflies, one rounding) and the quantisation
// are the device functions of rotate.hpp.

// Work split.  G = K/256 groups per row.  K <= 4096: a row block of
// floor(16/G) rows per 256-thread workgroup; K <= 16384: one row per block,
// 16*G threads.  These whole-row blocks run in a persistent grid
// (prologue_persistent_kernel) that loads the next block while it works on
// the current one.  Longer rows (prologue_kernel): 1024 threads walk the row
// in chunks of 64 groups twice (maximum, then quantise or scale),
// recomputing the transform instead of holding the row.

#include "launch.hpp"
#include "lora_body.hpp"
#include "rotate.hpp"

namespace convrot {
namespace {

struct Split {
  int rows_per_wg;   // rows handled by one workgroup
  int gpc;           // groups per chunk (groups of one row handled at once)
  int chunks;        // chunks per row
  int xcd_band;      // persistent kernel: block of workgroup b is (b % 8) (grid / 8) + b / 8
};

enum PrologueMode { kQuantInt8 = 0, kRotateF16 = 1, kRotateScaledF16 = 2 };

// Row maximum of non-negative doubles across 16-lane segments: the bit
// patterns of non-negative doubles order like unsigned integers.
__device__ __forceinline__ double seg_max_f64(double v) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) v = fmax(v, __shfl_xor(v, m));
  return v;
}

// kQuantInt8: Q_X, s_X.  kRotateF16: X16 = fp16(X H).  kRotateScaledF16 (range
// safe, [P4] "Design"): X16 = fp16(X H 2^-e) with e the smallest integer such
// that the row's max |X H| <= 2^e (0 for a zero row), and e per row.  kBF16:
// the input is bf16 (kRotateScaledF16 only).
template <int kMode, bool kBF16>
__global__ void __launch_bounds__(1024)
prologue_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K, Split sp,
                int8_t* __restrict__ QX, float* __restrict__ sX, __half* __restrict__ X16,
                int* __restrict__ rowexp) {
  extern __shared__ __align__(16) char smem[];
  __shared__ uint32_t rowmax[16];             // per row: max |fp32(16 X_rot)| as bits (non-negative: uint order)
  __shared__ unsigned long long rowmax64[16]; // the same as fp64 bits (row-scaled mode)

  const int tid = threadIdx.x;
  const int slot_id = tid >> 4;     // group slot in the workgroup
  const int lane = tid & 15;        // lane within the group
  const int G = (int)(K / kGroup);
  const int row_in_wg = slot_id / sp.gpc;
  const int gi = slot_id - row_in_wg * sp.gpc;       // group index inside a chunk
  const int64_t row = (int64_t)blockIdx.x * sp.rows_per_wg + row_in_wg;
  const bool active = row_in_wg < sp.rows_per_wg && row < M;
  char* slot = smem + slot_id * kSlotBytes;

  const uint16_t* xrow = X + row * K;
  double y[16];
  float f[16];

  if (kMode == kQuantInt8 && tid < 16) rowmax[tid] = 0u;
  if (kMode == kRotateScaledF16 && tid < 16) rowmax64[tid] = 0ull;
  if constexpr (kMode == kRotateF16) {
    // Weight-only path: no row scale, just fp16(X H) per group.
    if (active) {
      for (int c = 0; c < sp.chunks; ++c) {
        const int g = c * sp.gpc + gi;
        if (g >= G) break;
        rotate_group<kBF16>(xrow + (int64_t)g * kGroup, slot, lane, y);
        __half h[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) h[i] = f64_to_f16_rn(y[i] * 0.0625);
        uint4* dst = reinterpret_cast<uint4*>(X16 + row * K + (int64_t)g * kGroup + 16 * lane);
        dst[0] = *reinterpret_cast<const uint4*>(&h[0]);
        dst[1] = *reinterpret_cast<const uint4*>(&h[8]);
      }
    }
    return;
  }

  if constexpr (kMode == kRotateScaledF16) {
    __syncthreads();   // rowmax64 cleared
    // pass 1: transform, keep the values when the row fits in one chunk, take max
    double amax = 0.0;
    if (active) {
      for (int c = 0; c < sp.chunks; ++c) {
        const int g = c * sp.gpc + gi;
        if (g >= G) break;
        rotate_group<kBF16>(xrow + (int64_t)g * kGroup, slot, lane, y);
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmax(amax, fabs(y[i] * 0.0625));
      }
    }
    amax = seg_max_f64(amax);
    if (active && lane == 0) atomicMax(&rowmax64[row_in_wg], (unsigned long long)__double_as_longlong(amax));
    __syncthreads();
    if (!active) return;
    // e: max = 1.f 2^ex (normal double) -> e = ex, or ex + 1 when f > 0
    const unsigned long long mb = rowmax64[row_in_wg];
    int e = 0;
    if (mb != 0ull) {
      const int ex = (int)((mb >> 52) & 0x7FF) - 1023;
      e = (mb & ((1ull << 52) - 1)) == 0ull ? ex : ex + 1;
    }
    const double down = ldexp(0.0625, -e);   // exact power of two
    if (slot_id == row_in_wg * sp.gpc && lane == 0) rowexp[row] = e;
    // pass 2: scale, round once to fp16, store
    for (int c = 0; c < sp.chunks; ++c) {
      const int g = c * sp.gpc + gi;
      if (g >= G) break;
      if (sp.chunks > 1) rotate_group<kBF16>(xrow + (int64_t)g * kGroup, slot, lane, y);
      __half h[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) h[i] = f64_to_f16_rn(y[i] * down);
      uint4* dst = reinterpret_cast<uint4*>(X16 + row * K + (int64_t)g * kGroup + 16 * lane);
      dst[0] = *reinterpret_cast<const uint4*>(&h[0]);
      dst[1] = *reinterpret_cast<const uint4*>(&h[8]);
    }
    return;
  }

  __syncthreads();   // rowmax cleared
  // pass 1: transform, keep the values when the row fits in one chunk, take max
  float amax = 0.0f;
  if (active) {
    for (int c = 0; c < sp.chunks; ++c) {
      const int g = c * sp.gpc + gi;
      if (g >= G) break;
      rotate_group<kBF16>(xrow + (int64_t)g * kGroup, slot, lane, y);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        f[i] = (float)y[i];   // fp32(16 X_rot): the single rounding
        amax = fmaxf(amax, fabsf(f[i]));
      }
    }
  }
  // row maximum: within each 16-lane segment, then one LDS atomic per segment
  const uint32_t amax_bits = seg_max16_bits(__float_as_uint(amax));
  if (active && lane == 0) atomicMax(&rowmax[row_in_wg], amax_bits);
  __syncthreads();
  if (!active) return;
  // The factor 16 of the unnormalised transform stays in the values: with
  // F = fp32(16 X_rot) = 16 fp32(X_rot) and S = fp32(max|F|) / 127 (IEEE fp32
  // division) = 16 s_X -- scaling by 2^4 commutes with fp32 rounding, every
  // nonzero value here being at least 2^-35, far above the subnormals --
  // F / S equals X_rot / s_X exactly, so the codes are the same.
  const float s = __uint_as_float(rowmax[row_in_wg]) / 127.0f;
  if (slot_id == row_in_wg * sp.gpc && lane == 0) sX[row] = s * 0.0625f;   // exact

  // pass 2: quantise and store
  for (int c = 0; c < sp.chunks; ++c) {
    const int g = c * sp.gpc + gi;
    if (g >= G) break;
    if (sp.chunks > 1) {
      rotate_group<kBF16>(xrow + (int64_t)g * kGroup, slot, lane, y);
#pragma unroll
      for (int i = 0; i < 16; ++i) f[i] = (float)y[i];
    }
    const uint4 packed = quantize16(f, s);
    *reinterpret_cast<uint4*>(QX + row * K + (int64_t)g * kGroup + 16 * lane) = packed;
  }
}

// Rows of at most 16384 values (one chunk per row), every mode, as a
// persistent grid: a workgroup walks row blocks b, b + grid, ... and
// issues the loads of its next block before it rotates (and, with a row
// scale, reduces and quantises or scales) the current one, so at large M
// the memory traffic of one block overlaps the vector work of the previous
// one.  Row maxima of iteration i go through LDS buffer i % 3; buffer
// (i + 2) % 3 is cleared after the iteration's barrier, which every thread
// passes only after its last read of that buffer (iteration i - 1) and
// before its next atomic on it (iteration i + 2, behind the barrier of
// iteration i + 1).  Arithmetic as in prologue_kernel.
// One workgroup of the persistent prologue: block `bid` of a grid of `grid`
// workgroups walks row blocks bid, bid + grid, ...  `smem` holds the slots,
// rowmax / rowmax64 the three buffers of row maxima.
template <int kMode, bool kBF16>
__device__ __forceinline__ void prologue_persistent_block(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                          Split sp, int8_t* __restrict__ QX,
                                                          float* __restrict__ sX, __half* __restrict__ X16,
                                                          int* __restrict__ rowexp, int64_t bid, int64_t grid,
                                                          char* smem, uint32_t (*rowmax)[16],
                                                          unsigned long long (*rowmax64)[16]) {
  const int tid = threadIdx.x;
  const int slot_id = tid >> 4;       // group slot in the workgroup
  const int lane = tid & 15;          // lane within the group
  const int row_in_wg = slot_id / sp.gpc;
  const int gi = slot_id - row_in_wg * sp.gpc;   // group of the row (one chunk: all of them)
  const bool in_wg = row_in_wg < sp.rows_per_wg;
  char* slot = smem + slot_id * kSlotBytes;
  const int64_t blocks = (M + sp.rows_per_wg - 1) / sp.rows_per_wg;

  if (kMode == kQuantInt8 && tid < 48) rowmax[tid >> 4][tid & 15] = 0u;
  if (kMode == kRotateScaledF16 && tid < 48) rowmax64[tid >> 4][tid & 15] = 0ull;
  __syncthreads();

  auto has_row = [&](int64_t b) { return in_wg && b < blocks && b * sp.rows_per_wg + row_in_wg < M; };
  // Loads are issued by every lane, unconditionally, so that the compiler
  // counts them exactly and waits only for the block it is about to use:
  // lanes without a row of block b read the last row of the matrix instead
  // (in bounds, never used).  Element offsets advance by one grid stride of
  // rows per step; the clamp to the last row is a minimum of offsets (they
  // grow with the row), taken before the offset becomes an address.
  const int rclamp = row_in_wg < sp.rows_per_wg ? row_in_wg : sp.rows_per_wg - 1;
  const int64_t lane_off = (int64_t)gi * kGroup + 16 * lane;          // elements
  const int64_t stride = grid * sp.rows_per_wg * K;     // elements per step
  const int64_t x_last = (M - 1) * K + lane_off;
  int64_t x_next = (bid * sp.rows_per_wg + rclamp) * K + lane_off;
  auto src = [&](int64_t off) { return reinterpret_cast<const v4i*>(X + (off < x_last ? off : x_last)); };
  int64_t out_off = (bid * sp.rows_per_wg + row_in_wg) * K + lane_off;   // current block's row
  // Block b's data (r0, r1) is parked in the segment's LDS slot first; then
  // the same registers receive the loads of block b + grid, which are in
  // flight while block b is rotated and quantised.  A block's results are
  // held in registers and stored one iteration later, right after the next
  // loads go out: whatever the compiler makes the next iteration wait for
  // (it cannot count stores under a branch, so it waits for all memory
  // operations) was then issued a whole block of work earlier.
  uint4 pend[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  bool pend_active = false;
  int64_t pend_row = 0;
  int64_t pend_off = 0;   // element offset of the held row's 16 values
  float pend_s = 0.0f;   // s_X of the held row (kQuantInt8)
  int pend_e = 0;        // exponent of the held row (kRotateScaledF16)
  auto flush = [&]() {
    if (!pend_active) return;
    if constexpr (kMode == kQuantInt8) {
      *reinterpret_cast<uint4*>(QX + pend_off) = pend[0];
      if (gi == 0 && lane == 0) sX[pend_row] = pend_s;
    } else {
      uint4* dst = reinterpret_cast<uint4*>(X16 + pend_off);
      dst[0] = pend[0];
      dst[1] = pend[1];
      if (kMode == kRotateScaledF16 && gi == 0 && lane == 0) rowexp[pend_row] = pend_e;
    }
  };

  v4i r0 = __builtin_nontemporal_load(src(x_next));
  v4i r1 = __builtin_nontemporal_load(src(x_next) + 1);
  int it = 0;
  for (int64_t b = bid; b < blocks; b += grid, ++it) {   // uniform trip count
    const bool active = has_row(b);
    const int64_t row = b * sp.rows_per_wg + row_in_wg;
    if (active) park_row(slot, lane, r0, r1);
    x_next += stride;
    r0 = __builtin_nontemporal_load(src(x_next));
    r1 = __builtin_nontemporal_load(src(x_next) + 1);
    flush();
    pend_active = active;
    pend_row = row;
    pend_off = out_off;
    out_off += stride;
    double y[16];
    if (active) rotate_staged<kBF16>(slot, lane, y);
    if constexpr (kMode == kRotateF16) {
      // weight-only: fp16(X H) per group, no row scale
      if (active) {
        __half h[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) h[i] = f64_to_f16_rn(y[i] * 0.0625);
        pend[0] = *reinterpret_cast<const uint4*>(&h[0]);
        pend[1] = *reinterpret_cast<const uint4*>(&h[8]);
      }
    } else if constexpr (kMode == kRotateScaledF16) {
      // range safe: e = the smallest integer with max |X_rot| <= 2^e (0 for a
      // zero row), X16 = fp16(X_rot 2^-e) rounded once
      double amax = 0.0;
      if (active) {
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmax(amax, fabs(y[i] * 0.0625));
      }
      amax = seg_max_f64(amax);
      unsigned long long* rm = rowmax64[it % 3];
      if (active && lane == 0) atomicMax(&rm[row_in_wg], (unsigned long long)__double_as_longlong(amax));
      __syncthreads();
      if (tid < 16) rowmax64[(it + 2) % 3][tid] = 0ull;
      if (active) {
        const unsigned long long mb = rm[row_in_wg];
        int e = 0;
        if (mb != 0ull) {
          const int ex = (int)((mb >> 52) & 0x7FF) - 1023;
          e = (mb & ((1ull << 52) - 1)) == 0ull ? ex : ex + 1;
        }
        const double down = ldexp(0.0625, -e);   // exact power of two
        __half h[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) h[i] = f64_to_f16_rn(y[i] * down);
        pend[0] = *reinterpret_cast<const uint4*>(&h[0]);
        pend[1] = *reinterpret_cast<const uint4*>(&h[8]);
        pend_e = e;
      }
    } else {
      float f[16];
      float amax = 0.0f;
      if (active) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          f[i] = (float)y[i];   // fp32(16 X_rot): the single rounding
          amax = fmaxf(amax, fabsf(f[i]));
        }
      }
      const uint32_t amax_bits = seg_max16_bits(__float_as_uint(amax));
      uint32_t* rm = rowmax[it % 3];
      if (active && lane == 0) atomicMax(&rm[row_in_wg], amax_bits);
      __syncthreads();
      if (tid < 16) rowmax[(it + 2) % 3][tid] = 0u;
      if (active) {
        // S = fp32(max|16 X_rot|) / 127 = 16 s_X exactly; F / S = X_rot / s_X
        const float sc = __uint_as_float(rm[row_in_wg]) / 127.0f;
        pend_s = sc * 0.0625f;
        pend[0] = quantize16(f, sc);
      }
    }
  }
  flush();
}


template <int kMode, bool kBF16>
__global__ void __launch_bounds__(1024)
prologue_persistent_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K, Split sp,
                           int8_t* __restrict__ QX, float* __restrict__ sX, __half* __restrict__ X16,
                           int* __restrict__ rowexp) {
  extern __shared__ __align__(16) char smem[];
  __shared__ uint32_t rowmax[3][16];            // kQuantInt8: max |fp32(16 X_rot)| bits (uint order)
  __shared__ unsigned long long rowmax64[3][16];  // kRotateScaledF16: max |X_rot| as fp64 bits
  // XCD bands: workgroup b runs on XCD b % 8; with a grid of one block per
  // workgroup (a multiple of 8) XCD x then takes the x-th eighth of the blocks
  const int64_t b = blockIdx.x;
  const int64_t bid = sp.xcd_band ? (b & 7) * (int64_t)(gridDim.x >> 3) + (b >> 3) : b;
  prologue_persistent_block<kMode, kBF16>(X, M, K, sp, QX, sX, X16, rowexp, bid, gridDim.x, smem, rowmax,
                                          rowmax64);
}

// The prologue and the LoRA down projection in one launch: both read only X,
// so neither waits for the other.  Workgroups 0 .. pgrid - 1 run the
// persistent prologue (256 threads: rows of at most 16 groups), the rest
// the down projection's (row blocks + up blocks) x splits workgroups.
struct LoraJob {
  const float* down;
  const float* up;
  float scale;
  int64_t N;
  int rank;
  int64_t kc, bx_count, splits;
  float* P;
  __half* T;
  __half* U;
};

template <int kMode, int NFR>
__global__ void __launch_bounds__(256)
prologue_lora_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K, Split sp, int8_t* __restrict__ QX,
                     float* __restrict__ sX, __half* __restrict__ X16, int64_t pgrid, LoraJob lj) {
  extern __shared__ __align__(16) char smem[];
  __shared__ uint32_t rowmax[3][16];
  __shared__ unsigned long long rowmax64[3][16];
  const int64_t b = blockIdx.x;
  if (b < pgrid) {
    const int64_t bid = sp.xcd_band ? (b & 7) * (pgrid >> 3) + (b >> 3) : b;   // XCD bands, as above
    prologue_persistent_block<kMode, false>(X, M, K, sp, QX, sX, X16, nullptr, bid, pgrid, smem, rowmax, rowmax64);
    return;
  }
  const int64_t l = b - pgrid;
  int64_t bx = l % lj.bx_count, by = l / lj.bx_count;
  if (sp.xcd_band) {
    // with the prologue's rows in XCD bands, the down projection's row jobs
    // (row block, K range) of band x go to the workgroups on XCD x (b % 8 =
    // l % 8: pgrid is a multiple of 8), the up-weight blocks after them
    const int64_t rb = (M + kLoraRows - 1) / kLoraRows, per_band = rb >> 3, R = rb * lj.splits;
    if (l < R) {
      const int64_t i = l >> 3;
      bx = (l & 7) * per_band + i % per_band;
      by = i / per_band;
    } else {
      const int64_t ub = lj.bx_count - rb, u = l - R;
      bx = rb + u % ub;
      by = u / ub;
    }
  }
  lora_down_block<NFR>(reinterpret_cast<const __half*>(X), lj.down, lj.up, lj.scale, M, lj.N, K, lj.rank, lj.kc, lj.P,
                       lj.T, lj.U, bx, by, lj.splits, smem);
}

Split choose_split(int64_t K) {
  const int G = (int)(K / kGroup);
  Split sp;
  sp.xcd_band = 0;
  if (G <= 16) {
    sp.rows_per_wg = 16 / G;
    sp.gpc = G;
    sp.chunks = 1;
  } else if (G <= 64) {
    sp.rows_per_wg = 1;
    sp.gpc = G;
    sp.chunks = 1;
  } else {
    sp.rows_per_wg = 1;
    sp.gpc = 64;
    sp.chunks = (G + 63) / 64;
  }
  return sp;
}

// banded != null: assign the row blocks by XCD where the grid holds every
// block once and the blocks split into 8 equal bands; *banded tells whether.
template <int kMode, bool kBF16>
hipError_t launch(const void* X, int64_t M, int64_t K, int8_t* QX, float* sX, __half* X16, int* rowexp,
                  hipStream_t stream, bool* banded = nullptr) {
  Split sp = choose_split(K);
  const int slots = sp.rows_per_wg * sp.gpc;
  const int threads = ((slots * 16 + 63) / 64) * 64;
  const int64_t blocks = (M + sp.rows_per_wg - 1) / sp.rows_per_wg;
  const size_t lds = (size_t)(threads / 16) * kSlotBytes;
  if (sp.chunks == 1) {   // whole rows: the persistent, pipelined kernel
    auto fn = &prologue_persistent_kernel<kMode, kBF16>;
    const void* f = reinterpret_cast<const void*>(fn);
    if (const hipError_t e = allow_dynamic_lds(f, lds); e != hipSuccess) return e;
    int64_t resident = 0;
    if (const hipError_t e = resident_grid(f, threads, lds, &resident); e != hipSuccess) return e;
    const int64_t grid = blocks < resident ? blocks : resident;
    if (banded) {
      *banded = grid == blocks && M % (8 * (int64_t)sp.rows_per_wg) == 0;
      sp.xcd_band = *banded ? 1 : 0;
    }
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(threads), lds, stream,
                       reinterpret_cast<const uint16_t*>(X), M, K, sp, QX, sX, X16, rowexp);
    return hipGetLastError();
  }
  if (banded) *banded = false;
  auto fn = &prologue_kernel<kMode, kBF16>;
  if (const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(fn), lds); e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(threads), lds, stream,
                     reinterpret_cast<const uint16_t*>(X), M, K, sp, QX, sX, X16, rowexp);
  return hipGetLastError();
}

}  // namespace

namespace {

template <int kMode, int NFR>
hipError_t launch_pl(const void* X, int64_t M, int64_t K, int8_t* QX, float* sX, __half* X16, Split sp,
                     LoraJob lj, hipStream_t stream, bool* banded) {
  auto fn = &prologue_lora_kernel<kMode, NFR>;
  const void* f = reinterpret_cast<const void*>(fn);
  const size_t pro_lds = (size_t)sp.rows_per_wg * sp.gpc * kSlotBytes;
  const size_t lds = pro_lds > (size_t)lora_lds_bytes(NFR) ? pro_lds : (size_t)lora_lds_bytes(NFR);
  if (const hipError_t e = allow_dynamic_lds(f, lds); e != hipSuccess) return e;
  int64_t resident = 0;
  if (const hipError_t e = resident_grid(f, 256, lds, &resident); e != hipSuccess) return e;
  const int64_t blocks = (M + sp.rows_per_wg - 1) / sp.rows_per_wg;
  const int64_t pgrid = blocks < resident ? blocks : resident;
  if (banded) {   // the down projection's 32-row blocks must split into the same 8 bands
    *banded = pgrid == blocks && M % (8 * (int64_t)sp.rows_per_wg) == 0 && M % (8 * (int64_t)kLoraRows) == 0;
    sp.xcd_band = *banded ? 1 : 0;
  }
  const int64_t total = pgrid + lj.bx_count * lj.splits;
  hipLaunchKernelGGL(fn, dim3((unsigned)total), dim3(256), lds, stream, reinterpret_cast<const uint16_t*>(X), M, K,
                     sp, QX, sX, X16, pgrid, lj);
  if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (lj.splits == 1) return hipSuccess;
  return launch_lora_sum(lj.P, lj.splits, M, 16 * NFR, lj.rank, lj.T, stream);
}

template <int kMode>
hipError_t launch_with_lora(const void* X, int64_t M, int64_t K, int8_t* QX, float* sX, __half* X16,
                            const float* down, const float* up, float scale, int64_t N, int rank, int t_ld, float* P,
                            __half* T, __half* U, hipStream_t stream, bool* banded) {
  const Split sp = choose_split(K);
  if (sp.chunks != 1 || sp.rows_per_wg * sp.gpc != 16) {   // not 256-thread workgroups: two launches
    hipError_t e;
    if constexpr (kMode == kQuantInt8)
      e = launch<kQuantInt8, false>(X, M, K, QX, sX, nullptr, nullptr, stream, banded);
    else
      e = launch<kRotateF16, false>(X, M, K, nullptr, nullptr, X16, nullptr, stream, banded);
    if (e != hipSuccess) return e;
    return launch_lora_prep(X, down, up, scale, M, N, K, rank, t_ld, P, T, U, stream);
  }
  LoraJob lj;
  lj.down = down; lj.up = up; lj.scale = scale; lj.N = N; lj.rank = rank;
  lj.splits = lora_splits(K);
  lj.kc = K / lj.splits;
  lj.bx_count = (M + kLoraRows - 1) / kLoraRows + (N + 31) / 32;
  lj.P = P; lj.T = T; lj.U = U;
  return t_ld > 32 ? launch_pl<kMode, 4>(X, M, K, QX, sX, X16, sp, lj, stream, banded)
                   : launch_pl<kMode, 2>(X, M, K, QX, sX, X16, sp, lj, stream, banded);
}

}  // namespace

hipError_t launch_act_quant_lora(const void* X, int64_t M, int64_t K, int8_t* QX, float* sX, const float* down,
                                 const float* up, float scale, int64_t N, int rank, int t_ld, float* P, __half* T,
                                 __half* U, hipStream_t stream, bool* banded) {
  return launch_with_lora<kQuantInt8>(X, M, K, QX, sX, nullptr, down, up, scale, N, rank, t_ld, P, T, U, stream,
                                      banded);
}

hipError_t launch_act_rotate_f16_lora(const void* X, int64_t M, int64_t K, void* X16, const float* down,
                                      const float* up, float scale, int64_t N, int rank, int t_ld, float* P,
                                      __half* T, __half* U, hipStream_t stream, bool* banded) {
  return launch_with_lora<kRotateF16>(X, M, K, nullptr, nullptr, reinterpret_cast<__half*>(X16), down, up, scale, N,
                                      rank, t_ld, P, T, U, stream, banded);
}

hipError_t launch_act_quant(const void* X, int64_t M, int64_t K, int8_t* QX, float* sX,
                            hipStream_t stream, bool* banded) {
  return launch<kQuantInt8, false>(X, M, K, QX, sX, nullptr, nullptr, stream, banded);
}

hipError_t launch_act_rotate_f16(const void* X, int64_t M, int64_t K, void* X16,
                                 hipStream_t stream, bool* banded) {
  return launch<kRotateF16, false>(X, M, K, nullptr, nullptr, reinterpret_cast<__half*>(X16), nullptr,
                                   stream, banded);
}

hipError_t launch_act_rotate_scaled(const void* X, bool bf16, int64_t M, int64_t K, void* X16,
                                    int* rowexp, hipStream_t stream, bool* banded) {
  if (bf16)
    return launch<kRotateScaledF16, true>(X, M, K, nullptr, nullptr, reinterpret_cast<__half*>(X16), rowexp,
                                          stream, banded);
  return launch<kRotateScaledF16, false>(X, M, K, nullptr, nullptr, reinterpret_cast<__half*>(X16), rowexp,
                                         stream, banded);
}

}  // namespace convrot
