// Host-side launchers of the INT8ConvRot kernels (internal to the library).
#pragma once

#include "common.hpp"

namespace convrot {

enum class GemmMode { kI8toI32, kI8toF16, kF16, kW8A16 };

struct GemmArgs {
  const void* X;        // [M, K] int8 (kI8*) or fp16
  const void* W;        // [N, K] int8 (kI8*, kW8A16) or fp16 (kF16)
  const float* sX;      // [M]   (kI8toF16)
  const float* sW;      // [N]   (kI8toF16, kW8A16)
  const float* bias;    // [N] or null (kI8toF16, kW8A16, kF16)
  const __half* R;      // [M, N] fp16 residual added to the fp16 output (kI8toF16), or null
  const __half* T;      // [M, t_ld] fp16 LoRA activation X down^T (kI8toF16, kW8A16)
  const __half* U;      // [N, t_ld] fp16 LoRA up weight U' = fp16(scale * up), zero past the rank
  int t_ld;             // LoRA rank rounded up to 32 (0 = no LoRA)
  const int* rowexp;    // [M] power of two per row to restore (range-safe kW8A16), or null
  int out_bf16;         // kW8A16: output (and residual) bf16 instead of fp16
  void* out;            // [M, N] int32 or fp16; with kc: [K / kc, M, N] int32 partials
  int64_t M, N, K;
  int64_t kc;           // 0, or K per split (kI8toI32 only; a multiple of 256 dividing K)
  int64_t group_m;      // row tiles per group of the tile order (set by the launcher)
  int xcd_row_bands;    // 1: the activation rows were written in 8 bands of M / 8 rows, band x by the
                        // workgroups on XCD x (launch_act_quant with banded); the tile order then gives XCD x
                        // the same rows where the tiles allow it (a hint: any value is correct)
};

template <GemmMode MODE>
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);

// Pipelined direct-to-LDS GEMM (every mode) with an explicit tile
// configuration id, and the id the library picks for a problem size.
template <GemmMode MODE>
hipError_t launch_gemm_dma_cfg(const GemmArgs& a, int cfg, hipStream_t stream);
int choose_gemm_cfg(GemmMode mode, int64_t M, int64_t N, int64_t K);

// Few-row W8A8 product (M <= 16): K ranges for a size, and the launch
// (parts == nullptr: one range and the scale epilogue [+ bias, residual] in
// the kernel; else int32 partials [splits, M, N] for launch_splitk_epilogue).
int64_t skinny_splits(int64_t M, int64_t N, int64_t K);
hipError_t launch_skinny(const GemmArgs& a, int64_t splits, int32_t* parts, hipStream_t stream);
// The whole W8A8 layer in one launch for M K <= 8192 (every workgroup
// quantises the activations X fp16 [M, K] itself); a.X is unused.
bool skinny_fusable(int64_t M, int64_t K);
hipError_t launch_skinny_fused(const GemmArgs& a, const void* X, hipStream_t stream);

// The whole W8A8 layer in one launch for K = 256 (each row one rotation
// group), 16 < M <= 2048 and N a multiple of 4: every workgroup quantises
// its band of 32 rows itself; a.X and a.sX are unused, X is the fp16
// activation [M, 256].
bool band_fusable(int64_t M, int64_t N, int64_t K);
hipError_t launch_band(const GemmArgs& a, const void* X, hipStream_t stream);
// The whole W8A8 layer in one launch for narrow layers: K = 512 or 1024,
// M > 16, 4 <= N <= 256 with N % 4 == 0, and ceil(M / 8) ceil(N / 128) <= 256
// workgroups; each quantises its band of 8 rows itself (a.X and a.sX are
// unused, X is the fp16 activation [M, K]).
bool narrow_fusable(int64_t M, int64_t N, int64_t K);
hipError_t launch_narrow(const GemmArgs& a, const void* X, hipStream_t stream);

// Split-K plan of the W8A8 tiled-GEMM path with few rows (M <= 128; 1 = no
// split, always for more rows).
int64_t w8a8_splits(int64_t M, int64_t N, int64_t K);

// How the W8A8 linear runs for a size: one fused launch (few rows, short
// rows, no LoRA), one fused launch over row bands (K = 256, or narrow layers
// with K = 512 / 1024; no LoRA), the
// prologue and the few-row kernel (M <= 8, N <= 4096), or the prologue and
// the tiled GEMM; `parts` says whether int32 partials [splits, M, N] go
// through the workspace to the K-split epilogue.
struct W8A8Plan {
  enum Kind { kFused, kBand, kNarrow, kSkinny, kGemm } kind;
  int64_t splits;
  bool parts;
};
W8A8Plan w8a8_plan(int64_t M, int64_t N, int64_t K, bool lora);
// Y = fp16(fp32(sum_z A_z) * fp32(s_X s_W) [+ bias]) from the int32 partials,
// then the optional LoRA term (a.T, a.U, a.t_ld) before the fp16 rounding and
// the optional residual a.R after it.
hipError_t launch_splitk_epilogue(const int32_t* parts, int64_t splits, const GemmArgs& a,
                                  hipStream_t stream);

// Dequantise-every-call baseline: W16 fp16 [N, K] = fp16((Q_W (.) s_W) H).
hipError_t launch_dequantize(const int8_t* QW, const float* sW, int64_t N, int64_t K, void* W16,
                             hipStream_t stream);
hipError_t launch_quantize_weights(const float* W, int64_t N, int64_t K, int8_t* QW, float* sW,
                                   hipStream_t stream);
// Activation prologues.  With banded != null the row blocks are assigned by
// XCD where the whole grid is resident and M splits into 8 equal bands of
// blocks: workgroup b (on XCD b mod 8) takes block (b mod 8) (blocks / 8) +
// b / 8, so XCD x writes rows [x M / 8, (x + 1) M / 8); *banded tells whether
// it did (GemmArgs::xcd_row_bands).  The results are the same either way.
hipError_t launch_act_quant(const void* X, int64_t M, int64_t K, int8_t* QX, float* sX,
                            hipStream_t stream, bool* banded = nullptr);
hipError_t launch_act_rotate_f16(const void* X, int64_t M, int64_t K, void* X16,
                                 hipStream_t stream, bool* banded = nullptr);
// Range-safe weight-only prologue: X fp16 or bf16 [M, K] -> X16 = fp16(X H 2^-e) and e [M].
hipError_t launch_act_rotate_scaled(const void* X, bool bf16, int64_t M, int64_t K, void* X16,
                                    int* rowexp, hipStream_t stream, bool* banded = nullptr);

// LoRA operands of the GEMM epilogue: T fp16 [M, t_ld] = X down^T and
// U' fp16 [N, t_ld] = fp16(scale * up) (columns past the rank zero).  K is
// split into lora_splits(K) ranges; with more than one, the fp32 partial sums
// P [splits, M, t_ld] go through the workspace.
int64_t lora_splits(int64_t K);
hipError_t launch_lora_prep(const void* X, const float* down, const float* up, float scale, int64_t M,
                            int64_t N, int64_t K, int rank, int t_ld, float* P, __half* T, __half* U,
                            hipStream_t stream);
// T = fp16(sum of the K ranges' partial sums P, in range order).
hipError_t launch_lora_sum(const float* P, int64_t splits, int64_t M, int t_ld, int rank, __half* T,
                           hipStream_t stream);
// The prologue (Q_X, s_X; or X16 = fp16(X H) with rotate_f16) and the LoRA
// down projection (T, U', the same values as launch_lora_prep) in one launch
// where the prologue runs 256-thread workgroups (K <= 4096), else in two.
hipError_t launch_act_quant_lora(const void* X, int64_t M, int64_t K, int8_t* QX, float* sX, const float* down,
                                 const float* up, float scale, int64_t N, int rank, int t_ld, float* P, __half* T,
                                 __half* U, hipStream_t stream, bool* banded = nullptr);
hipError_t launch_act_rotate_f16_lora(const void* X, int64_t M, int64_t K, void* X16, const float* down,
                                      const float* up, float scale, int64_t N, int rank, int t_ld, float* P,
                                      __half* T, __half* U, hipStream_t stream, bool* banded = nullptr);

// Lets kernel `fn` use `bytes` of dynamic LDS on the current device (above
// the 64 KiB default), calling hipFuncSetAttribute only when this kernel has
// not yet been allowed that much on this device.
hipError_t allow_dynamic_lds(const void* fn, size_t bytes);
// Workgroups of kernel `fn` (with `threads` threads and `lds` bytes of
// dynamic LDS) that the current device holds at once: CUs x workgroups per
// CU (remembered per kernel, device and size).
hipError_t resident_grid(const void* fn, int threads, size_t lds, int64_t* wgs);

// Empty contractions (K = 0).  Y [M, N] = +0 + bias[n] (or +0) rounded to
// the output type, then the residual R (same type, may be Y) added once;
// int32 output: all zero.  fill32 writes n copies of a 32-bit word.
enum EmptyOut { kEmptyF16 = 0, kEmptyBF16 = 1, kEmptyI32 = 2 };
hipError_t launch_empty_linear(int64_t M, int64_t N, const float* bias, const void* R, EmptyOut out, void* Y,
                               hipStream_t stream);
hipError_t launch_fill32(void* p, int64_t n, uint32_t value, hipStream_t stream);

}  // namespace convrot
