/*
 * convrot.h -- C ABI of the INT8ConvRot linear layer for AMD MI355X (gfx950).
 *
 * The method is the one defined on the page "INT8ConvRot GEMM vs fp16 on M1
 * Max with Metal, MPSMatrix, and MLX (fp16 Wins)", section "What changed in
 * the computation":
 *
 *   H      = (H4 (x) H4 (x) H4 (x) H4) / 16, a symmetric 256x256 matrix with
 *            HH = I, applied to the last dimension in groups of 256;
 *   weights (once):  W_rot = W H^T, s_W[n] = max_k |W_rot[n,k]| / 127,
 *                    Q_W = round(W_rot / s_W) clamped to [-128, 127];
 *   activations (every call): X_rot = X H, s_X[m] = max_k |X_rot[m,k]| / 127,
 *                    Q_X = round(X_rot / s_X) clamped to [-128, 127];
 *   A = Q_X Q_W^T accumulated in int32, Y = A (.) s_X s_W^T.
 *
 * Arithmetic contract (the pages leave precision open; this library fixes it):
 *   - H4 is Sylvester's [[1,1],[1,-1]] (x) [[1,1],[1,-1]];
 *   - W_rot and X_rot are the exact products rounded once to fp32;
 *   - s = fp32(max|v|) / 127 and Q = round_half_even(v / s), both IEEE fp32
 *     divisions; an all-zero row gives s = 0 and Q = 0;
 *   - Y = fp16( fp32(A) * fp32(s_X[m] * s_W[n]) [+ bias[n]] ), round to nearest
 *     even at every step, no fused multiply-add.
 * Under this contract Q_W, s_W, Q_X, s_X, A and the W8A8 output Y are fully
 * determined, and the library returns exactly those bits.
 *
 * Conventions for every entry point:
 *   - Tensors are dense and row-major: X, Q_X, Q_W, W and lora.down have
 *     row stride K; Y and A have row stride N; lora.up has row stride rank.
 *   - Every tensor pointer is a device pointer on the current HIP device and
 *     must be 16-byte aligned.  The caller owns every buffer; the library
 *     allocates nothing, frees nothing and keeps no state between calls
 *     beyond per-device caches of the device check, of the kernels'
 *     dynamic-LDS attributes and of how many workgroups of a kernel the
 *     device holds at once.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without synchronising.  All argument checks run on
 *     the host before anything is enqueued; on an error nothing is enqueued
 *     and no output is touched.
 *   - Sizes are int64_t.  K must be a multiple of 256 and at most 131072
 *     (so 127 * 127 * K < 2^31 and the int32 accumulator cannot overflow).
 *     M == 0 or N == 0 is a valid empty call: nothing is launched.
 *   - K == 0 is an empty contraction (page "[PR #249] Add an mps backend
 *     ...", commit list: empty contractions return early): every sum over k
 *     is empty, so A = 0, a row maximum is 0 (s_X, s_W and the range-safe
 *     exponent are 0, as for a zero row), a LoRA term is 0, and a linear
 *     writes Y = out(+0 + bias[n]) (+0 without a bias) plus its residual as
 *     usual.  Arrays with no elements (X, Q_X, Q_W, W16, X16, lora.down) are
 *     not touched and may be NULL; no workspace is needed.
 *   - Outputs must not overlap inputs or the workspace (one exception: the
 *     residual of convrot_linear_w8a8_ex may be its output buffer).
 *   - Errors are returned as status codes; nothing is printed, thrown or
 *     aborted.  A non-finite input gives unspecified (but in-bounds) output.
 *   - Calls are thread-safe; calls that share an output buffer race.
 */
#ifndef CONVROT_H
#define CONVROT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CONVROT_ABI_VERSION 1
#define CONVROT_GROUP 256
#define CONVROT_K_MAX 131072
#define CONVROT_LORA_RANK_MAX 64
/* Size of the fixed device scratch of convrot_linear_w8a8_noalloc. */
#define CONVROT_NOALLOC_SCRATCH_BYTES (32u << 20)

typedef enum convrot_status {
  CONVROT_OK = 0,
  CONVROT_ERR_INVALID_ARG = 1, /* null pointer with nonzero extent, output overlapping an input */
  CONVROT_ERR_SHAPE = 2,       /* negative size, K % 256 != 0, K > 131072, bad LoRA rank */
  CONVROT_ERR_ALIGNMENT = 3,   /* a tensor pointer not aligned to 16 bytes */
  CONVROT_ERR_DEVICE = 4,      /* current device is not gfx950 or cannot be queried */
  CONVROT_ERR_LAUNCH = 5,      /* a kernel launch reported an error */
  CONVROT_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than convrot_workspace_bytes() */
  CONVROT_ERR_TOO_LARGE = 7    /* convrot_linear_w8a8_noalloc: the problem needs more than
                                  CONVROT_NOALLOC_SCRATCH_BYTES of scratch */
} convrot_status;

typedef enum convrot_path {
  CONVROT_PATH_W8A8 = 0,
  CONVROT_PATH_W8A16 = 1,
  CONVROT_PATH_DEQUANT = 2,
  CONVROT_PATH_W8A16_RS = 3
} convrot_path;

/* 16-bit floating-point formats of the range-safe weight-only path. */
typedef enum convrot_dtype {
  CONVROT_DTYPE_F16 = 0,  /* IEEE binary16 */
  CONVROT_DTYPE_BF16 = 1  /* bfloat16: the upper half of an IEEE binary32 */
} convrot_dtype;

/* Unmerged LoRA of the int8 linears.  Page "[PR #249] Add an mps
 * backend: weight-only INT8 and W4A8/W6A8 linears for Apple GPUs", sections
 * "What" and "Design": lora_down [R, K], lora_up [N, R], lora_scale;
 * Y += scale * (X down^T) up^T. */
typedef struct convrot_lora {
  const float* down; /* device fp32 [rank, K] */
  const float* up;   /* device fp32 [N, rank] */
  int64_t rank;      /* 1 .. CONVROT_LORA_RANK_MAX */
  float scale;
} convrot_lora;

/* Version of this ABI (CONVROT_ABI_VERSION). */
int convrot_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* convrot_status_string(int status);

/* Offline weight preparation (the weight equation of "What changed in the
 * computation"): W fp32 [N, K] -> Q_W int8 [N, K] (rotated and quantised,
 * one scale per output channel) and s_W fp32 [N].  The rotation is computed
 * exactly in wide fixed point and rounded once to fp32. */
convrot_status convrot_quantize_weights(const float* W, int64_t N, int64_t K,
                                        int8_t* Q_W, float* s_W, void* stream);

/* Bytes of workspace that convrot_linear_w8a8 / convrot_linear_w8a8_ex
 * (path = CONVROT_PATH_W8A8), convrot_linear_w8a16 (path =
 * CONVROT_PATH_W8A16) or convrot_linear_dequant (path =
 * CONVROT_PATH_DEQUANT, lora_rank 0) need for these sizes, with lora_rank = 0
 * without LoRA; 0 for an empty problem (M, N or K zero), (size_t)-1 for
 * invalid sizes. */
size_t convrot_workspace_bytes(int path, int64_t M, int64_t N, int64_t K, int64_t lora_rank);

/* The W8A8 ConvRot linear ("What changed in the computation", activation
 * and product equations): X fp16 [M, K], Q_W int8 [N, K], s_W fp32 [N],
 * optional bias fp32 [N] (NULL = none) -> Y fp16 [M, N].  Runs the fused
 * rotate/absmax/quantise prologue (Q_X and s_X go to the workspace) and the
 * int8 MFMA GEMM with the scale epilogue -- or, when every row is a single
 * rotation group (K = 256, 16 < M <= 2048, N a multiple of 4), the layer is
 * narrow (K = 512 or 1024, M > 16, 4 <= N <= 256 with N a multiple of 4,
 * ceil(M / 8) ceil(N / 128) <= 256) or there are few short rows (M <= 16,
 * M K <= 8192), one launch that quantises the rows in each workgroup and
 * leaves the workspace unused.  The result is the same bits on every path. */
convrot_status convrot_linear_w8a8(const void* X, int64_t M, int64_t K,
                                   const int8_t* Q_W, const float* s_W, int64_t N,
                                   const float* bias, void* Y,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* The W8A8 ConvRot linear with the extras a model layer needs: page "[PR
 * #249] Add an mps backend ...", section "What" (the int8 linear takes an
 * unmerged LoRA: lora_down [R, K], lora_up [N, R], lora_scale) and section
 * "Design" (bias and residual added in eager's order).  Computes
 *   Y = fp16( fp32(A) * fp32(s_X[m] * s_W[n]) [+ bias[n]] [+ LoRA] )
 *   then, with a residual, Y = fp16( Y + residual[m, n] ),
 * where LoRA = scale * (X down^T) up^T.  Without a LoRA, Y is exact under the
 * arithmetic contract above (the residual step is one correctly rounded fp16
 * addition).  With a LoRA, the LoRA term is computed on fp16 MFMA with fp32
 * accumulation (down, the low-rank activation and scale * up rounded to fp16),
 * so Y matches the exact value within that term's rounding error.
 *   lora:     NULL = none; otherwise rank 1 .. CONVROT_LORA_RANK_MAX and the
 *             workspace must be sized with convrot_workspace_bytes(
 *             CONVROT_PATH_W8A8, M, N, K, rank).
 *   residual: NULL = none; otherwise device fp16 [M, N] (row stride N).  It
 *             may be Y itself (in-place update: each element is read before
 *             it is written, by the same thread) but must not otherwise
 *             overlap Y, and must not overlap the workspace.
 * With lora == NULL and residual == NULL this is convrot_linear_w8a8. */
convrot_status convrot_linear_w8a8_ex(const void* X, int64_t M, int64_t K,
                                      const int8_t* Q_W, const float* s_W, int64_t N,
                                      const float* bias, const convrot_lora* lora,
                                      const void* residual, void* Y,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* The W8A8 linear of convrot_linear_w8a8 without a caller workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments,
 * arithmetic, checks and bits as convrot_linear_w8a8 (workspace aside); the
 * caller still passes X, Q_W, s_W, the optional bias and Y.  Q_X, s_X and
 * any int32 K-split partials go to a fixed device array of
 * CONVROT_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds per GPU from
 * its load until the process ends, so this call allocates nothing.  A problem
 * whose convrot_workspace_bytes(CONVROT_PATH_W8A8, M, N, K, 0) exceeds that
 * size returns CONVROT_ERR_TOO_LARGE with nothing enqueued (e.g. M = 1024 at
 * any K <= 16384 fits; M * K of more than about 32 Mi does not).  Every call
 * on one GPU shares that GPU's array: calls that overlap in time on one GPU
 * (on different streams, or from several threads without ordering) race and
 * give undefined results; order them on one stream or with events. */
convrot_status convrot_linear_w8a8_noalloc(const void* X, int64_t M, int64_t K,
                                           const int8_t* Q_W, const float* s_W, int64_t N,
                                           const float* bias, void* Y, void* stream);

/* The weight-only (W8A16) ConvRot linear: the weight-only listing of "What
 * changed in the computation" (x_rot fp16 [M,K], qweight int8 [N,K], one
 * scale per output channel), plus an optional unmerged LoRA (NULL = none).
 * X16 = fp16(X H) (rounded once from the exact product) goes to the
 * workspace; Y = fp16(s_W[n] * sum_k X16 Q_W + scale * (X down^T) up^T + bias)
 * with fp32 accumulation on fp16 MFMA, so Y matches the exact value within
 * accumulation error, not bit for bit. */
convrot_status convrot_linear_w8a16(const void* X, int64_t M, int64_t K,
                                    const int8_t* Q_W, const float* s_W, int64_t N,
                                    const float* bias, const convrot_lora* lora, void* Y,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* The dequantise-every-call baseline the pages compare against (page
 * "INT8ConvRot GEMM vs fp16 on M1 Max ...", section "What changed in the
 * computation": the int8 weights and their scale are turned back into fp16
 * and un-rotated on every call, then a plain fp16 X W^T runs; its three-way
 * table times this path).  W_deq = fp16((Q_W (.) s_W) H) goes to the workspace
 * (fp16 [N, K], exact before its one rounding); then Y fp16 [M, N] =
 * fp16(X W_deq^T [+ bias]) on fp16 MFMA with fp32 accumulation, so Y matches
 * the exact value within accumulation error, not bit for bit. */
convrot_status convrot_linear_dequant(const void* X, int64_t M, int64_t K,
                                      const int8_t* Q_W, const float* s_W, int64_t N,
                                      const float* bias, void* Y,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* The range-safe weight-only linear: page "[PR #249] Add an mps backend
 * ...", section "Design" (range safety by construction).  X [M, K] is fp16 or
 * bf16 (x_dtype); each row is rotated (exact fp64 transform; for bf16 rows
 * exact while a group's values span at most 45 binades) and divided by 2^e,
 * e the smallest integer with max |X H| <= 2^e (0 for a zero row), before the
 * one rounding to fp16, so no row can overflow fp16 whatever its range; the
 * workspace holds that fp16 activation [M, K] and e [M] (int32).  The fp16
 * MFMA accumulates in fp32 (no K limit), the epilogue restores 2^e exactly
 * (ldexp), multiplies by s_W, adds the optional bias and rounds once to
 * y_dtype (fp16 or bf16, round to nearest even); an optional residual of
 * y_dtype [M, N] (which may be Y itself) is then added as one addition in
 * y_dtype.  Y matches the exact value within accumulation error.  Workspace:
 * convrot_workspace_bytes(CONVROT_PATH_W8A16_RS, M, N, K, 0).  A dtype other
 * than the two above is CONVROT_ERR_INVALID_ARG. */
convrot_status convrot_linear_w8a16_rs(const void* X, int x_dtype, int64_t M, int64_t K,
                                       const int8_t* Q_W, const float* s_W, int64_t N,
                                       const float* bias, const void* residual, void* Y, int y_dtype,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* ---- stages (exported for parity tests and per-kernel measurement) ---- */

/* The range-safe prologue alone: X fp16 or bf16 [M, K] -> X16 fp16 [M, K] =
 * fp16(X H 2^-e) (rounded once) and e int32 [M]. */
convrot_status convrot_act_rotate_scaled(const void* X, int x_dtype, int64_t M, int64_t K,
                                         void* X16, int32_t* rowexp, void* stream);

/* The baseline's weight step alone: Q_W int8 [N, K], s_W fp32 [N] ->
 * W16 fp16 [N, K] = fp16((Q_W (.) s_W) H), correctly rounded. */
convrot_status convrot_dequantize_weights(const int8_t* Q_W, const float* s_W, int64_t N, int64_t K,
                                          void* W16, void* stream);

/* Prologue alone: page "INT8ConvRot GEMM vs fp16 on M1 Max with Metal,
 * MPSMatrix, and MLX (fp16 Wins)", section "What changed in the computation",
 * activation equation: X_rot = X H per 256-group, s_X[m] = max_k |X_rot| / 127
 * over the whole row, Q_X = round(X_rot / s_X).  X fp16 [M, K] -> Q_X int8
 * [M, K] and s_X fp32 [M] (caller-owned, row-major), bit-exact under the
 * arithmetic contract above.  Errors as for every entry point; K == 0 writes
 * s_X = 0. */
convrot_status convrot_act_quant(const void* X, int64_t M, int64_t K,
                                 int8_t* Q_X, float* s_X, void* stream);

/* Weight-only prologue alone: same page and section, the weight-only
 * listing (the activations are rotated online and handed over as fp16
 * x_rot).  X fp16 [M, K] -> X16 fp16 [M, K] = fp16(X H), rounded once from
 * the exact product (bit-exact).  K == 0 launches nothing. */
convrot_status convrot_act_rotate_f16(const void* X, int64_t M, int64_t K,
                                      void* X16, void* stream);

/* Integer product alone: same page, section "What changed in the
 * computation", product equation (A = Q_X Q_W^T accumulated in int32; the
 * section "Running int8xint8 in a Metal kernel" checks exactly this integer
 * result against a CPU matmul).  Q_X int8 [M, K], Q_W int8 [N, K] -> A int32
 * [M, N], bit-exact (integer sums, any order).  Inputs are expected in
 * [-127, 127] as the quantisers produce them (with -128 codes A is exact only
 * while 128 * 128 * K < 2^31).  K == 0 writes A = 0. */
convrot_status convrot_gemm_i8_i32(const int8_t* Q_X, const int8_t* Q_W,
                                   int64_t M, int64_t N, int64_t K,
                                   int32_t* A, void* stream);

/* Integer product with the scale epilogue: same page and section, product
 * equation Y = A (.) s_X s_W^T.  Q_X int8 [M, K], s_X fp32 [M], Q_W int8
 * [N, K], s_W fp32 [N], optional bias fp32 [N] -> Y fp16 [M, N] =
 * fp16(fp32(A) * fp32(s_X[m] * s_W[n]) [+ bias[n]]), bit-exact under the
 * arithmetic contract above.  K == 0 writes Y = +0 [+ bias]. */
convrot_status convrot_gemm_i8_f16(const int8_t* Q_X, const float* s_X,
                                   const int8_t* Q_W, const float* s_W, const float* bias,
                                   int64_t M, int64_t N, int64_t K, void* Y, void* stream);

/* fp16 baseline GEMM: the fp16 column of the six-shape table on the page
 * "INT8ConvRot GEMM vs fp16 on M1 Max with Metal, MPSMatrix, and MLX (fp16
 * Wins)", section "Testing the MPS weight-only INT8 path in isolation" (the
 * comparison point of every table there).  Y fp16 [M, N] = X fp16 [M, K] .
 * W fp16 [N, K]^T with fp32 accumulation on fp16 MFMA, so Y matches the
 * exact value within accumulation error, not bit for bit.  K must be a
 * multiple of 256 here as well (K == 0 gives Y = +0). */
convrot_status convrot_gemm_f16(const void* X, const void* W,
                                int64_t M, int64_t N, int64_t K, void* Y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_H */
