// C ABI of the INT8ConvRot library: argument checks, workspace layout and
// the launches on the caller's stream.  Declarations and the full contract
// are in include/convrot.h.

#include <atomic>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "convrot.h"
#include "launch.hpp"


using namespace convrot;

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other / error
std::atomic<int> g_device_state[kMaxDevices];

convrot_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CONVROT_ERR_DEVICE;
  int st = g_device_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      st = 2;
    } else {
      st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    }
    g_device_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? CONVROT_OK : CONVROT_ERR_DEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// K = 0 is an empty contraction (see empty_linear); otherwise a multiple of
// the group size up to kKMax.
bool k_ok(int64_t K) { return K >= 0 && K % kGroup == 0 && K <= kKMax; }

// [a, a + na) and [b, b + nb) overlap?  (null or empty ranges never overlap)
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

int lora_ld(int64_t rank) { return rank > 0 ? (int)((rank + 31) / 32 * 32) : 0; }

// LoRA part of a workspace: T fp16 [M, t_ld], U' fp16 [N, t_ld], then (when
// K is split) the fp32 partial sums [splits, M, t_ld].
struct LoraWs {
  __half* T = nullptr;
  __half* U = nullptr;
  float* P = nullptr;
};

size_t lora_ws_bytes(int64_t M, int64_t N, int64_t K, int64_t rank) {
  if (rank <= 0) return 0;
  const size_t t_ld = (size_t)lora_ld(rank);
  const int64_t splits = lora_splits(K);
  return round256((size_t)M * t_ld * 2) + round256((size_t)N * t_ld * 2) +
         (splits > 1 ? round256((size_t)splits * M * t_ld * 4) : 0);
}

LoraWs lora_ws(char* base, int64_t M, int64_t N, int64_t K, int64_t rank) {
  LoraWs w;
  if (rank <= 0) return w;
  const size_t t_ld = (size_t)lora_ld(rank);
  w.T = reinterpret_cast<__half*>(base);
  size_t off = round256((size_t)M * t_ld * 2);
  w.U = reinterpret_cast<__half*>(base + off);
  off += round256((size_t)N * t_ld * 2);
  if (lora_splits(K) > 1) w.P = reinterpret_cast<float*>(base + off);
  return w;
}

convrot_status launched(hipError_t e) { return e == hipSuccess ? CONVROT_OK : CONVROT_ERR_LAUNCH; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

struct In {
  const void* p;
  size_t bytes;
};

// A linear with K = 0 (an empty contraction): every sum over k is empty, so
// Y = out(+0 + bias) (+0 without a bias) plus the residual (which may be Y
// itself); an int32 output is all zero.  `required` are the inputs with
// elements (scales), which must be present, aligned and apart from Y; the
// arrays with no elements (X, Q_X, Q_W, lora.down) are not touched and may
// be null.  No workspace is used.
convrot_status empty_linear(int64_t M, int64_t N, std::initializer_list<In> required, const float* bias,
                            const convrot_lora* lora, const void* residual, void* Y, EmptyOut out,
                            void* stream) {
  if (!Y || (lora && !lora->up)) return CONVROT_ERR_INVALID_ARG;
  for (const In& r : required)
    if (!r.p) return CONVROT_ERR_INVALID_ARG;
  bool aligned = aligned16(Y) && (!bias || aligned16(bias)) && (!residual || aligned16(residual)) &&
                 (!lora || (aligned16(lora->up) && (!lora->down || aligned16(lora->down))));
  for (const In& r : required) aligned = aligned && aligned16(r.p);
  if (!aligned) return CONVROT_ERR_ALIGNMENT;
  const size_t yb = (size_t)M * N * (out == kEmptyI32 ? 4 : 2);
  if (overlap(Y, yb, bias, bias ? (size_t)N * 4 : 0) ||
      (residual != Y && overlap(Y, yb, residual, residual ? yb : 0)) ||
      (lora && overlap(Y, yb, lora->up, (size_t)N * lora->rank * 4)))
    return CONVROT_ERR_INVALID_ARG;
  for (const In& r : required)
    if (overlap(Y, yb, r.p, r.bytes)) return CONVROT_ERR_INVALID_ARG;
  if (convrot_status st = check_device()) return st;
  return launched(launch_empty_linear(M, N, bias, residual, out, Y, as_stream(stream)));
}

// K = 0 for a per-row output (a scale or an exponent): the row maximum over
// no elements is 0.
convrot_status empty_rows(void* v, int64_t rows, void* stream) {
  if (!v) return CONVROT_ERR_INVALID_ARG;
  if (!aligned16(v)) return CONVROT_ERR_ALIGNMENT;
  if (convrot_status st = check_device()) return st;
  return launched(launch_fill32(v, rows, 0u, as_stream(stream)));
}

}  // namespace

extern "C" {

int convrot_abi_version(void) { return CONVROT_ABI_VERSION; }

const char* convrot_status_string(int status) {
  switch (status) {
    case CONVROT_OK: return "ok";
    case CONVROT_ERR_INVALID_ARG: return "invalid argument (null pointer or overlapping output)";
    case CONVROT_ERR_SHAPE: return "invalid shape (negative size, K not a multiple of 256 in 0..131072, or bad LoRA rank)";
    case CONVROT_ERR_ALIGNMENT: return "tensor pointer not 16-byte aligned";
    case CONVROT_ERR_DEVICE: return "current HIP device is not gfx950 or cannot be queried";
    case CONVROT_ERR_LAUNCH: return "kernel launch failed";
    case CONVROT_ERR_WORKSPACE: return "workspace missing or too small";
    case CONVROT_ERR_TOO_LARGE:
      return "problem needs more scratch than the allocation-free entry point holds "
             "(CONVROT_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

size_t convrot_workspace_bytes(int path, int64_t M, int64_t N, int64_t K, int64_t lora_rank) {
  if (M < 0 || N < 0 || K < 0 || lora_rank < 0 || lora_rank > CONVROT_LORA_RANK_MAX) return (size_t)-1;
  if (M == 0 || N == 0) return 0;
  if (!k_ok(K)) return (size_t)-1;
  if (K == 0) {   // an empty contraction needs no workspace
    if (path == CONVROT_PATH_W8A8 || path == CONVROT_PATH_W8A16) return 0;
    if (path == CONVROT_PATH_DEQUANT || path == CONVROT_PATH_W8A16_RS) return lora_rank == 0 ? 0 : (size_t)-1;
    return (size_t)-1;
  }
  if (path == CONVROT_PATH_W8A8) {
    const W8A8Plan plan = w8a8_plan(M, N, K, lora_rank > 0);
    return round256((size_t)M * K) + round256((size_t)M * 4) +
           (plan.parts ? round256((size_t)plan.splits * M * N * 4) : 0) + lora_ws_bytes(M, N, K, lora_rank);
  }
  if (path == CONVROT_PATH_W8A16) return round256((size_t)M * K * 2) + lora_ws_bytes(M, N, K, lora_rank);
  if (path == CONVROT_PATH_DEQUANT) return lora_rank == 0 ? round256((size_t)N * K * 2) : (size_t)-1;
  if (path == CONVROT_PATH_W8A16_RS)
    return lora_rank == 0 ? round256((size_t)M * K * 2) + round256((size_t)M * 4) : (size_t)-1;
  return (size_t)-1;
}

convrot_status convrot_quantize_weights(const float* W, int64_t N, int64_t K, int8_t* Q_W,
                                        float* s_W, void* stream) {
  if (N < 0 || K < 0) return CONVROT_ERR_SHAPE;
  if (N == 0) return CONVROT_OK;
  if (!k_ok(K)) return CONVROT_ERR_SHAPE;
  if (K == 0) return empty_rows(s_W, N, stream);   // s_W = 0, Q_W has no elements
  if (!W || !Q_W || !s_W) return CONVROT_ERR_INVALID_ARG;
  if (!aligned16(W) || !aligned16(Q_W) || !aligned16(s_W)) return CONVROT_ERR_ALIGNMENT;
  const size_t wb = (size_t)N * K * 4, qb = (size_t)N * K, sb = (size_t)N * 4;
  if (overlap(Q_W, qb, W, wb) || overlap(s_W, sb, W, wb) || overlap(Q_W, qb, s_W, sb))
    return CONVROT_ERR_INVALID_ARG;
  if (convrot_status st = check_device()) return st;
  return launched(launch_quantize_weights(W, N, K, Q_W, s_W, as_stream(stream)));
}

convrot_status convrot_act_quant(const void* X, int64_t M, int64_t K, int8_t* Q_X, float* s_X,
                                 void* stream) {
  if (M < 0 || K < 0) return CONVROT_ERR_SHAPE;
  if (M == 0) return CONVROT_OK;
  if (!k_ok(K)) return CONVROT_ERR_SHAPE;
  if (K == 0) return empty_rows(s_X, M, stream);   // s_X = 0, Q_X has no elements
  if (!X || !Q_X || !s_X) return CONVROT_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(Q_X) || !aligned16(s_X)) return CONVROT_ERR_ALIGNMENT;
  const size_t xb = (size_t)M * K * 2, qb = (size_t)M * K, sb = (size_t)M * 4;
  if (overlap(Q_X, qb, X, xb) || overlap(s_X, sb, X, xb) || overlap(Q_X, qb, s_X, sb))
    return CONVROT_ERR_INVALID_ARG;
  if (convrot_status st = check_device()) return st;
  return launched(launch_act_quant(X, M, K, Q_X, s_X, as_stream(stream)));
}

convrot_status convrot_act_rotate_f16(const void* X, int64_t M, int64_t K, void* X16,
                                      void* stream) {
  if (M < 0 || K < 0) return CONVROT_ERR_SHAPE;
  if (M == 0) return CONVROT_OK;
  if (!k_ok(K)) return CONVROT_ERR_SHAPE;
  if (K == 0) return check_device();               // X16 has no elements
  if (!X || !X16) return CONVROT_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(X16)) return CONVROT_ERR_ALIGNMENT;
  if (overlap(X16, (size_t)M * K * 2, X, (size_t)M * K * 2)) return CONVROT_ERR_INVALID_ARG;
  if (convrot_status st = check_device()) return st;
  return launched(launch_act_rotate_f16(X, M, K, X16, as_stream(stream)));
}

convrot_status convrot_gemm_i8_i32(const int8_t* Q_X, const int8_t* Q_W, int64_t M, int64_t N,
                                   int64_t K, int32_t* A, void* stream) {
  if (M < 0 || N < 0 || K < 0) return CONVROT_ERR_SHAPE;
  if (M == 0 || N == 0) return CONVROT_OK;
  if (!k_ok(K)) return CONVROT_ERR_SHAPE;
  if (K == 0) return empty_linear(M, N, {}, nullptr, nullptr, nullptr, A, kEmptyI32, stream);
  if (!Q_X || !Q_W || !A) return CONVROT_ERR_INVALID_ARG;
  if (!aligned16(Q_X) || !aligned16(Q_W) || !aligned16(A)) return CONVROT_ERR_ALIGNMENT;
  const size_t ab = (size_t)M * N * 4;
  if (overlap(A, ab, Q_X, (size_t)M * K) || overlap(A, ab, Q_W, (size_t)N * K))
    return CONVROT_ERR_INVALID_ARG;
  if (convrot_status st = check_device()) return st;
  GemmArgs g{};
  g.X = Q_X; g.W = Q_W; g.out = A; g.M = M; g.N = N; g.K = K;
  return launched(launch_gemm<GemmMode::kI8toI32>(g, as_stream(stream)));
}

static convrot_status check_gemm_i8_f16(const int8_t* Q_X, const float* s_X, const int8_t* Q_W,
                                        const float* s_W, const float* bias, int64_t M, int64_t N,
                                        int64_t K, const void* Y) {
  if (!Q_X || !s_X || !Q_W || !s_W || !Y) return CONVROT_ERR_INVALID_ARG;
  if (!aligned16(Q_X) || !aligned16(s_X) || !aligned16(Q_W) || !aligned16(s_W) || !aligned16(Y) ||
      (bias && !aligned16(bias)))
    return CONVROT_ERR_ALIGNMENT;
  const size_t yb = (size_t)M * N * 2;
  if (overlap(Y, yb, Q_X, (size_t)M * K) || overlap(Y, yb, s_X, (size_t)M * 4) ||
      overlap(Y, yb, Q_W, (size_t)N * K) || overlap(Y, yb, s_W, (size_t)N * 4) ||
      overlap(Y, yb, bias, bias ? (size_t)N * 4 : 0))
    return CONVROT_ERR_INVALID_ARG;
  return CONVROT_OK;
}

convrot_status convrot_gemm_i8_f16(const int8_t* Q_X, const float* s_X, const int8_t* Q_W,
                                   const float* s_W, const float* bias, int64_t M, int64_t N,
                                   int64_t K, void* Y, void* stream) {
  if (M < 0 || N < 0 || K < 0) return CONVROT_ERR_SHAPE;
  if (M == 0 || N == 0) return CONVROT_OK;
  if (!k_ok(K)) return CONVROT_ERR_SHAPE;
  if (K == 0)
    return empty_linear(M, N, {{s_X, (size_t)M * 4}, {s_W, (size_t)N * 4}}, bias, nullptr, nullptr, Y, kEmptyF16,
                        stream);
  if (convrot_status st = check_gemm_i8_f16(Q_X, s_X, Q_W, s_W, bias, M, N, K, Y)) return st;
  if (convrot_status st = check_device()) return st;
  GemmArgs g{};
  g.X = Q_X; g.W = Q_W; g.sX = s_X; g.sW = s_W; g.bias = bias; g.out = Y;
  g.M = M; g.N = N; g.K = K;
  return launched(launch_gemm<GemmMode::kI8toF16>(g, as_stream(stream)));
}

convrot_status convrot_gemm_f16(const void* X, const void* W, int64_t M, int64_t N, int64_t K,
                                void* Y, void* stream) {
  if (M < 0 || N < 0 || K < 0) return CONVROT_ERR_SHAPE;
  if (M == 0 || N == 0) return CONVROT_OK;
  if (!k_ok(K)) return CONVROT_ERR_SHAPE;
  if (K == 0) return empty_linear(M, N, {}, nullptr, nullptr, nullptr, Y, kEmptyF16, stream);
  if (!X || !W || !Y) return CONVROT_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(W) || !aligned16(Y)) return CONVROT_ERR_ALIGNMENT;
  const size_t yb = (size_t)M * N * 2;
  if (overlap(Y, yb, X, (size_t)M * K * 2) || overlap(Y, yb, W, (size_t)N * K * 2))
    return CONVROT_ERR_INVALID_ARG;
  if (convrot_status st = check_device()) return st;
  GemmArgs g{};
  g.X = X; g.W = W; g.out = Y; g.M = M; g.N = N; g.K = K;
  return launched(launch_gemm<GemmMode::kF16>(g, as_stream(stream)));
}

}  // extern "C"

namespace {

// The W8A8 linear with its optional extras.  Workspace layout (each part
// rounded up to 256 bytes): Q_X int8 [M, K], s_X fp32 [M], the int32
// partials of a K split [splits, M, N] (only when split), the LoRA part
// (only with a LoRA).
convrot_status linear_w8a8_impl(const void* X, int64_t M, int64_t K, const int8_t* Q_W,
                                const float* s_W, int64_t N, const float* bias,
                                const convrot_lora* lora, const void* residual, void* Y,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || N < 0 || K < 0) return CONVROT_ERR_SHAPE;
  const int64_t rank = lora ? lora->rank : 0;
  if (lora && (rank < 1 || rank > CONVROT_LORA_RANK_MAX)) return CONVROT_ERR_SHAPE;
  if (M == 0 || N == 0) return CONVROT_OK;
  if (!k_ok(K)) return CONVROT_ERR_SHAPE;
  if (K == 0) return empty_linear(M, N, {{s_W, (size_t)N * 4}}, bias, lora, residual, Y, kEmptyF16, stream);
  if (!X || !Q_W || !s_W || !Y) return CONVROT_ERR_INVALID_ARG;
  if (lora && (!lora->down || !lora->up)) return CONVROT_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(Q_W) || !aligned16(s_W) || !aligned16(Y) ||
      (bias && !aligned16(bias)) || (workspace && !aligned16(workspace)) ||
      (residual && !aligned16(residual)) ||
      (lora && (!aligned16(lora->down) || !aligned16(lora->up))))
    return CONVROT_ERR_ALIGNMENT;
  const size_t need = convrot_workspace_bytes(CONVROT_PATH_W8A8, M, N, K, rank);
  if (!workspace || workspace_bytes < need) return CONVROT_ERR_WORKSPACE;
  const size_t yb = (size_t)M * N * 2;
  const size_t xb = (size_t)M * K * 2, qb = (size_t)N * K, sb = (size_t)N * 4;
  const size_t bb = bias ? (size_t)N * 4 : 0, rb = residual ? yb : 0;
  const size_t db = lora ? (size_t)rank * K * 4 : 0, ub = lora ? (size_t)N * rank * 4 : 0;
  const void* dp = lora ? lora->down : nullptr;
  const void* up = lora ? lora->up : nullptr;
  // The residual may be the output buffer itself (an in-place residual
  // update), but may not overlap it otherwise, nor the workspace.
  if (overlap(Y, yb, X, xb) || overlap(Y, yb, Q_W, qb) || overlap(Y, yb, s_W, sb) ||
      overlap(Y, yb, bias, bb) || overlap(Y, yb, workspace, need) || overlap(Y, yb, dp, db) ||
      overlap(Y, yb, up, ub) || (residual != Y && overlap(Y, yb, residual, rb)) ||
      overlap(workspace, need, X, xb) || overlap(workspace, need, Q_W, qb) ||
      overlap(workspace, need, s_W, sb) || overlap(workspace, need, bias, bb) ||
      overlap(workspace, need, dp, db) || overlap(workspace, need, up, ub) ||
      overlap(workspace, need, residual, rb))
    return CONVROT_ERR_INVALID_ARG;
  if (convrot_status st = check_device()) return st;
  hipStream_t s = as_stream(stream);
  const W8A8Plan plan = w8a8_plan(M, N, K, lora != nullptr);
  const int64_t splits = plan.splits;
  char* ws = reinterpret_cast<char*>(workspace);
  int8_t* QX = reinterpret_cast<int8_t*>(ws);
  size_t off = round256((size_t)M * K);
  float* sX = reinterpret_cast<float*>(ws + off);
  off += round256((size_t)M * 4);
  int32_t* parts = reinterpret_cast<int32_t*>(ws + off);
  if (plan.parts) off += round256((size_t)splits * M * N * 4);
  const LoraWs lw = lora_ws(ws + off, M, N, K, rank);
  const int t_ld = lora_ld(rank);

  if (plan.kind == W8A8Plan::kFused) {   // one launch: quantisation, product and epilogue
    GemmArgs g{};
    g.W = Q_W; g.sW = s_W; g.bias = bias; g.out = Y;
    g.R = reinterpret_cast<const __half*>(residual);
    g.M = M; g.N = N; g.K = K;
    return launched(launch_skinny_fused(g, X, s));
  }
  if (plan.kind == W8A8Plan::kBand) {    // one launch over row bands (K = 256)
    GemmArgs g{};
    g.W = Q_W; g.sW = s_W; g.bias = bias; g.out = Y;
    g.R = reinterpret_cast<const __half*>(residual);
    g.M = M; g.N = N; g.K = K;
    return launched(launch_band(g, X, s));
  }
  if (plan.kind == W8A8Plan::kNarrow) {  // one launch over row bands (narrow layers)
    GemmArgs g{};
    g.W = Q_W; g.sW = s_W; g.bias = bias; g.out = Y;
    g.R = reinterpret_cast<const __half*>(residual);
    g.M = M; g.N = N; g.K = K;
    return launched(launch_narrow(g, X, s));
  }
  // Q_X is written in row bands by XCD where the prologue's grid allows it,
  // so that the GEMM's workgroups on each XCD read the rows that XCD's L2 has
  // just written (with LoRA, the down projection's row blocks follow the
  // same bands)
  bool banded = false;
  if (lora) {   // the prologue and the LoRA down projection share a launch where they can
    if (convrot_status st = launched(launch_act_quant_lora(X, M, K, QX, sX, lora->down, lora->up, lora->scale, N,
                                                           (int)rank, t_ld, lw.P, lw.T, lw.U, s, &banded)))
      return st;
  } else if (convrot_status st = launched(launch_act_quant(X, M, K, QX, sX, s, &banded))) {
    return st;
  }
  GemmArgs g{};
  g.xcd_row_bands = banded ? 1 : 0;
  g.X = QX; g.W = Q_W; g.sX = sX; g.sW = s_W; g.bias = bias; g.out = Y;
  g.R = reinterpret_cast<const __half*>(residual);
  g.T = lw.T; g.U = lw.U; g.t_ld = t_ld;
  g.M = M; g.N = N; g.K = K;
  if (plan.kind == W8A8Plan::kSkinny) {
    if (!plan.parts) return launched(launch_skinny(g, 1, nullptr, s));
    if (convrot_status st = launched(launch_skinny(g, splits, parts, s))) return st;
    return launched(launch_splitk_epilogue(parts, splits, g, s));
  }
  if (plan.parts) {   // few rows: int32 partials over K splits, then the epilogue
    GemmArgs gi{};
    gi.X = QX; gi.W = Q_W; gi.out = parts; gi.M = M; gi.N = N; gi.K = K; gi.kc = K / splits;
    if (convrot_status st = launched(launch_gemm<GemmMode::kI8toI32>(gi, s))) return st;
    return launched(launch_splitk_epilogue(parts, splits, g, s));
  }
  return launched(launch_gemm<GemmMode::kI8toF16>(g, s));
}

}  // namespace

extern "C" {

convrot_status convrot_linear_w8a8(const void* X, int64_t M, int64_t K, const int8_t* Q_W,
                                   const float* s_W, int64_t N, const float* bias, void* Y,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return linear_w8a8_impl(X, M, K, Q_W, s_W, N, bias, nullptr, nullptr, Y, workspace,
                          workspace_bytes, stream);
}

convrot_status convrot_linear_w8a8_ex(const void* X, int64_t M, int64_t K, const int8_t* Q_W,
                                      const float* s_W, int64_t N, const float* bias,
                                      const convrot_lora* lora, const void* residual, void* Y,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return linear_w8a8_impl(X, M, K, Q_W, s_W, N, bias, lora, residual, Y, workspace,
                          workspace_bytes, stream);
}

convrot_status convrot_dequantize_weights(const int8_t* Q_W, const float* s_W, int64_t N, int64_t K,
                                          void* W16, void* stream) {
  if (N < 0 || K < 0) return CONVROT_ERR_SHAPE;
  if (N == 0) return CONVROT_OK;
  if (!k_ok(K)) return CONVROT_ERR_SHAPE;
  if (K == 0) return check_device();               // W16 has no elements
  if (!Q_W || !s_W || !W16) return CONVROT_ERR_INVALID_ARG;
  if (!aligned16(Q_W) || !aligned16(s_W) || !aligned16(W16)) return CONVROT_ERR_ALIGNMENT;
  const size_t wb = (size_t)N * K * 2;
  if (overlap(W16, wb, Q_W, (size_t)N * K) || overlap(W16, wb, s_W, (size_t)N * 4))
    return CONVROT_ERR_INVALID_ARG;
  if (convrot_status st = check_device()) return st;
  return launched(launch_dequantize(Q_W, s_W, N, K, W16, as_stream(stream)));
}

convrot_status convrot_linear_dequant(const void* X, int64_t M, int64_t K, const int8_t* Q_W,
                                      const float* s_W, int64_t N, const float* bias, void* Y,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || N < 0 || K < 0) return CONVROT_ERR_SHAPE;
  if (M == 0 || N == 0) return CONVROT_OK;
  if (!k_ok(K)) return CONVROT_ERR_SHAPE;
  if (K == 0) return empty_linear(M, N, {{s_W, (size_t)N * 4}}, bias, nullptr, nullptr, Y, kEmptyF16, stream);
  if (!X || !Q_W || !s_W || !Y) return CONVROT_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(Q_W) || !aligned16(s_W) || !aligned16(Y) ||
      (bias && !aligned16(bias)) || (workspace && !aligned16(workspace)))
    return CONVROT_ERR_ALIGNMENT;
  const size_t need = convrot_workspace_bytes(CONVROT_PATH_DEQUANT, M, N, K, 0);
  if (!workspace || workspace_bytes < need) return CONVROT_ERR_WORKSPACE;
  const size_t yb = (size_t)M * N * 2, xb = (size_t)M * K * 2, qb = (size_t)N * K, sb = (size_t)N * 4;
  const size_t bb = bias ? (size_t)N * 4 : 0;
  if (overlap(Y, yb, X, xb) || overlap(Y, yb, Q_W, qb) || overlap(Y, yb, s_W, sb) ||
      overlap(Y, yb, bias, bb) || overlap(Y, yb, workspace, need) || overlap(workspace, need, X, xb) ||
      overlap(workspace, need, Q_W, qb) || overlap(workspace, need, s_W, sb) ||
      overlap(workspace, need, bias, bb))
    return CONVROT_ERR_INVALID_ARG;
  if (convrot_status st = check_device()) return st;
  hipStream_t s = as_stream(stream);
  if (convrot_status st = launched(launch_dequantize(Q_W, s_W, N, K, workspace, s))) return st;
  GemmArgs g{};
  g.X = X; g.W = workspace; g.bias = bias; g.out = Y; g.M = M; g.N = N; g.K = K;
  return launched(launch_gemm<GemmMode::kF16>(g, s));
}

convrot_status convrot_act_rotate_scaled(const void* X, int x_dtype, int64_t M, int64_t K, void* X16,
                                         int32_t* rowexp, void* stream) {
  if (M < 0 || K < 0) return CONVROT_ERR_SHAPE;
  if (x_dtype != CONVROT_DTYPE_F16 && x_dtype != CONVROT_DTYPE_BF16) return CONVROT_ERR_INVALID_ARG;
  if (M == 0) return CONVROT_OK;
  if (!k_ok(K)) return CONVROT_ERR_SHAPE;
  if (K == 0) return empty_rows(rowexp, M, stream);   // e = 0, X16 has no elements
  if (!X || !X16 || !rowexp) return CONVROT_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(X16) || !aligned16(rowexp)) return CONVROT_ERR_ALIGNMENT;
  const size_t xb = (size_t)M * K * 2, eb = (size_t)M * 4;
  if (overlap(X16, xb, X, xb) || overlap(rowexp, eb, X, xb) || overlap(rowexp, eb, X16, xb))
    return CONVROT_ERR_INVALID_ARG;
  if (convrot_status st = check_device()) return st;
  return launched(launch_act_rotate_scaled(X, x_dtype == CONVROT_DTYPE_BF16, M, K, X16, rowexp, as_stream(stream)));
}

convrot_status convrot_linear_w8a16_rs(const void* X, int x_dtype, int64_t M, int64_t K, const int8_t* Q_W,
                                       const float* s_W, int64_t N, const float* bias, const void* residual,
                                       void* Y, int y_dtype, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (M < 0 || N < 0 || K < 0) return CONVROT_ERR_SHAPE;
  if ((x_dtype != CONVROT_DTYPE_F16 && x_dtype != CONVROT_DTYPE_BF16) ||
      (y_dtype != CONVROT_DTYPE_F16 && y_dtype != CONVROT_DTYPE_BF16))
    return CONVROT_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return CONVROT_OK;
  if (!k_ok(K)) return CONVROT_ERR_SHAPE;
  if (K == 0)
    return empty_linear(M, N, {{s_W, (size_t)N * 4}}, bias, nullptr, residual, Y,
                        y_dtype == CONVROT_DTYPE_BF16 ? kEmptyBF16 : kEmptyF16, stream);
  if (!X || !Q_W || !s_W || !Y) return CONVROT_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(Q_W) || !aligned16(s_W) || !aligned16(Y) ||
      (bias && !aligned16(bias)) || (residual && !aligned16(residual)) || (workspace && !aligned16(workspace)))
    return CONVROT_ERR_ALIGNMENT;
  const size_t need = convrot_workspace_bytes(CONVROT_PATH_W8A16_RS, M, N, K, 0);
  if (!workspace || workspace_bytes < need) return CONVROT_ERR_WORKSPACE;
  const size_t yb = (size_t)M * N * 2, xb = (size_t)M * K * 2, qb = (size_t)N * K, sb = (size_t)N * 4;
  const size_t bb = bias ? (size_t)N * 4 : 0, rb = residual ? yb : 0;
  if (overlap(Y, yb, X, xb) || overlap(Y, yb, Q_W, qb) || overlap(Y, yb, s_W, sb) || overlap(Y, yb, bias, bb) ||
      overlap(Y, yb, workspace, need) || (residual != Y && overlap(Y, yb, residual, rb)) ||
      overlap(workspace, need, X, xb) || overlap(workspace, need, Q_W, qb) || overlap(workspace, need, s_W, sb) ||
      overlap(workspace, need, bias, bb) || overlap(workspace, need, residual, rb))
    return CONVROT_ERR_INVALID_ARG;
  if (convrot_status st = check_device()) return st;
  hipStream_t s = as_stream(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  void* X16 = ws;
  int* rowexp = reinterpret_cast<int*>(ws + round256((size_t)M * K * 2));
  bool banded = false;   // X16 in row bands by XCD, as for Q_X
  if (convrot_status st =
          launched(launch_act_rotate_scaled(X, x_dtype == CONVROT_DTYPE_BF16, M, K, X16, rowexp, s, &banded)))
    return st;
  GemmArgs g{};
  g.xcd_row_bands = banded ? 1 : 0;
  g.X = X16; g.W = Q_W; g.sW = s_W; g.bias = bias; g.out = Y;
  g.R = reinterpret_cast<const __half*>(residual);
  g.rowexp = rowexp; g.out_bf16 = y_dtype == CONVROT_DTYPE_BF16;
  g.M = M; g.N = N; g.K = K;
  return launched(launch_gemm<GemmMode::kW8A16>(g, s));
}

convrot_status convrot_linear_w8a16(const void* X, int64_t M, int64_t K, const int8_t* Q_W,
                                    const float* s_W, int64_t N, const float* bias,
                                    const convrot_lora* lora, void* Y, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (M < 0 || N < 0 || K < 0) return CONVROT_ERR_SHAPE;
  const int64_t rank = lora ? lora->rank : 0;
  if (lora && (rank < 1 || rank > CONVROT_LORA_RANK_MAX)) return CONVROT_ERR_SHAPE;
  if (M == 0 || N == 0) return CONVROT_OK;
  if (!k_ok(K)) return CONVROT_ERR_SHAPE;
  if (K == 0) return empty_linear(M, N, {{s_W, (size_t)N * 4}}, bias, lora, nullptr, Y, kEmptyF16, stream);
  if (!X || !Q_W || !s_W || !Y) return CONVROT_ERR_INVALID_ARG;
  if (lora && (!lora->down || !lora->up)) return CONVROT_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(Q_W) || !aligned16(s_W) || !aligned16(Y) ||
      (bias && !aligned16(bias)) || (workspace && !aligned16(workspace)) ||
      (lora && (!aligned16(lora->down) || !aligned16(lora->up))))
    return CONVROT_ERR_ALIGNMENT;
  const size_t need = convrot_workspace_bytes(CONVROT_PATH_W8A16, M, N, K, rank);
  if (!workspace || workspace_bytes < need) return CONVROT_ERR_WORKSPACE;
  const size_t yb = (size_t)M * N * 2;
  const size_t db = lora ? (size_t)rank * K * 4 : 0, ub = lora ? (size_t)N * rank * 4 : 0;
  const void* dp = lora ? lora->down : nullptr;
  const void* up = lora ? lora->up : nullptr;
  if (overlap(Y, yb, X, (size_t)M * K * 2) || overlap(Y, yb, Q_W, (size_t)N * K) ||
      overlap(Y, yb, s_W, (size_t)N * 4) || overlap(Y, yb, bias, bias ? (size_t)N * 4 : 0) ||
      overlap(Y, yb, workspace, need) || overlap(Y, yb, dp, db) || overlap(Y, yb, up, ub) ||
      overlap(workspace, need, X, (size_t)M * K * 2) || overlap(workspace, need, Q_W, (size_t)N * K) ||
      overlap(workspace, need, s_W, (size_t)N * 4) ||
      overlap(workspace, need, bias, bias ? (size_t)N * 4 : 0) || overlap(workspace, need, dp, db) ||
      overlap(workspace, need, up, ub))
    return CONVROT_ERR_INVALID_ARG;
  if (convrot_status st = check_device()) return st;
  hipStream_t s = as_stream(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  void* X16 = ws;
  const LoraWs lw = lora_ws(ws + round256((size_t)M * K * 2), M, N, K, rank);
  const int t_ld = lora_ld(rank);
  bool banded = false;   // X16 in row bands by XCD, as for Q_X
  if (lora) {   // the prologue and the LoRA down projection share a launch where they can
    if (convrot_status st = launched(launch_act_rotate_f16_lora(X, M, K, X16, lora->down, lora->up, lora->scale, N,
                                                                (int)rank, t_ld, lw.P, lw.T, lw.U, s, &banded)))
      return st;
  } else if (convrot_status st = launched(launch_act_rotate_f16(X, M, K, X16, s, &banded))) {
    return st;
  }
  GemmArgs g{};
  g.xcd_row_bands = banded ? 1 : 0;
  g.X = X16; g.W = Q_W; g.sW = s_W; g.bias = bias; g.out = Y;
  g.T = lw.T; g.U = lw.U; g.t_ld = t_ld;
  g.M = M; g.N = N; g.K = K;
  return launched(launch_gemm<GemmMode::kW8A16>(g, s));
}

}  // extern "C"

// ------------------------------------------------ allocation-free W8A8 call
// For callers that cannot allocate device memory.  The W8A8 path's scratch
// (Q_X, s_X and, with few rows, the int32 K-split partials; the same layout
// as a caller workspace) lives in this fixed device array: every GPU the
// library runs on holds its own copy from the code object's load until the
// process ends.  Nothing in it has to start at zero (the prologue writes Q_X
// and s_X, and the split GEMM every partial, before anything reads them).

static __device__ __align__(256) char scratch[CONVROT_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mutex;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of this GPU's scratch array, looked up once per device with
// that device current.  In host code `scratch` names a host-side stand-in,
// so only this address is ever handed to a kernel.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" convrot_status convrot_linear_w8a8_noalloc(const void* X, int64_t M, int64_t K, const int8_t* Q_W,
                                                      const float* s_W, int64_t N, const float* bias, void* Y,
                                                      void* stream) {
  if (M < 0 || N < 0 || K < 0) return CONVROT_ERR_SHAPE;
  if (M == 0 || N == 0) return CONVROT_OK;
  if (!k_ok(K)) return CONVROT_ERR_SHAPE;
  if (K == 0)   // an empty contraction uses no scratch
    return linear_w8a8_impl(X, M, K, Q_W, s_W, N, bias, nullptr, nullptr, Y, nullptr, 0, stream);
  const size_t need = convrot_workspace_bytes(CONVROT_PATH_W8A8, M, N, K, 0);
  if (need == (size_t)-1) return CONVROT_ERR_SHAPE;
  if (need > (size_t)CONVROT_NOALLOC_SCRATCH_BYTES) return CONVROT_ERR_TOO_LARGE;
  // the pointer checks come before the device lookup, as in every entry point
  if (!X || !Q_W || !s_W || !Y) return CONVROT_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(Q_W) || !aligned16(s_W) || !aligned16(Y) || (bias && !aligned16(bias)))
    return CONVROT_ERR_ALIGNMENT;
  const size_t yb = (size_t)M * N * 2;
  if (overlap(Y, yb, X, (size_t)M * K * 2) || overlap(Y, yb, Q_W, (size_t)N * K) ||
      overlap(Y, yb, s_W, (size_t)N * 4) || overlap(Y, yb, bias, bias ? (size_t)N * 4 : 0))
    return CONVROT_ERR_INVALID_ARG;
  if (convrot_status st = check_device()) return st;
  void* ws = scratch_for_current_device();
  if (!ws) return CONVROT_ERR_DEVICE;
  return linear_w8a8_impl(X, M, K, Q_W, s_W, N, bias, nullptr, nullptr, Y, ws,
                          (size_t)CONVROT_NOALLOC_SCRATCH_BYTES, stream);
}
