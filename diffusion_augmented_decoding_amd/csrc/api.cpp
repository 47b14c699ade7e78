// libunospec C ABI: argument validation and dispatch.  Every check runs on
// the host before anything is enqueued; no C++ exception leaves this file.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>

#include "internal.h"

namespace uno {

static thread_local char g_err[512] = "";

uno_status fail(uno_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

uno_status check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return UNO_OK;
  return fail(UNO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace uno

using namespace uno;

extern "C" {

int uno_abi_version(void) { return UNO_ABI_VERSION; }

const char* uno_status_string(uno_status s) {
  switch (s) {
    case UNO_OK: return "ok";
    case UNO_ERR_INVALID_ARGUMENT: return "invalid argument";
    case UNO_ERR_UNSUPPORTED: return "unsupported";
    case UNO_ERR_WORKSPACE: return "workspace too small";
    case UNO_ERR_HIP: return "HIP error";
    case UNO_ERR_INTERNAL: return "internal error";
  }
  return "unknown status";
}

const char* uno_last_error(void) { return g_err; }

// ------------------------------------------------------------------ gated LoRA
static uno_status check_gated_lora_shape(uno_dtype dtype, int64_t M, int64_t N, int64_t K, int64_t r) {
  if (dtype != UNO_F32 && dtype != UNO_BF16) return fail(UNO_ERR_INVALID_ARGUMENT, "unknown dtype %d", int(dtype));
  if (M < 1 || N < 1 || K < 1 || r < 0)
    return fail(UNO_ERR_INVALID_ARGUMENT, "sizes must be M,N,K >= 1 and r >= 0 (got %lld,%lld,%lld,%lld)",
                (long long)M, (long long)N, (long long)K, (long long)r);
  if (M > (1ll << 30) || N > (1ll << 30) || K > (1ll << 30) || r > 4096)
    return fail(UNO_ERR_UNSUPPORTED, "sizes beyond the supported range");
  if (dtype == UNO_BF16 && (K % 8 != 0 || r % 8 != 0))
    return fail(UNO_ERR_UNSUPPORTED, "bf16 path needs K and r multiples of 8 (got K=%lld r=%lld)", (long long)K,
                (long long)r);
  return UNO_OK;
}

uno_status uno_gated_lora_linear_workspace(uno_dtype dtype, int64_t M, int64_t N, int64_t K, int64_t r,
                                           size_t* bytes) {
  UNO_GUARD_BEGIN
  if (!bytes) return fail(UNO_ERR_INVALID_ARGUMENT, "bytes is NULL");
  uno_status s = check_gated_lora_shape(dtype, M, N, K, r);
  if (s != UNO_OK) return s;
  *bytes = gated_lora_workspace_bytes(dtype, M, N, K, r);
  return UNO_OK;
  UNO_GUARD_END
}

uno_status uno_gated_lora_linear(hipStream_t stream, uno_dtype dtype, int64_t M, int64_t N, int64_t K, int64_t r,
                                 const void* x, int64_t ldx, const void* W, int64_t ldw, const void* A, int64_t lda,
                                 const void* B, int64_t ldb, const uint8_t* gate, float lora_scale, void* y,
                                 int64_t ldy, void* workspace, size_t workspace_bytes) {
  UNO_GUARD_BEGIN
  uno_status s = check_gated_lora_shape(dtype, M, N, K, r);
  if (s != UNO_OK) return s;
  if (!x || !W || !y) return fail(UNO_ERR_INVALID_ARGUMENT, "x, W and y must be non-NULL");
  const bool lora = r > 0 && gate != nullptr;
  if (lora && (!A || !B)) return fail(UNO_ERR_INVALID_ARGUMENT, "A and B must be non-NULL when r > 0 and gate is set");
  if (ldx < K || ldw < K || ldy < N || (lora && (lda < K || ldb < r)))
    return fail(UNO_ERR_INVALID_ARGUMENT, "leading dimension smaller than the row width");
  if (!std::isfinite(lora_scale)) return fail(UNO_ERR_INVALID_ARGUMENT, "lora_scale must be finite");
  if (dtype == UNO_BF16) {
    if (ldx % 8 || ldw % 8 || (lora && (lda % 8 || ldb % 8)))
      return fail(UNO_ERR_UNSUPPORTED, "bf16 path needs input leading dimensions that are multiples of 8");
    if (!aligned16(x) || !aligned16(W) || (lora && (!aligned16(A) || !aligned16(B))))
      return fail(UNO_ERR_UNSUPPORTED, "bf16 path needs 16-byte aligned input matrices");
    if ((reinterpret_cast<uintptr_t>(y) & 1u) != 0) return fail(UNO_ERR_INVALID_ARGUMENT, "y is not 2-byte aligned");
  }
  const size_t need = gated_lora_workspace_bytes(dtype, M, N, K, lora ? r : 0);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(UNO_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  GatedLoraArgs a{};
  a.dtype = dtype;
  a.M = M;
  a.N = N;
  a.K = K;
  a.r = lora ? r : 0;
  a.x = x;
  a.ldx = ldx;
  a.w = W;
  a.ldw = ldw;
  a.a = A;
  a.lda = lda;
  a.b = B;
  a.ldb = ldb;
  a.gate = lora ? gate : nullptr;
  a.lora_scale = lora_scale;
  a.y = y;
  a.ldy = ldy;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  return check_hip(launch_gated_lora(a, stream), "uno_gated_lora_linear launch");
  UNO_GUARD_END
}

// ------------------------------------------------------------------ LoRA merge
uno_status uno_lora_merge(hipStream_t stream, int64_t N, int64_t K, int64_t r, const void* W, int64_t ldw,
                          const void* A, int64_t lda, const void* B, int64_t ldb, float lora_scale, void* out,
                          int64_t ldo) {
  UNO_GUARD_BEGIN
  if (N < 1 || K < 1 || r < 1) return fail(UNO_ERR_INVALID_ARGUMENT, "N, K and r must be >= 1");
  if (N > 65535) return fail(UNO_ERR_UNSUPPORTED, "N above 65535 (got %lld)", (long long)N);
  if (K > (int64_t(1) << 30) || r > (int64_t(1) << 20)) return fail(UNO_ERR_UNSUPPORTED, "K or r too large");
  if (!W || !A || !B || !out) return fail(UNO_ERR_INVALID_ARGUMENT, "W, A, B and out must be non-NULL");
  if (ldw < K || lda < K || ldb < r || ldo < K)
    return fail(UNO_ERR_INVALID_ARGUMENT, "leading dimension smaller than the row width");
  if (!std::isfinite(lora_scale)) return fail(UNO_ERR_INVALID_ARGUMENT, "lora_scale must be finite");
  if (((reinterpret_cast<uintptr_t>(W) | reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B) |
        reinterpret_cast<uintptr_t>(out)) & 1u) != 0)
    return fail(UNO_ERR_INVALID_ARGUMENT, "bf16 matrices must be 2-byte aligned");
  LoraMergeArgs m{N, K, r, W, ldw, A, lda, B, ldb, lora_scale, out, ldo};
  return check_hip(launch_lora_merge(m, stream), "uno_lora_merge launch");
  UNO_GUARD_END
}

// ------------------------------------------------------------------ linear verify
static uno_status check_verify_linear_shape(int32_t batch, int32_t k, int32_t vocab) {
  if (batch < 1) return fail(UNO_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", batch);
  if (k < 0 || k > 64) return fail(UNO_ERR_INVALID_ARGUMENT, "k must be in 0..64 (got %d)", k);
  if (vocab < 1) return fail(UNO_ERR_INVALID_ARGUMENT, "vocab must be >= 1 (got %d)", vocab);
  if (vocab > (1 << 20)) return fail(UNO_ERR_UNSUPPORTED, "vocab above 2^20 (got %d)", vocab);
  if (int64_t(batch) * (2 * k + 1) > (int64_t(1) << 31) - 1) return fail(UNO_ERR_UNSUPPORTED, "too many rows");
  return UNO_OK;
}

// ------------------------------------------------------------------ gated-LoRA backward
static uno_status check_lora_backward(int64_t M, int64_t N, int64_t K, int64_t r) {
  if (M < 1 || N < 1 || K < 1 || r < 1) return fail(UNO_ERR_INVALID_ARGUMENT, "M, N, K and r must be >= 1");
  if (M > (int64_t(1) << 24) || N > (int64_t(1) << 20) || K > (int64_t(1) << 20) || r > 4096)
    return fail(UNO_ERR_UNSUPPORTED, "shape above the supported range");
  if (N % 32 || K % 8 || r % 8)
    return fail(UNO_ERR_UNSUPPORTED, "N must be a multiple of 32, K and r multiples of 8");
  return UNO_OK;
}

uno_status uno_gated_lora_backward_workspace(int64_t M, int64_t N, int64_t K, int64_t r, int32_t with_w_t,
                                            size_t* bytes) {
  UNO_GUARD_BEGIN
  if (!bytes) return fail(UNO_ERR_INVALID_ARGUMENT, "bytes is NULL");
  uno_status s = check_lora_backward(M, N, K, r);
  if (s != UNO_OK) return s;
  *bytes = lora_backward_workspace_bytes(M, N, K, r, with_w_t ? 1 : 0);
  return UNO_OK;
  UNO_GUARD_END
}

uno_status uno_gated_lora_backward(hipStream_t stream, int64_t M, int64_t N, int64_t K, int64_t r, const void* x,
                                   int64_t ldx, const void* W, int64_t ldw, const void* A, int64_t lda, const void* B,
                                   int64_t ldb, const uint8_t* gate, float lora_scale, const void* dy, int64_t lddy,
                                   void* dx, int64_t lddx, float* dA, int64_t ldda, float* dB, int64_t lddb,
                                   const void* W_t, int64_t ldwt, void* workspace, size_t workspace_bytes) {
  UNO_GUARD_BEGIN
  uno_status s = check_lora_backward(M, N, K, r);
  if (s != UNO_OK) return s;
  if (!x || !A || !B || !dy || !dA || !dB || (dx && !W))
    return fail(UNO_ERR_INVALID_ARGUMENT, "required pointer is NULL");
  if (ldx < K || lda < K || ldb < r || lddy < N || ldda < K || lddb < r || (dx && (ldw < K || lddx < K)))
    return fail(UNO_ERR_INVALID_ARGUMENT, "leading dimension smaller than the row width");
  if (ldx % 8 || lda % 8 || ldb % 8 || lddy % 8 || ldda % 8 || lddb % 8 || (dx && (ldw % 8 || lddx % 8)))
    return fail(UNO_ERR_UNSUPPORTED, "leading dimensions must be multiples of 8");
  if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(dy) || !aligned16(dA) || !aligned16(dB) ||
      (dx && (!aligned16(W) || !aligned16(dx))))
    return fail(UNO_ERR_UNSUPPORTED, "matrices must be 16-byte aligned");
  if (!std::isfinite(lora_scale)) return fail(UNO_ERR_INVALID_ARGUMENT, "lora_scale must be finite");
  if (W_t && (ldwt < N || ldwt % 8 || !aligned16(W_t)))
    return fail(UNO_ERR_INVALID_ARGUMENT, "W_t needs ldwt >= N, a multiple of 8, and 16-byte alignment");
  const size_t need = lora_backward_workspace_bytes(M, N, K, r, W_t ? 1 : 0);
  if (workspace_bytes < need || !workspace)
    return fail(UNO_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(UNO_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  LoraBackwardArgs a{};
  a.M = M;
  a.N = N;
  a.K = K;
  a.r = r;
  a.x = x;
  a.ldx = ldx;
  a.w = W;
  a.ldw = ldw;
  a.a = A;
  a.lda = lda;
  a.b = B;
  a.ldb = ldb;
  a.gate = gate;
  a.lora_scale = lora_scale;
  a.dy = dy;
  a.lddy = lddy;
  a.dx = dx;
  a.lddx = lddx;
  a.da = dA;
  a.ldda = ldda;
  a.db = dB;
  a.lddb = lddb;
  a.w_t = W_t;
  a.ldwt = ldwt;
  a.ws = workspace;
  return check_hip(launch_lora_backward(a, stream), "uno_gated_lora_backward launch");
  UNO_GUARD_END
}

uno_status uno_transpose_bf16(hipStream_t stream, int64_t rows, int64_t cols, const void* src, int64_t ld_src,
                              void* dst, int64_t ld_dst) {
  UNO_GUARD_BEGIN
  if (rows < 1 || cols < 1) return fail(UNO_ERR_INVALID_ARGUMENT, "rows and cols must be >= 1");
  if (rows > (int64_t(1) << 30) || cols > (int64_t(1) << 30)) return fail(UNO_ERR_UNSUPPORTED, "too large");
  if (((cols + 63) / 64) * ((rows + 63) / 64) > 0x7fffffff) return fail(UNO_ERR_UNSUPPORTED, "too many tiles");
  if (!src || !dst) return fail(UNO_ERR_INVALID_ARGUMENT, "src and dst must be non-NULL");
  if (ld_src < cols || ld_dst < rows) return fail(UNO_ERR_INVALID_ARGUMENT, "leading dimension below the row width");
  if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 1u) != 0)
    return fail(UNO_ERR_INVALID_ARGUMENT, "src and dst must be 2-byte aligned");
  return check_hip(launch_transpose_bf16(src, ld_src, dst, ld_dst, rows, cols, stream), "uno_transpose_bf16 launch");
  UNO_GUARD_END
}

// ------------------------------------------------------------------ distillation losses
uno_status uno_distill_loss(hipStream_t stream, uno_dtype logit_dtype, int32_t batch, int32_t rows, int32_t vocab,
                            const void* teacher, int64_t t_seq_stride, int64_t t_row_stride, const void* student,
                            int64_t s_seq_stride, int64_t s_row_stride, float temperature, float alpha, float beta,
                            float grad_scale, float* out_kl, float* out_tv, void* grad, int64_t g_seq_stride,
                            int64_t g_row_stride) {
  UNO_GUARD_BEGIN
  if (logit_dtype != UNO_F32 && logit_dtype != UNO_BF16)
    return fail(UNO_ERR_INVALID_ARGUMENT, "unknown dtype %d", int(logit_dtype));
  if (batch < 1 || rows < 1 || vocab < 1) return fail(UNO_ERR_INVALID_ARGUMENT, "batch, rows and vocab must be >= 1");
  if (int64_t(batch) * rows > 0x7fffffff) return fail(UNO_ERR_UNSUPPORTED, "more than 2^31 - 1 row pairs");
  if (vocab > (1 << 20)) return fail(UNO_ERR_UNSUPPORTED, "vocab above 2^20");
  if (!teacher || !student || !out_kl || !out_tv) return fail(UNO_ERR_INVALID_ARGUMENT, "required pointer is NULL");
  if (t_row_stride < vocab || s_row_stride < vocab || (grad && g_row_stride < vocab))
    return fail(UNO_ERR_INVALID_ARGUMENT, "a row stride is below vocab");
  if (t_seq_stride < 0 || s_seq_stride < 0 || (grad && g_seq_stride < 0))
    return fail(UNO_ERR_INVALID_ARGUMENT, "negative sequence stride");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(UNO_ERR_INVALID_ARGUMENT, "temperature must be finite and > 0");
  if (!std::isfinite(alpha) || !std::isfinite(beta) || !std::isfinite(grad_scale))
    return fail(UNO_ERR_INVALID_ARGUMENT, "alpha, beta and grad_scale must be finite");
  DistillArgs a{};
  a.dtype = logit_dtype;
  a.batch = batch;
  a.rows = rows;
  a.vocab = vocab;
  a.teacher = teacher;
  a.t_seq = t_seq_stride;
  a.t_row = t_row_stride;
  a.student = student;
  a.s_seq = s_seq_stride;
  a.s_row = s_row_stride;
  a.scale_log2 = float(1.4426950408889634 / double(temperature));
  a.inv_t = float(1.0 / double(temperature));
  a.alpha = alpha;
  a.beta = beta;
  a.grad_scale = grad_scale;
  a.out_kl = out_kl;
  a.out_tv = out_tv;
  a.grad = grad;
  a.g_seq = g_seq_stride;
  a.g_row = g_row_stride;
  return check_hip(launch_distill(a, stream), "uno_distill_loss launch");
  UNO_GUARD_END
}

// ------------------------------------------------------------------ tree construction
static uno_status check_tree_build(int32_t batch, int32_t max_depth, const int32_t* branching, int32_t vocab,
                                   int32_t n_tree, int32_t without) {
  if (batch < 1 || batch > 65535) return fail(UNO_ERR_INVALID_ARGUMENT, "batch must be in [1, 65535]");
  if (max_depth < 1 || max_depth > 64) return fail(UNO_ERR_INVALID_ARGUMENT, "max_depth must be in [1, 64]");
  if (vocab < 1) return fail(UNO_ERR_INVALID_ARGUMENT, "vocab must be >= 1");
  if (vocab > (1 << 20)) return fail(UNO_ERR_UNSUPPORTED, "vocab above 2^20");
  if (!branching) return fail(UNO_ERR_INVALID_ARGUMENT, "branching is NULL");
  int64_t n = 1, width = 1;
  for (int d = 0; d < max_depth; ++d) {
    const int32_t br = branching[d];
    if (br < 1 || br > kMaxBranch) return fail(UNO_ERR_INVALID_ARGUMENT, "branching[%d] must be in [1, %d]", d, kMaxBranch);
    if (without && br > vocab)
      return fail(UNO_ERR_INVALID_ARGUMENT, "branching[%d] = %d above vocab without replacement", d, br);
    width *= br;
    n += width;
    if (n > 1024) return fail(UNO_ERR_UNSUPPORTED, "tree above 1024 nodes");
  }
  if (n_tree != n) return fail(UNO_ERR_INVALID_ARGUMENT, "n_tree %d, the branching gives %lld nodes", n_tree, (long long)n);
  return UNO_OK;
}

uno_status uno_psi_spec_build_tree_workspace(int32_t batch, int32_t max_depth, int32_t vocab, size_t* bytes) {
  UNO_GUARD_BEGIN
  if (!bytes) return fail(UNO_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (batch < 1 || batch > 65535) return fail(UNO_ERR_INVALID_ARGUMENT, "batch must be in [1, 65535]");
  if (max_depth < 1 || max_depth > 64) return fail(UNO_ERR_INVALID_ARGUMENT, "max_depth must be in [1, 64]");
  if (vocab < 1) return fail(UNO_ERR_INVALID_ARGUMENT, "vocab must be >= 1");
  if (vocab > (1 << 20)) return fail(UNO_ERR_UNSUPPORTED, "vocab above 2^20");
  *bytes = tree_build_workspace_bytes(batch, max_depth, vocab);
  return UNO_OK;
  UNO_GUARD_END
}

uno_status uno_psi_spec_build_tree(hipStream_t stream, uno_dtype logit_dtype, int32_t batch, int32_t max_depth,
                                   const int32_t* branching, int32_t vocab, const void* q_logits,
                                   int64_t q_seq_stride, int64_t q_row_stride, const float* u_draw, int32_t n_tree,
                                   float temperature, int32_t without_replacement, int32_t* out_parent,
                                   int32_t* out_tokens, void* workspace, size_t workspace_bytes) {
  UNO_GUARD_BEGIN
  if (logit_dtype != UNO_F32 && logit_dtype != UNO_BF16)
    return fail(UNO_ERR_INVALID_ARGUMENT, "unknown dtype %d", int(logit_dtype));
  if (without_replacement != 0 && without_replacement != 1)
    return fail(UNO_ERR_INVALID_ARGUMENT, "without_replacement must be 0 or 1");
  uno_status s = check_tree_build(batch, max_depth, branching, vocab, n_tree, without_replacement);
  if (s != UNO_OK) return s;
  if (!q_logits || !u_draw || !out_parent || !out_tokens)
    return fail(UNO_ERR_INVALID_ARGUMENT, "required pointer is NULL");
  if (q_row_stride < vocab || q_seq_stride < 0)
    return fail(UNO_ERR_INVALID_ARGUMENT, "q_row_stride below vocab or negative q_seq_stride");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(UNO_ERR_INVALID_ARGUMENT, "temperature must be finite and > 0");
  const size_t need = tree_build_workspace_bytes(batch, max_depth, vocab);
  if (workspace_bytes < need || !workspace)
    return fail(UNO_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  TreeBuildArgs a{};
  a.dtype = logit_dtype;
  a.batch = batch;
  a.max_depth = max_depth;
  a.vocab = vocab;
  a.n = n_tree;
  for (int d = 0; d < max_depth; ++d) a.branching[d] = branching[d];
  a.q = q_logits;
  a.q_seq = q_seq_stride;
  a.q_row = q_row_stride;
  a.u = u_draw;
  a.scale_log2 = float(1.4426950408889634 / double(temperature));
  a.without = without_replacement;
  a.out_parent = out_parent;
  a.out_tokens = out_tokens;
  a.ws = workspace;
  if (debug_checks()) {
    const uno_status d = debug_check_unit(stream, u_draw, int64_t(batch) * n_tree, "u_draw");
    if (d != UNO_OK) return d;
  }
  return check_hip(launch_tree_build(a, stream), "uno_psi_spec_build_tree launch");
  UNO_GUARD_END
}

}  // extern "C"

namespace uno {

// Host validation of a linear verify call (everything but the workspace) and
// its kernel arguments; shared by the workspace and the allocation-free
// entry points.
uno_status verify_linear_args(uno_dtype logit_dtype, int32_t batch, int32_t k, int32_t vocab, const void* p_logits,
                              int64_t p_seq_stride, int64_t p_row_stride, const void* q_logits,
                              int64_t q_seq_stride, int64_t q_row_stride, const int32_t* draft_tokens,
                              const float* u_accept, const float* u_sample, float temperature,
                              int32_t* out_accept_len, int32_t* out_token, float* out_p_draft, float* out_q_draft,
                              float* out_residual_mass, VerifyLinearArgs* out) {
  if (logit_dtype != UNO_F32 && logit_dtype != UNO_BF16)
    return fail(UNO_ERR_INVALID_ARGUMENT, "unknown dtype %d", int(logit_dtype));
  uno_status s = check_verify_linear_shape(batch, k, vocab);
  if (s != UNO_OK) return s;
  if (!p_logits || !u_sample || !out_accept_len || !out_token)
    return fail(UNO_ERR_INVALID_ARGUMENT, "p_logits, u_sample, out_accept_len and out_token must be non-NULL");
  if (k > 0 && (!q_logits || !draft_tokens || !u_accept))
    return fail(UNO_ERR_INVALID_ARGUMENT, "q_logits, draft_tokens and u_accept must be non-NULL when k > 0");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(UNO_ERR_INVALID_ARGUMENT, "temperature must be finite and > 0");
  // the sequence strides are never used with a single sequence
  if (p_row_stride < vocab || (batch > 1 && p_seq_stride < int64_t(k + 1) * p_row_stride))
    return fail(UNO_ERR_INVALID_ARGUMENT, "p strides must cover [k+1][vocab]");
  if (k > 0 && (q_row_stride < vocab || (batch > 1 && q_seq_stride < int64_t(k) * q_row_stride)))
    return fail(UNO_ERR_INVALID_ARGUMENT, "q strides must cover [k][vocab]");
  VerifyLinearArgs a{};
  a.dtype = logit_dtype;
  a.batch = batch;
  a.k = k;
  a.vocab = vocab;
  a.p = p_logits;
  a.p_seq = p_seq_stride;
  a.p_row = p_row_stride;
  a.q = q_logits;
  a.q_seq = q_seq_stride;
  a.q_row = q_row_stride;
  a.drafts = draft_tokens;
  a.drafts_seq = k;
  a.u_acc = u_accept;
  a.u_s = u_sample;
  a.scale_log2 = float(1.4426950408889634 / double(temperature));
  a.out_len = out_accept_len;
  a.out_tok = out_token;
  a.out_pd = out_p_draft;
  a.out_qd = out_q_draft;
  a.out_mass = out_residual_mass;
  *out = a;
  return UNO_OK;
}

}  // namespace uno

extern "C" {

uno_status uno_psi_spec_verify_linear_workspace(int32_t batch, int32_t k, int32_t vocab, size_t* bytes) {
  UNO_GUARD_BEGIN
  if (!bytes) return fail(UNO_ERR_INVALID_ARGUMENT, "bytes is NULL");
  uno_status s = check_verify_linear_shape(batch, k, vocab);
  if (s != UNO_OK) return s;
  *bytes = verify_linear_workspace_bytes(batch, k, vocab);
  return UNO_OK;
  UNO_GUARD_END
}

uno_status uno_psi_spec_verify_linear(hipStream_t stream, uno_dtype logit_dtype, int32_t batch, int32_t k,
                                      int32_t vocab, const void* p_logits, int64_t p_seq_stride,
                                      int64_t p_row_stride, const void* q_logits, int64_t q_seq_stride,
                                      int64_t q_row_stride, const int32_t* draft_tokens, const float* u_accept,
                                      const float* u_sample, float temperature, int32_t* out_accept_len,
                                      int32_t* out_token, float* out_p_draft, float* out_q_draft,
                                      float* out_residual_mass, void* workspace, size_t workspace_bytes) {
  UNO_GUARD_BEGIN
  VerifyLinearArgs a{};
  uno_status s = verify_linear_args(logit_dtype, batch, k, vocab, p_logits, p_seq_stride, p_row_stride, q_logits,
                                    q_seq_stride, q_row_stride, draft_tokens, u_accept, u_sample, temperature,
                                    out_accept_len, out_token, out_p_draft, out_q_draft, out_residual_mass, &a);
  if (s != UNO_OK) return s;
  const size_t need = verify_linear_workspace_bytes(batch, k, vocab);
  if (workspace_bytes < need || !workspace)
    return fail(UNO_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  a.ws = workspace;
  s = debug_check_verify_linear(stream, a);
  if (s != UNO_OK) return s;
  return check_hip(launch_verify_linear(a, stream), "uno_psi_spec_verify_linear launch");
  UNO_GUARD_END
}

// ------------------------------------------------------------------ early-exit linear verify
uno_status uno_psi_spec_verify_linear_early_exit_workspace(int32_t batch, int32_t k, int32_t vocab, size_t* bytes) {
  UNO_GUARD_BEGIN
  if (!bytes) return fail(UNO_ERR_INVALID_ARGUMENT, "bytes is NULL");
  const uno_status s = check_verify_linear_shape(batch, k, vocab);
  if (s != UNO_OK) return s;
  *bytes = verify_linear_ee_workspace_bytes(batch, k, vocab);
  return UNO_OK;
  UNO_GUARD_END
}

uno_status uno_psi_spec_verify_linear_early_exit(hipStream_t stream, uno_dtype logit_dtype, int32_t batch, int32_t k,
                                                 int32_t vocab, const void* p_logits, int64_t p_seq_stride,
                                                 int64_t p_row_stride, const void* q_logits, int64_t q_seq_stride,
                                                 int64_t q_row_stride, const int32_t* draft_tokens,
                                                 const float* u_accept, const float* u_sample, float temperature,
                                                 int32_t* out_accept_len, int32_t* out_token, float* out_p_draft,
                                                 float* out_q_draft, float* out_residual_mass, void* workspace,
                                                 size_t workspace_bytes) {
  UNO_GUARD_BEGIN
  VerifyLinearArgs a{};
  uno_status s = verify_linear_args(logit_dtype, batch, k, vocab, p_logits, p_seq_stride, p_row_stride, q_logits,
                                    q_seq_stride, q_row_stride, draft_tokens, u_accept, u_sample, temperature,
                                    out_accept_len, out_token, out_p_draft, out_q_draft, out_residual_mass, &a);
  if (s != UNO_OK) return s;
  const size_t need = verify_linear_ee_workspace_bytes(batch, k, vocab);
  if (workspace_bytes < need || !workspace)
    return fail(UNO_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  a.ws = workspace;
  s = debug_check_verify_linear(stream, a);
  if (s != UNO_OK) return s;
  return check_hip(launch_verify_linear_ee(a, stream), "uno_psi_spec_verify_linear_early_exit launch");
  UNO_GUARD_END
}

// ------------------------------------------------------------------ sampled linear verify
static uno_status check_sampling(int32_t vocab, int32_t top_k, float top_p, int32_t greedy) {
  if (top_k < 0) return fail(UNO_ERR_INVALID_ARGUMENT, "top_k must be >= 0 (0: off; got %d)", top_k);
  if (!(top_p > 0.f) || !(top_p <= 1.f)) return fail(UNO_ERR_INVALID_ARGUMENT, "top_p must be in (0, 1]");
  if (greedy != 0 && greedy != 1) return fail(UNO_ERR_INVALID_ARGUMENT, "greedy must be 0 or 1");
  (void)vocab;
  return UNO_OK;
}

uno_status uno_psi_spec_verify_linear_sampled_workspace(int32_t batch, int32_t k, int32_t vocab, size_t* bytes) {
  UNO_GUARD_BEGIN
  if (!bytes) return fail(UNO_ERR_INVALID_ARGUMENT, "bytes is NULL");
  uno_status s = check_verify_linear_shape(batch, k, vocab);
  if (s != UNO_OK) return s;
  *bytes = verify_linear_sampled_workspace_bytes(batch, k, vocab);
  return UNO_OK;
  UNO_GUARD_END
}

uno_status uno_psi_spec_verify_linear_sampled(hipStream_t stream, uno_dtype logit_dtype, int32_t batch, int32_t k,
                                              int32_t vocab, const void* p_logits, int64_t p_seq_stride,
                                              int64_t p_row_stride, const void* q_logits, int64_t q_seq_stride,
                                              int64_t q_row_stride, const int32_t* draft_tokens,
                                              const float* u_accept, const float* u_sample, float temperature,
                                              int32_t top_k, float top_p, int32_t greedy, int32_t* out_accept_len,
                                              int32_t* out_token, float* out_p_draft, float* out_q_draft,
                                              float* out_residual_mass, void* workspace, size_t workspace_bytes) {
  UNO_GUARD_BEGIN
  VerifyLinearArgs a{};
  uno_status s = verify_linear_args(logit_dtype, batch, k, vocab, p_logits, p_seq_stride, p_row_stride, q_logits,
                                    q_seq_stride, q_row_stride, draft_tokens, u_accept, u_sample, temperature,
                                    out_accept_len, out_token, out_p_draft, out_q_draft, out_residual_mass, &a);
  if (s != UNO_OK) return s;
  s = check_sampling(vocab, top_k, top_p, greedy);
  if (s != UNO_OK) return s;
  const size_t need = verify_linear_sampled_workspace_bytes(batch, k, vocab);
  if (workspace_bytes < need || !workspace)
    return fail(UNO_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  a.ws = workspace;
  s = debug_check_verify_linear(stream, a);
  if (s != UNO_OK) return s;
  return check_hip(launch_verify_linear_sampled(a, top_k, top_p, greedy, stream),
                   "uno_psi_spec_verify_linear_sampled launch");
  UNO_GUARD_END
}

// ------------------------------------------------------------------ tree attention
static uno_status check_tree_attn_shape(int32_t batch, int32_t n_tree, int32_t ctx, int32_t nh, int32_t nkv,
                                        int32_t hd) {
  if (batch < 1 || n_tree < 1 || ctx < 0 || nh < 1 || nkv < 1)
    return fail(UNO_ERR_INVALID_ARGUMENT, "sizes must be batch,n_tree,n_heads,n_kv_heads >= 1 and ctx_len >= 0");
  if (hd != 128) return fail(UNO_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", hd);
  if (nh % nkv != 0) return fail(UNO_ERR_INVALID_ARGUMENT, "n_heads must be a multiple of n_kv_heads");
  if (nh / nkv > 8) return fail(UNO_ERR_UNSUPPORTED, "at most 8 query heads per KV head");
  if (n_tree > 256) return fail(UNO_ERR_UNSUPPORTED, "n_tree above 256 (got %d)", n_tree);
  if (int64_t(ctx) + n_tree > (int64_t(1) << 30)) return fail(UNO_ERR_UNSUPPORTED, "context too long");
  if (batch > 65535 || nkv > 65535) return fail(UNO_ERR_UNSUPPORTED, "grid too large");
  return UNO_OK;
}

uno_status uno_tree_verify_attention_workspace(int32_t batch, int32_t n_tree, int32_t ctx_len, int32_t n_heads,
                                               int32_t n_kv_heads, int32_t head_dim, size_t* bytes) {
  UNO_GUARD_BEGIN
  if (!bytes) return fail(UNO_ERR_INVALID_ARGUMENT, "bytes is NULL");
  uno_status s = check_tree_attn_shape(batch, n_tree, ctx_len, n_heads, n_kv_heads, head_dim);
  if (s != UNO_OK) return s;
  *bytes = tree_attention_workspace_bytes(batch, n_tree, ctx_len, n_heads, n_kv_heads, head_dim);
  return UNO_OK;
  UNO_GUARD_END
}

uno_status uno_tree_verify_attention(hipStream_t stream, int32_t batch, int32_t n_tree, int32_t ctx_len,
                                     int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, const void* q,
                                     const void* k_cache, const void* v_cache, const void* k_tree,
                                     const void* v_tree, const int32_t* parent, float softmax_scale, void* out,
                                     float* out_lse, void* workspace, size_t workspace_bytes) {
  UNO_GUARD_BEGIN
  uno_status s = check_tree_attn_shape(batch, n_tree, ctx_len, n_heads, n_kv_heads, head_dim);
  if (s != UNO_OK) return s;
  if (!q || !k_tree || !v_tree || !parent || !out || (ctx_len > 0 && (!k_cache || !v_cache)))
    return fail(UNO_ERR_INVALID_ARGUMENT, "required pointer is NULL");
  if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(out) ||
      (ctx_len > 0 && (!aligned16(k_cache) || !aligned16(v_cache))))
    return fail(UNO_ERR_UNSUPPORTED, "bf16 tensors must be 16-byte aligned");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(UNO_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
  const size_t need = tree_attention_workspace_bytes(batch, n_tree, ctx_len, n_heads, n_kv_heads, head_dim);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(UNO_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  TreeAttnArgs a{};
  a.batch = batch;
  a.n_tree = n_tree;
  a.ctx = ctx_len;
  a.n_heads = n_heads;
  a.n_kv = n_kv_heads;
  a.head_dim = head_dim;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_tree = k_tree;
  a.v_tree = v_tree;
  a.parent = parent;
  a.scale = softmax_scale;
  a.out = out;
  a.out_lse = out_lse;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  return check_hip(launch_tree_attention(a, stream), "uno_tree_verify_attention launch");
  UNO_GUARD_END
}

// ------------------------------------------------------------------ tree verify
static uno_status check_tree_verify_shape(int32_t batch, int32_t n_tree, int32_t max_depth, int32_t max_children,
                                          int32_t vocab) {
  if (batch < 1 || n_tree < 1 || max_depth < 1 || vocab < 1)
    return fail(UNO_ERR_INVALID_ARGUMENT, "batch, n_tree, max_depth and vocab must be >= 1");
  if (max_children < 0 || max_children > 1023)
    return fail(UNO_ERR_INVALID_ARGUMENT, "max_children must be in 0..1023 (got %d)", max_children);
  if (batch > 65535) return fail(UNO_ERR_UNSUPPORTED, "batch above 65535");
  if (n_tree > 1024) return fail(UNO_ERR_UNSUPPORTED, "n_tree above 1024 (got %d)", n_tree);
  if (max_depth > 64) return fail(UNO_ERR_UNSUPPORTED, "max_depth above 64 (got %d)", max_depth);
  if (vocab > (1 << 20)) return fail(UNO_ERR_UNSUPPORTED, "vocab above 2^20 (got %d)", vocab);
  if (int64_t(batch) * (n_tree + max_depth) > (int64_t(1) << 31) - 1) return fail(UNO_ERR_UNSUPPORTED, "too many rows");
  return UNO_OK;
}

static uno_status tree_workspace(int32_t batch, int32_t n_tree, int32_t max_depth, int32_t max_children,
                                 int32_t vocab, int wor, size_t* bytes) {
  if (!bytes) return fail(UNO_ERR_INVALID_ARGUMENT, "bytes is NULL");
  uno_status s = check_tree_verify_shape(batch, n_tree, max_depth, max_children, vocab);
  if (s != UNO_OK) return s;
  if (wor && max_children > 64)
    return fail(UNO_ERR_UNSUPPORTED, "without replacement: max_children above 64 (got %d)", max_children);
  *bytes = tree_verify_workspace_bytes(batch, n_tree, max_depth, max_children, vocab, wor);
  return UNO_OK;
}

static uno_status verify_tree(hipStream_t stream, uno_dtype logit_dtype, int32_t batch, int32_t n_tree,
                              int32_t max_depth, int32_t max_children, int32_t vocab, const int32_t* parent,
                              const int32_t* tokens, const void* p_logits, const void* q_logits,
                              const float* u_accept, const float* u_sample, float temperature,
                              int32_t* out_accept_len, int32_t* out_path, int32_t* out_token, void* workspace,
                              size_t workspace_bytes, int wor, const char* name) {
  if (logit_dtype != UNO_F32 && logit_dtype != UNO_BF16)
    return fail(UNO_ERR_INVALID_ARGUMENT, "unknown dtype %d", int(logit_dtype));
  uno_status s = check_tree_verify_shape(batch, n_tree, max_depth, max_children, vocab);
  if (s != UNO_OK) return s;
  if (wor && max_children > 64)
    return fail(UNO_ERR_UNSUPPORTED, "without replacement: max_children above 64 (got %d)", max_children);
  if (!parent || !tokens || !p_logits || !q_logits || !u_accept || !u_sample || !out_accept_len || !out_path ||
      !out_token)
    return fail(UNO_ERR_INVALID_ARGUMENT, "required pointer is NULL");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(UNO_ERR_INVALID_ARGUMENT, "temperature must be finite and > 0");
  const size_t need = tree_verify_workspace_bytes(batch, n_tree, max_depth, max_children, vocab, wor);
  if (workspace_bytes < need || !workspace)
    return fail(UNO_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  TreeVerifyArgs a{};
  a.dtype = logit_dtype;
  a.batch = batch;
  a.n_tree = n_tree;
  a.max_depth = max_depth;
  a.max_children = max_children;
  a.vocab = vocab;
  a.parent = parent;
  a.tokens = tokens;
  a.p = p_logits;
  a.q = q_logits;
  a.u_acc = u_accept;
  a.u_s = u_sample;
  a.scale_log2 = float(1.4426950408889634 / double(temperature));
  a.out_len = out_accept_len;
  a.out_path = out_path;
  a.out_tok = out_token;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  a.wor = wor;
  if (debug_checks()) {   // node tokens (the root's is unused) and the uniforms
    uno_status d = debug_check_ids(stream, tokens, batch, n_tree, n_tree, 1, 0, vocab, "tokens");
    if (d == UNO_OK) d = debug_check_unit(stream, u_accept, int64_t(batch) * n_tree, "u_accept");
    if (d == UNO_OK) d = debug_check_unit(stream, u_sample, batch, "u_sample");
    if (d != UNO_OK) return d;
  }
  return check_hip(launch_tree_verify(a, stream), name);
}

uno_status uno_psi_spec_verify_tree_workspace(int32_t batch, int32_t n_tree, int32_t max_depth, int32_t max_children,
                                              int32_t vocab, size_t* bytes) {
  UNO_GUARD_BEGIN
  return tree_workspace(batch, n_tree, max_depth, max_children, vocab, 0, bytes);
  UNO_GUARD_END
}

uno_status uno_psi_spec_verify_tree(hipStream_t stream, uno_dtype logit_dtype, int32_t batch, int32_t n_tree,
                                    int32_t max_depth, int32_t max_children, int32_t vocab, const int32_t* parent,
                                    const int32_t* tokens, const void* p_logits, const void* q_logits,
                                    const float* u_accept, const float* u_sample, float temperature,
                                    int32_t* out_accept_len, int32_t* out_path, int32_t* out_token, void* workspace,
                                    size_t workspace_bytes) {
  UNO_GUARD_BEGIN
  return verify_tree(stream, logit_dtype, batch, n_tree, max_depth, max_children, vocab, parent, tokens, p_logits,
                     q_logits, u_accept, u_sample, temperature, out_accept_len, out_path, out_token, workspace,
                     workspace_bytes, 0, "uno_psi_spec_verify_tree launch");
  UNO_GUARD_END
}

uno_status uno_psi_spec_verify_tree_wor_workspace(int32_t batch, int32_t n_tree, int32_t max_depth,
                                                  int32_t max_children, int32_t vocab, size_t* bytes) {
  UNO_GUARD_BEGIN
  return tree_workspace(batch, n_tree, max_depth, max_children, vocab, 1, bytes);
  UNO_GUARD_END
}

uno_status uno_psi_spec_verify_tree_wor(hipStream_t stream, uno_dtype logit_dtype, int32_t batch, int32_t n_tree,
                                        int32_t max_depth, int32_t max_children, int32_t vocab, const int32_t* parent,
                                        const int32_t* tokens, const void* p_logits, const void* q_logits,
                                        const float* u_accept, const float* u_sample, float temperature,
                                        int32_t* out_accept_len, int32_t* out_path, int32_t* out_token,
                                        void* workspace, size_t workspace_bytes) {
  UNO_GUARD_BEGIN
  return verify_tree(stream, logit_dtype, batch, n_tree, max_depth, max_children, vocab, parent, tokens, p_logits,
                     q_logits, u_accept, u_sample, temperature, out_accept_len, out_path, out_token, workspace,
                     workspace_bytes, 1, "uno_psi_spec_verify_tree_wor launch");
  UNO_GUARD_END
}

}  // extern "C"
