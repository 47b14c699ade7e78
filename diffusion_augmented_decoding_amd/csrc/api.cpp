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

// ------------------------------------------------------------------ linear verify
static uno_status check_verify_linear_shape(int32_t batch, int32_t k, int32_t vocab) {
  if (batch < 1) return fail(UNO_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", batch);
  if (k < 0 || k > 64) return fail(UNO_ERR_INVALID_ARGUMENT, "k must be in 0..64 (got %d)", k);
  if (vocab < 1) return fail(UNO_ERR_INVALID_ARGUMENT, "vocab must be >= 1 (got %d)", vocab);
  if (vocab > (1 << 20)) return fail(UNO_ERR_UNSUPPORTED, "vocab above 2^20 (got %d)", vocab);
  if (int64_t(batch) * (2 * k + 1) > (int64_t(1) << 31) - 1) return fail(UNO_ERR_UNSUPPORTED, "too many rows");
  return UNO_OK;
}

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
  if (p_row_stride < vocab || p_seq_stride < int64_t(k + 1) * p_row_stride)
    return fail(UNO_ERR_INVALID_ARGUMENT, "p strides must cover [k+1][vocab]");
  if (k > 0 && (q_row_stride < vocab || q_seq_stride < int64_t(k) * q_row_stride))
    return fail(UNO_ERR_INVALID_ARGUMENT, "q strides must cover [k][vocab]");
  const size_t need = verify_linear_workspace_bytes(batch, k, vocab);
  if (workspace_bytes < need || !workspace)
    return fail(UNO_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
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
  a.u_acc = u_accept;
  a.u_s = u_sample;
  a.scale_log2 = float(1.4426950408889634 / double(temperature));
  a.out_len = out_accept_len;
  a.out_tok = out_token;
  a.out_pd = out_p_draft;
  a.out_qd = out_q_draft;
  a.out_mass = out_residual_mass;
  a.ws = workspace;
  return check_hip(launch_verify_linear(a, stream), "uno_psi_spec_verify_linear launch");
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

uno_status uno_psi_spec_verify_tree_workspace(int32_t batch, int32_t n_tree, int32_t max_depth, int32_t max_children,
                                              int32_t vocab, size_t* bytes) {
  UNO_GUARD_BEGIN
  if (!bytes) return fail(UNO_ERR_INVALID_ARGUMENT, "bytes is NULL");
  uno_status s = check_tree_verify_shape(batch, n_tree, max_depth, max_children, vocab);
  if (s != UNO_OK) return s;
  *bytes = tree_verify_workspace_bytes(batch, n_tree, max_depth, max_children, vocab);
  return UNO_OK;
  UNO_GUARD_END
}

uno_status uno_psi_spec_verify_tree(hipStream_t stream, uno_dtype logit_dtype, int32_t batch, int32_t n_tree,
                                    int32_t max_depth, int32_t max_children, int32_t vocab, const int32_t* parent,
                                    const int32_t* tokens, const void* p_logits, const void* q_logits,
                                    const float* u_accept, const float* u_sample, float temperature,
                                    int32_t* out_accept_len, int32_t* out_path, int32_t* out_token, void* workspace,
                                    size_t workspace_bytes) {
  UNO_GUARD_BEGIN
  if (logit_dtype != UNO_F32 && logit_dtype != UNO_BF16)
    return fail(UNO_ERR_INVALID_ARGUMENT, "unknown dtype %d", int(logit_dtype));
  uno_status s = check_tree_verify_shape(batch, n_tree, max_depth, max_children, vocab);
  if (s != UNO_OK) return s;
  if (!parent || !tokens || !p_logits || !q_logits || !u_accept || !u_sample || !out_accept_len || !out_path ||
      !out_token)
    return fail(UNO_ERR_INVALID_ARGUMENT, "required pointer is NULL");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(UNO_ERR_INVALID_ARGUMENT, "temperature must be finite and > 0");
  const size_t need = tree_verify_workspace_bytes(batch, n_tree, max_depth, max_children, vocab);
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
  return check_hip(launch_tree_verify(a, stream), "uno_psi_spec_verify_tree launch");
  UNO_GUARD_END
}

}  // extern "C"
