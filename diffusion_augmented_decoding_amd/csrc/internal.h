// Host-side internals of libunospec: launcher declarations, error reporting,
// kernel timing hooks.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>

#include "../../include/uno.h"

namespace uno {

// Thread-local error message set by the entry points.
uno_status fail(uno_status s, const char* fmt, ...);
uno_status check_hip(hipError_t e, const char* what);
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// every exported function body sits in a try block: no exception crosses the ABI
#define UNO_GUARD_BEGIN try {
#define UNO_GUARD_END                                                            \
  }                                                                              \
  catch (...) {                                                                  \
    return ::uno::fail(UNO_ERR_INTERNAL, "internal error (exception caught)");   \
  }

// Kernel timing: bracket a launch with events when profiling is on.
struct ProfileScope {
  ProfileScope(const char* name, hipStream_t stream);
  ~ProfileScope();
  const char* name;
  hipStream_t stream;
  int slot;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Tuning overrides for sweeps: a build compiled with -DUNO_TUNING reads them
// from the environment; the library as built for use ignores the environment.
inline const char* tuning_env(const char* name) {
#ifdef UNO_TUNING
  return getenv(name);
#else
  (void)name;
  return nullptr;
#endif
}

// Data-contract checks (UNO_DEBUG / uno_debug_checks): on when enabled; each
// check waits for the device and returns UNO_ERR_INVALID_ARGUMENT on a
// violation.  ids[r * stride + c], r < rows, first_col <= c < cols, in [lo, hi).
bool debug_checks();
uno_status debug_check_ids(hipStream_t stream, const int32_t* ids, int64_t rows, int64_t cols, int64_t stride,
                           int64_t first_col, int32_t lo, int32_t hi, const char* what);
uno_status debug_check_unit(hipStream_t stream, const float* u, int64_t n, const char* what);
// The checks of a linear verify call (draft ids, both uniforms), when enabled.
inline uno_status debug_check_verify_linear(hipStream_t stream, const struct VerifyLinearArgs& a);

// Raise a kernel's dynamic-LDS limit to `bytes` once per device: `done` holds
// one bit per device id (ids >= 64 set the attribute on every launch).
inline hipError_t ensure_dynamic_lds(const void* kern, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t(1) << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// ---------------------------------------------------------------- sampler
struct RowStat {   // per logit row, log2 domain: y = logit * log2(e) / T
  float m;         // max_v y_v
  float s;         // sum_v 2^(y_v - m)
  float yd;        // y at the draft token (p rows 0..k-1, q rows); unused otherwise
  float pad;
};

struct VerifyLinearArgs {
  uno_dtype dtype;
  int batch, k, vocab;
  const void* p; int64_t p_seq, p_row;
  const void* q; int64_t q_seq, q_row;
  const int32_t* drafts; int64_t drafts_seq;   // draft i of sequence b at drafts[b * drafts_seq + i]
  const float* u_acc;
  const float* u_s;
  float scale_log2;   // log2(e) / T
  int32_t* out_len;
  int32_t* out_tok;
  float* out_pd;
  float* out_qd;
  float* out_mass;
  void* ws;           // workspace (verify_linear_workspace_bytes)
};
inline uno_status debug_check_verify_linear(hipStream_t stream, const VerifyLinearArgs& a) {
  if (!debug_checks()) return UNO_OK;
  uno_status s = debug_check_ids(stream, a.drafts, a.batch, a.k, a.drafts_seq, 0, 0, a.vocab, "draft_tokens");
  if (s == UNO_OK) s = debug_check_unit(stream, a.u_acc, int64_t(a.batch) * a.k, "u_accept");
  if (s == UNO_OK) s = debug_check_unit(stream, a.u_s, a.batch, "u_sample");
  return s;
}
// Gated-LoRA backward (bf16 operands): dx = dY W + dT A (bf16, optional),
// dA = dT^T x and dB = s dY^T U (fp32), U = g (x A^T), dT = s g (dY B).
struct LoraBackwardArgs {
  int64_t M, N, K, r;
  const void* x; int64_t ldx;
  const void* w; int64_t ldw;
  const void* a; int64_t lda;
  const void* b; int64_t ldb;
  const uint8_t* gate;                  // NULL: every row gate 0
  float lora_scale;
  const void* dy; int64_t lddy;
  void* dx; int64_t lddx;               // optional
  float* da; int64_t ldda;
  float* db; int64_t lddb;
  const void* w_t; int64_t ldwt;        // optional: W^T [K][N]; dx and U / dT then run on the forward's kernels
  void* ws;                             // U and dT (bf16 [M][r] each), transposes, partials
};
size_t lora_backward_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r, int with_wt);
hipError_t launch_transpose_bf16(const void* src, int64_t lds, void* dst, int64_t ldd, int64_t rows, int64_t cols,
                                 hipStream_t stream);
hipError_t launch_lora_backward(const LoraBackwardArgs& a, hipStream_t stream);

// Distillation losses of row pairs (student rows against teacher rows).
struct DistillArgs {
  uno_dtype dtype;
  int batch, rows, vocab;                // pair i of sequence b: teacher/student row i
  const void* teacher; int64_t t_seq, t_row;
  const void* student; int64_t s_seq, s_row;
  float scale_log2, inv_t;               // log2(e) / T, 1 / T
  float alpha, beta, grad_scale;
  float* out_kl;                         // [batch * rows]
  float* out_tv;                         // [batch * rows]
  void* grad; int64_t g_seq, g_row;      // optional, the logits' dtype
};
hipError_t launch_distill(const DistillArgs& a, hipStream_t stream);

// Candidate trees from the per-depth draft marginals (breadth first, branching[d]
// children for every node at depth d), tokens drawn with or without replacement.
constexpr int kMaxBranch = 64;
struct TreeBuildArgs {
  uno_dtype dtype;
  int batch, max_depth, vocab, n;
  int branching[64];
  const void* q; int64_t q_seq, q_row;   // q row d of tree b at q + b * q_seq + d * q_row
  const float* u;                        // [batch][n]
  float scale_log2;
  int without;
  int32_t* out_parent;                   // [batch][n]
  int32_t* out_tokens;                   // [batch][n]
  void* ws;
};
size_t tree_build_workspace_bytes(int batch, int max_depth, int vocab);
hipError_t launch_tree_build(const TreeBuildArgs& a, hipStream_t stream);

size_t verify_linear_workspace_bytes(int batch, int k, int vocab);
hipError_t launch_verify_linear(const VerifyLinearArgs& a, hipStream_t stream);
// early exit: the rows after each sequence's first rejection are not read
size_t verify_linear_ee_workspace_bytes(int batch, int k, int vocab);
hipError_t launch_verify_linear_ee(const VerifyLinearArgs& a, hipStream_t stream);
// The same verify on rows transformed by top-k (0: off), top-p (1: off) or greedy.
size_t verify_linear_sampled_workspace_bytes(int batch, int k, int vocab);
hipError_t launch_verify_linear_sampled(const VerifyLinearArgs& a, int top_k, float top_p, int greedy,
                                        hipStream_t stream);
// Host validation of a linear verify call (all but the workspace); fills the
// kernel arguments (ws left null).
uno_status verify_linear_args(uno_dtype logit_dtype, int32_t batch, int32_t k, int32_t vocab, const void* p_logits,
                              int64_t p_seq_stride, int64_t p_row_stride, const void* q_logits,
                              int64_t q_seq_stride, int64_t q_row_stride, const int32_t* draft_tokens,
                              const float* u_accept, const float* u_sample, float temperature,
                              int32_t* out_accept_len, int32_t* out_token, float* out_p_draft, float* out_q_draft,
                              float* out_residual_mass, VerifyLinearArgs* out);

// ---------------------------------------------------------------- gated LoRA
struct GatedLoraArgs {
  uno_dtype dtype;
  int64_t M, N, K, r;
  const void* x; int64_t ldx;
  const void* w; int64_t ldw;
  const void* a; int64_t lda;
  const void* b; int64_t ldb;
  const uint8_t* gate;
  float lora_scale;
  void* y; int64_t ldy;
  void* ws; size_t ws_bytes;
  const void* t_pre; int64_t ldt_pre;   // optional (bf16 path): T = s g (x A^T) computed by the caller
  int gate_block;                       // > 0: the gate is 0 on rows j < gate_block and 1 on the rest of
                                        // every 2 * gate_block rows (as the decode step builds it); the
                                        // LoRA-down then reads only the gated rows (`gate` is not read)
  const void* w_merged;                 // optional (bf16, with gate_block > 0): w + lora_scale * b a, ld ldw;
                                        // the gated rows then read it and no LoRA-down runs
};
// Gate-merged GEMM rows: M rows of the structured gate (gate_block) split into
// clean and gated halves of whole bm-row tiles, gathered by load groups of
// threads / 8 rows.
bool merged_rows_ok(int64_t M, int gate_block, int bm, int threads);

// out[n][k] = bf16(w[n][k] + scale * sum_j b[n][j] a[j][k]) (bf16 operands)
struct LoraMergeArgs {
  int64_t N, K, r;
  const void* w; int64_t ldw;
  const void* a; int64_t lda;
  const void* b; int64_t ldb;
  float scale;
  void* out; int64_t ldo;
};
hipError_t launch_lora_merge(const LoraMergeArgs& m, hipStream_t stream);
size_t gated_lora_workspace_bytes(uno_dtype dtype, int64_t M, int64_t N, int64_t K, int64_t r);

// bf16 LoRA-down of n adapter rows: t [M][n] = bf16(s * g[m] * (x A^T)[m]), 0 where g = 0.
struct LoraDownArgs {
  int64_t M, K, n;
  const void* x; int64_t ldx;
  const void* a; int64_t lda;        // [n][K]
  const uint8_t* gate;
  float lora_scale;
  uint16_t* t;                       // [M][n]
  void* part;                        // fp32 partials, lora_down_part_bytes(M, n, K)
  int gather_blk;                    // > 0: structured gate as GatedLoraArgs::gate_block
};
size_t lora_down_part_bytes(int64_t M, int64_t n, int64_t K);
hipError_t launch_lora_down(const LoraDownArgs& a, hipStream_t stream);
hipError_t launch_gated_lora(const GatedLoraArgs& a, hipStream_t stream);
// Two bf16 projections of the same input and shapes (k and v), T of each
// computed by the caller (t_pre), as one GEMM launch over both outputs.
bool gated_lora_pair_ok(const GatedLoraArgs& a, const GatedLoraArgs& b);
hipError_t launch_gated_lora_pair(const GatedLoraArgs& a, const GatedLoraArgs& b, hipStream_t stream);

// bf16 gate and up projections with the SwiGLU product fused into the GEMM
// epilogue: y[m][f] = bf16(silu(g) * u), g = x Wg^T + t_g Bg^T, u = x Wu^T +
// t_u Bu^T in fp32, t = [t_g | t_u] (M x 2r, both adapters' T side by side,
// as one grouped LoRA-down writes them).  N = features.  Needs K and r
// multiples of 64 and operands within the buffer-load window
// (swiglu_fused_ok); the caller falls back to two projections otherwise.
struct SwigluArgs {
  int64_t M, N, K, r;
  const void* x; int64_t ldx;
  const void* wg; const void* wu; int64_t ldw;     // [N][K] each
  const void* bg; const void* bu; int64_t ldb;     // [N][r] each
  const void* t; int64_t ldt;                      // [M][2r]; unused when r == 0 or merged
  void* y; int64_t ldy;
  // optional: gate-merged weights (both), with the structured gate of
  // gate_block; the gated rows read them and t, bg, bu are not used
  const void* wg_merged; const void* wu_merged;
  int gate_block;
};
bool swiglu_fused_ok(const SwigluArgs& a);
hipError_t launch_gated_lora_swiglu(const SwigluArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- tree attention
struct TreeAttnArgs {
  int batch, n_tree, ctx, n_heads, n_kv, head_dim;
  int block;                 // 0: prefix-tree mask from parent; > 0: clean/noisy block mask
  const int32_t* ctx_lens;   // block mask only: valid cache rows per sequence, clamped to
                             // [0, ctx]; ctx is then the rows of capacity per sequence
                             // (nullptr: every sequence has ctx rows)
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const void* k_tree;
  const void* v_tree;
  const int32_t* parent;
  float scale;
  void* out;
  float* out_lse;
  void* ws; size_t ws_bytes;
};
size_t tree_attention_workspace_bytes(int batch, int n_tree, int ctx, int n_heads, int n_kv, int head_dim);
hipError_t launch_tree_attention(const TreeAttnArgs& a, hipStream_t stream);

// Split-key partials shared by the attention kernels: [batch * n_kv * ks
// groups][tiles32 tiles][32 rows] x (unnormalised O[128] fp32), then the same
// rows x (max in the log2 domain, sum); merged by launch_attn_combine.
size_t attn_part_bytes(int batch, int n_kv, int tiles32, int ks);
hipError_t launch_attn_combine(const TreeAttnArgs& a, int tiles32, int ks, void* ws, hipStream_t stream,
                               const char* name);

// Block-masked attention (a.block > 0, a.n_tree = 2 * a.block) over a long
// cache: K/V blocks staged in LDS and shared by 128 query rows.
size_t block_attention_workspace_bytes(int batch, int block, int ctx, int n_heads, int n_kv);
hipError_t launch_block_attention(const TreeAttnArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- tree verify
struct TreeVerifyArgs {
  uno_dtype dtype;
  int batch, n_tree, max_depth, max_children, vocab;
  const int32_t* parent;
  const int32_t* tokens;
  const void* p;
  const void* q;
  const float* u_acc;
  const float* u_s;
  float scale_log2;
  int32_t* out_len;
  int32_t* out_path;
  int32_t* out_tok;
  void* ws; size_t ws_bytes;
  int wor;   // siblings drawn without replacement (max_children <= 64)
};
size_t tree_verify_workspace_bytes(int batch, int n_tree, int max_depth, int max_children, int vocab, int wor);
hipError_t launch_tree_verify(const TreeVerifyArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- row sampler
struct SampleRowsArgs {
  uno_dtype dtype;
  int rows, vocab;
  const void* logits; int64_t row_stride;
  int per_seq; int64_t seq_stride;   // row i at (i / per_seq) * seq_stride + (i % per_seq) * row_stride
  const float* u;
  float scale_log2;   // log2(e) / T
  int32_t* out_tok;
  void* ws;
};
size_t sample_rows_workspace_bytes(int rows, int vocab);
hipError_t launch_sample_rows(const SampleRowsArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- layer ops
struct RmsNormArgs {
  int64_t rows;
  int dim;
  const void* x; int64_t ldx;
  const void* res; int64_t ldr;      // optional: s = x + res first
  void* sum_out; int64_t lds;        // bf16(s) (required with res; may alias x)
  const void* weight;
  float eps;
  void* out; int64_t ldo;            // optional: bf16(s / rms(s) * weight)
};
int rms_norm_max_dim();
hipError_t launch_rms_norm(const RmsNormArgs& a, hipStream_t stream);

struct RopeArgs {
  int64_t rows;
  int n_heads;
  void* x; int64_t ldx;              // [rows][n_heads * 128], rotated in place
  const int32_t* positions;          // [rows]
  float theta;
  int n_heads2;                      // optional second tensor at the same positions (0: none)
  void* x2; int64_t ldx2;
  // Optional append into a KV cache (cache_len != nullptr; needs x2): rows are
  // sequences of 2*block (block clean, then block noisy); clean row j of
  // sequence b writes its rotated x2 row to k_cache and its v row to v_cache
  // at slot cache_len[b] + j when 0 <= slot < cap.  Caches [batch][cap][n_heads2][128].
  const int32_t* cache_len;
  int block, cap;
  void* k_cache; void* v_cache;
  const void* v; int64_t ldv;
  // Optional per-head RMSNorm before the rotation (bf16 weights of 128):
  // head <- head / sqrt(mean(head^2) + norm_eps) * weight, for x with norm_w
  // and for x2 with norm_w2 (nullptr: no norm on that tensor)
  const void* norm_w;
  const void* norm_w2;
  float norm_eps;
};
hipError_t launch_rope(const RopeArgs& a, hipStream_t stream);

struct SiluMulArgs {
  int64_t rows;
  int dim;
  const void* g; int64_t ldg;
  const void* u; int64_t ldu;
  void* out; int64_t ldo;
};
hipError_t launch_silu_mul(const SiluMulArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- decoder layer
struct DecoderLayerArgs {
  int batch, block, ctx, hidden, inter, n_heads, n_kv, r;
  const uno_layer_weights* w;
  const uint8_t* gate;               // [rows]; null: adapter off everywhere
  const int32_t* positions;          // [rows]
  const int32_t* cache_len;          // [batch] valid cache rows (nullptr: ctx rows each); when set,
                                     // ctx is the capacity and the clean rows' k, v are appended
                                     // at slots cache_len[b] + j (the length itself is not changed)
  int gate_block;                    // > 0: `gate` follows the step's clean/noisy pattern (GatedLoraArgs)
  // Chaining layers (the decode step): norm_ready = the scratch buffer `a`
  // already holds rmsnorm(h, attn_norm) (written by the previous layer), so the
  // first norm is skipped; next_norm != nullptr = the closing residual add also
  // writes rmsnorm(h, next_norm) to next_out (nullptr: this layer's `a`).
  bool norm_ready;
  const void* next_norm;
  void* next_out;
  float rms_eps, rope_theta, lora_scale;
  void* h;                           // bf16 [rows][hidden], updated in place
  void* ws; size_t ws_bytes;
};
size_t decoder_layer_workspace_bytes(int batch, int block, int ctx, int hidden, int inter, int nh, int nkv, int r);
hipError_t launch_decoder_layer(const DecoderLayerArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- step set-up
// Row j of sequence b (rows of a sequence: block clean, then block noisy):
// h[row] = embed[tokens[row]] (a zero row for an id outside [0, vocab)),
// gate[row] = (j >= block), positions[row] = ctx + j (clean row j at ctx + j,
// noisy row j at ctx + block + j), with ctx replaced by cache_len[b] clamped
// to [0, cap] when cache_len is given.
struct StepSetupArgs {
  int64_t rows;
  int block, ctx, hidden, vocab;
  const int32_t* cache_len;          // [batch] or nullptr
  int cap;                           // rows of capacity per sequence (with cache_len)
  const int32_t* tokens;
  const void* embed;                 // bf16 [vocab][hidden]
  void* h;                           // bf16 [rows][hidden]
  uint8_t* gate;
  int32_t* positions;
};
hipError_t launch_step_setup(const StepSetupArgs& a, hipStream_t stream);


// KV commit after verification, for b < batch: with len = cache_len[b]
// (clamped to [0, cap]) and L = accept_len[b], cache_len[b] = len + L + 1 when
// L >= 0 and len + L + 1 <= cap (the rows themselves were appended during the
// forward pass; the rejected and noisy rows are dropped by not counting
// them); otherwise the length is left as it is and accept_len[b] = -1.
hipError_t launch_kv_commit(int batch, int cap, int32_t* accept_len, int32_t* cache_len, hipStream_t stream);

// The end of a decode step, one sequence per 2*block threads: the commit
// above (when cache_len is given; a flagged sequence also gets token -1),
// then the next step's ids [y, d_0 .. d_{k-1}, noisy ids] (next may alias
// tokens: each id is read and written by the same thread).
struct StepFinishArgs {
  int batch, block, cap;
  int32_t* accept_len;               // [batch], set to -1 on overflow
  int32_t* token;                    // [batch], set to -1 on overflow
  int32_t* cache_len;                // [batch] or nullptr
  const int32_t* drafts;             // [batch][block - 1]
  const int32_t* tokens;             // [batch][2 * block]
  int32_t* next;                     // [batch][2 * block] or nullptr
};
hipError_t launch_step_finish(const StepFinishArgs& a, hipStream_t stream);

}  // namespace uno
