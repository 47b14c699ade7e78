/*
 * libunospec -- the data-parallel hot path of one Psi-Spec decode step of Uno,
 * a diffusion-augmented LLM, for AMD Instinct MI355X (gfx950).
 *
 * Method source: "Uno" (arXiv 2609.04010) as summarised on hyper.ai, section
 * "方法" (method): LoRA adapters on every AR weight matrix, a per-position
 * gate over one concatenated clean + noisy forward, and the Psi-Spec sampler
 * (rejection sampling against the AR distribution that keeps the longest
 * valid prefix, with a linear and a tree candidate strategy).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Memory: every data pointer is device memory of the current HIP device,
 *   owned by the caller.  The library never allocates or frees device memory
 *   in a call; scratch space is the caller's `workspace`, sized by the
 *   matching *_workspace query (a size of 0 allows workspace == NULL).
 * - Layout: row-major (C order).  "ld"/"stride" arguments are in elements.
 * - Ordering: work is enqueued on `stream` (NULL = the null stream) and the
 *   call returns without synchronising.  Device-side faults surface at the
 *   caller's next synchronisation.
 * - Errors: arguments are validated on the host before anything is enqueued;
 *   an invalid call enqueues nothing and returns a non-zero uno_status.
 *   uno_last_error() returns a message for the calling thread's last error.
 *   No C++ exception crosses this interface.
 * - Threads: calls are reentrant; concurrent calls must not share a workspace.
 * - Aliasing: outputs must not alias inputs or each other.
 * - Data contract: token ids in [0, vocab), finite logits, uniforms in [0, 1).
 *   These are not checked on the device.
 */
#ifndef UNO_H
#define UNO_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  UNO_OK = 0,
  UNO_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, bad stride, bad tree */
  UNO_ERR_UNSUPPORTED = 2,      /* valid but outside what the kernels implement */
  UNO_ERR_WORKSPACE = 3,        /* workspace smaller than the query returned */
  UNO_ERR_HIP = 4,              /* a HIP runtime call or a launch failed */
  UNO_ERR_INTERNAL = 5
} uno_status;

typedef enum { UNO_F32 = 0, UNO_BF16 = 1 } uno_dtype;

#define UNO_ABI_VERSION 2

int uno_abi_version(void);
const char* uno_status_string(uno_status s);
/* Message describing the calling thread's most recent error ("" if none). */
const char* uno_last_error(void);

/* --------------------------------------------------------------------------
 * Gated-LoRA linear layer.
 * Source: Uno summary (hyper.ai), section "方法": the diffusion weights are
 * low-rank adapters on every AR weight matrix; drafting uses AR + adapter
 * weights, verification the AR weights only; one forward over concatenated
 * clean and noisy sequences, with a mask that disables the adapter on clean
 * positions and enables it on noisy ones.
 *
 *   y[m, :] = x[m, :] W^T + lora_scale * gate[m] * (x[m, :] A^T) B^T
 *
 * dtype   UNO_BF16: x, W, A, B, y are bf16; products accumulate in fp32 on
 *         matrix cores; the low-rank intermediate x A^T is held as bf16.
 *         UNO_F32: everything fp32 (vector ALU).
 * x [M, K] (row stride ldx >= K), W [N, K] (ldw >= K), A [r, K] (lda >= K),
 * B [N, r] (ldb >= r), y [M, N] (ldy >= N).
 * gate    uint8 [M]; 0 = clean/verify row (AR weights only), non-zero = noisy/
 *         draft row (adapter on).  NULL = all rows 0.  r = 0 is allowed (A, B
 *         unused, may be NULL): a plain GEMM.
 * Requirements: M, N, K >= 1, r >= 0.  UNO_BF16 also needs K and r multiples
 * of 8, ldx, ldw, lda, ldb multiples of 8 and 16-byte aligned x, W, A, B
 * (else UNO_ERR_UNSUPPORTED); y and ldy are unconstrained.
 * Rows whose gate is 0 give results bit-identical to the same call with r = 0.
 * ------------------------------------------------------------------------ */
uno_status uno_gated_lora_linear_workspace(uno_dtype dtype, int64_t M, int64_t N, int64_t K,
                                           int64_t r, size_t* bytes);
uno_status uno_gated_lora_linear(hipStream_t stream, uno_dtype dtype,
                                 int64_t M, int64_t N, int64_t K, int64_t r,
                                 const void* x, int64_t ldx, const void* W, int64_t ldw,
                                 const void* A, int64_t lda, const void* B, int64_t ldb,
                                 const uint8_t* gate, float lora_scale,
                                 void* y, int64_t ldy,
                                 void* workspace, size_t workspace_bytes);

/* --------------------------------------------------------------------------
 * Psi-Spec linear verify sampler.
 * Source: Uno summary (hyper.ai), section "方法", last paragraph: a block
 * proposed by the diffusion path is rejection-sampled against the base AR
 * distribution and the longest valid prefix is accepted; the linear sampler
 * draws one candidate sequence from the marginals; the block's first token
 * comes from the AR weights.  The acceptance rule and residual are standard
 * speculative sampling (Leviathan et al. 2023; Chen et al. 2023):
 *
 *   p_i = softmax(p_logits[b, i] / T), i = 0..k      (row k = bonus row)
 *   q_i = softmax(q_logits[b, i] / T), i = 0..k-1
 *   accept draft i  iff  u_accept[b, i] * q_i[d_i] < p_i[d_i]
 *   L = first rejected i (k if none)
 *   L < k: w = max(0, p_L - q_L) (falls back to p_L if sum(w) == 0); L = k: w = p_k
 *   y = smallest v (token-id order) with cumsum(w)[v] > u_sample[b] * sum(w)
 *
 * p_logits [batch][k+1][vocab] with strides (p_seq_stride, p_row_stride),
 *   row i = AR distribution of the position of draft i (the logit row of the
 *   preceding token), row k = the position after the last draft.
 * q_logits [batch][k][vocab] with strides (q_seq_stride, q_row_stride).
 * draft_tokens int32 [batch][k]; u_accept f32 [batch][k]; u_sample f32 [batch].
 * Outputs: out_accept_len int32 [batch] (L in 0..k), out_token int32 [batch]
 *   (the correction or bonus token y; the step emits d[0:L] then y).
 *   Optional (may be NULL): out_p_draft f32 [batch][k] = p_i[d_i],
 *   out_q_draft f32 [batch][k] = q_i[d_i], out_residual_mass f32 [batch] =
 *   sum(w) of the row y was drawn from (1 for a bonus draw).
 * Requirements: batch >= 1, 0 <= k <= 64, 1 <= vocab <= 2^20, temperature > 0,
 *   row strides >= vocab, sequence strides >= the rows they hold.
 * ------------------------------------------------------------------------ */
uno_status uno_psi_spec_verify_linear_workspace(int32_t batch, int32_t k, int32_t vocab, size_t* bytes);
uno_status uno_psi_spec_verify_linear(hipStream_t stream, uno_dtype logit_dtype,
                                      int32_t batch, int32_t k, int32_t vocab,
                                      const void* p_logits, int64_t p_seq_stride, int64_t p_row_stride,
                                      const void* q_logits, int64_t q_seq_stride, int64_t q_row_stride,
                                      const int32_t* draft_tokens,
                                      const float* u_accept, const float* u_sample,
                                      float temperature,
                                      int32_t* out_accept_len, int32_t* out_token,
                                      float* out_p_draft, float* out_q_draft, float* out_residual_mass,
                                      void* workspace, size_t workspace_bytes);

/* --------------------------------------------------------------------------
 * Tree-masked grouped-query attention for tree verification.
 * Source: Uno summary (hyper.ai), section "方法", last paragraph: the tree
 * sampler verifies several candidates concurrently as a prefix tree with tree
 * attention.  Node i of the tree attends to every cached position and to the
 * tree nodes that are its ancestors or itself:
 *
 *   O[b,i,h] = sum_j softmax_j(scale * <Q[b,i,h], K_j>) V_j,
 *   j over cache rows 0..ctx_len-1 and tree nodes {ancestors of i} + {i},
 *   K_j, V_j taken from KV head h / (n_heads / n_kv_heads).
 *
 * q       bf16 [batch][n_tree][n_heads][head_dim]   (RoPE already applied)
 * k_cache, v_cache bf16 [batch][ctx_len][n_kv_heads][head_dim]
 * k_tree,  v_tree  bf16 [batch][n_tree][n_kv_heads][head_dim]
 * parent  int32 [batch][n_tree]: parent[b][0] = -1, 0 <= parent[b][i] < i.
 *         Checked on the device; a bad tree makes that batch element's
 *         outputs NaN.
 * out     bf16 [batch][n_tree][n_heads][head_dim]
 * out_lse optional f32 [batch][n_tree][n_heads]: natural-log log-sum-exp of
 *         the scaled scores.
 * workspace: device memory of at least the size the _workspace query gives
 *   (0 when the call has enough query tiles to fill the device on its own;
 *   otherwise per-split partial results, fp32).  K and V must be finite: a
 *   masked key still enters the products with weight 0.
 * Requirements: head_dim == 128, n_heads a multiple of n_kv_heads,
 *   n_heads / n_kv_heads <= 8, 1 <= n_tree <= 256, ctx_len >= 0, batch >= 1.
 * ------------------------------------------------------------------------ */
uno_status uno_tree_verify_attention_workspace(int32_t batch, int32_t n_tree, int32_t ctx_len,
                                               int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                               size_t* bytes);
uno_status uno_tree_verify_attention(hipStream_t stream,
                                     int32_t batch, int32_t n_tree, int32_t ctx_len,
                                     int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                     const void* q, const void* k_cache, const void* v_cache,
                                     const void* k_tree, const void* v_tree,
                                     const int32_t* parent, float softmax_scale,
                                     void* out, float* out_lse,
                                     void* workspace, size_t workspace_bytes);

/* --------------------------------------------------------------------------
 * Psi-Spec tree verify: per-node rejection over a prefix tree.
 * Source: Uno summary (hyper.ai), section "方法", last paragraph (tree
 * sampler; lossless in both the linear and the tree case).  Read as
 * multi-candidate speculative sampling (SpecInfer, Miao et al. 2023):
 *   cur = root, r = p_root;
 *   children c of cur in ascending node id, token t, depth d:
 *     accept iff u_accept[b][c] * q_d[t] < r[t] -> cur = c, r = p_c, repeat;
 *     reject -> r = max(0, r - q_d) / sum (unchanged if the sum is 0);
 *   no child accepted (or no child): y = smallest v with cumsum(r)[v] > u_sample * sum(r).
 *   L = depth of cur; the path is the accepted node ids.
 * Siblings are read as i.i.d. draws from the per-depth marginal q_d.
 *
 * parent, tokens int32 [batch][n_tree] (parent[b][0] = -1, parent[b][i] < i;
 *   tokens[b][0] unused).
 * p_logits [batch][n_tree][vocab]: AR row of each node (scores its children).
 * q_logits [batch][max_depth][vocab]: draft marginal of depth 1..max_depth.
 * u_accept f32 [batch][n_tree] (entry 0 unused), u_sample f32 [batch].
 * max_children: upper bound on the children of any node (the caller builds
 *   the tree and knows its branching); the residual masses are computed in
 *   max_children chunk-parallel rounds.
 * Outputs: out_accept_len int32 [batch]; out_path int32 [batch][max_depth]
 *   (accepted node ids, -1 padded); out_token int32 [batch].
 * Requirements: 1 <= batch <= 65535, 1 <= n_tree <= 1024, 1 <= max_depth <= 64,
 *   0 <= max_children <= 1023, 1 <= vocab <= 2^20, temperature > 0.  The tree
 *   is checked on the device: parent[0] = -1, 0 <= parent[i] < i, depth at
 *   most max_depth, at most max_children children per node; a tree that
 *   fails yields out_accept_len = -1, out_token = -1 and an all -1 path.
 * ------------------------------------------------------------------------ */
uno_status uno_psi_spec_verify_tree_workspace(int32_t batch, int32_t n_tree, int32_t max_depth,
                                              int32_t max_children, int32_t vocab, size_t* bytes);
uno_status uno_psi_spec_verify_tree(hipStream_t stream, uno_dtype logit_dtype,
                                    int32_t batch, int32_t n_tree, int32_t max_depth, int32_t max_children,
                                    int32_t vocab,
                                    const int32_t* parent, const int32_t* tokens,
                                    const void* p_logits, const void* q_logits,
                                    const float* u_accept, const float* u_sample,
                                    float temperature,
                                    int32_t* out_accept_len, int32_t* out_path, int32_t* out_token,
                                    void* workspace, size_t workspace_bytes);

/* ==========================================================================
 * The composed decode step.  Source: Uno summary (hyper.ai), section 方法
 * (one forward over the concatenated clean and noisy rows of a block, the
 * adapter switched per row) and section 实验 (adapters on an open-weight
 * Qwen3-8B model, rank 128, a KV cache shared by the draft and verify paths,
 * full attention).  The pages give no layer internals; the functions below
 * implement a Qwen3-shaped pre-norm layer: RMSNorm, rotary embeddings on q
 * and k ("rotate half" pairing), grouped-query attention, SwiGLU MLP,
 * residual stream.  Rows of one sequence are its `block` clean rows followed
 * by its `block` noisy rows; sequences are consecutive.  All activations are
 * bf16, row-major, 16-byte aligned with leading dimensions that are
 * multiples of 8 elements.
 * ======================================================================== */

/* RMSNorm with an optional fused residual add.
 *   res == NULL: out = bf16(x / sqrt(mean(x^2) + eps) * weight)
 *   res != NULL: s = bf16(x + res) is written to sum_out (which may be x
 *                itself), then out = bf16(s / sqrt(mean(s^2) + eps) * weight);
 *                out may be NULL (residual add only).
 * rows >= 1, 8 <= dim <= 16384, dim % 8 == 0; one pass over the inputs. */
uno_status uno_rms_norm(hipStream_t stream, int64_t rows, int32_t dim,
                        const void* x, int64_t ldx, const void* res, int64_t ldr,
                        void* sum_out, int64_t ld_sum, const void* weight, float eps,
                        void* out, int64_t ldo);

/* Rotary position embedding, in place, on x [rows][n_heads][128]: element
 * pair (i, i + 64) of every head is rotated by positions[row] * theta^(-i/64)
 * (angle formed in double precision).  positions int32 [rows], >= 0. */
uno_status uno_rope(hipStream_t stream, int64_t rows, int32_t n_heads, void* x, int64_t ldx,
                    const int32_t* positions, float theta);

/* SwiGLU product out = bf16(silu(g) * u), silu(g) = g / (1 + e^-g);
 * [rows][dim], dim % 8 == 0; out may be g or u. */
uno_status uno_silu_mul(hipStream_t stream, int64_t rows, int32_t dim, const void* g, int64_t ldg,
                        const void* u, int64_t ldu, void* out, int64_t ldo);

/* Block-masked GQA attention of the 2*block rows of every sequence over its
 * KV cache and the block's own keys: clean row i (i < block) sees the whole
 * cache and clean rows 0..i; a noisy row sees the whole cache and all 2*block
 * rows of the block.  Layouts as uno_tree_verify_attention with
 * n_tree = 2*block: q [batch][2*block][n_heads][128], k_block/v_block
 * [batch][2*block][n_kv_heads][128], caches [batch][ctx_len][n_kv_heads][128].
 * 1 <= block <= 128; workspace from the query (fp32 split partials).
 * cache_len (optional, device int32 [batch]): sequence b's cache holds
 * cache_len[b] valid rows (clamped to [0, ctx_len]) and only those are
 * attended; ctx_len is then the capacity, the row distance between
 * sequences.  NULL = every sequence has ctx_len rows. */
uno_status uno_block_verify_attention_workspace(int32_t batch, int32_t block, int32_t ctx_len,
                                                int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                                size_t* bytes);
uno_status uno_block_verify_attention(hipStream_t stream,
                                      int32_t batch, int32_t block, int32_t ctx_len,
                                      int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                      const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* cache_len,
                                      const void* k_block, const void* v_block, float softmax_scale,
                                      void* out, float* out_lse,
                                      void* workspace, size_t workspace_bytes);

/* Row sampler: out_token[i] = smallest v with cumsum(softmax(logits[i] / T))_v
 * > u[i] (the last token with mass if rounding leaves none), in token order --
 * the same inverse-CDF rule as the verify samplers' draws.  Used to draw the
 * draft tokens from the noisy rows' distributions.  logits [rows] rows of
 * `vocab` at row_stride elements (bf16 or fp32); u f32 [rows] in [0, 1). */
uno_status uno_sample_rows_workspace(int32_t rows, int32_t vocab, size_t* bytes);
uno_status uno_sample_rows(hipStream_t stream, uno_dtype logit_dtype, int32_t rows, int32_t vocab,
                           const void* logits, int64_t row_stride, const float* u, float temperature,
                           int32_t* out_token, void* workspace, size_t workspace_bytes);

/* One decoder layer over the residual stream, in place.
 * Weights (bf16, row-major): attn_norm and mlp_norm [hidden]; for each
 * projection p in (q, k, v, o, gate, up, down), w[p] [out][in], a[p]
 * [r][in], b[p] [out][r] with (out, in) = (n_heads*128, hidden),
 * (n_kv_heads*128, hidden) twice, (hidden, n_heads*128), (inter, hidden)
 * twice, (hidden, inter).  k_cache/v_cache [batch][ctx][n_kv_heads][128].
 *   a = rmsnorm(h); q, k, v = gated_lora(a); rope(q), rope(k);
 *   att = block_attention(q, cache + (k, v)); h += gated_lora(att, o);
 *   a = rmsnorm(h); h += gated_lora(silu(gated_lora(a, gate)) * gated_lora(a, up), down)
 * with every gated_lora as uno_gated_lora_linear under `gate` [rows] and
 * lora_scale.  When the adapters a[q], a[k], a[v] are stored back to back
 * (one [3r][hidden] array), and likewise a[gate], a[up], each group's
 * LoRA-down runs as one launch over the shared input.  hidden_state [rows][hidden], rows = batch * 2 * block;
 * positions int32 [rows].
 * cache_len NULL: every sequence's cache holds ctx_len rows and the block's
 * k and v are not written to it.  cache_len (device int32 [batch]) set:
 * sequence b's cache holds cache_len[b] valid rows out of a capacity of
 * ctx_len (attention sees those rows only), and clean row j of sequence b
 * writes its k (after RoPE) and v into slot cache_len[b] + j of the cache
 * when that slot is below ctx_len; cache_len itself is not changed (see
 * uno_kv_commit).  The caches are then written: k_cache/v_cache must not be
 * read by concurrent work.
 * hidden and inter multiples of 8, r a multiple of 8, n_heads / n_kv_heads
 * <= 8, 1 <= block <= 128. */
enum { UNO_PROJ_Q = 0, UNO_PROJ_K, UNO_PROJ_V, UNO_PROJ_O, UNO_PROJ_GATE, UNO_PROJ_UP, UNO_PROJ_DOWN,
       UNO_NUM_PROJ };
typedef struct {
  const void* attn_norm;
  const void* mlp_norm;
  const void* w[UNO_NUM_PROJ];
  const void* a[UNO_NUM_PROJ];
  const void* b[UNO_NUM_PROJ];
  void* k_cache;   /* read; written only by calls given a cache_len */
  void* v_cache;
} uno_layer_weights;

uno_status uno_decoder_layer_workspace(int32_t batch, int32_t block, int32_t ctx_len, int32_t hidden,
                                       int32_t inter, int32_t n_heads, int32_t n_kv_heads, int32_t r,
                                       size_t* bytes);
uno_status uno_decoder_layer(hipStream_t stream, int32_t batch, int32_t block, int32_t ctx_len,
                             int32_t hidden, int32_t inter, int32_t n_heads, int32_t n_kv_heads, int32_t r,
                             const uno_layer_weights* weights, const uint8_t* gate, const int32_t* positions,
                             const int32_t* cache_len, float rms_eps, float rope_theta, float lora_scale,
                             void* hidden_state, void* workspace, size_t workspace_bytes);

/* KV commit after verification.  Source: Uno summary (hyper.ai), section
 * 方法 (the AR path keeps the longest valid prefix of the block; the block's
 * first token comes from the AR weights alone) and section 实验 (drafting
 * and verification share one KV cache).  The clean rows of a block carry
 * the adapter gate 0 and see only the cache and earlier clean rows, so
 * their keys and values are the AR model's; uno_decoder_layer with a
 * cache_len has already written them after each sequence's valid rows.
 * This call keeps clean rows 0..L (the block's AR token and the accepted
 * drafts) and drops the rest by not counting them:
 *   cache_len[b] = min(capacity, cache_len[b] + accept_len[b] + 1), b < batch.
 * accept_len, cache_len: device int32 [batch]; cache_len updated in place.
 * The correction token is not in the cache: it is the next block's first
 * clean row.  batch >= 1, capacity >= 0. */
uno_status uno_kv_commit(hipStream_t stream, int32_t batch, int32_t capacity, const int32_t* accept_len,
                         int32_t* cache_len);

/* One whole Psi-Spec decode step.  Source: Uno summary (hyper.ai), section
 * 方法 (the diffusion path proposes a block, the AR path verifies it by
 * rejection sampling and keeps the longest valid prefix; the linear sampler
 * draws one candidate from the marginals; one forward pass runs over the
 * concatenated clean and noisy rows with the adapter gated per row) and
 * section 实验 (Qwen3-8B base, rank-128 adapters, shared KV cache).
 *
 * Per sequence b the step takes 2*block token ids: `block` clean ids (the
 * AR token, then k = block - 1 drafts) and `block` noisy ids.  It runs
 *   h = embed[tokens]; gate = 0 on clean rows, 1 on noisy rows;
 *   positions: clean row j and noisy row j at ctx_len + j;
 *   n_layers x uno_decoder_layer (layer l uses layers[l], its KV cache holds
 *     ctx_len positions per sequence; the block is not written to it);
 *   logits = rmsnorm(h, final_norm) . lm_head^T     (bf16 [rows][vocab], no adapter);
 *   drafts[b][i] = inverse-CDF draw from softmax(noisy row i / T) at u_draft[b][i], i < k
 *     (the uno_sample_rows rule);
 *   uno_psi_spec_verify_linear with p = the k + 1 clean rows and q = the first k
 *     noisy rows of the same logits, on the drafts just drawn.
 * Reading: the pages leave open which forward's q a draft is verified against;
 * here the drafts a step verifies are drawn from that step's own noisy rows,
 * which is the same work per step as carrying them over from the previous
 * step (one draw of k rows, one verify of 2k + 1 rows per sequence).
 *
 * layers: host array of n_layers uno_layer_weights (device pointers); embed and
 * lm_head bf16 [vocab][hidden]; final_norm bf16 [hidden]; tokens int32
 * [batch][2*block]; u_draft, u_accept f32 [batch][k]; u_sample f32 [batch];
 * logits (output, caller-owned) bf16 [batch*2*block][vocab]; out_drafts int32
 * [batch][k]; out_accept_len, out_token int32 [batch].  1 <= block <= 65,
 * head_dim 128, hidden and inter multiples of 8, r a multiple of 8 (0: no
 * adapter).  A token id outside [0, vocab) embeds as a zero row.
 *
 * cache_len (optional, device int32 [batch], updated in place): the decode
 * loop's form.  Sequence b's caches hold cache_len[b] valid rows out of a
 * capacity of ctx_len per sequence; clean row j and noisy row j sit at
 * position cache_len[b] + j; every layer writes the clean rows' k and v into
 * its cache after the valid rows (uno_decoder_layer), and after verification
 * the step commits the kept rows (uno_kv_commit), so the next step's
 * cache_len[b] is the old one + out_accept_len[b] + 1.  A slot at or past
 * ctx_len is not written and the length stops at ctx_len.  NULL: every
 * cache holds ctx_len rows, the caches are only read and positions are
 * ctx_len + j. */
typedef struct {
  int32_t batch, block, ctx_len;
  int32_t hidden, inter, n_heads, n_kv_heads, r, n_layers, vocab;
  float rms_eps, rope_theta, lora_scale, temperature;
} uno_step_config;

uno_status uno_psi_spec_step_workspace(const uno_step_config* config, size_t* bytes);
uno_status uno_psi_spec_step(hipStream_t stream, const uno_step_config* config, const uno_layer_weights* layers,
                             const void* embed, const void* final_norm, const void* lm_head,
                             const int32_t* tokens, int32_t* cache_len, const float* u_draft, const float* u_accept,
                             const float* u_sample, void* logits, int32_t* out_drafts,
                             int32_t* out_accept_len, int32_t* out_token,
                             void* workspace, size_t workspace_bytes);

/* --------------------------------------------------------------------------
 * Kernel timing (measurement support, not part of the method).
 * When enabled, every kernel the library launches whose name contains
 * `name_filter` (NULL or "" = every kernel) is bracketed by HIP events
 * recorded on its launch stream; uno_profile_query returns the summed
 * duration in milliseconds and the launch count of recorded kernels whose
 * name contains `name`, over launches since the last reset.  Querying
 * synchronises on the recorded events.  Not thread-safe; for benchmarks.
 * ------------------------------------------------------------------------ */
void uno_profile_enable(int on, const char* name_filter);
void uno_profile_reset(void);
uno_status uno_profile_query(const char* name, double* total_ms, int64_t* count);

#ifdef __cplusplus
}
#endif
#endif /* UNO_H */
