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
 * - Data contract: token ids in [0, vocab), finite logits with |logit / T| <=
 *   1e4 (the softmax kernels subtract a separately rounded row maximum inside
 *   a fused multiply-add; exp(-1e4) is already 0 in fp32, so -1e4 stands for
 *   probability 0), uniforms in [0, 1).  These are not checked on the device,
 *   unless the data-contract checks are on (UNO_DEBUG set to anything but "0"
 *   in the environment, or uno_debug_checks(1)): the verify, sampler and step
 *   calls then check their token ids and uniforms on the device first, wait
 *   for the result, and return UNO_ERR_INVALID_ARGUMENT on a violation.  (A
 *   debugging aid: the calls then synchronise their stream.)
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

#define UNO_ABI_VERSION 8

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

/* The data-contract checks (see the conventions above): on = 1 / off = 0; the
 * default comes from the UNO_DEBUG environment variable. */
void uno_debug_checks(int32_t on);
int32_t uno_debug_checks_enabled(void);

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
 *   row strides >= vocab, sequence strides >= the rows they hold (not
 *   checked, and not used, when batch is 1).
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

/* Early-exit variant of uno_psi_spec_verify_linear: the same accept rule,
 * residual and draw, but most rows of positions after the first rejection are
 * not read (drafts are tested in order, and the first rejection ends the
 * block, so those rows cannot change the result).  Source: the same passage
 * (the longest valid prefix of the block is kept).  Same arguments, same
 * requirements, same outputs bit for bit (the row statistics are those of
 * uno_psi_spec_verify_linear, merged in the same order), except that
 * out_p_draft / out_q_draft entries of positions after the first rejection
 * are NaN (not evaluated).  Positions are taken in rounds of 2, 2, 4, then 8
 * positions: a sequence reads the rows of the rounds up to the one holding
 * its first rejection (at most 7 positions past it), and each round costs two
 * kernel launches. */
uno_status uno_psi_spec_verify_linear_early_exit_workspace(int32_t batch, int32_t k, int32_t vocab, size_t* bytes);
uno_status uno_psi_spec_verify_linear_early_exit(hipStream_t stream, uno_dtype logit_dtype,
                                                 int32_t batch, int32_t k, int32_t vocab,
                                                 const void* p_logits, int64_t p_seq_stride, int64_t p_row_stride,
                                                 const void* q_logits, int64_t q_seq_stride, int64_t q_row_stride,
                                                 const int32_t* draft_tokens,
                                                 const float* u_accept, const float* u_sample,
                                                 float temperature,
                                                 int32_t* out_accept_len, int32_t* out_token,
                                                 float* out_p_draft, float* out_q_draft, float* out_residual_mass,
                                                 void* workspace, size_t workspace_bytes);

/* Allocation-free variant of uno_psi_spec_verify_linear, for callers that
 * cannot allocate device memory or hand over a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments (minus the workspace), same kernels, same outputs bit for bit.
 * Its scratch is a 16 MiB array of the library's own in device memory, one per
 * GPU, held until the process ends: a call whose workspace query
 * (uno_psi_spec_verify_linear_workspace) exceeds 16 MiB returns
 * UNO_ERR_UNSUPPORTED (16 MiB covers batch 4096 x 64 drafts at vocab
 * 151,936).  The call allocates nothing.  Every call on one GPU shares that
 * GPU's array: calls that overlap on a GPU (other streams, other threads)
 * race on it and must be serialised by the caller. */
uno_status uno_psi_spec_verify_linear_noalloc(hipStream_t stream, uno_dtype logit_dtype,
                                              int32_t batch, int32_t k, int32_t vocab,
                                              const void* p_logits, int64_t p_seq_stride, int64_t p_row_stride,
                                              const void* q_logits, int64_t q_seq_stride, int64_t q_row_stride,
                                              const int32_t* draft_tokens,
                                              const float* u_accept, const float* u_sample,
                                              float temperature,
                                              int32_t* out_accept_len, int32_t* out_token,
                                              float* out_p_draft, float* out_q_draft, float* out_residual_mass);

/* Linear verify under a sampling transform.  Source: 4sapi.net blog on Uno,
 * its checklist (a changed temperature or top_p changes the distribution the
 * AR model samples from); Uno summary (hyper.ai), section "方法" (the verify
 * is lossless with respect to the AR sampling distribution).  Every p and q
 * row is replaced by its transformed distribution, then the rules of
 * uno_psi_spec_verify_linear run unchanged (drafts must come from the
 * transformed q rows):
 *   top_k >= 1: keep the tokens whose logit is at least the top_k-th largest
 *     logit of the row (ties at the boundary all kept); 0 = off;
 *   0 < top_p < 1: after top-k, keep the tokens whose strictly larger logits
 *     carry less than top_p of the kept mass (whole tie groups, largest
 *     first, until the mass reaches top_p); 1 = off;
 *   greedy = 1: the row is one-hot at its first largest logit (temperature,
 *     top_k and top_p ignored).
 * Kept rows are renormalised.  out_p_draft / out_q_draft are the transformed
 * probabilities and out_residual_mass the transformed residual's mass.  The
 * kept set is found exactly per row (radix selection on the logit order with
 * integer and 2^-40 fixed-point counts); a top-p boundary whose mass above
 * lies within 2^-40 * 2^20 of top_p times the kept mass may resolve either
 * way.  Arguments and requirements as uno_psi_spec_verify_linear, plus top_k
 * >= 0, 0 < top_p <= 1, greedy in {0, 1}. */
uno_status uno_psi_spec_verify_linear_sampled_workspace(int32_t batch, int32_t k, int32_t vocab, size_t* bytes);
uno_status uno_psi_spec_verify_linear_sampled(hipStream_t stream, uno_dtype logit_dtype,
                                              int32_t batch, int32_t k, int32_t vocab,
                                              const void* p_logits, int64_t p_seq_stride, int64_t p_row_stride,
                                              const void* q_logits, int64_t q_seq_stride, int64_t q_row_stride,
                                              const int32_t* draft_tokens,
                                              const float* u_accept, const float* u_sample,
                                              float temperature, int32_t top_k, float top_p, int32_t greedy,
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

/* --------------------------------------------------------------------------
 * Psi-Spec tree verify for siblings drawn WITHOUT REPLACEMENT ("wor"), e.g. by
 * uno_psi_spec_build_tree with without_replacement = 1.  Source: Uno summary
 * (hyper.ai), section "方法", last paragraph (lossless tree verify); read as
 * recursive rejection sampling without replacement (Jeon et al. 2024):
 *   cur = root, r = p_root; the children c of cur in ascending node id, with
 *   R the tokens of the children of cur tried before c:
 *     q_c = q_d with the tokens in R set to 0, renormalised (left at 0 when no
 *       mass remains);
 *     accept iff u_accept[b][c] * q_c[t] < r[t] -> cur = c, r = p_c, repeat;
 *     reject -> r = max(0, r - q_c) / sum (unchanged, and for the node's later
 *       children too, once the sum is 0);
 *   no child accepted (or no child): y = inverse CDF of r at u_sample.
 * Arguments, layouts, outputs and the checks on the tree as for
 * uno_psi_spec_verify_tree, with max_children <= 64.  A remaining draft mass
 * below 1e-6 of the row counts as none (fp32 cannot resolve less).
 * ------------------------------------------------------------------------ */
uno_status uno_psi_spec_verify_tree_wor_workspace(int32_t batch, int32_t n_tree, int32_t max_depth,
                                                  int32_t max_children, int32_t vocab, size_t* bytes);
uno_status uno_psi_spec_verify_tree_wor(hipStream_t stream, uno_dtype logit_dtype,
                                        int32_t batch, int32_t n_tree, int32_t max_depth, int32_t max_children,
                                        int32_t vocab,
                                        const int32_t* parent, const int32_t* tokens,
                                        const void* p_logits, const void* q_logits,
                                        const float* u_accept, const float* u_sample,
                                        float temperature,
                                        int32_t* out_accept_len, int32_t* out_path, int32_t* out_token,
                                        void* workspace, size_t workspace_bytes);

/* --------------------------------------------------------------------------
 * Psi-Spec candidate tree from the per-depth draft marginals.
 * Source: Uno summary (hyper.ai), section "方法", last paragraph (the tree
 * sampler draws several candidates from the diffusion path's marginals and
 * verifies them as a prefix tree).  The pages fix neither the shape nor the
 * draw; this call builds a breadth-first tree with a budget per depth: every
 * node at depth d (the root is depth 0) has branching[d] children; node ids
 * run level by level, the children of one node consecutive.  The children of
 * a depth-d node draw their tokens from q row d (the draft marginal of depth
 * d + 1) at temperature T, child c with uniform u_draw[b][c], by the inverse
 * CDF of every other draw (smallest v with cumsum(q)_v > u * sum(q)):
 *   without_replacement = 0: siblings are independent draws (duplicates
 *     possible) -- verify with uno_psi_spec_verify_tree;
 *   without_replacement = 1: sibling j draws from q with the tokens of the
 *     earlier siblings removed and the rest renormalised; if no mass is left
 *     (every token of positive mass drawn) the token is the smallest id not
 *     drawn yet, so siblings are distinct -- verify with
 *     uno_psi_spec_verify_tree_wor.
 *
 * branching: HOST int32 [max_depth], each in [1, 64] (<= vocab without
 *   replacement); n_tree must equal 1 + sum_d prod_{i<=d} branching[i] and be
 *   at most 1024.
 * q_logits: q row d of tree b at q_logits + b * q_seq_stride + d * q_row_stride
 *   elements (bf16 or fp32), q_row_stride >= vocab, q_seq_stride >= 0 (the
 *   noisy rows of a decode step's logits can be passed in place).
 * u_draw f32 [batch][n_tree] in [0, 1) (entry 0 of each tree unused).
 * Outputs int32 [batch][n_tree]: out_parent (parent[0] = -1), out_tokens
 *   (tokens[0] = -1: the root's token is the caller's).
 * 1 <= batch <= 65535, 1 <= max_depth <= 64, 1 <= vocab <= 2^20, T > 0;
 * workspace from the query (row statistics, draw descriptors, segment
 * masses).
 * ------------------------------------------------------------------------ */
uno_status uno_psi_spec_build_tree_workspace(int32_t batch, int32_t max_depth, int32_t vocab, size_t* bytes);
uno_status uno_psi_spec_build_tree(hipStream_t stream, uno_dtype logit_dtype, int32_t batch, int32_t max_depth,
                                   const int32_t* branching, int32_t vocab, const void* q_logits,
                                   int64_t q_seq_stride, int64_t q_row_stride, const float* u_draw, int32_t n_tree,
                                   float temperature, int32_t without_replacement, int32_t* out_parent,
                                   int32_t* out_tokens, void* workspace, size_t workspace_bytes);

/* --------------------------------------------------------------------------
 * dst[c][r] = src[r][c] for a rows x cols bf16 matrix (src ld ld_src >=
 * cols, dst ld ld_dst >= rows, both 2-byte aligned, not overlapping).  For
 * callers of uno_gated_lora_backward: the frozen AR weight W [N][K] is
 * transposed once into W^T [K][N].  At most 2^31 - 1 tiles of 64 x 64.
 * ------------------------------------------------------------------------ */
uno_status uno_transpose_bf16(hipStream_t stream, int64_t rows, int64_t cols, const void* src, int64_t ld_src,
                              void* dst, int64_t ld_dst);

/* --------------------------------------------------------------------------
 * Gated-LoRA backward (the training side of the gated concatenated forward).
 * Source: Uno summary (hyper.ai), section "方法": the diffusion weights are
 * low-rank adapters on every AR weight matrix, trained by diffusion
 * distillation after the AR weights are frozen; one forward runs over the
 * concatenated clean and noisy rows with the adapter masked off on clean
 * rows.  For y = x W^T + s diag(g) (x A^T) B^T (uno_gated_lora_linear) and
 * dY = dL/dy, with U = diag(g) (x A^T) and dT = s diag(g) (dY B):
 *   dB = s dY^T U            f32 [N][r] (ld lddb)
 *   dA = dT^T x              f32 [r][K] (ld ldda)
 *   dx = dY W + dT A         bf16 [M][K] (ld lddx); dx = NULL skips it (and W)
 * W is frozen (no gradient).  bf16 operands x [M][K], W [N][K], A [r][K],
 * B [N][r], dY [M][N]; gate u8 [M] (0 = clean row, nonzero = gated row;
 * NULL = every row clean: dA = dB = 0, dx = dY W).  U and dT are rounded to
 * bf16 between the products (as the forward's adapter input is).
 * W_t (optional, bf16 [K][N], ld ldwt): the frozen weight transposed once
 * (uno_transpose_bf16).  With it (and a gate) dx, U and dT run on the
 * forward's tuned kernels (every operand with the reduction index
 * contiguous; A^T and B^T are transposed per call); without it every
 * product runs on a generic kernel that reads W as stored.  The workspace
 * query takes with_w_t accordingly.
 * Requirements: N % 32 == 0, K % 8 == 0, r % 8 == 0, every leading dimension
 * a multiple of 8 and at least its row width, every matrix and the
 * workspace 16-byte aligned; workspace from the query (U and dT).
 * ------------------------------------------------------------------------ */
uno_status uno_gated_lora_backward_workspace(int64_t M, int64_t N, int64_t K, int64_t r, int32_t with_w_t,
                                            size_t* bytes);
uno_status uno_gated_lora_backward(hipStream_t stream, int64_t M, int64_t N, int64_t K, int64_t r,
                                   const void* x, int64_t ldx, const void* W, int64_t ldw,
                                   const void* A, int64_t lda, const void* B, int64_t ldb,
                                   const uint8_t* gate, float lora_scale,
                                   const void* dy, int64_t lddy,
                                   void* dx, int64_t lddx, float* dA, int64_t ldda, float* dB, int64_t lddb,
                                   const void* W_t, int64_t ldwt,
                                   void* workspace, size_t workspace_bytes);

/* --------------------------------------------------------------------------
 * Distillation losses of row pairs (the training side of the gated forward).
 * Source: Uno summary (hyper.ai), section "方法", the paragraphs on diffusion
 * distillation: the objective alpha * L_DCD + beta * L_TV; one forward over
 * the concatenated clean and noisy rows with the adapter off on clean rows
 * (teacher logits, AR weights only) and on on noisy rows (student logits);
 * the block-level KL between the student and the teacher distribution; the
 * TV distance between the diffusion and the AR distribution, which lengthens
 * the accepted draft prefix.  Readings: student row i pairs with teacher row
 * i; the block KL is the sum of the per-row KL(student || teacher) (product
 * of per-position marginals against the teacher's per-position
 * conditionals); the TV loss is the sum of per-row TV.  Per pair, with
 * p = softmax(teacher / T) and q = softmax(student / T):
 *   out_kl = sum_v q_v (ln q_v - ln p_v),   out_tv = 1/2 sum_v |q_v - p_v|,
 *   grad (optional) = d/dz [grad_scale * (alpha KL + beta TV)] in the
 *     student logits z: grad_scale / T * q_v * (alpha (ln q_v - ln p_v - KL)
 *     + beta / 2 (sign(q_v - p_v) - sum_u sign(q_u - p_u) q_u)), sign(0) = 0.
 *
 * Row i of sequence b: teacher + b * t_seq_stride + i * t_row_stride
 * elements (likewise student and grad), bf16 or fp32 (grad in the logits'
 * dtype); strides >= vocab per row, >= 0 per sequence.  With the decode
 * step's logits [batch][2*block][vocab]: teacher = logits, student = logits +
 * block * vocab, both strides 2*block*vocab and vocab, rows = block.
 * out_kl, out_tv: f32 [batch * rows].  grad = NULL: losses only.
 * batch, rows >= 1, batch * rows < 2^31, 1 <= vocab <= 2^20, T > 0, alpha,
 * beta, grad_scale finite.  No workspace: one workgroup per pair, three
 * passes over it, fixed summation order (deterministic).
 * ------------------------------------------------------------------------ */
uno_status uno_distill_loss(hipStream_t stream, uno_dtype logit_dtype, int32_t batch, int32_t rows, int32_t vocab,
                            const void* teacher, int64_t t_seq_stride, int64_t t_row_stride,
                            const void* student, int64_t s_seq_stride, int64_t s_row_stride,
                            float temperature, float alpha, float beta, float grad_scale,
                            float* out_kl, float* out_tv,
                            void* grad, int64_t g_seq_stride, int64_t g_row_stride);

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
 * (angle formed in double precision).  positions int32 [rows], >= 0.
 * norm_weight (optional, bf16 [128], 2-byte aligned; NULL: none): every head
 * is first scaled to head / sqrt(mean(head^2) + norm_eps) * norm_weight
 * (Qwen3's per-head q/k norm), in fp32, with one bf16 rounding after the
 * rotation; norm_eps finite and >= 0.  Source: Uno summary (hyper.ai),
 * section 实验 (a Qwen3-8B base). */
uno_status uno_rope(hipStream_t stream, int64_t rows, int32_t n_heads, void* x, int64_t ldx,
                    const int32_t* positions, float theta, const void* norm_weight, float norm_eps);

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
 *   a = rmsnorm(h); q, k, v = gated_lora(a); rope(qnorm(q)), rope(knorm(k));
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
 * qnorm / knorm: Qwen3's per-head RMSNorm (rms_eps) of every 128-wide q and
 * k head with the bf16 weights q_norm / k_norm [128], before the rotation,
 * in fp32 with one bf16 rounding after it (the identity when both weights
 * are NULL).
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
  /* Optional gate-merged weights, all seven or none: w_merged[p] =
   * bf16(w[p] + lora_scale * b[p] a[p]) as uno_lora_merge writes it, with the
   * lora_scale of the call.  Used by uno_psi_spec_step, whose gate is 0 on
   * every clean row and 1 on every noisy row: there the noisy rows read
   * w_merged and the clean rows w, and no LoRA-down runs.  Ignored by
   * uno_decoder_layer (its gate is arbitrary). */
  const void* w_merged[UNO_NUM_PROJ];
  /* Optional per-head q/k RMSNorm weights, bf16 [128] each, 16-byte
   * aligned, both or neither (NULL: the layer has no per-head norm).
   * Source: Uno summary (hyper.ai), section 实验 (a Qwen3-8B base, whose
   * attention normalises every q and k head before the rotary embedding). */
  const void* q_norm;
  const void* k_norm;
} uno_layer_weights;

/* Gate-merged weights for uno_layer_weights.w_merged.  Source: Uno summary
 * (hyper.ai), section 方法 (the gated LoRA: a row with gate 1 adds the
 * low-rank update to the AR weights, a row with gate 0 keeps them); with a
 * 0/1 gate, a gated row computes x (W + s B A)^T, the LoRA merge identity.
 * out[n][k] = bf16(W[n][k] + lora_scale * sum_j B[n][j] A[j][k]), the sum
 * over j = 0..r-1 in order with fp32 fused multiply-adds and one rounding at
 * the end.  bf16 only: W [N][K] (ld ldw), A [r][K] (ld lda), B [N][r] (ld
 * ldb), out [N][K] (ld ldo), device memory, out aliasing none of the inputs.
 * 1 <= N <= 65535, K >= 1, r >= 1.  A one-time set-up call (weights load);
 * every leading dimension a multiple of 8 with 16-byte aligned W, A and out
 * takes the vector path. */
uno_status uno_lora_merge(hipStream_t stream, int64_t N, int64_t K, int64_t r, const void* W, int64_t ldw,
                          const void* A, int64_t lda, const void* B, int64_t ldb, float lora_scale, void* out,
                          int64_t ldo);

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
 * drafts) and drops the rest by not counting them.  For b < batch, with
 * len = cache_len[b] clamped to [0, capacity] and L = accept_len[b]:
 *   L >= 0 and len + L + 1 <= capacity:  cache_len[b] = len + L + 1;
 *   otherwise (the kept rows do not all fit, or L is already -1): cache_len[b]
 *   is left as it is and accept_len[b] = -1 (the sequence is flagged: its
 *   emitted tokens would no longer match its cache).
 * accept_len, cache_len: device int32 [batch], both updated in place.
 * The correction token is not in the cache: it is the next block's first
 * clean row.  batch >= 1, capacity >= 0. */
uno_status uno_kv_commit(hipStream_t stream, int32_t batch, int32_t capacity, int32_t* accept_len,
                         int32_t* cache_len);

/* One whole Psi-Spec decode step of the decode loop.  Source: Uno summary
 * (hyper.ai), section 方法 (both weight sets draft, only the AR weights
 * verify; the diffusion path keeps the next-token parametrisation and
 * predicts the next clean token from a noisy sequence; a block proposed on
 * the diffusion path is rejection-sampled against the AR distribution and
 * the longest valid prefix is kept; the first token of a block comes from
 * the AR weights; the linear sampler draws one candidate from the marginals;
 * one forward pass runs over the concatenated clean and noisy rows with the
 * adapter gated per row) and section 实验 (Qwen3-8B base, rank-128 adapters,
 * one KV cache shared by drafting and verification).
 *
 * Per sequence b the step takes 2*block token ids: `block` clean ids -- the
 * previous step's AR token y, then the k = block - 1 drafts d that step drew
 * -- and `block` noisy ids (the caller's noise/mask ids for the next block).
 * It runs
 *   h = embed[tokens]; gate = 0 on clean rows, 1 on noisy rows;
 *   positions: clean row j at ctx + j, noisy row j at ctx + block + j (the
 *     noisy rows stand for the next block; ctx = cache_len[b] or ctx_len);
 *   n_layers x uno_decoder_layer (layer l uses layers[l]);
 *   logits = rmsnorm(h, final_norm) . lm_head^T  (bf16 [rows][vocab], no adapter);
 *   out_drafts[b][i] = inverse-CDF draw from softmax(noisy row i / T) at
 *     u_draft[b][i], i < k (the uno_sample_rows rule): the next step's drafts;
 *   uno_psi_spec_verify_linear of the clean drafts d against p = the k + 1
 *     clean rows and q = prev_q, the previous step's noisy-row logits the
 *     drafts were drawn from (the caller keeps that step's logits buffer and
 *     passes its noisy rows 0..k-1 with strides; nothing is copied).  With
 *     prev_q NULL (the loop's first step) no draft is verified: L = 0 and y
 *     is drawn from clean row 0.
 *   out_next_tokens[b] (optional) = [y, out_drafts[b][0..k-1], the noisy ids
 *     of tokens[b]]: the next step's ids, assembled on the device; may be
 *     `tokens` itself.
 *
 * layers: host array of n_layers uno_layer_weights (device pointers); embed and
 * lm_head bf16 [vocab][hidden]; final_norm bf16 [hidden]; tokens int32
 * [batch][2*block]; prev_q bf16, row i of sequence b at prev_q +
 * b * prev_q_seq_stride + i * prev_q_row_stride (elements; row stride >=
 * vocab, sequence stride >= k row strides), must not alias logits; u_draft,
 * u_accept f32 [batch][k]; u_sample f32 [batch]; logits (output,
 * caller-owned) bf16 [batch*2*block][vocab]; out_drafts int32 [batch][k];
 * out_accept_len, out_token int32 [batch].  1 <= block <= 65, head_dim 128,
 * hidden and inter multiples of 8, r a multiple of 8 (0: no adapter).  A
 * token id outside [0, vocab) embeds as a zero row.
 *
 * cache_len (optional, device int32 [batch], updated in place): the decode
 * loop's form.  Sequence b's caches hold cache_len[b] valid rows (clamped to
 * [0, ctx_len]) out of a capacity of ctx_len per sequence; every layer writes
 * the clean rows' k and v into its cache after the valid rows
 * (uno_decoder_layer), and after verification the step commits the kept
 * rows as uno_kv_commit does, so the next step's cache_len[b] is the old one
 * + out_accept_len[b] + 1.  A sequence whose kept rows do not fit is
 * flagged: out_accept_len[b] = out_token[b] = -1, its length unchanged.
 * NULL: every cache holds ctx_len rows, the caches are only read and
 * positions start at ctx_len. */
typedef struct {
  int32_t batch, block, ctx_len;
  int32_t hidden, inter, n_heads, n_kv_heads, r, n_layers, vocab;
  float rms_eps, rope_theta, lora_scale, temperature;
} uno_step_config;

uno_status uno_psi_spec_step_workspace(const uno_step_config* config, size_t* bytes);
uno_status uno_psi_spec_step(hipStream_t stream, const uno_step_config* config, const uno_layer_weights* layers,
                             const void* embed, const void* final_norm, const void* lm_head,
                             const int32_t* tokens, int32_t* cache_len,
                             const void* prev_q, int64_t prev_q_seq_stride, int64_t prev_q_row_stride,
                             const float* u_draft, const float* u_accept, const float* u_sample,
                             void* logits, int32_t* out_drafts, int32_t* out_accept_len, int32_t* out_token,
                             int32_t* out_next_tokens, void* workspace, size_t workspace_bytes);

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
