// libunospec C ABI: one whole Psi-Spec decode step (token ids in, accepted
// length and correction/bonus token out).  Validation runs on the host before
// anything is enqueued; no C++ exception leaves this file.
#include <algorithm>
#include <cmath>

#include "internal.h"

using namespace uno;

namespace {

constexpr int kHeadDim = 128;

struct StepWs {
  size_t h, a, gate, pos, scratch, total;
};

size_t up256(size_t b) { return align_up(b, 256); }

// h and the final-norm output, the set-up arrays, then one scratch region
// shared by the stages that run one after another (decoder layers, LM head,
// draft draw, verify).
StepWs step_ws(const uno_step_config& c) {
  const size_t rows = size_t(c.batch) * 2 * c.block;
  const int k = c.block - 1;
  StepWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += up256(bytes);
    return at;
  };
  w.h = take(rows * c.hidden * 2);
  w.a = take(rows * c.hidden * 2);
  w.gate = take(rows);
  w.pos = take(rows * 4);
  size_t scratch = decoder_layer_workspace_bytes(c.batch, c.block, c.ctx_len, c.hidden, c.inter, c.n_heads,
                                                 c.n_kv_heads, c.r);
  scratch = std::max(scratch, gated_lora_workspace_bytes(UNO_BF16, int64_t(rows), c.vocab, c.hidden, 0));
  if (k > 0) scratch = std::max(scratch, sample_rows_workspace_bytes(c.batch * k, c.vocab));
  scratch = std::max(scratch, verify_linear_workspace_bytes(c.batch, k, c.vocab));
  w.scratch = take(scratch);
  w.total = off;
  return w;
}

uno_status check_config(const uno_step_config* c) {
  if (!c) return fail(UNO_ERR_INVALID_ARGUMENT, "config is NULL");
  if (c->batch < 1 || c->block < 1 || c->ctx_len < 0 || c->n_heads < 1 || c->n_kv_heads < 1 || c->n_layers < 0 ||
      c->vocab < 1)
    return fail(UNO_ERR_INVALID_ARGUMENT, "batch, block, n_heads, n_kv_heads, vocab >= 1; ctx_len, n_layers >= 0");
  if (c->n_heads % c->n_kv_heads != 0) return fail(UNO_ERR_INVALID_ARGUMENT, "n_heads must be a multiple of n_kv_heads");
  if (c->n_heads / c->n_kv_heads > 8) return fail(UNO_ERR_UNSUPPORTED, "at most 8 query heads per KV head");
  if (c->block - 1 > 64) return fail(UNO_ERR_UNSUPPORTED, "block above 65 (at most 64 drafts per sequence)");
  if (int64_t(c->ctx_len) + 2 * c->block > (int64_t(1) << 30)) return fail(UNO_ERR_UNSUPPORTED, "context too long");
  if (c->batch > 65535 || int64_t(c->batch) * (c->block - 1) > 65535)
    return fail(UNO_ERR_UNSUPPORTED, "batch above 65535 or more than 65535 draft rows");
  if (c->hidden < 8 || c->hidden % 8 != 0 || c->inter < 8 || c->inter % 8 != 0)
    return fail(UNO_ERR_UNSUPPORTED, "hidden and inter must be positive multiples of 8");
  if (c->hidden > rms_norm_max_dim()) return fail(UNO_ERR_UNSUPPORTED, "hidden above %d", rms_norm_max_dim());
  if (c->r < 0 || c->r % 8 != 0) return fail(UNO_ERR_UNSUPPORTED, "r must be a non-negative multiple of 8");
  if (c->vocab > (1 << 20)) return fail(UNO_ERR_UNSUPPORTED, "vocab above 2^20");
  if (int64_t(c->batch) * 2 * c->block > 0x7fffffff / 8) return fail(UNO_ERR_UNSUPPORTED, "too many rows");
  if (!(c->rms_eps >= 0.f) || !std::isfinite(c->rms_eps) || !(c->rope_theta > 1.f) || !std::isfinite(c->rope_theta) ||
      !std::isfinite(c->lora_scale) || !(c->temperature > 0.f) || !std::isfinite(c->temperature))
    return fail(UNO_ERR_INVALID_ARGUMENT, "rms_eps >= 0, rope_theta > 1, finite lora_scale and temperature > 0 required");
  return UNO_OK;
}

}  // namespace

extern "C" {

uno_status uno_psi_spec_step_workspace(const uno_step_config* config, size_t* bytes) {
  UNO_GUARD_BEGIN
  if (!bytes) return fail(UNO_ERR_INVALID_ARGUMENT, "bytes is NULL");
  uno_status s = check_config(config);
  if (s != UNO_OK) return s;
  *bytes = step_ws(*config).total;
  return UNO_OK;
  UNO_GUARD_END
}

uno_status uno_psi_spec_step(hipStream_t stream, const uno_step_config* config, const uno_layer_weights* layers,
                             const void* embed, const void* final_norm, const void* lm_head, const int32_t* tokens,
                             int32_t* cache_len, const void* prev_q, int64_t prev_q_seq_stride,
                             int64_t prev_q_row_stride, const float* u_draft, const float* u_accept,
                             const float* u_sample, void* logits, int32_t* out_drafts, int32_t* out_accept_len,
                             int32_t* out_token, int32_t* out_next_tokens, void* workspace, size_t workspace_bytes) {
  UNO_GUARD_BEGIN
  uno_status s = check_config(config);
  if (s != UNO_OK) return s;
  const uno_step_config c = *config;
  const int k = c.block - 1;
  if (!embed || !final_norm || !lm_head || !tokens || !u_sample || !logits || !out_accept_len || !out_token ||
      (c.n_layers > 0 && !layers))
    return fail(UNO_ERR_INVALID_ARGUMENT, "required pointer is NULL");
  if (k > 0 && (!u_draft || !out_drafts))
    return fail(UNO_ERR_INVALID_ARGUMENT, "u_draft and out_drafts are required when block > 1");
  // the drafts verified this step are the clean ids 1..k, drawn by the previous step from prev_q
  const int kv = (prev_q && k > 0) ? k : 0;
  if (kv > 0) {
    if (!u_accept) return fail(UNO_ERR_INVALID_ARGUMENT, "u_accept is required with prev_q");
    if (prev_q_row_stride < c.vocab || (c.batch > 1 && prev_q_seq_stride < int64_t(k) * prev_q_row_stride))
      return fail(UNO_ERR_INVALID_ARGUMENT, "prev_q strides must cover [k][vocab]");
    if (reinterpret_cast<uintptr_t>(prev_q) & 1u) return fail(UNO_ERR_UNSUPPORTED, "prev_q must be 2-byte aligned");
  }
  if (!aligned16(embed) || !aligned16(final_norm) || !aligned16(lm_head) || (reinterpret_cast<uintptr_t>(logits) & 7u))
    return fail(UNO_ERR_UNSUPPORTED, "embed, final_norm, lm_head 16-byte and logits 8-byte aligned required");
  for (int l = 0; l < c.n_layers; ++l) {
    const uno_layer_weights& w = layers[l];
    if (!w.attn_norm || !w.mlp_norm || !aligned16(w.attn_norm) || !aligned16(w.mlp_norm))
      return fail(UNO_ERR_INVALID_ARGUMENT, "layer %d: norm weights NULL or unaligned", l);
    for (int p = 0; p < UNO_NUM_PROJ; ++p) {
      if (!w.w[p] || !aligned16(w.w[p])) return fail(UNO_ERR_INVALID_ARGUMENT, "layer %d: w[%d] NULL or unaligned", l, p);
      if (c.r > 0 && (!w.a[p] || !w.b[p] || !aligned16(w.a[p]) || !aligned16(w.b[p])))
        return fail(UNO_ERR_INVALID_ARGUMENT, "layer %d: a[%d] / b[%d] NULL or unaligned", l, p, p);
    }
    if (c.ctx_len > 0 && (!w.k_cache || !w.v_cache || !aligned16(w.k_cache) || !aligned16(w.v_cache)))
      return fail(UNO_ERR_INVALID_ARGUMENT, "layer %d: KV cache NULL or unaligned", l);
    if (!w.q_norm != !w.k_norm) return fail(UNO_ERR_INVALID_ARGUMENT, "layer %d: q_norm and k_norm: both or neither", l);
    if ((w.q_norm && !aligned16(w.q_norm)) || (w.k_norm && !aligned16(w.k_norm)))
      return fail(UNO_ERR_UNSUPPORTED, "layer %d: q_norm / k_norm must be 16-byte aligned", l);
  }
  const StepWs W = step_ws(c);
  if (workspace_bytes < W.total || !workspace)
    return fail(UNO_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, W.total);

  if (debug_checks()) {   // ids of every row and the uniforms the step uses
    uno_status d = debug_check_ids(stream, tokens, c.batch, 2 * c.block, 2 * c.block, 0, 0, c.vocab, "tokens");
    if (d == UNO_OK && k > 0) d = debug_check_unit(stream, u_draft, int64_t(c.batch) * k, "u_draft");
    if (d == UNO_OK && kv > 0) d = debug_check_unit(stream, u_accept, int64_t(c.batch) * kv, "u_accept");
    if (d == UNO_OK) d = debug_check_unit(stream, u_sample, c.batch, "u_sample");
    if (d != UNO_OK) return d;
  }
  char* ws = static_cast<char*>(workspace);
  const int64_t rows = int64_t(c.batch) * 2 * c.block;
  void* h = ws + W.h;
  void* a = ws + W.a;
  uint8_t* gate = reinterpret_cast<uint8_t*>(ws + W.gate);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + W.pos);
  void* scratch = ws + W.scratch;
  const size_t scratch_bytes = workspace_bytes - W.scratch;
  const float scale_log2 = float(1.4426950408889634 / double(c.temperature));

  // token embeddings, gates (clean 0 / noisy 1) and positions
  StepSetupArgs sa{};
  sa.rows = rows;
  sa.block = c.block;
  sa.ctx = c.ctx_len;
  sa.cache_len = cache_len;
  sa.cap = c.ctx_len;
  sa.hidden = c.hidden;
  sa.vocab = c.vocab;
  sa.tokens = tokens;
  sa.embed = embed;
  sa.h = h;
  sa.gate = gate;
  sa.positions = pos;
  hipError_t e = launch_step_setup(sa, stream);

  // the decoder stack over the concatenated clean + noisy rows
  for (int l = 0; l < c.n_layers && e == hipSuccess; ++l) {
    DecoderLayerArgs la{};
    la.batch = c.batch;
    la.block = c.block;
    la.ctx = c.ctx_len;
    la.hidden = c.hidden;
    la.inter = c.inter;
    la.n_heads = c.n_heads;
    la.n_kv = c.n_kv_heads;
    la.r = c.r;
    la.w = &layers[l];
    la.gate = c.r > 0 ? gate : nullptr;
    la.gate_block = c.block;   // the gates step_setup writes: 0 on each sequence's clean rows, 1 on its noisy rows
    // each layer's closing residual add also normalises for what follows: the
    // next layer's attention norm, or the final norm before the LM head
    la.norm_ready = l > 0;
    la.next_norm = l + 1 < c.n_layers ? layers[l + 1].attn_norm : final_norm;
    la.next_out = l + 1 < c.n_layers ? nullptr : a;
    la.positions = pos;
    la.cache_len = cache_len;
    la.rms_eps = c.rms_eps;
    la.rope_theta = c.rope_theta;
    la.lora_scale = c.lora_scale;
    la.h = h;
    la.ws = scratch;
    la.ws_bytes = scratch_bytes;
    e = launch_decoder_layer(la, stream);
  }

  // final norm (done by the last layer's closing pass when there are layers)
  // and LM head (no adapter): logits [rows][vocab]
  if (e == hipSuccess && c.n_layers == 0) {
    RmsNormArgs na{};
    na.rows = rows;
    na.dim = c.hidden;
    na.x = h;
    na.ldx = c.hidden;
    na.weight = final_norm;
    na.eps = c.rms_eps;
    na.out = a;
    na.ldo = c.hidden;
    e = launch_rms_norm(na, stream);
  }
  if (e == hipSuccess) {
    GatedLoraArgs ga{};
    ga.dtype = UNO_BF16;
    ga.M = rows;
    ga.N = c.vocab;
    ga.K = c.hidden;
    ga.r = 0;
    ga.x = a;
    ga.ldx = c.hidden;
    ga.w = lm_head;
    ga.ldw = c.hidden;
    ga.y = logits;
    ga.ldy = c.vocab;
    ga.ws = scratch;
    ga.ws_bytes = scratch_bytes;
    e = launch_gated_lora(ga, stream);
  }

  // drafts: one inverse-CDF draw from each of the first k noisy rows' q
  const int64_t seq_stride = 2 * int64_t(c.block) * c.vocab;
  const uint16_t* lg = static_cast<const uint16_t*>(logits);
  if (e == hipSuccess && k > 0) {
    SampleRowsArgs ra{};
    ra.dtype = UNO_BF16;
    ra.rows = c.batch * k;
    ra.vocab = c.vocab;
    ra.logits = lg + int64_t(c.block) * c.vocab;
    ra.row_stride = c.vocab;
    ra.per_seq = k;
    ra.seq_stride = seq_stride;
    ra.u = u_draft;
    ra.scale_log2 = scale_log2;
    ra.out_tok = out_drafts;
    ra.ws = scratch;
    e = launch_sample_rows(ra, stream);
  }

  // verify the clean drafts: p from the kv + 1 clean rows, q from the previous
  // step's noisy rows (prev_q); without prev_q no draft is verified (L = 0, y
  // drawn from clean row 0)
  if (e == hipSuccess) {
    VerifyLinearArgs va{};
    va.dtype = UNO_BF16;
    va.batch = c.batch;
    va.k = kv;
    va.vocab = c.vocab;
    va.p = lg;
    va.p_seq = seq_stride;
    va.p_row = c.vocab;
    va.q = prev_q;
    va.q_seq = prev_q_seq_stride;
    va.q_row = prev_q_row_stride;
    va.drafts = tokens + 1;
    va.drafts_seq = 2 * int64_t(c.block);
    va.u_acc = u_accept;
    va.u_s = u_sample;
    va.scale_log2 = scale_log2;
    va.out_len = out_accept_len;
    va.out_tok = out_token;
    va.ws = scratch;
    e = launch_verify_linear(va, stream);
  }
  // commit (the block's AR token and its accepted drafts, appended by every
  // layer during the forward pass, join each sequence's valid cache prefix;
  // a sequence whose kept rows do not fit is flagged) and the next step's ids
  if (e == hipSuccess && (cache_len || out_next_tokens)) {
    StepFinishArgs fa{};
    fa.batch = c.batch;
    fa.block = c.block;
    fa.cap = c.ctx_len;
    fa.accept_len = out_accept_len;
    fa.token = out_token;
    fa.cache_len = cache_len;
    fa.drafts = out_drafts;
    fa.tokens = tokens;
    fa.next = out_next_tokens;
    e = launch_step_finish(fa, stream);
  }
  return check_hip(e, "uno_psi_spec_step launch");
  UNO_GUARD_END
}

}  // extern "C"
