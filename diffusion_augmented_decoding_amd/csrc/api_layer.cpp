// libunospec C ABI, composed decode step: layer operations, block attention,
// the row sampler and one decoder layer.  Validation runs on the host before
// anything is enqueued; no C++ exception leaves this file.
#include <algorithm>
#include <cmath>

#include "internal.h"

using namespace uno;

namespace {

constexpr int kHeadDim = 128;

bool ld_ok(int64_t ld, int64_t width) { return ld >= width && ld % 8 == 0; }

uno_status check_block_attn(int32_t batch, int32_t block, int32_t ctx, int32_t nh, int32_t nkv, int32_t hd) {
  if (batch < 1 || block < 1 || ctx < 0 || nh < 1 || nkv < 1)
    return fail(UNO_ERR_INVALID_ARGUMENT, "sizes must be batch,block,n_heads,n_kv_heads >= 1 and ctx_len >= 0");
  if (hd != kHeadDim) return fail(UNO_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", hd);
  if (nh % nkv != 0) return fail(UNO_ERR_INVALID_ARGUMENT, "n_heads must be a multiple of n_kv_heads");
  if (nh / nkv > 8) return fail(UNO_ERR_UNSUPPORTED, "at most 8 query heads per KV head");
  if (block > 128) return fail(UNO_ERR_UNSUPPORTED, "block above 128 (got %d)", block);
  if (int64_t(ctx) + 2 * block > (int64_t(1) << 30)) return fail(UNO_ERR_UNSUPPORTED, "context too long");
  if (batch > 65535 || nkv > 65535) return fail(UNO_ERR_UNSUPPORTED, "grid too large");
  return UNO_OK;
}

}  // namespace

namespace uno {

// Workspace layout of one decoder layer.
struct LayerWs {
  size_t a, q, k, v, att, o, g, u, lora, attn, tqkv, tgu, lpart, total;
};

static size_t up256(size_t b) { return align_up(b, 256); }

static LayerWs layer_ws(int batch, int block, int ctx, int hidden, int inter, int nh, int nkv, int r) {
  const size_t rows = size_t(batch) * 2 * block;
  const int qd = nh * kHeadDim, kvd = nkv * kHeadDim;
  LayerWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += up256(bytes);
    return at;
  };
  w.a = take(rows * hidden * 2);
  w.q = take(rows * qd * 2);
  w.k = take(rows * kvd * 2);
  w.v = take(rows * kvd * 2);
  w.att = take(rows * qd * 2);
  w.o = take(rows * hidden * 2);
  w.g = take(rows * size_t(inter) * 2);
  w.u = take(rows * size_t(inter) * 2);
  const int64_t M = int64_t(rows);
  const int64_t shapes[UNO_NUM_PROJ][2] = {{qd, hidden}, {kvd, hidden}, {kvd, hidden}, {hidden, qd},
                                           {inter, hidden}, {inter, hidden}, {hidden, inter}};
  size_t lora = 0;
  for (const auto& s : shapes) lora = std::max(lora, gated_lora_workspace_bytes(UNO_BF16, M, s[0], s[1], r));
  w.lora = take(lora);
  w.attn = take(block_attention_workspace_bytes(batch, block, ctx, nh, nkv));
  // grouped LoRA-down (adapters of q/k/v, and of gate/up, stored back to back)
  w.tqkv = take(rows * 3 * size_t(r) * 2);
  w.tgu = take(rows * 2 * size_t(r) * 2);
  w.lpart = take(r > 0 ? std::max(lora_down_part_bytes(M, 3 * r, hidden), lora_down_part_bytes(M, 2 * r, hidden)) : 0);
  w.total = off;
  return w;
}

size_t decoder_layer_workspace_bytes(int batch, int block, int ctx, int hidden, int inter, int nh, int nkv, int r) {
  return layer_ws(batch, block, ctx, hidden, inter, nh, nkv, r).total;
}

// One pre-norm decoder layer on the residual stream d.h, in place:
//   a = rmsnorm(h); q, k, v = gated_lora(a); rope(q), rope(k);
//   att = block_attention(q, cache + (k, v)); h += gated_lora(att, o);
//   a = rmsnorm(h); h += gated_lora(silu(gated_lora(a, gate)) * gated_lora(a, up), down)
hipError_t launch_decoder_layer(const DecoderLayerArgs& d, hipStream_t stream) {
  const LayerWs L = layer_ws(d.batch, d.block, d.ctx, d.hidden, d.inter, d.n_heads, d.n_kv, d.r);
  char* ws = static_cast<char*>(d.ws);
  const int64_t rows = int64_t(d.batch) * 2 * d.block;
  const int qd = d.n_heads * kHeadDim, kvd = d.n_kv * kHeadDim;
  void* a = ws + L.a;
  void* q = ws + L.q;
  void* k = ws + L.k;
  void* v = ws + L.v;
  void* att = ws + L.att;
  void* o = ws + L.o;
  void* g = ws + L.g;
  void* u = ws + L.u;
  void* h = d.h;
  // gate-merged weights (all seven projections) under the structured gate:
  // the gated rows read w + s b a and no LoRA-down runs
  bool merged = d.gate && d.r > 0 && d.gate_block > 0;
  for (int p = 0; p < UNO_NUM_PROJ && merged; ++p) merged = d.w->w_merged[p] != nullptr;

  auto proj_args = [&](int p, const void* x, int64_t K, int64_t N, void* y, const uint16_t* t_pre = nullptr,
                       int64_t ldt_pre = 0) {
    GatedLoraArgs ga{};
    ga.dtype = UNO_BF16;
    ga.M = rows;
    ga.N = N;
    ga.K = K;
    ga.r = (d.gate && d.r > 0) ? d.r : 0;
    ga.x = x;
    ga.ldx = K;
    ga.w = d.w->w[p];
    ga.ldw = K;
    ga.a = d.w->a[p];
    ga.lda = K;
    ga.b = d.w->b[p];
    ga.ldb = d.r;
    ga.gate = d.gate;
    ga.lora_scale = d.lora_scale;
    ga.y = y;
    ga.ldy = N;
    ga.t_pre = t_pre;
    ga.ldt_pre = ldt_pre;
    ga.gate_block = d.gate_block;
    ga.w_merged = merged ? d.w->w_merged[p] : nullptr;
    ga.ws = ws + L.lora;
    ga.ws_bytes = d.ws_bytes - L.lora;
    return ga;
  };
  auto proj = [&](int p, const void* x, int64_t K, int64_t N, void* y, const uint16_t* t_pre = nullptr,
                  int64_t ldt_pre = 0) {
    return launch_gated_lora(proj_args(p, x, K, N, y, t_pre, ldt_pre), stream);
  };
  auto norm = [&](const void* res, const void* weight, void* out) {
    RmsNormArgs na{};
    na.rows = rows;
    na.dim = d.hidden;
    na.x = h;
    na.ldx = d.hidden;
    na.res = res;
    na.ldr = d.hidden;
    na.sum_out = res ? h : nullptr;
    na.lds = d.hidden;
    na.weight = weight;
    na.eps = d.rms_eps;
    na.out = out;
    na.ldo = d.hidden;
    return launch_rms_norm(na, stream);
  };
  auto rope_qk = [&]() {
    RopeArgs ra{};
    ra.rows = rows;
    ra.n_heads = d.n_heads;
    ra.x = q;
    ra.ldx = int64_t(d.n_heads) * kHeadDim;
    ra.positions = d.positions;
    ra.theta = d.rope_theta;
    ra.n_heads2 = d.n_kv;
    ra.x2 = k;
    ra.ldx2 = int64_t(d.n_kv) * kHeadDim;
    ra.norm_w = d.w->q_norm;    // per-head q/k norm (both or neither)
    ra.norm_w2 = d.w->k_norm;
    ra.norm_eps = d.rms_eps;
    if (d.cache_len) {   // the clean rows' keys (rotated) and values join the cache's free slots
      ra.cache_len = d.cache_len;
      ra.block = d.block;
      ra.cap = d.ctx;
      ra.k_cache = const_cast<void*>(d.w->k_cache);
      ra.v_cache = const_cast<void*>(d.w->v_cache);
      ra.v = v;
      ra.ldv = int64_t(d.n_kv) * kHeadDim;
    }
    return launch_rope(ra, stream);
  };

  // Adapters stored back to back (q, k, v; gate, up) share one LoRA-down
  // launch over the common input; each projection then reads its slice of T.
  const bool lora = d.gate && d.r > 0;
  const int64_t rK = int64_t(d.r) * d.hidden;
  auto packed = [&](int p0, int n) {
    if (!lora) return false;
    const uint16_t* base = static_cast<const uint16_t*>(d.w->a[p0]);
    for (int i = 1; i < n; ++i)
      if (static_cast<const uint16_t*>(d.w->a[p0 + i]) != base + i * rK) return false;
    return true;
  };
  auto group_down = [&](int p0, int n, const void* x, uint16_t* t) {
    LoraDownArgs ld{};
    ld.M = rows;
    ld.K = d.hidden;
    ld.n = int64_t(n) * d.r;
    ld.x = x;
    ld.ldx = d.hidden;
    ld.a = d.w->a[p0];
    ld.lda = d.hidden;
    ld.gate = d.gate;
    ld.lora_scale = d.lora_scale;
    ld.t = t;
    ld.part = ws + L.lpart;
    ld.gather_blk = d.gate_block;
    return launch_lora_down(ld, stream);
  };
  uint16_t* tqkv = reinterpret_cast<uint16_t*>(ws + L.tqkv);
  uint16_t* tgu = reinterpret_cast<uint16_t*>(ws + L.tgu);
  const bool qkv_grouped = !merged && packed(UNO_PROJ_Q, 3);
  const bool gu_grouped = !merged && packed(UNO_PROJ_GATE, 2);
  const int64_t r3 = 3 * int64_t(d.r), r2 = 2 * int64_t(d.r);

  hipError_t e = d.norm_ready ? hipSuccess : norm(nullptr, d.w->attn_norm, a);
  if (e == hipSuccess && qkv_grouped) e = group_down(UNO_PROJ_Q, 3, a, tqkv);
  if (e == hipSuccess) e = proj(UNO_PROJ_Q, a, d.hidden, qd, q, qkv_grouped ? tqkv : nullptr, r3);
  if (e == hipSuccess) {
    // k and v: one launch over both outputs where the shapes allow
    const GatedLoraArgs ak = proj_args(UNO_PROJ_K, a, d.hidden, kvd, k, qkv_grouped ? tqkv + d.r : nullptr, r3);
    const GatedLoraArgs av = proj_args(UNO_PROJ_V, a, d.hidden, kvd, v, qkv_grouped ? tqkv + 2 * d.r : nullptr, r3);
    if (gated_lora_pair_ok(ak, av)) {
      e = launch_gated_lora_pair(ak, av, stream);
    } else {
      e = launch_gated_lora(ak, stream);
      if (e == hipSuccess) e = launch_gated_lora(av, stream);
    }
  }
  if (e == hipSuccess) e = rope_qk();
  if (e == hipSuccess) {
    TreeAttnArgs ta{};
    ta.batch = d.batch;
    ta.n_tree = 2 * d.block;
    ta.block = d.block;
    ta.ctx = d.ctx;
    ta.ctx_lens = d.cache_len;
    ta.n_heads = d.n_heads;
    ta.n_kv = d.n_kv;
    ta.head_dim = kHeadDim;
    ta.q = q;
    ta.k_cache = d.w->k_cache;
    ta.v_cache = d.w->v_cache;
    ta.k_tree = k;
    ta.v_tree = v;
    ta.scale = 1.f / std::sqrt(float(kHeadDim));
    ta.out = att;
    ta.out_lse = nullptr;
    ta.ws = ws + L.attn;
    ta.ws_bytes = d.ws_bytes - L.attn;
    e = launch_block_attention(ta, stream);
  }
  if (e == hipSuccess) e = proj(UNO_PROJ_O, att, qd, d.hidden, o);
  if (e == hipSuccess) e = norm(o, d.w->mlp_norm, a);                 // h += o; a = rmsnorm(h)
  if (e == hipSuccess && gu_grouped) e = group_down(UNO_PROJ_GATE, 2, a, tgu);
  // gate, up and SwiGLU in one GEMM when T of both adapters sits side by side
  // (or there is no adapter); else two projections and the SwiGLU kernel
  SwigluArgs sw{};
  sw.M = rows;
  sw.N = d.inter;
  sw.K = d.hidden;
  sw.r = lora ? d.r : 0;
  sw.x = a;
  sw.ldx = d.hidden;
  sw.wg = d.w->w[UNO_PROJ_GATE];
  sw.wu = d.w->w[UNO_PROJ_UP];
  sw.ldw = d.hidden;
  sw.bg = d.w->b[UNO_PROJ_GATE];
  sw.bu = d.w->b[UNO_PROJ_UP];
  sw.ldb = d.r;
  sw.t = tgu;
  sw.ldt = r2;
  sw.y = g;
  sw.ldy = d.inter;
  if (merged) {
    sw.wg_merged = d.w->w_merged[UNO_PROJ_GATE];
    sw.wu_merged = d.w->w_merged[UNO_PROJ_UP];
    sw.gate_block = d.gate_block;
  }
  const bool fused = (!lora || gu_grouped || merged) && swiglu_fused_ok(sw);
  if (e == hipSuccess && fused) e = launch_gated_lora_swiglu(sw, stream);
  if (e == hipSuccess && !fused) e = proj(UNO_PROJ_GATE, a, d.hidden, d.inter, g, gu_grouped ? tgu : nullptr, r2);
  if (e == hipSuccess && !fused) e = proj(UNO_PROJ_UP, a, d.hidden, d.inter, u, gu_grouped ? tgu + d.r : nullptr, r2);
  if (e == hipSuccess && !fused) {
    SiluMulArgs sa{};
    sa.rows = rows;
    sa.dim = d.inter;
    sa.g = g;
    sa.ldg = d.inter;
    sa.u = u;
    sa.ldu = d.inter;
    sa.out = g;
    sa.ldo = d.inter;
    e = launch_silu_mul(sa, stream);
  }
  if (e == hipSuccess) e = proj(UNO_PROJ_DOWN, g, d.inter, d.hidden, o);
  // h += down; with a next norm in the chain, the same pass writes its output
  // (the gate/up GEMM has consumed `a` by now, so it may be overwritten)
  if (e == hipSuccess) e = norm(o, d.next_norm ? d.next_norm : d.w->attn_norm,
                                d.next_norm ? (d.next_out ? d.next_out : a) : nullptr);
  return e;
}

}  // namespace uno

extern "C" {

// ------------------------------------------------------------------ rms norm
uno_status uno_rms_norm(hipStream_t stream, int64_t rows, int32_t dim, const void* x, int64_t ldx, const void* res,
                        int64_t ldr, void* sum_out, int64_t ld_sum, const void* weight, float eps, void* out,
                        int64_t ldo) {
  UNO_GUARD_BEGIN
  if (rows < 1 || rows > 0x7fffffff) return fail(UNO_ERR_INVALID_ARGUMENT, "rows must be in [1, 2^31)");
  if (dim < 8 || dim % 8 != 0) return fail(UNO_ERR_UNSUPPORTED, "dim must be a positive multiple of 8");
  if (dim > rms_norm_max_dim()) return fail(UNO_ERR_UNSUPPORTED, "dim above %d", rms_norm_max_dim());
  if (!x || !weight) return fail(UNO_ERR_INVALID_ARGUMENT, "x and weight are required");
  if (!res && !out) return fail(UNO_ERR_INVALID_ARGUMENT, "nothing to compute (res and out both NULL)");
  if (res && !sum_out) return fail(UNO_ERR_INVALID_ARGUMENT, "sum_out is required with res");
  if (!ld_ok(ldx, dim) || (res && (!ld_ok(ldr, dim) || !ld_ok(ld_sum, dim))) || (out && !ld_ok(ldo, dim)))
    return fail(UNO_ERR_UNSUPPORTED, "leading dimensions must be >= dim and multiples of 8");
  if (!aligned16(x) || !aligned16(weight) || (res && (!aligned16(res) || !aligned16(sum_out))) ||
      (out && !aligned16(out)))
    return fail(UNO_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(UNO_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  RmsNormArgs a{};
  a.rows = rows;
  a.dim = dim;
  a.x = x;
  a.ldx = ldx;
  a.res = res;
  a.ldr = ldr;
  a.sum_out = sum_out;
  a.lds = ld_sum;
  a.weight = weight;
  a.eps = eps;
  a.out = out;
  a.ldo = ldo;
  return check_hip(launch_rms_norm(a, stream), "uno_rms_norm launch");
  UNO_GUARD_END
}

// ------------------------------------------------------------------ rope
uno_status uno_rope(hipStream_t stream, int64_t rows, int32_t n_heads, void* x, int64_t ldx,
                    const int32_t* positions, float theta, const void* norm_weight, float norm_eps) {
  UNO_GUARD_BEGIN
  if (rows < 1 || n_heads < 1) return fail(UNO_ERR_INVALID_ARGUMENT, "rows and n_heads must be >= 1");
  if (rows > 0x7fffffff) return fail(UNO_ERR_UNSUPPORTED, "rows above 2^31 - 1");
  if (!x || !positions) return fail(UNO_ERR_INVALID_ARGUMENT, "x and positions are required");
  if (ldx < int64_t(n_heads) * kHeadDim) return fail(UNO_ERR_INVALID_ARGUMENT, "ldx below n_heads * 128");
  if (!(theta > 1.f) || !std::isfinite(theta)) return fail(UNO_ERR_INVALID_ARGUMENT, "theta must be finite and > 1");
  if (norm_weight && (!(norm_eps >= 0.f) || !std::isfinite(norm_eps)))
    return fail(UNO_ERR_INVALID_ARGUMENT, "norm_eps must be finite and >= 0");
  if (reinterpret_cast<uintptr_t>(norm_weight) & 1u) return fail(UNO_ERR_UNSUPPORTED, "norm_weight must be 2-byte aligned");
  RopeArgs a{};
  a.rows = rows;
  a.n_heads = n_heads;
  a.x = x;
  a.ldx = ldx;
  a.positions = positions;
  a.theta = theta;
  a.norm_w = norm_weight;
  a.norm_eps = norm_eps;
  return check_hip(launch_rope(a, stream), "uno_rope launch");
  UNO_GUARD_END
}

// ------------------------------------------------------------------ silu * mul
uno_status uno_silu_mul(hipStream_t stream, int64_t rows, int32_t dim, const void* g, int64_t ldg, const void* u,
                        int64_t ldu, void* out, int64_t ldo) {
  UNO_GUARD_BEGIN
  if (rows < 1 || dim < 8 || dim % 8 != 0)
    return fail(UNO_ERR_INVALID_ARGUMENT, "rows >= 1 and dim a positive multiple of 8 required");
  if (rows * (dim / 8) / 256 >= 0x7fffffff) return fail(UNO_ERR_UNSUPPORTED, "too many elements");
  if (!g || !u || !out) return fail(UNO_ERR_INVALID_ARGUMENT, "g, u and out are required");
  if (!ld_ok(ldg, dim) || !ld_ok(ldu, dim) || !ld_ok(ldo, dim))
    return fail(UNO_ERR_UNSUPPORTED, "leading dimensions must be >= dim and multiples of 8");
  if (!aligned16(g) || !aligned16(u) || !aligned16(out))
    return fail(UNO_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
  SiluMulArgs a{};
  a.rows = rows;
  a.dim = dim;
  a.g = g;
  a.ldg = ldg;
  a.u = u;
  a.ldu = ldu;
  a.out = out;
  a.ldo = ldo;
  return check_hip(launch_silu_mul(a, stream), "uno_silu_mul launch");
  UNO_GUARD_END
}

// ------------------------------------------------------------------ block attention
uno_status uno_block_verify_attention_workspace(int32_t batch, int32_t block, int32_t ctx_len, int32_t n_heads,
                                                int32_t n_kv_heads, int32_t head_dim, size_t* bytes) {
  UNO_GUARD_BEGIN
  if (!bytes) return fail(UNO_ERR_INVALID_ARGUMENT, "bytes is NULL");
  uno_status s = check_block_attn(batch, block, ctx_len, n_heads, n_kv_heads, head_dim);
  if (s != UNO_OK) return s;
  *bytes = block_attention_workspace_bytes(batch, block, ctx_len, n_heads, n_kv_heads);
  return UNO_OK;
  UNO_GUARD_END
}

uno_status uno_block_verify_attention(hipStream_t stream, int32_t batch, int32_t block, int32_t ctx_len,
                                      int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, const void* q,
                                      const void* k_cache, const void* v_cache, const int32_t* cache_len,
                                      const void* k_block, const void* v_block, float softmax_scale, void* out,
                                      float* out_lse, void* workspace, size_t workspace_bytes) {
  UNO_GUARD_BEGIN
  uno_status s = check_block_attn(batch, block, ctx_len, n_heads, n_kv_heads, head_dim);
  if (s != UNO_OK) return s;
  if (!q || !k_block || !v_block || !out || (ctx_len > 0 && (!k_cache || !v_cache)))
    return fail(UNO_ERR_INVALID_ARGUMENT, "required pointer is NULL");
  if (!aligned16(q) || !aligned16(k_block) || !aligned16(v_block) || !aligned16(out) ||
      (ctx_len > 0 && (!aligned16(k_cache) || !aligned16(v_cache))))
    return fail(UNO_ERR_UNSUPPORTED, "bf16 tensors must be 16-byte aligned");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(UNO_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
  const size_t need = block_attention_workspace_bytes(batch, block, ctx_len, n_heads, n_kv_heads);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(UNO_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  TreeAttnArgs a{};
  a.batch = batch;
  a.n_tree = 2 * block;
  a.block = block;
  a.ctx = ctx_len;
  a.ctx_lens = cache_len;
  a.n_heads = n_heads;
  a.n_kv = n_kv_heads;
  a.head_dim = head_dim;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_tree = k_block;
  a.v_tree = v_block;
  a.parent = nullptr;
  a.scale = softmax_scale;
  a.out = out;
  a.out_lse = out_lse;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  return check_hip(launch_block_attention(a, stream), "uno_block_verify_attention launch");
  UNO_GUARD_END
}

// ------------------------------------------------------------------ row sampler
uno_status uno_sample_rows_workspace(int32_t rows, int32_t vocab, size_t* bytes) {
  UNO_GUARD_BEGIN
  if (!bytes) return fail(UNO_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (rows < 1 || vocab < 1) return fail(UNO_ERR_INVALID_ARGUMENT, "rows and vocab must be >= 1");
  if (vocab > (1 << 20)) return fail(UNO_ERR_UNSUPPORTED, "vocab above 2^20");
  *bytes = sample_rows_workspace_bytes(rows, vocab);
  return UNO_OK;
  UNO_GUARD_END
}

uno_status uno_sample_rows(hipStream_t stream, uno_dtype logit_dtype, int32_t rows, int32_t vocab,
                           const void* logits, int64_t row_stride, const float* u, float temperature,
                           int32_t* out_token, void* workspace, size_t workspace_bytes) {
  UNO_GUARD_BEGIN
  if (logit_dtype != UNO_F32 && logit_dtype != UNO_BF16) return fail(UNO_ERR_INVALID_ARGUMENT, "bad dtype");
  if (rows < 1 || vocab < 1) return fail(UNO_ERR_INVALID_ARGUMENT, "rows and vocab must be >= 1");
  if (vocab > (1 << 20)) return fail(UNO_ERR_UNSUPPORTED, "vocab above 2^20");
  if (rows > 65535) return fail(UNO_ERR_UNSUPPORTED, "rows above 65535");
  if (!logits || !u || !out_token) return fail(UNO_ERR_INVALID_ARGUMENT, "required pointer is NULL");
  if (row_stride < vocab) return fail(UNO_ERR_INVALID_ARGUMENT, "row_stride below vocab");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(UNO_ERR_INVALID_ARGUMENT, "temperature must be finite and > 0");
  const size_t need = sample_rows_workspace_bytes(rows, vocab);
  if (workspace_bytes < need || !workspace)
    return fail(UNO_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  SampleRowsArgs a{};
  a.dtype = logit_dtype;
  a.rows = rows;
  a.vocab = vocab;
  a.logits = logits;
  a.row_stride = row_stride;
  a.per_seq = rows;
  a.seq_stride = 0;
  a.u = u;
  a.scale_log2 = 1.4426950408889634f / temperature;
  a.out_tok = out_token;
  a.ws = workspace;
  if (debug_checks()) {
    const uno_status d = debug_check_unit(stream, u, rows, "u");
    if (d != UNO_OK) return d;
  }
  return check_hip(launch_sample_rows(a, stream), "uno_sample_rows launch");
  UNO_GUARD_END
}

// ------------------------------------------------------------------ decoder layer
static uno_status check_layer(int32_t batch, int32_t block, int32_t ctx, int32_t hidden, int32_t inter,
                              int32_t nh, int32_t nkv, int32_t r) {
  uno_status s = check_block_attn(batch, block, ctx, nh, nkv, kHeadDim);
  if (s != UNO_OK) return s;
  if (hidden < 8 || hidden % 8 != 0 || inter < 8 || inter % 8 != 0)
    return fail(UNO_ERR_UNSUPPORTED, "hidden and inter must be positive multiples of 8");
  if (hidden > rms_norm_max_dim()) return fail(UNO_ERR_UNSUPPORTED, "hidden above %d", rms_norm_max_dim());
  if (r < 0 || r % 8 != 0) return fail(UNO_ERR_UNSUPPORTED, "r must be a non-negative multiple of 8");
  if (int64_t(batch) * 2 * block > 0x7fffffff / 8) return fail(UNO_ERR_UNSUPPORTED, "too many rows");
  return UNO_OK;
}

uno_status uno_decoder_layer_workspace(int32_t batch, int32_t block, int32_t ctx_len, int32_t hidden, int32_t inter,
                                       int32_t n_heads, int32_t n_kv_heads, int32_t r, size_t* bytes) {
  UNO_GUARD_BEGIN
  if (!bytes) return fail(UNO_ERR_INVALID_ARGUMENT, "bytes is NULL");
  uno_status s = check_layer(batch, block, ctx_len, hidden, inter, n_heads, n_kv_heads, r);
  if (s != UNO_OK) return s;
  *bytes = decoder_layer_workspace_bytes(batch, block, ctx_len, hidden, inter, n_heads, n_kv_heads, r);
  return UNO_OK;
  UNO_GUARD_END
}

uno_status uno_decoder_layer(hipStream_t stream, int32_t batch, int32_t block, int32_t ctx_len, int32_t hidden,
                             int32_t inter, int32_t n_heads, int32_t n_kv_heads, int32_t r,
                             const uno_layer_weights* wt, const uint8_t* gate, const int32_t* positions,
                             const int32_t* cache_len, float rms_eps, float rope_theta, float lora_scale,
                             void* hidden_state, void* workspace, size_t workspace_bytes) {
  UNO_GUARD_BEGIN
  uno_status s = check_layer(batch, block, ctx_len, hidden, inter, n_heads, n_kv_heads, r);
  if (s != UNO_OK) return s;
  if (!wt || !hidden_state || !positions || !wt->attn_norm || !wt->mlp_norm)
    return fail(UNO_ERR_INVALID_ARGUMENT, "required pointer is NULL");
  for (int p = 0; p < UNO_NUM_PROJ; ++p) {
    if (!wt->w[p] || !aligned16(wt->w[p])) return fail(UNO_ERR_INVALID_ARGUMENT, "w[%d] NULL or unaligned", p);
    if (r > 0 && gate && (!wt->a[p] || !wt->b[p] || !aligned16(wt->a[p]) || !aligned16(wt->b[p])))
      return fail(UNO_ERR_INVALID_ARGUMENT, "a[%d] / b[%d] NULL or unaligned", p, p);
  }
  if (ctx_len > 0 && (!wt->k_cache || !wt->v_cache || !aligned16(wt->k_cache) || !aligned16(wt->v_cache)))
    return fail(UNO_ERR_INVALID_ARGUMENT, "KV cache NULL or unaligned");
  if (!wt->q_norm != !wt->k_norm) return fail(UNO_ERR_INVALID_ARGUMENT, "q_norm and k_norm: both or neither");
  if ((wt->q_norm && !aligned16(wt->q_norm)) || (wt->k_norm && !aligned16(wt->k_norm)))
    return fail(UNO_ERR_UNSUPPORTED, "q_norm / k_norm must be 16-byte aligned");
  if (!aligned16(hidden_state) || !aligned16(wt->attn_norm) || !aligned16(wt->mlp_norm))
    return fail(UNO_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
  if (!(rms_eps >= 0.f) || !std::isfinite(rms_eps) || !(rope_theta > 1.f) || !std::isfinite(rope_theta) ||
      !std::isfinite(lora_scale))
    return fail(UNO_ERR_INVALID_ARGUMENT, "rms_eps >= 0, rope_theta > 1 and a finite lora_scale required");
  const size_t need = decoder_layer_workspace_bytes(batch, block, ctx_len, hidden, inter, n_heads, n_kv_heads, r);
  if (workspace_bytes < need || !workspace)
    return fail(UNO_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);

  DecoderLayerArgs la{};
  la.batch = batch;
  la.block = block;
  la.ctx = ctx_len;
  la.hidden = hidden;
  la.inter = inter;
  la.n_heads = n_heads;
  la.n_kv = n_kv_heads;
  la.r = r;
  la.w = wt;
  la.gate = gate;
  la.positions = positions;
  la.cache_len = cache_len;
  la.rms_eps = rms_eps;
  la.rope_theta = rope_theta;
  la.lora_scale = lora_scale;
  la.h = hidden_state;
  la.ws = workspace;
  la.ws_bytes = workspace_bytes;
  const hipError_t e = launch_decoder_layer(la, stream);
  return check_hip(e, "uno_decoder_layer launch");
  UNO_GUARD_END
}

// ------------------------------------------------------------------ KV commit
uno_status uno_kv_commit(hipStream_t stream, int32_t batch, int32_t capacity, int32_t* accept_len,
                         int32_t* cache_len) {
  UNO_GUARD_BEGIN
  if (batch < 1 || capacity < 0) return fail(UNO_ERR_INVALID_ARGUMENT, "batch >= 1 and capacity >= 0 required");
  if (!accept_len || !cache_len) return fail(UNO_ERR_INVALID_ARGUMENT, "accept_len and cache_len are required");
  return check_hip(launch_kv_commit(batch, capacity, accept_len, cache_len, stream), "uno_kv_commit launch");
  UNO_GUARD_END
}

}  // extern "C"
