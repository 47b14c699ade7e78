// Drives every host-validated entry point of the C ABI with valid and
// invalid arguments, linked against launcher stand-ins (stubs.cpp), under
// AddressSanitizer and UndefinedBehaviorSanitizer.  "Device" buffers are
// host memory here; validation never reads them.  Exit status 0 when every
// call returned the expected class of status and the sanitizers stayed
// quiet (they abort the process otherwise).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "uno.h"

namespace uno {
extern int g_stub_launches;
}

static int g_fail = 0;

static void expect(const char* what, uno_status got, bool want_ok) {
  if ((got == UNO_OK) != want_ok) {
    fprintf(stderr, "%s: status %d (%s), expected %s\n", what, int(got), uno_last_error(),
            want_ok ? "ok" : "an error");
    ++g_fail;
  }
}

int main() {
  std::vector<unsigned char> mem(1 << 22);
  void* D = mem.data() + 256 - (reinterpret_cast<uintptr_t>(mem.data()) & 255);   // 256-byte aligned
  void* odd = static_cast<char*>(D) + 1;
  const size_t big = size_t(1) << 40;
  size_t bytes = 0;
  hipStream_t s = nullptr;

  if (uno_abi_version() < 1) ++g_fail;
  for (int i = -1; i < 8; ++i) (void)uno_status_string(uno_status(i));

  // gated LoRA
  expect("lora ws", uno_gated_lora_linear_workspace(UNO_BF16, 64, 128, 256, 16, &bytes), true);
  expect("lora ws null", uno_gated_lora_linear_workspace(UNO_BF16, 64, 128, 256, 16, nullptr), false);
  expect("lora", uno_gated_lora_linear(s, UNO_BF16, 64, 128, 256, 16, D, 256, D, 256, D, 256, D, 16,
                                       (const uint8_t*)D, 1.f, D, 128, D, big), true);
  expect("lora bad M", uno_gated_lora_linear(s, UNO_BF16, -1, 128, 256, 16, D, 256, D, 256, D, 256, D, 16,
                                             (const uint8_t*)D, 1.f, D, 128, D, big), false);
  expect("lora odd x", uno_gated_lora_linear(s, UNO_BF16, 64, 128, 256, 16, odd, 256, D, 256, D, 256, D, 16,
                                             (const uint8_t*)D, 1.f, D, 128, D, big), false);
  expect("lora ld", uno_gated_lora_linear(s, UNO_F32, 64, 128, 256, 16, D, 8, D, 256, D, 256, D, 16,
                                          (const uint8_t*)D, 1.f, D, 128, D, big), false);
  expect("merge", uno_lora_merge(s, 128, 256, 16, D, 256, D, 256, D, 16, 0.5f, D, 256), true);
  expect("merge r", uno_lora_merge(s, 128, 256, 0, D, 256, D, 256, D, 16, 0.5f, D, 256), false);

  // linear verify, plain and sampled
  const int B = 3, K = 4, V = 1000;
  for (int pass = 0; pass < 3; ++pass) {
    auto call = [&](int batch, int k, int vocab, const void* p, int64_t ps, int64_t pr, float t, int top_k,
                    float top_p, void* ws, size_t wsb) {
      if (pass == 0)
        return uno_psi_spec_verify_linear(s, UNO_BF16, batch, k, vocab, p, ps, pr, D, int64_t(K) * V, V,
                                          (const int32_t*)D, (const float*)D, (const float*)D, t, (int32_t*)D,
                                          (int32_t*)D, nullptr, nullptr, nullptr, ws, wsb);
      if (pass == 2)
        return uno_psi_spec_verify_linear_early_exit(s, UNO_BF16, batch, k, vocab, p, ps, pr, D, int64_t(K) * V, V,
                                                     (const int32_t*)D, (const float*)D, (const float*)D, t,
                                                     (int32_t*)D, (int32_t*)D, nullptr, nullptr, nullptr, ws, wsb);
      return uno_psi_spec_verify_linear_sampled(s, UNO_BF16, batch, k, vocab, p, ps, pr, D, int64_t(K) * V, V,
                                                (const int32_t*)D, (const float*)D, (const float*)D, t, top_k,
                                                top_p, 0, (int32_t*)D, (int32_t*)D, nullptr, nullptr, nullptr, ws,
                                                wsb);
    };
    expect("verify", call(B, K, V, D, int64_t(K + 1) * V, V, 1.f, 5, 0.9f, D, big), true);
    expect("verify k", call(B, 65, V, D, int64_t(66) * V, V, 1.f, 5, 0.9f, D, big), false);
    expect("verify T", call(B, K, V, D, int64_t(K + 1) * V, V, 0.f, 5, 0.9f, D, big), false);
    expect("verify stride", call(B, K, V, D, int64_t(K + 1) * V, V - 1, 1.f, 5, 0.9f, D, big), false);
    expect("verify p", call(B, K, V, nullptr, int64_t(K + 1) * V, V, 1.f, 5, 0.9f, D, big), false);
    expect("verify ws", call(B, K, V, D, int64_t(K + 1) * V, V, 1.f, 5, 0.9f, D, 8), false);
    expect("verify vocab", call(B, K, (1 << 20) + 1, D, int64_t(K + 1) << 21, 1 << 21, 1.f, 5, 0.9f, D, big), false);
    if (pass == 1) {
      expect("sampled top_p", call(B, K, V, D, int64_t(K + 1) * V, V, 1.f, 5, 0.f, D, big), false);
      expect("sampled top_k", call(B, K, V, D, int64_t(K + 1) * V, V, 1.f, -2, 0.9f, D, big), false);
    }
  }
  expect("verify ws q", uno_psi_spec_verify_linear_workspace(256, 15, 151936, &bytes), true);
  expect("early exit ws q", uno_psi_spec_verify_linear_early_exit_workspace(256, 15, 151936, &bytes), true);
  expect("sampled ws q", uno_psi_spec_verify_linear_sampled_workspace(256, 15, 151936, &bytes), true);

  // tree attention and tree verify
  expect("tree attn ws", uno_tree_verify_attention_workspace(1, 65, 1024, 32, 8, 128, &bytes), true);
  expect("tree attn", uno_tree_verify_attention(s, 1, 65, 1024, 32, 8, 128, D, D, D, D, D, (const int32_t*)D, 0.08f,
                                                D, (float*)D, D, big), true);
  expect("tree attn hd", uno_tree_verify_attention(s, 1, 65, 1024, 32, 8, 64, D, D, D, D, D, (const int32_t*)D,
                                                   0.08f, D, (float*)D, D, big), false);
  expect("tree ws", uno_psi_spec_verify_tree_workspace(2, 65, 3, 4, V, &bytes), true);
  expect("tree", uno_psi_spec_verify_tree(s, UNO_BF16, 2, 65, 3, 4, V, (const int32_t*)D, (const int32_t*)D, D, D,
                                          (const float*)D, (const float*)D, 1.f, (int32_t*)D, (int32_t*)D,
                                          (int32_t*)D, D, big), true);
  expect("tree n", uno_psi_spec_verify_tree(s, UNO_BF16, 2, 2000, 3, 4, V, (const int32_t*)D, (const int32_t*)D, D,
                                            D, (const float*)D, (const float*)D, 1.f, (int32_t*)D, (int32_t*)D,
                                            (int32_t*)D, D, big), false);

  expect("tree wor ws", uno_psi_spec_verify_tree_wor_workspace(2, 65, 3, 4, V, &bytes), true);
  expect("tree wor", uno_psi_spec_verify_tree_wor(s, UNO_BF16, 2, 65, 3, 4, V, (const int32_t*)D, (const int32_t*)D,
                                                  D, D, (const float*)D, (const float*)D, 1.f, (int32_t*)D,
                                                  (int32_t*)D, (int32_t*)D, D, big), true);
  expect("tree wor children", uno_psi_spec_verify_tree_wor(s, UNO_BF16, 2, 65, 3, 65, V, (const int32_t*)D,
                                                           (const int32_t*)D, D, D, (const float*)D, (const float*)D,
                                                           1.f, (int32_t*)D, (int32_t*)D, (int32_t*)D, D, big),
         false);

  // gated-LoRA backward
  expect("lora bwd ws", uno_gated_lora_backward_workspace(1024, 4096, 4096, 128, 1, &bytes), true);
  expect("lora bwd", uno_gated_lora_backward(s, 64, 256, 128, 16, D, 128, D, 128, D, 128, D, 16, (const uint8_t*)D,
                                             1.f, D, 256, D, 128, (float*)D, 128, (float*)D, 16, nullptr, 0, D, big),
         true);
  expect("lora bwd wt", uno_gated_lora_backward(s, 64, 256, 128, 16, D, 128, D, 128, D, 128, D, 16,
                                                (const uint8_t*)D, 1.f, D, 256, D, 128, (float*)D, 128, (float*)D, 16,
                                                D, 256, D, big), true);
  expect("lora bwd N", uno_gated_lora_backward(s, 64, 250, 128, 16, D, 128, D, 128, D, 128, D, 16,
                                               (const uint8_t*)D, 1.f, D, 256, D, 128, (float*)D, 128, (float*)D, 16,
                                               nullptr, 0, D, big), false);
  expect("transpose", uno_transpose_bf16(s, 100, 60, D, 64, D, 104), true);
  expect("transpose ld", uno_transpose_bf16(s, 100, 60, D, 50, D, 104), false);

  // distillation losses
  expect("distill", uno_distill_loss(s, UNO_BF16, 2, 8, V, D, 16 * V, V, D, 16 * V, V, 1.f, 1.f, 1.f, 1.f, (float*)D,
                                     (float*)D, D, 16 * V, V), true);
  expect("distill no grad", uno_distill_loss(s, UNO_F32, 2, 8, V, D, 16 * V, V, D, 16 * V, V, 0.7f, 1.f, 0.f, 1.f,
                                             (float*)D, (float*)D, nullptr, 0, 0), true);
  expect("distill stride", uno_distill_loss(s, UNO_BF16, 2, 8, V, D, 16 * V, V - 1, D, 16 * V, V, 1.f, 1.f, 1.f, 1.f,
                                            (float*)D, (float*)D, D, 16 * V, V), false);

  // tree construction (branching is a host array read by the call)
  const int32_t br[3] = {4, 2, 2};   // 1 + 4 + 8 + 16 = 29 nodes
  const int32_t br_bad[3] = {4, 0, 2};
  expect("build ws", uno_psi_spec_build_tree_workspace(2, 3, V, &bytes), true);
  expect("build", uno_psi_spec_build_tree(s, UNO_BF16, 2, 3, br, V, D, 3 * V, V, (const float*)D, 29, 1.f, 1,
                                          (int32_t*)D, (int32_t*)D, D, big), true);
  expect("build n", uno_psi_spec_build_tree(s, UNO_BF16, 2, 3, br, V, D, 3 * V, V, (const float*)D, 30, 1.f, 0,
                                            (int32_t*)D, (int32_t*)D, D, big), false);
  expect("build branch", uno_psi_spec_build_tree(s, UNO_BF16, 2, 3, br_bad, V, D, 3 * V, V, (const float*)D, 29,
                                                 1.f, 0, (int32_t*)D, (int32_t*)D, D, big), false);
  expect("build null", uno_psi_spec_build_tree(s, UNO_BF16, 2, 3, nullptr, V, D, 3 * V, V, (const float*)D, 29,
                                               1.f, 0, (int32_t*)D, (int32_t*)D, D, big), false);

  // layer ops
  expect("norm", uno_rms_norm(s, 16, 256, D, 256, nullptr, 0, nullptr, 0, D, 1e-6f, D, 256), true);
  expect("norm dim", uno_rms_norm(s, 16, 0, D, 256, nullptr, 0, nullptr, 0, D, 1e-6f, D, 256), false);
  expect("rope", uno_rope(s, 16, 4, D, 512, (const int32_t*)D, 1e6f, nullptr, 1e-6f), true);
  expect("rope norm", uno_rope(s, 16, 4, D, 512, (const int32_t*)D, 1e6f, D, 1e-6f), true);
  expect("rope theta", uno_rope(s, 16, 4, D, 512, (const int32_t*)D, 0.5f, nullptr, 1e-6f), false);
  expect("rope norm eps", uno_rope(s, 16, 4, D, 512, (const int32_t*)D, 1e6f, D, -1.f), false);
  expect("silu", uno_silu_mul(s, 16, 256, D, 256, D, 256, D, 256), true);
  expect("silu null", uno_silu_mul(s, 16, 256, nullptr, 256, D, 256, D, 256), false);
  expect("block attn ws", uno_block_verify_attention_workspace(4, 16, 128, 32, 8, 128, &bytes), true);
  expect("block attn", uno_block_verify_attention(s, 4, 16, 128, 32, 8, 128, D, D, D, nullptr, D, D, 0.08f, D,
                                                  (float*)D, D, big), true);
  expect("block attn heads", uno_block_verify_attention(s, 4, 16, 128, 32, 3, 128, D, D, D, nullptr, D, D, 0.08f, D,
                                                        (float*)D, D, big), false);
  expect("sample ws", uno_sample_rows_workspace(8, V, &bytes), true);
  expect("sample", uno_sample_rows(s, UNO_BF16, 8, V, D, V, (const float*)D, 1.f, (int32_t*)D, D, big), true);
  expect("sample stride", uno_sample_rows(s, UNO_BF16, 8, V, D, V - 3, (const float*)D, 1.f, (int32_t*)D, D, big),
         false);

  // decoder layer, with and without merged weights
  uno_layer_weights w;
  memset(&w, 0, sizeof(w));
  w.attn_norm = D;
  w.mlp_norm = D;
  for (int p = 0; p < UNO_NUM_PROJ; ++p) {
    w.w[p] = D;
    w.a[p] = D;
    w.b[p] = D;
  }
  w.k_cache = D;
  w.v_cache = D;
  expect("layer ws", uno_decoder_layer_workspace(2, 4, 40, 256, 512, 4, 2, 16, &bytes), true);
  expect("layer", uno_decoder_layer(s, 2, 4, 40, 256, 512, 4, 2, 16, &w, (const uint8_t*)D, (const int32_t*)D, nullptr,
                                    1e-6f, 1e6f, 1.f, D, D, big), true);
  w.q_norm = D;
  w.k_norm = D;
  expect("layer qk norm", uno_decoder_layer(s, 2, 4, 40, 256, 512, 4, 2, 16, &w, (const uint8_t*)D, (const int32_t*)D,
                                            nullptr, 1e-6f, 1e6f, 1.f, D, D, big), true);
  w.k_norm = nullptr;
  expect("layer q norm alone", uno_decoder_layer(s, 2, 4, 40, 256, 512, 4, 2, 16, &w, (const uint8_t*)D,
                                                 (const int32_t*)D, nullptr, 1e-6f, 1e6f, 1.f, D, D, big), false);
  w.q_norm = nullptr;
  expect("layer weights", uno_decoder_layer(s, 2, 4, 40, 256, 512, 4, 2, 16, nullptr, (const uint8_t*)D,
                                            (const int32_t*)D, nullptr, 1e-6f, 1e6f, 1.f, D, D, big), false);
  expect("commit", uno_kv_commit(s, 4, 100, (int32_t*)D, (int32_t*)D), true);
  expect("commit null", uno_kv_commit(s, 4, 100, nullptr, (int32_t*)D), false);

  // decode step over several layers (the host array of layer weights is read)
  uno_step_config c;
  memset(&c, 0, sizeof(c));
  c.batch = 2;
  c.block = 4;
  c.ctx_len = 40;
  c.hidden = 256;
  c.inter = 512;
  c.n_heads = 4;
  c.n_kv_heads = 2;
  c.r = 16;
  c.n_layers = 3;
  c.vocab = V;
  c.rms_eps = 1e-6f;
  c.rope_theta = 1e6f;
  c.lora_scale = 1.f;
  c.temperature = 1.f;
  std::vector<uno_layer_weights> layers(3, w);
  expect("step ws", uno_psi_spec_step_workspace(&c, &bytes), true);
  expect("step", uno_psi_spec_step(s, &c, layers.data(), D, D, D, (const int32_t*)D, (int32_t*)D, D, int64_t(3) * V, V,
                                   (const float*)D, (const float*)D, (const float*)D, D, (int32_t*)D, (int32_t*)D,
                                   (int32_t*)D, (int32_t*)D, D, big), true);
  for (int p = 0; p < UNO_NUM_PROJ; ++p) layers[1].w_merged[p] = D;
  expect("step merged", uno_psi_spec_step(s, &c, layers.data(), D, D, D, (const int32_t*)D, nullptr, nullptr, 0, 0,
                                          (const float*)D, (const float*)D, (const float*)D, D, (int32_t*)D,
                                          (int32_t*)D, (int32_t*)D, nullptr, D, big), true);
  layers[2].w[3] = nullptr;
  expect("step null w", uno_psi_spec_step(s, &c, layers.data(), D, D, D, (const int32_t*)D, nullptr, nullptr, 0, 0,
                                          (const float*)D, (const float*)D, (const float*)D, D, (int32_t*)D,
                                          (int32_t*)D, (int32_t*)D, nullptr, D, big), false);
  c.block = 0;
  expect("step block", uno_psi_spec_step_workspace(&c, &bytes), false);

  // profiling with no records
  double ms = 0;
  int64_t cnt = 0;
  expect("profile", uno_profile_query("uno_gemm_bf16", &ms, &cnt), true);
  expect("profile null", uno_profile_query(nullptr, &ms, &cnt), false);

  if (uno::g_stub_launches == 0) ++g_fail;
  printf("%d launches reached, %d unexpected statuses\n", uno::g_stub_launches, g_fail);
  return g_fail == 0 ? 0 : 1;
}
