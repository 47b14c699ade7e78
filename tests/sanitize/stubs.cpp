// Host-only stand-ins for the library's kernel launchers and workspace
// queries, so that the C ABI's argument validation (api*.cpp) can be built
// and run under AddressSanitizer / UndefinedBehaviorSanitizer on a machine
// without a GPU.  Every launcher counts its calls and succeeds; workspace
// queries return small fixed sizes.
#include "../../diffusion_augmented_decoding_amd/csrc/internal.h"

namespace uno {

int g_stub_launches = 0;

static hipError_t launched() {
  ++g_stub_launches;
  return hipSuccess;
}

bool debug_checks() { return false; }
uno_status debug_check_ids(hipStream_t, const int32_t*, int64_t, int64_t, int64_t, int64_t, int32_t, int32_t,
                           const char*) {
  return UNO_OK;
}
uno_status debug_check_unit(hipStream_t, const float*, int64_t, const char*) { return UNO_OK; }

size_t block_attention_workspace_bytes(int, int, int, int, int) { return 256; }
size_t gated_lora_workspace_bytes(uno_dtype, int64_t, int64_t, int64_t, int64_t) { return 256; }
size_t lora_down_part_bytes(int64_t, int64_t, int64_t) { return 256; }
size_t sample_rows_workspace_bytes(int, int) { return 256; }
size_t tree_attention_workspace_bytes(int, int, int, int, int, int) { return 256; }
size_t lora_backward_workspace_bytes(int64_t, int64_t, int64_t, int64_t, int) { return 256; }
size_t tree_build_workspace_bytes(int, int, int) { return 256; }
size_t tree_verify_workspace_bytes(int, int, int, int, int, int) { return 256; }
size_t verify_linear_workspace_bytes(int, int, int) { return 256; }
size_t verify_linear_ee_workspace_bytes(int, int, int) { return 256; }
size_t verify_linear_sampled_workspace_bytes(int, int, int) { return 256; }
int rms_norm_max_dim() { return 1 << 16; }

bool gated_lora_pair_ok(const GatedLoraArgs&, const GatedLoraArgs&) { return true; }
bool swiglu_fused_ok(const SwigluArgs&) { return true; }

hipError_t launch_block_attention(const TreeAttnArgs&, hipStream_t) { return launched(); }
hipError_t launch_gated_lora(const GatedLoraArgs&, hipStream_t) { return launched(); }
hipError_t launch_gated_lora_pair(const GatedLoraArgs&, const GatedLoraArgs&, hipStream_t) { return launched(); }
hipError_t launch_gated_lora_swiglu(const SwigluArgs&, hipStream_t) { return launched(); }
hipError_t launch_kv_commit(int, int, int32_t*, int32_t*, hipStream_t) { return launched(); }
hipError_t launch_lora_down(const LoraDownArgs&, hipStream_t) { return launched(); }
hipError_t launch_lora_merge(const LoraMergeArgs&, hipStream_t) { return launched(); }
hipError_t launch_rms_norm(const RmsNormArgs&, hipStream_t) { return launched(); }
hipError_t launch_rope(const RopeArgs&, hipStream_t) { return launched(); }
hipError_t launch_sample_rows(const SampleRowsArgs&, hipStream_t) { return launched(); }
hipError_t launch_silu_mul(const SiluMulArgs&, hipStream_t) { return launched(); }
hipError_t launch_step_finish(const StepFinishArgs&, hipStream_t) { return launched(); }
hipError_t launch_step_setup(const StepSetupArgs&, hipStream_t) { return launched(); }
hipError_t launch_tree_attention(const TreeAttnArgs&, hipStream_t) { return launched(); }
hipError_t launch_distill(const DistillArgs&, hipStream_t) { return launched(); }
hipError_t launch_lora_backward(const LoraBackwardArgs&, hipStream_t) { return launched(); }
hipError_t launch_transpose_bf16(const void*, int64_t, void*, int64_t, int64_t, int64_t, hipStream_t) {
  return launched();
}
hipError_t launch_tree_build(const TreeBuildArgs&, hipStream_t) { return launched(); }
hipError_t launch_tree_verify(const TreeVerifyArgs&, hipStream_t) { return launched(); }
hipError_t launch_verify_linear(const VerifyLinearArgs&, hipStream_t) { return launched(); }
hipError_t launch_verify_linear_ee(const VerifyLinearArgs&, hipStream_t) { return launched(); }
hipError_t launch_verify_linear_sampled(const VerifyLinearArgs&, int, float, int, hipStream_t) { return launched(); }

}  // namespace uno
