"""CPU oracle for the Psi-Spec decode-step hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) imports, calls or links this package; only the tests, the
`smoke()` check and the CPU-baseline leg of the benchmark do.

Every function here is a plain, slow, float64 restatement of what the method
computes, written from the pages:

* Uno: diffusion-augmented LLM (hyper.ai summary of arXiv 2609.04010),
  section "方法" (method) -- gated LoRA over concatenated clean + noisy rows,
  the Psi-Spec sampler with its linear and tree candidate strategies.
* The same paper's abstract (chatpaper.ai, English part) -- lossless
  acceleration.
* ainews.surl.tw article on Uno -- "lossless" means the samples follow the
  base AR distribution, not bit-identical text.

Each module states the passage it follows and every reading taken where the
pages are silent.  Pins that tie these functions to something other than
themselves live in `tests/test_oracle_*.py`.
"""

from .gated_lora import gated_lora_linear, merged_weight
from .distill import log_softmax_rows, distill_losses, gated_lora_backward
from .verify_linear import (
    softmax_rows,
    row_log_stats,
    accept_draft,
    residual_weights,
    inverse_cdf,
    verify_linear,
)
from .sampling import kth_largest, top_k_mask, top_p_mask, transform_probs
from .tree_attention import ancestors_or_self, tree_attention, tree_attention_dense_mask
from .verify_tree import node_depths, children_lists, verify_tree
from .tree_build import tree_layout, draw_without, build_tree
from .decoder import (
    round_bf16,
    rms_norm,
    rope,
    block_mask,
    block_attention,
    silu_mul,
    decoder_layer,
    lm_head,
)
from .step import step_rows, decode_step, decode_loop, emitted_tokens
from .kv_commit import kv_commit

__all__ = [
    "gated_lora_linear",
    "merged_weight",
    "log_softmax_rows",
    "distill_losses",
    "gated_lora_backward",
    "softmax_rows",
    "row_log_stats",
    "accept_draft",
    "residual_weights",
    "inverse_cdf",
    "verify_linear",
    "kth_largest",
    "top_k_mask",
    "top_p_mask",
    "transform_probs",
    "ancestors_or_self",
    "tree_attention",
    "tree_attention_dense_mask",
    "node_depths",
    "children_lists",
    "verify_tree",
    "tree_layout",
    "draw_without",
    "build_tree",
    "round_bf16",
    "rms_norm",
    "rope",
    "block_mask",
    "block_attention",
    "silu_mul",
    "decoder_layer",
    "lm_head",
    "step_rows",
    "decode_step",
    "decode_loop",
    "emitted_tokens",
    "kv_commit",
]
