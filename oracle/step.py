"""Oracle: one whole Psi-Spec decode step (token ids to accepted length and
correction/bonus token).  Test infrastructure only.

Source: Uno paper summary (hyper.ai, arXiv 2609.04010), section "方法": the
diffusion path proposes a block of tokens, the AR weights verify it by
rejection sampling and keep the longest valid prefix; the linear sampler
draws a single candidate from the marginals; one forward pass runs over the
concatenated clean and noisy sequences with the adapter switched off on the
clean positions and on for the noisy ones.  Section "实验": Qwen3-8B base,
rank-128 adapters, one KV cache shared by drafting and verification.

Readings taken here (the pages leave them open):
* per sequence, 2*block token ids: `block` clean ids (the AR token, then
  k = block - 1 drafts) followed by `block` noisy ids;
* the rows' gates are 0 (clean) and 1 (noisy); clean row j and noisy row j
  sit at position ctx + j;
* logits = lm_head(final hidden state), stored as bf16;
* the drafts a step verifies are drawn from the same step's noisy rows:
  d[b, i] = inverse-CDF draw from softmax(noisy row i / T) at u_draft[b, i],
  for i < k (the same per-step work as carrying them over from the previous
  step);
* verification is `verify_linear` with p = the k + 1 clean rows and q = the
  first k noisy rows.

Float64 throughout, with bf16 rounding at the storage points of
`decoder_layer` and of the logits.
"""

import numpy as np

from .decoder import decoder_layer, lm_head, round_bf16
from .verify_linear import inverse_cdf, softmax_rows, verify_linear


def step_rows(batch, block, ctx):
    """(gate [rows], positions [rows]) of the concatenated clean + noisy rows.
    ctx: the cache length, one number for every sequence or one per sequence."""
    j = np.tile(np.arange(2 * block), batch)
    gate = (j >= block).astype(np.uint8)
    per_seq = np.broadcast_to(np.asarray(ctx), (batch,))
    pos = np.repeat(per_seq, 2 * block) + (j % block)
    return gate, pos


def decode_step(tokens, embed, layers, k_caches, v_caches, final_norm, w_lm, u_draft, u_accept, u_sample,
                block, n_heads, n_kv_heads, eps=1e-6, theta=1.0e6, lora_scale=1.0, temperature=1.0,
                cache_len=None):
    """tokens int [B, 2*block]; embed, w_lm [V, hidden]; layers: list of weight
    dicts as taken by `decoder_layer`; k_caches/v_caches: per layer
    [B, C, Hkv, 128]; u_draft, u_accept [B, block-1]; u_sample [B];
    cache_len [B] (optional): valid cache rows per sequence (None: all C).

    Returns dict: logits [B*2*block, V] (bf16-rounded float64), drafts [B, k],
    accept_len [B], token [B], and k_clean / v_clean: per layer the stored
    (bf16, after RoPE for k) keys and values of the clean rows [B, block, Hkv, 128],
    the rows `kv_commit` appends to the cache."""
    tokens = np.asarray(tokens)
    bsz = tokens.shape[0]
    k = block - 1
    cap = np.asarray(k_caches[0]).shape[1] if len(layers) else 0
    lens = np.full(bsz, cap) if cache_len is None else np.asarray(cache_len)
    gate, pos = step_rows(bsz, block, lens)
    h = np.asarray(embed, dtype=np.float64)[tokens.reshape(-1)]
    k_clean, v_clean = [], []
    for lw, kc, vc in zip(layers, k_caches, v_caches):
        h, st = decoder_layer(h, lw, gate, pos, kc, vc, block, n_heads, n_kv_heads, eps, theta, lora_scale,
                              lens)
        k_clean.append(st["k"].reshape(bsz, 2 * block, n_kv_heads, -1)[:, :block])
        v_clean.append(st["v"].reshape(bsz, 2 * block, n_kv_heads, -1)[:, :block])
    logits = round_bf16(lm_head(h, final_norm, w_lm, eps))
    lg = logits.reshape(bsz, 2 * block, -1)
    drafts = np.zeros((bsz, k), dtype=np.int64)
    for b in range(bsz):
        for i in range(k):
            drafts[b, i] = inverse_cdf(softmax_rows(lg[b, block + i], temperature), u_draft[b, i])
    v = verify_linear(lg[:, :block], lg[:, block:block + k], drafts, u_accept, u_sample, temperature)
    return {"logits": logits, "drafts": drafts, "accept_len": v["accept_len"], "token": v["token"],
            "p_draft": v["p_draft"], "q_draft": v["q_draft"], "k_clean": k_clean, "v_clean": v_clean}
