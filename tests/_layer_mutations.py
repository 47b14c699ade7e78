"""Planted wiring mistakes in the decoder layer, for measuring test power.

`mutated_layer` restates `oracle.decoder_layer` step by step from the
oracle's own pieces (gated LoRA, RMSNorm, RoPE, SwiGLU, bf16 storage
rounding), with the attention written here over an explicit mask, and
plants one mistake selected by name.  With no mistake it reproduces the
oracle exactly (pinned in tests/test_layer_mutations.py), so each mutation
differs from the oracle by that one mistake alone.

The mistakes are the ones a GPU wiring bug would make:
  mask_leak              clean rows also see the noisy rows of their block
  positions_at_ctx       every row of a block rotated at the block's first position
  positions_shift        every row rotated one position further
  swiglu_swap            silu(up) * gate instead of silu(gate) * up
  drop_qkv_adapters      no adapter on q, k and v
  drop_o_adapter         no adapter on o
  drop_gate_up_adapters  no adapter on gate and up
  drop_down_adapter      no adapter on down
  no_attention           the attention output replaced by zeros
  mlp_norm_of_input      the MLP norm reads the layer input h instead of h + o
  drop_qk_norm           no per-head RMSNorm of q and k (layers that have it)

Test infrastructure only.
"""

import numpy as np

import oracle

MUTATIONS = ("mask_leak", "positions_at_ctx", "positions_shift", "swiglu_swap", "drop_qkv_adapters",
             "drop_o_adapter", "drop_gate_up_adapters", "drop_down_adapter", "no_attention",
             "mlp_norm_of_input", "drop_qk_norm")
ADAPTER_MUTATIONS = ("drop_qkv_adapters", "drop_o_adapter", "drop_gate_up_adapters", "drop_down_adapter")


def _attention(q, kc, vc, kb, vb, block, scale, lens, leak):
    """Masked softmax attention per sequence; q [B, n, H, D], caches [B, C, Hkv, D]."""
    bsz, n, nh, hd = q.shape
    group = nh // kc.shape[2]
    out = np.zeros_like(q)
    allow = np.zeros((n, n), dtype=bool)
    for i in range(n):
        if i < block and not leak:
            allow[i, : i + 1] = True
        else:
            allow[i, :] = True
    for b in range(bsz):
        c = int(lens[b])
        for h in range(nh):
            g = h // group
            keys = np.concatenate([kc[b, :c, g], kb[b, :, g]], axis=0)
            vals = np.concatenate([vc[b, :c, g], vb[b, :, g]], axis=0)
            s = scale * (q[b, :, h] @ keys.T)
            ok = np.concatenate([np.ones((n, c), dtype=bool), allow], axis=1)
            s = np.where(ok, s, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            out[b, :, h] = (e / e.sum(axis=1, keepdims=True)) @ vals
    return out


def mutated_layer(h, w, gate, positions, k_cache, v_cache, block, n_heads, n_kv_heads, mutation=None,
                  ctx_lens=None, eps=1e-6, theta=1.0e6):
    """oracle.decoder_layer with the named mistake planted (None: no mistake)."""
    assert mutation is None or mutation in MUTATIONS, mutation
    bf = oracle.round_bf16
    h = np.asarray(h, dtype=np.float64)
    rows, hidden = h.shape
    n = 2 * block
    bsz = rows // n
    hd = 128
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    lens = np.full(bsz, kc.shape[1]) if ctx_lens is None else np.asarray(ctx_lens)
    dropped = {"drop_qkv_adapters": "qkv", "drop_o_adapter": "o", "drop_gate_up_adapters": "gu",
               "drop_down_adapter": "d"}.get(mutation, "")

    def proj(x, p):
        g = np.zeros_like(gate) if p in dropped else gate
        return bf(oracle.gated_lora_linear(x, w["w" + p], w["a" + p], w["b" + p], g))

    pos = np.asarray(positions).copy()
    if mutation == "positions_at_ctx":
        pos = pos.reshape(bsz, n)
        pos = np.repeat(pos.min(axis=1, keepdims=True), n, axis=1).reshape(-1)
    elif mutation == "positions_shift":
        pos = pos + 1
    a = bf(oracle.rms_norm(h, w["attn_norm"], eps))
    q = proj(a, "q").reshape(rows, n_heads, hd)
    k = proj(a, "k").reshape(rows, n_kv_heads, hd)
    if "q_norm" in w and mutation != "drop_qk_norm":
        q = oracle.rms_norm(q, w["q_norm"], eps)
        k = oracle.rms_norm(k, w["k_norm"], eps)
    q = bf(oracle.rope(q, pos, theta))
    k = bf(oracle.rope(k, pos, theta))
    v = proj(a, "v").reshape(rows, n_kv_heads, hd)
    att = _attention(q.reshape(bsz, n, n_heads, hd), kc, vc, k.reshape(bsz, n, n_kv_heads, hd),
                     v.reshape(bsz, n, n_kv_heads, hd), block, 1.0 / np.sqrt(hd), lens, mutation == "mask_leak")
    att = bf(att.reshape(rows, n_heads * hd))
    if mutation == "no_attention":
        att = np.zeros_like(att)
    h1 = bf(h + proj(att, "o"))
    a2 = bf(oracle.rms_norm(h if mutation == "mlp_norm_of_input" else h1, w["mlp_norm"], eps))
    gg, uu = proj(a2, "g"), proj(a2, "u")
    m = bf(oracle.silu_mul(uu, gg) if mutation == "swiglu_swap" else oracle.silu_mul(gg, uu))
    return bf(h1 + proj(m, "d"))


def row_relerr(got, ref):
    """max over rows of ||got - ref||_inf / ||ref||_inf."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    return float(np.max(np.max(np.abs(got - ref), axis=1) / np.maximum(np.max(np.abs(ref), axis=1), 1e-300)))
