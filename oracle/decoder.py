"""Oracle: one decoder layer of the composed decode step, and the LM head.
Test infrastructure only.

Source: Uno paper summary (hyper.ai, arXiv 2609.04010), section "方法" (one
forward pass over the concatenated clean and noisy sequences of a block, LoRA
adapters on every AR weight matrix switched by a per-position mask) and
section "实验" (the adapters sit on an open-weight Qwen3-8B model, rank 128;
the draft and verify paths share one KV cache; full attention).  The pages
give no layer internals.  Readings taken here:

* Qwen3-8B shapes: hidden 4096, MLP 12288, 32 query / 8 KV heads of 128;
  pre-norm RMSNorm (eps 1e-6) before attention and before the MLP, SwiGLU MLP
  (silu(gate) * up), residual adds, no biases;
* Qwen3's per-head RMSNorm of q and k (weights q_norm, k_norm of 128, the
  same eps) over each 128-wide head, after the projection and before the
  rotation; optional (a layer without the two weights skips it).  The normed
  values are not stored: the one bf16 rounding comes after the rotation;
* rotary position embedding on q and k, base 1e6, "rotate half" pairing
  (element i with element i + 64 of a 128-wide head);
* rows of one sequence: `block` clean rows (adapter off) then `block` noisy
  rows (adapter on); clean row i and noisy row i both sit at position ctx + i;
* block mask: clean row i attends to the whole cache and to clean rows 0..i;
  a noisy row attends to the whole cache and to every row of the block;
* LM head: final RMSNorm then a plain projection (no adapter);
* between kernels every activation is stored as bf16 (round to nearest even);
  each function below returns exact float64 results, and `decoder_layer`
  applies the bf16 rounding at the same storage points as the GPU path.

Float64 throughout.
"""

import numpy as np

from .gated_lora import gated_lora_linear


def round_bf16(x):
    """float64 values rounded to bfloat16 (nearest, ties to even), returned as float64."""
    f = np.asarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(f)
    out = rounded.astype(np.uint32).view(np.float32).astype(np.float64)
    out[nan] = np.nan
    return out


def rms_norm(x, weight, eps=1e-6):
    """x / sqrt(mean(x^2) + eps) * weight, over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def rope(x, positions, theta=1.0e6):
    """Rotary embedding of x [rows, heads, D] at integer positions [rows].

    Pair (i, i + D/2) of every head is rotated by the angle pos * theta^(-2i/D).
    """
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(positions, dtype=np.float64).reshape(-1)
    d = x.shape[-1]
    half = d // 2
    inv_freq = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = pos[:, None] * inv_freq[None, :]             # [rows, half]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def block_mask(block):
    """Allowed block keys per block row, [2*block, 2*block] bool (clean rows first)."""
    n = 2 * block
    allow = np.zeros((n, n), dtype=bool)
    for i in range(n):
        if i < block:
            allow[i, : i + 1] = True        # clean row: causal over the clean rows
        else:
            allow[i, :] = True              # noisy row: the whole block
    return allow


def block_attention(q, k_cache, v_cache, k_blk, v_blk, block, scale, ctx_lens=None):
    """Attention of the block rows over cache + block under `block_mask`.

    q [B, n, H, D] with n = 2*block; k_cache/v_cache [B, C, Hkv, D];
    k_blk/v_blk [B, n, Hkv, D].  ctx_lens [B] (optional): sequence b's cache
    holds ctx_lens[b] <= C valid rows; rows from ctx_lens[b] on are unused
    capacity and are not attended.  None means every sequence has C rows.
    Returns (out [B, n, H, D], lse [B, n, H]).
    """
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    kb = np.asarray(k_blk, dtype=np.float64)
    vb = np.asarray(v_blk, dtype=np.float64)
    bsz, n, nh, hd = q.shape
    nkv = kc.shape[2]
    group = nh // nkv
    ctx = kc.shape[1]
    allow = block_mask(block)
    lens = np.full(bsz, ctx) if ctx_lens is None else np.asarray(ctx_lens)
    out = np.zeros((bsz, n, nh, hd))
    lse = np.zeros((bsz, n, nh))
    for b in range(bsz):
        c = int(lens[b])
        for h in range(nh):
            g = h // group
            keys = np.concatenate([kc[b, :c, g, :], kb[b, :, g, :]], axis=0)     # [c + n, D]
            vals = np.concatenate([vc[b, :c, g, :], vb[b, :, g, :]], axis=0)
            s = scale * (q[b, :, h, :] @ keys.T)                               # [n, c + n]
            ok = np.concatenate([np.ones((n, c), dtype=bool), allow], axis=1)
            s = np.where(ok, s, -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            e = np.exp(s - m)
            z = np.sum(e, axis=1, keepdims=True)
            out[b, :, h, :] = (e / z) @ vals
            lse[b, :, h] = (m + np.log(z))[:, 0]
    return out, lse


def silu_mul(g, u):
    """silu(g) * u = g / (1 + exp(-g)) * u."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    return g / (1.0 + np.exp(-g)) * u


def decoder_layer(h, w, gate, positions, k_cache, v_cache, block, n_heads, n_kv_heads,
                  eps=1e-6, theta=1.0e6, lora_scale=1.0, ctx_lens=None):
    """One layer on the residual stream h [rows, hidden], rows = B * 2 * block.
    ctx_lens: per-sequence valid cache rows, as in `block_attention`.

    w: dict with attn_norm, mlp_norm [hidden] and, for p in q k v o g u d,
    w{p} [out, in], a{p} [r, in], b{p} [out, r]; optionally q_norm and k_norm
    [128] (both or neither).  Every stored intermediate is rounded to bf16;
    returns (h_out, dict of the stored intermediates).
    """
    bf = round_bf16
    h = np.asarray(h, dtype=np.float64)
    rows, hidden = h.shape
    bsz = rows // (2 * block)
    hd = 128

    def proj(x, p):
        return bf(gated_lora_linear(x, w["w" + p], w["a" + p], w["b" + p], gate, lora_scale))

    a = bf(rms_norm(h, w["attn_norm"], eps))
    q = proj(a, "q").reshape(rows, n_heads, hd)
    k = proj(a, "k").reshape(rows, n_kv_heads, hd)
    v = proj(a, "v").reshape(rows, n_kv_heads, hd)
    assert ("q_norm" in w) == ("k_norm" in w), "q_norm and k_norm come together"
    if "q_norm" in w:
        q = rms_norm(q, w["q_norm"], eps)          # over each head's 128 values
        k = rms_norm(k, w["k_norm"], eps)
    q = bf(rope(q, positions, theta))
    k = bf(rope(k, positions, theta))
    n = 2 * block
    att, _ = block_attention(q.reshape(bsz, n, n_heads, hd), k_cache, v_cache,
                             k.reshape(bsz, n, n_kv_heads, hd), v.reshape(bsz, n, n_kv_heads, hd),
                             block, 1.0 / np.sqrt(hd), ctx_lens)
    att = bf(att.reshape(rows, n_heads * hd))
    o = proj(att, "o")
    h1 = bf(h + o)
    a2 = bf(rms_norm(h1, w["mlp_norm"], eps))
    gg = proj(a2, "g")
    uu = proj(a2, "u")
    m = bf(silu_mul(gg, uu))
    d = proj(m, "d")
    h2 = bf(h1 + d)
    return h2, {"a": a, "q": q, "k": k, "v": v, "att": att, "h1": h1, "a2": a2, "m": m}


def lm_head(h, norm_w, w_lm, eps=1e-6):
    """Logits [rows, V] = bf16(rms_norm(h)) W_lm^T (float64, before output rounding)."""
    a = round_bf16(rms_norm(h, norm_w, eps))
    return a @ np.asarray(w_lm, dtype=np.float64).T
