"""Oracle: one whole Psi-Spec decode step of the decode loop, and a chain of
them.  Test infrastructure only.

Source: Uno paper summary (hyper.ai, arXiv 2609.04010), section "方法":
both weight sets draft and only the AR weights verify; the diffusion path
keeps the next-token parametrisation and predicts the next clean token from a
noisy sequence; the sampler proposes a block on the diffusion path and keeps
the longest prefix that passes rejection sampling against the AR
distribution; the first token of a block comes from the AR weights alone; the
linear sampler draws one candidate from the marginals; one forward pass runs
over the concatenated clean and noisy sequences with the adapter off on the
clean positions and on for the noisy ones.  Section "实验": Qwen3-8B base,
rank-128 adapters, one KV cache shared by drafting and verification.

Readings taken here (the pages leave them open):
* per sequence, 2*block token ids: `block` clean ids -- the AR token y of the
  previous step, then the k = block - 1 drafts d that step drew -- followed
  by `block` noisy ids (the caller's noise/mask ids for the next block);
* gates 0 on the clean rows, 1 on the noisy rows; clean row j sits at
  position ctx + j and noisy row j at ctx + block + j: the noisy rows stand
  for the next block, whose first position is where this step's AR token
  will go, and noisy row i (next-token parametrisation) gives the marginal
  of the token at ctx + block + i + 1;
* the drafts in the clean rows are verified against p = this step's clean
  rows 0..k (row i scores draft i, row k gives the bonus) and against the q
  they were drawn from, which the previous step produced and the caller
  carries over (`prev_q`); a step without a carried q (the loop's first)
  verifies no draft: L = 0 and y is drawn from clean row 0;
* this step's drafts are drawn from its noisy rows 0..k-1 by the
  inverse-CDF rule with u_draft; their logits are this step's `q_next`,
  carried to the next step;
* the next step's ids are [y, d_0 .. d_{k-1}] followed by the same noisy ids;
* with per-sequence cache lengths the clean rows 0..L are kept (they hold
  the previous step's AR token and the L accepted drafts: the tokens emitted
  so far apart from this step's y, which is the next block's first clean
  row); a sequence whose kept rows do not fit the capacity is flagged
  (accept_len = token = -1) and keeps nothing;
* a token id outside [0, V) embeds as a zero row (the next step of a flagged
  sequence carries y = -1).

Float64 throughout, with bf16 rounding at the storage points of
`decoder_layer` and of the logits.
"""

import numpy as np

from .decoder import decoder_layer, lm_head, round_bf16
from .kv_commit import kv_commit
from .verify_linear import inverse_cdf, softmax_rows, verify_linear


def step_rows(batch, block, ctx):
    """(gate [rows], positions [rows]) of the concatenated clean + noisy rows:
    clean row j at ctx + j, noisy row j at ctx + block + j.  ctx: the cache
    length, one number for every sequence or one per sequence."""
    j = np.tile(np.arange(2 * block), batch)
    gate = (j >= block).astype(np.uint8)
    per_seq = np.broadcast_to(np.asarray(ctx), (batch,))
    pos = np.repeat(per_seq, 2 * block) + j
    return gate, pos


def decode_step(tokens, embed, layers, k_caches, v_caches, final_norm, w_lm, prev_q, u_draft, u_accept, u_sample,
                block, n_heads, n_kv_heads, eps=1e-6, theta=1.0e6, lora_scale=1.0, temperature=1.0,
                cache_len=None, capacity=None):
    """tokens int [B, 2*block] (clean ids [y, d_0..d_{k-1}], then noisy ids);
    embed, w_lm [V, hidden]; layers: list of weight dicts as taken by
    `decoder_layer`; k_caches/v_caches: per layer [B, C, Hkv, 128]; prev_q
    [B, k, V] (the stored logits the clean drafts were drawn from) or None;
    u_draft, u_accept [B, block-1]; u_sample [B]; cache_len [B] (optional):
    valid cache rows per sequence (None: all C, nothing is kept); capacity:
    rows of cache per sequence (default: the caches' C; with no layers and no
    capacity the kept rows always fit).

    Returns dict: logits [B*2*block, V] (bf16-rounded float64); accept_len,
    token [B] (-1 for a sequence whose kept rows do not fit); drafts [B, k]
    (drawn from this step's noisy rows); q_next [B, k, V] (their logits);
    next_tokens [B, 2*block]; p_draft, q_draft [B, k] (zeros when no draft is
    verified); k_clean / v_clean: per layer the stored (bf16, after RoPE for
    k) keys and values of the clean rows [B, block, Hkv, 128]."""
    tokens = np.asarray(tokens)
    bsz = tokens.shape[0]
    k = block - 1
    if capacity is None and len(layers):
        capacity = np.asarray(k_caches[0]).shape[1]
    lens = np.full(bsz, capacity if capacity is not None else 0) if cache_len is None else np.asarray(cache_len)
    gate, pos = step_rows(bsz, block, lens)
    # an id outside [0, V) (e.g. the -1 of a flagged sequence) embeds as a zero row
    ids = tokens.reshape(-1)
    emb = np.asarray(embed, dtype=np.float64)
    ok = (ids >= 0) & (ids < emb.shape[0])
    h = np.where(ok[:, None], emb[np.where(ok, ids, 0)], 0.0)
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
    kv = k if prev_q is not None else 0
    v = verify_linear(lg[:, :kv + 1], np.asarray(prev_q)[:, :kv] if kv else np.zeros((bsz, 0, lg.shape[2])),
                      tokens[:, 1:kv + 1], np.asarray(u_accept)[:, :kv], u_sample, temperature)
    acc, tok = v["accept_len"].copy(), v["token"].copy()
    if cache_len is not None and capacity is not None:
        over = lens + acc + 1 > capacity
        acc[over] = -1
        tok[over] = -1
    nxt = tokens.copy()
    nxt[:, 0] = tok
    nxt[:, 1:block] = drafts
    pd = np.zeros((bsz, k))
    qd = np.zeros((bsz, k))
    pd[:, :kv], qd[:, :kv] = v["p_draft"], v["q_draft"]
    return {"logits": logits, "drafts": drafts, "accept_len": acc, "token": tok, "q_next": lg[:, block:block + k],
            "next_tokens": nxt, "p_draft": pd, "q_draft": qd, "k_clean": k_clean, "v_clean": v_clean}


def decode_loop(tokens, embed, layers, k_caches, v_caches, final_norm, w_lm, uniforms, block, n_heads, n_kv_heads,
                cache_len, prev_q=None, **kw):
    """A chain of decode steps on the shared caches: step t + 1 takes step t's
    next_tokens and q_next, and each step's kept clean rows are committed
    (kv_commit) before the next one runs.

    uniforms: list over steps of (u_draft, u_accept, u_sample).  Returns
    (list of per-step results of `decode_step`, each with its `cache_len`
    after the commit, final k_caches, final v_caches)."""
    kcs = [np.asarray(x, dtype=np.float64) for x in k_caches]
    vcs = [np.asarray(x, dtype=np.float64) for x in v_caches]
    lens = np.asarray(cache_len).copy()
    out = []
    for ud, ua, us in uniforms:
        r = decode_step(tokens, embed, layers, kcs, vcs, final_norm, w_lm, prev_q, ud, ua, us, block, n_heads,
                        n_kv_heads, cache_len=lens, **kw)
        new_len = np.where(r["accept_len"] >= 0, lens + r["accept_len"] + 1, lens)
        for l in range(len(layers)):
            kcs[l], vcs[l], new_len, _ = kv_commit(kcs[l], vcs[l], lens, r["k_clean"][l], r["v_clean"][l],
                                                   r["accept_len"])
        r["cache_len"] = new_len
        out.append(r)
        lens = new_len
        tokens = r["next_tokens"]
        prev_q = r["q_next"]
    return out, kcs, vcs


def emitted_tokens(steps, tokens0):
    """Per sequence, the token stream a chain produced: the first step's
    clean row 0 id, then for each step the drafts it accepted (the clean ids
    it verified) and its y.  A flagged step (accept_len -1) ends the stream."""
    tokens0 = np.asarray(tokens0)
    bsz = tokens0.shape[0]
    out = [[int(tokens0[b, 0])] for b in range(bsz)]
    alive = [True] * bsz
    verified = tokens0[:, 1:]
    for r in steps:
        for b in range(bsz):
            L = int(r["accept_len"][b])
            if not alive[b] or L < 0:
                alive[b] = False
                continue
            out[b].extend(int(x) for x in verified[b, :L])
            out[b].append(int(r["token"][b]))
        verified = r["drafts"]
    return out
