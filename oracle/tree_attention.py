"""Oracle: tree-masked GQA attention for tree verification.  Test infrastructure only.

Source: Uno paper summary (hyper.ai, arXiv 2609.04010), section "方法", last
paragraph: the tree sampler draws several candidates and verifies them
concurrently as a prefix tree using tree attention.  The pages give no mask,
layout or head configuration; the readings taken here are:

* node 0 is the root (the block's first token, produced by the AR weights and
  not yet in the KV cache); nodes are numbered so that parent[i] < i;
* node i attends to every cached position plus the tree nodes that are its
  ancestors or itself (the usual prefix-tree mask);
* no causal constraint inside the cache; RoPE is applied by the caller;
* grouped-query attention: query head h reads KV head h // (H / H_kv);
* O = softmax(scale * Q K^T) V over the allowed keys, plus the natural-log
  log-sum-exp of the scaled scores (LSE) per (node, head).

Float64 throughout, from the exact values of the (bf16) inputs.
"""

import numpy as np


def ancestors_or_self(parent):
    """List of ascending node-id lists: the ancestors of i plus i itself."""
    parent = [int(x) for x in np.asarray(parent).reshape(-1)]
    out = []
    for i in range(len(parent)):
        chain = []
        j = i
        while j >= 0:
            chain.append(j)
            j = parent[j]
        out.append(sorted(chain))
    return out


def tree_attention(q, k_cache, v_cache, k_tree, v_tree, parent, scale):
    """Per-(node, head) loop form.

    q       [B, n, H, D]
    k_cache [B, C, Hkv, D], v_cache [B, C, Hkv, D]
    k_tree  [B, n, Hkv, D], v_tree  [B, n, Hkv, D]
    parent  [B, n] (parent[b, 0] = -1)
    Returns (out [B, n, H, D] float64, lse [B, n, H] float64).
    """
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    k_tree = np.asarray(k_tree, dtype=np.float64)
    v_tree = np.asarray(v_tree, dtype=np.float64)
    parent = np.asarray(parent)
    bsz, n, nh, hd = q.shape
    nkv = k_cache.shape[2]
    group = nh // nkv
    out = np.zeros((bsz, n, nh, hd), dtype=np.float64)
    lse = np.zeros((bsz, n, nh), dtype=np.float64)
    for b in range(bsz):
        anc = ancestors_or_self(parent[b])
        for i in range(n):
            for h in range(nh):
                g = h // group
                keys = np.concatenate([k_cache[b, :, g, :], k_tree[b, anc[i], g, :]], axis=0)
                vals = np.concatenate([v_cache[b, :, g, :], v_tree[b, anc[i], g, :]], axis=0)
                s = scale * (keys @ q[b, i, h])
                mx = np.max(s)
                e = np.exp(s - mx)
                z = np.sum(e)
                out[b, i, h] = (e / z) @ vals
                lse[b, i, h] = mx + np.log(z)
    return out, lse


def tree_attention_dense_mask(q, k_cache, v_cache, k_tree, v_tree, parent, scale):
    """Second, independent form: one dense [n, C + n] boolean mask per batch.

    Used only to cross-check `tree_attention`; same arguments and results.
    """
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    k_tree = np.asarray(k_tree, dtype=np.float64)
    v_tree = np.asarray(v_tree, dtype=np.float64)
    parent = np.asarray(parent)
    bsz, n, nh, hd = q.shape
    ctx = k_cache.shape[1]
    nkv = k_cache.shape[2]
    group = nh // nkv
    out = np.zeros((bsz, n, nh, hd))
    lse = np.zeros((bsz, n, nh))
    for b in range(bsz):
        # allowed[i, j] for tree key j: walk i's parent chain once, marking.
        allowed_tree = np.zeros((n, n), dtype=bool)
        for i in range(n):
            j = i
            while j >= 0:
                allowed_tree[i, j] = True
                j = int(parent[b, j])
        mask = np.concatenate([np.ones((n, ctx), dtype=bool), allowed_tree], axis=1)
        for g in range(nkv):
            keys = np.concatenate([k_cache[b, :, g], k_tree[b, :, g]], axis=0)   # [C+n, D]
            vals = np.concatenate([v_cache[b, :, g], v_tree[b, :, g]], axis=0)
            for hh in range(group):
                h = g * group + hh
                s = scale * (q[b, :, h, :] @ keys.T)                             # [n, C+n]
                s = np.where(mask, s, -np.inf)
                mx = np.max(s, axis=1, keepdims=True)
                e = np.exp(s - mx)
                z = np.sum(e, axis=1, keepdims=True)
                out[b, :, h, :] = (e / z) @ vals
                lse[b, :, h] = (mx + np.log(z))[:, 0]
    return out, lse
