"""Pins of the tree oracles: tree-masked attention and per-node tree verify.

Source: Uno summary (hyper.ai, arXiv 2609.04010), section 方法, last paragraph:
the tree sampler samples several candidates and verifies them concurrently as
a prefix tree with tree attention; lossless in both the linear and the tree
case.
"""

import itertools

import numpy as np
import pytest
import torch
from scipy.special import softmax as sp_softmax

import oracle
import workloads
from _exact_law import explore, emitted_law


def _sdpa_reference(q, keys, vals, mask, scale):
    """torch CPU float64 scaled_dot_product_attention with a boolean mask.
    q [H, n, D]; keys/vals [H, C+n, D]; mask [n, C+n] (True = attend)."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(keys), torch.from_numpy(vals),
        attn_mask=torch.from_numpy(mask), scale=scale)
    return out.numpy()


def _case(parent, ctx=9, nh=4, nkv=2, hd=8, seed=0):
    c = workloads.tree_attention_case(1, parent, ctx, nh, nkv, hd, seed=seed)
    return c


def _expand_kv(x, group):
    # [C, Hkv, D] -> [H, C, D], query head h reads kv head h // group
    return np.repeat(x.transpose(1, 0, 2), group, axis=0).astype(np.float64)


@pytest.mark.parametrize("shape", ["chain", "star", "cfg", "random"])
def test_loop_form_matches_dense_mask_form(shape):
    n = 13
    parent = {"chain": workloads.chain_parent(n), "star": workloads.star_parent(n),
              "cfg": workloads.tree_parent_cfg(0, branching=3, depth=2, n_last=5),
              "random": workloads.random_parent(n, 5)}[shape]
    c = _case(parent)
    args = (c["q_f32"], c["k_cache_f32"], c["v_cache_f32"], c["k_tree_f32"], c["v_tree_f32"], c["parent"], c["scale"])
    o1, l1 = oracle.tree_attention(*args)
    o2, l2 = oracle.tree_attention_dense_mask(*args)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-13)


def test_chain_tree_is_causal_attention():
    n, ctx, nh, nkv, hd = 7, 11, 4, 2, 8
    c = _case(workloads.chain_parent(n), ctx, nh, nkv, hd, seed=1)
    o, _ = oracle.tree_attention(c["q_f32"], c["k_cache_f32"], c["v_cache_f32"], c["k_tree_f32"],
                                 c["v_tree_f32"], c["parent"], c["scale"])
    keys = np.concatenate([_expand_kv(c["k_cache_f32"][0], nh // nkv), _expand_kv(c["k_tree_f32"][0], nh // nkv)], 1)
    vals = np.concatenate([_expand_kv(c["v_cache_f32"][0], nh // nkv), _expand_kv(c["v_tree_f32"][0], nh // nkv)], 1)
    mask = np.concatenate([np.ones((n, ctx), bool), np.tril(np.ones((n, n), bool))], axis=1)
    ref = _sdpa_reference(c["q_f32"][0].transpose(1, 0, 2).astype(np.float64), keys, vals, mask, c["scale"])
    np.testing.assert_allclose(o[0], ref.transpose(1, 0, 2), rtol=1e-10, atol=1e-12)


def test_single_node_is_decode_attention_and_lse():
    ctx, nh, nkv, hd = 20, 8, 2, 16
    c = _case(np.array([-1], np.int32), ctx, nh, nkv, hd, seed=2)
    o, lse = oracle.tree_attention(c["q_f32"], c["k_cache_f32"], c["v_cache_f32"], c["k_tree_f32"],
                                   c["v_tree_f32"], c["parent"], c["scale"])
    keys = np.concatenate([_expand_kv(c["k_cache_f32"][0], 4), _expand_kv(c["k_tree_f32"][0], 4)], 1)
    vals = np.concatenate([_expand_kv(c["v_cache_f32"][0], 4), _expand_kv(c["v_tree_f32"][0], 4)], 1)
    q = c["q_f32"][0].transpose(1, 0, 2).astype(np.float64)
    ref = _sdpa_reference(q, keys, vals, np.ones((1, ctx + 1), bool), c["scale"])
    np.testing.assert_allclose(o[0], ref.transpose(1, 0, 2), rtol=1e-10, atol=1e-12)
    s = torch.from_numpy(c["scale"] * np.einsum("hd,hcd->hc", q[:, 0], keys))
    np.testing.assert_allclose(lse[0, 0], torch.logsumexp(s, dim=1).numpy(), rtol=1e-13)


def test_star_tree_sees_cache_root_and_self():
    n, ctx, nh, nkv, hd = 6, 5, 2, 1, 8
    c = _case(workloads.star_parent(n), ctx, nh, nkv, hd, seed=3)
    o, _ = oracle.tree_attention(c["q_f32"], c["k_cache_f32"], c["v_cache_f32"], c["k_tree_f32"],
                                 c["v_tree_f32"], c["parent"], c["scale"])
    for i in range(1, n):
        sub = [0, i]
        o2, _ = oracle.tree_attention(c["q_f32"][:, [i]], c["k_cache_f32"], c["v_cache_f32"],
                                      c["k_tree_f32"][:, sub], c["v_tree_f32"][:, sub],
                                      np.array([[-1, 0]]), c["scale"])
        # node i with keys [cache, root, self] == the same query as node 1 of a 2-chain
        keys = np.concatenate([c["k_cache_f32"][0, :, 0], c["k_tree_f32"][0, sub, 0]]).astype(np.float64)
        vals = np.concatenate([c["v_cache_f32"][0, :, 0], c["v_tree_f32"][0, sub, 0]]).astype(np.float64)
        for h in range(nh):
            sc = c["scale"] * keys @ c["q_f32"][0, i, h].astype(np.float64)
            np.testing.assert_allclose(o[0, i, h], sp_softmax(sc) @ vals, rtol=1e-11, atol=1e-13)


def test_cache_permutation_invariance():
    parent = workloads.tree_parent_cfg(0, branching=2, depth=3, n_last=6)
    c = _case(parent, ctx=16, seed=4)
    args = [c["q_f32"], c["k_cache_f32"], c["v_cache_f32"], c["k_tree_f32"], c["v_tree_f32"], c["parent"], c["scale"]]
    o1, l1 = oracle.tree_attention(*args)
    perm = np.random.default_rng(0).permutation(16)
    args[1] = c["k_cache_f32"][:, perm]
    args[2] = c["v_cache_f32"][:, perm]
    o2, l2 = oracle.tree_attention(*args)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


# ------------------------------------------------------------------ tree verify
def test_branching_one_equals_linear_sampler():
    k, v = 5, 200
    lin = workloads.verify_linear_case(8, k, v, 0.8, dtype="f32", seed=11, workers=1)
    parent = workloads.chain_parent(k + 1)
    for b in range(8):
        tokens = np.concatenate([[0], lin["drafts"][b]])[None]
        u_acc = np.concatenate([[0.0], lin["u_acc"][b]])[None]
        r = oracle.verify_tree(parent[None], tokens, lin["p_f32"][b][None], lin["q_f32"][b][None],
                               u_acc, lin["u_s"][b:b + 1])
        rl = oracle.verify_linear(lin["p_f32"][b:b + 1], lin["q_f32"][b:b + 1], lin["drafts"][b:b + 1],
                                  lin["u_acc"][b:b + 1], lin["u_s"][b:b + 1])
        assert r["accept_len"][0] == rl["accept_len"][0]
        assert r["token"][0] == rl["token"][0]
        L = rl["accept_len"][0]
        assert list(r["path"][0, :L]) == list(range(1, L + 1))


def test_identical_marginal_chain_accepts_all():
    k, v = 4, 50
    rng = np.random.default_rng(3)
    pl = rng.normal(size=(1, k + 1, v))
    ql = pl[:, :k].copy()
    parent = workloads.chain_parent(k + 1)[None]
    tokens = np.concatenate([[0], rng.integers(0, v, k)])[None]
    r = oracle.verify_tree(parent, tokens, pl, ql, np.full((1, k + 1), 0.9999), np.array([0.3]))
    assert r["accept_len"][0] == k


TREES = {
    "star3": np.array([-1, 0, 0, 0]),
    "two_chains": np.array([-1, 0, 0, 1, 2]),
    "fork_below": np.array([-1, 0, 1, 1]),
}


@pytest.mark.parametrize("name,vocab", [("star3", 3), ("two_chains", 3), ("fork_below", 4)])
def test_exhaustive_tree_law_equals_ar(name, vocab):
    """Siblings i.i.d. from the per-depth marginal; the emitted law at every
    position, given the emitted prefix, equals the AR distribution."""
    parent = TREES[name]
    n = len(parent)
    depth = oracle.node_depths(parent)
    dmax = max(depth)
    rng = np.random.default_rng(50 + n)
    ar = {}
    for j in range(dmax + 1):
        for pre in itertools.product(range(vocab), repeat=j):
            ar[pre] = rng.normal(0.0, 1.5, vocab)
    qlog = rng.normal(0.0, 1.5, (dmax, vocab))
    qprob = sp_softmax(qlog, axis=1)
    assigns = list(itertools.product(range(vocab), repeat=n - 1))
    tokens = np.array([[0] + list(a) for a in assigns])
    weight = np.array([np.prod([qprob[depth[i + 1] - 1, a[i]] for i in range(n - 1)]) for a in assigns])

    def path_tokens(tok, node):
        out = []
        while node > 0:
            out.append(int(tok[node]))
            node = parent[node]
        return tuple(reversed(out))

    pl = np.stack([[ar[path_tokens(t, i)] for i in range(n)] for t in tokens])
    ql = np.broadcast_to(qlog, (len(assigns), dmax, vocab)).copy()
    par = np.broadcast_to(parent, (len(assigns), n)).copy()

    def run(ci, ua, us):
        r = oracle.verify_tree(par[ci], tokens[ci], pl[ci], ql[ci], ua, us, return_visited=True)
        out = []
        for b in range(len(ci)):
            L = int(r["accept_len"][b])
            pre = tuple(int(tokens[ci[b], x]) for x in r["path"][b, :L])
            out.append((r["visited"][b], pre, int(r["token"][b])))
        return out

    leaves = explore(len(assigns), run, n, vocab)
    for c in range(len(assigns)):
        assert abs(sum(w for w, _, _ in leaves[c]) - 1.0) < 1e-12
    table = emitted_law(leaves, weight, vocab)
    checked = 0
    for pre, (reach, emit) in table.items():
        if reach < 1e-14:
            continue
        np.testing.assert_allclose(emit / reach, sp_softmax(ar[pre]), rtol=0, atol=1e-12,
                                   err_msg=f"{name} prefix {pre}")
        checked += 1
    assert checked >= 2


def test_handworked_tree_golden_cases():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "verify_tree_handworked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        pl = np.log(np.maximum(np.array(c["p"]), 1e-300))[None]
        ql = np.log(np.maximum(np.array(c["q"]), 1e-300))[None]
        r = oracle.verify_tree(np.array([c["parent"]]), np.array([c["tokens"]]), pl, ql,
                               np.array([c["u_accept"]]), np.array([c["u_sample"]]))
        e = c["expect"]
        L = e["accept_len"]
        assert r["accept_len"][0] == L, c["name"]
        assert list(r["path"][0, :L]) == e["path"], c["name"]
        assert r["token"][0] == e["token"], c["name"]
