"""GPU parity: uno_tree_verify_attention and uno_psi_spec_verify_tree.

Attention bar: per (node, head) row, ||o - o_ref||_inf / ||o_ref||_inf <= 2e-2
(bf16 output); LSE (fp32) within 1e-5 * max(1, |lse|): the log-sum-exp carries
the absolute rounding of the fp32 scores (~|s| 2^-24 sqrt(head_dim)), so the
fp32 relative bound is taken with a floor of 1 for values near zero.  Tree verify bar: accepted
length, path and token bit-exact unless the oracle reaches the GPU's outcome
with one visited uniform moved by at most 1e-5 (a near-tie, counted).
"""

import numpy as np
import pytest

import oracle
import workloads
from _parity import row_relerr, say, to_dev, to_host, tree_outcome_near

pytestmark = pytest.mark.gpu


def _attn(dad, c):
    import torch
    out, lse = dad.tree_verify_attention(to_dev(c["q"]), to_dev(c["k_cache"]), to_dev(c["v_cache"]),
                                         to_dev(c["k_tree"]), to_dev(c["v_tree"]),
                                         to_dev(c["parent"].astype(np.int32)), c["scale"])
    torch.cuda.synchronize()
    return to_host(out), to_host(lse)


def _check_lse(lse, ref):
    err = np.abs(lse - ref) / np.maximum(1.0, np.abs(ref))
    assert np.max(err) <= 1e-5, f"lse err {np.max(err):.3g}"


def _attn_ref(c):
    return oracle.tree_attention(c["q_f32"], c["k_cache_f32"], c["v_cache_f32"], c["k_tree_f32"],
                                 c["v_tree_f32"], c["parent"], c["scale"])


def test_attention_tree_workload(gpu_lib):
    """Root + 64 candidates (branching 4, depth 3), 1K-token cache, GQA 32/8."""
    say("tree attention n=65 ctx=1024 H=32/8")
    parent = workloads.tree_parent_cfg(0)
    c = workloads.tree_attention_case(1, parent, 1024, 32, 8, 128, seed=0)
    o, lse = _attn(gpu_lib, c)
    ro, rl = _attn_ref(c)
    err = row_relerr(o, ro)
    say(f"  row rel err {err:.3g}")
    assert err <= 2e-2
    _check_lse(lse, rl)


@pytest.mark.parametrize("name,n,ctx,nh,nkv,batch", [
    ("chain", 9, 37, 8, 2, 1),
    ("star", 40, 64, 4, 4, 2),          # G = 1
    ("random", 100, 5, 16, 2, 2),       # G = 8
    ("cfg", 65, 0, 32, 8, 1),           # no cache at all
    ("single", 1, 200, 32, 8, 3),       # plain decode attention
    ("random", 256, 96, 8, 8, 1),       # largest tree
    ("random", 256, 40, 32, 4, 3),      # enough query tiles for one key split per tile
    ("single", 1, 3000, 8, 1, 1),       # long cache, many key splits
])
def test_attention_shapes(gpu_lib, name, n, ctx, nh, nkv, batch):
    say(f"tree attention {name} n={n} ctx={ctx} H={nh}/{nkv} B={batch}")
    if name == "chain":
        parent = workloads.chain_parent(n)
    elif name == "star":
        parent = workloads.star_parent(n)
    elif name == "cfg":
        parent = workloads.tree_parent_cfg(3)
    elif name == "single":
        parent = np.array([-1], np.int32)
    else:
        parent = np.stack([workloads.random_parent(n, s) for s in range(batch)])
    c = workloads.tree_attention_case(batch, parent, ctx, nh, nkv, 128, seed=n + ctx)
    o, lse = _attn(gpu_lib, c)
    ro, rl = _attn_ref(c)
    assert row_relerr(o, ro) <= 2e-2
    _check_lse(lse, rl)


def test_attention_malformed_tree_gives_nan(gpu_lib):
    say("tree attention malformed parent")
    parent = workloads.chain_parent(6)
    parent[3] = 4                         # parent after child: invalid
    c = workloads.tree_attention_case(1, parent, 16, 8, 2, 128, seed=1)
    o, lse = _attn(gpu_lib, c)
    assert np.all(np.isnan(o)) and np.all(np.isnan(lse))


def _verify(dad, c, max_children=None):
    import torch
    if max_children is None:
        max_children = workloads.max_children(c["parent"])
    out = dad.psi_spec_verify_tree(to_dev(c["parent"].astype(np.int32)), to_dev(c["tokens"]), to_dev(c["p"]),
                                   to_dev(c["q"]), to_dev(c["u_acc"]), to_dev(c["u_s"]), c["temperature"],
                                   max_children=max_children)
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in out.items()}


def _check_verify(c, g):
    ties = 0
    for b in range(c["batch"]):
        r = oracle.verify_tree(c["parent"][b:b + 1], c["tokens"][b:b + 1], c["p_f32"][b:b + 1],
                               c["q_f32"][b:b + 1], c["u_acc"][b:b + 1], c["u_s"][b:b + 1], c["temperature"])
        Lo, Lg = int(r["accept_len"][0]), int(g["accept_len"][b])
        same = (Lo == Lg and list(r["path"][0]) == list(g["path"][b]) and int(r["token"][0]) == int(g["token"][b]))
        if not same:
            assert tree_outcome_near(c["parent"][b], c["tokens"][b], c["p_f32"][b], c["q_f32"][b], c["u_acc"][b],
                                     float(c["u_s"][b]), c["temperature"],
                                     (Lg, list(g["path"][b]), int(g["token"][b]))), f"batch {b}"
            ties += 1
    return ties


def test_verify_tree_workload(gpu_lib):
    """Per-node rejection over the 65-node tree at vocab 151,936 (bf16)."""
    say("tree verify n=65 V=151936")
    parent = workloads.tree_parent_cfg(0)
    c = workloads.tree_verify_case(parent, 151936, dtype="bf16", seed=0, batch=2)
    g = _verify(gpu_lib, c)
    say(f"  L = {g['accept_len']}, path = {g['path']}, y = {g['token']}")
    assert _check_verify(c, g) <= 1


@pytest.mark.parametrize("shape,vocab,dtype,seed", [
    ("chain", 1000, "f32", 1),
    ("cfg", 5000, "bf16", 2),
    ("star", 777, "bf16", 3),
    ("random", 20000, "f32", 4),
    ("wide_random", 3000, "bf16", 5),
])
def test_verify_tree_shapes(gpu_lib, shape, vocab, dtype, seed):
    say(f"tree verify {shape} V={vocab} {dtype}")
    parent = {"chain": workloads.chain_parent(6), "cfg": workloads.tree_parent_cfg(seed),
              "star": workloads.star_parent(30), "random": workloads.random_parent(40, seed),
              "wide_random": workloads.random_parent(500, seed)}[shape]
    ties = 0
    for q_std in (0.1, 0.5, 2.0):
        c = workloads.tree_verify_case(parent, vocab, dtype=dtype, seed=seed, q_std=q_std, batch=3)
        g = _verify(gpu_lib, c)
        ties += _check_verify(c, g)
    assert ties <= 1


def test_verify_tree_malformed(gpu_lib):
    say("tree verify malformed parent")
    parent = workloads.chain_parent(5)
    c = workloads.tree_verify_case(parent, 100, dtype="f32", seed=1)
    c["parent"][0, 2] = 3
    g = _verify(gpu_lib, c, max_children=1)
    assert g["accept_len"][0] == -1 and g["token"][0] == -1 and np.all(g["path"][0] == -1)


def test_verify_tree_more_children_than_declared(gpu_lib):
    say("tree verify max_children below the tree's branching")
    c = workloads.tree_verify_case(workloads.star_parent(6), 300, dtype="f32", seed=2, batch=2)
    g = _verify(gpu_lib, c, max_children=3)
    assert np.all(g["accept_len"] == -1) and np.all(g["token"] == -1)
    g = _verify(gpu_lib, c, max_children=5)
    assert _check_verify(c, g) <= 1


def test_verify_tree_batch_of_different_trees(gpu_lib):
    say("tree verify batch of different trees, one malformed")
    parents = np.stack([workloads.random_parent(30, s) for s in range(4)])
    cs = [workloads.tree_verify_case(parents[b], 2000, dtype="bf16", seed=10 + b) for b in range(4)]
    c = {k: np.concatenate([x[k] for x in cs]) for k in ("parent", "tokens", "p", "p_f32", "u_acc", "u_s")}
    dmax = max(x["max_depth"] for x in cs)
    for k in ("q", "q_f32"):      # pad the per-depth draft rows to a common depth
        c[k] = np.concatenate([np.pad(x[k], ((0, 0), (0, dmax - x["max_depth"]), (0, 0))) for x in cs])
    c.update(batch=4, temperature=1.0)
    c["parent"][3, 5] = 7         # malformed third tree
    g = _verify(gpu_lib, c, max_children=workloads.max_children(parents))
    assert g["accept_len"][3] == -1
    good = {k: (v[:3] if isinstance(v, np.ndarray) else v) for k, v in c.items()}
    good["batch"] = 3
    assert _check_verify(good, {k: v[:3] for k, v in g.items()}) <= 1


def test_tree_handworked_golden_cases(gpu_lib):
    """The hand-worked trees of tests/golden/verify_tree_handworked.json
    (ascending sibling order, a duplicate sibling rejected by the residual,
    every child rejected, the second depth's marginal) through the HIP
    kernels with fp32 logits ln(p): accepted length, path and token exactly
    as worked by hand."""
    import json
    import os
    import torch
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "verify_tree_handworked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        say(f"tree golden {c['name']}")
        parent = np.asarray([c["parent"]], np.int32)
        pl = np.log(np.maximum(np.array(c["p"]), 1e-300)).astype(np.float32)[None]
        ql = np.log(np.maximum(np.array(c["q"]), 1e-300)).astype(np.float32)[None]
        out = gpu_lib.psi_spec_verify_tree(to_dev(parent), to_dev(np.asarray([c["tokens"]], np.int32)), to_dev(pl),
                                           to_dev(ql), to_dev(np.asarray([c["u_accept"]], np.float32)),
                                           to_dev(np.asarray([c["u_sample"]], np.float32)),
                                           max_children=workloads.max_children(parent))
        torch.cuda.synchronize()
        e = c["expect"]
        L = int(to_host(out["accept_len"])[0])
        assert L == e["accept_len"], c["name"]
        assert list(to_host(out["path"])[0, :L]) == e["path"], c["name"]
        assert int(to_host(out["token"])[0]) == e["token"], c["name"]
