"""GPU parity of the tree verify for siblings drawn without replacement
(uno_psi_spec_verify_tree_wor) against oracle.verify_tree(without_replacement=True).

Source: Uno summary (hyper.ai, arXiv 2609.04010), section 方法, last
paragraph (lossless tree verify); the without-replacement rule is recursive
rejection sampling without replacement (Jeon et al. 2024), pinned in the
oracle by the exhaustive emitted law of built trees.  Bar: accepted length,
path and token bit-exact unless the oracle reaches the GPU's outcome with one
visited uniform moved by at most 1e-5 (a near-tie, counted)."""

import numpy as np
import pytest

import oracle
import workloads
from _parity import say, to_dev, to_host, tree_outcome_near, check_tree_build

pytestmark = pytest.mark.gpu

FULL_V = 151936


def _verify(dad, parent, tokens, p, q, ua, us, temperature=1.0, max_children=None):
    import torch
    out = dad.psi_spec_verify_tree(to_dev(np.asarray(parent, np.int32)), to_dev(np.asarray(tokens, np.int32)),
                                   to_dev(p), to_dev(q), to_dev(np.asarray(ua, np.float32)),
                                   to_dev(np.asarray(us, np.float32)), temperature, max_children=max_children,
                                   without_replacement=True)
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in out.items()}


def _check(parent, tokens, p32, q32, ua, us, g, temperature=1.0):
    ties = 0
    for b in range(parent.shape[0]):
        r = oracle.verify_tree(parent[b:b + 1], tokens[b:b + 1], p32[b:b + 1], q32[b:b + 1], ua[b:b + 1],
                               us[b:b + 1], temperature, without_replacement=True)
        Lo, Lg = int(r["accept_len"][0]), int(g["accept_len"][b])
        same = (Lo == Lg and list(r["path"][0]) == list(g["path"][b]) and int(r["token"][0]) == int(g["token"][b]))
        if not same:
            assert tree_outcome_near(parent[b], tokens[b], p32[b], q32[b], ua[b], float(us[b]), temperature,
                                     (Lg, list(g["path"][b]), int(g["token"][b])), without=True), \
                f"tree {b}: gpu L={Lg} path={list(g['path'][b])} y={int(g['token'][b])}, oracle L={Lo} " \
                f"path={list(r['path'][0])} y={int(r['token'][0])}"
            ties += 1
    return ties


def _built_case(batch, branching, vocab, dtype, seed, q_std, temperature=1.0, node_std=0.5):
    """Trees built by the oracle without replacement from the case's q.  A
    large node_std makes the AR rows nearly independent of the draft rows
    (long rejection chains)."""
    c = workloads.tree_build_case(batch, branching, vocab, dtype, seed=seed, q_std=q_std, node_std=node_std)
    parent, _ = oracle.tree_layout(branching)
    toks = np.stack([oracle.build_tree(c["q_f32"][b], branching, c["u_draw"][b], temperature, True)[1]
                     for b in range(batch)])
    c["parent"] = np.tile(parent.astype(np.int32), (batch, 1))
    c["tokens"] = np.where(toks < 0, 0, toks).astype(np.int32)      # the root's entry is unused
    return c


@pytest.mark.parametrize("batch,branching,vocab,dtype,q_std,node_std", [
    (3, [4, 2, 2], 1000, "f32", 0.5, 0.5),
    (3, [4, 2, 2], 1000, "f32", 2.0, 0.5),
    (2, [3, 3], 8193, "bf16", 1.0, 0.5),
    (2, [8, 4], 5000, "bf16", 2.0, 0.5),
    (2, [64], 100, "f32", 2.0, 0.5),
    (1, [2] * 6, 300, "f32", 3.0, 0.5),
    (16, [3, 2], 257, "bf16", 1.5, 0.5),
    (4, [64], 1000, "f32", 1.0, 4.0),      # chains of 64 rejections
    (8, [16, 2], 2000, "bf16", 0.5, 2.5),  # chains of 16 rejections
])
def test_verify_wor_matches_oracle(gpu_lib, batch, branching, vocab, dtype, q_std, node_std):
    say(f"tree verify wor {branching} V={vocab} {dtype} q_std={q_std} node_std={node_std}")
    c = _built_case(batch, branching, vocab, dtype, seed=vocab + len(branching), q_std=q_std, node_std=node_std)
    g = _verify(gpu_lib, c["parent"], c["tokens"], c["p"], c["q"], c["u_acc"], c["u_s"],
                max_children=max(branching))
    say(f"  L = {g['accept_len'].tolist()}")
    assert _check(c["parent"], c["tokens"], c["p_f32"], c["q_f32"], c["u_acc"], c["u_s"], g) <= 1


@pytest.mark.parametrize("branching,vocab,tree", [([64], 1000, 0), ([16, 2], 2000, 2)])
def test_verify_wor_residual_on_a_uniform_grid(gpu_lib, branching, vocab, tree):
    """One tree whose walk rejects every child of the root (or of a node),
    copied 128 times with u_sample on a grid: the draws trace the inverse
    CDF of the final residual, removed tokens' weights included, at 128
    points.  On this tree the with-replacement residual differs from the
    without-replacement one at some of the points, so the check separates
    the two rules."""
    c = _built_case(4, branching, vocab, "f32", seed=7, q_std=1.0 if branching == [64] else 0.5,
                    node_std=4.0 if branching == [64] else 2.5)
    k = 128
    rep = {key: np.repeat(c[key][tree:tree + 1], k, axis=0) for key in ("parent", "tokens", "p", "p_f32", "q",
                                                                       "q_f32", "u_acc")}
    us = ((np.arange(k) + 0.5) / k).astype(np.float32)
    say(f"tree verify wor residual grid {branching} V={vocab}")
    g = _verify(gpu_lib, rep["parent"], rep["tokens"], rep["p"], rep["q"], rep["u_acc"], us,
                max_children=max(branching))
    assert _check(rep["parent"], rep["tokens"], rep["p_f32"], rep["q_f32"], rep["u_acc"], us, g) <= 2
    sep = 0
    for i in range(k):
        a = oracle.verify_tree(rep["parent"][:1], rep["tokens"][:1], rep["p_f32"][:1], rep["q_f32"][:1],
                               rep["u_acc"][:1], us[i:i + 1], without_replacement=True)
        w = oracle.verify_tree(rep["parent"][:1], rep["tokens"][:1], rep["p_f32"][:1], rep["q_f32"][:1],
                               rep["u_acc"][:1], us[i:i + 1])
        sep += int(a["token"][0]) != int(w["token"][0])
    assert sep > 0


def test_verify_wor_full_vocabulary(gpu_lib):
    """V = 151,936 bf16, 69-node trees (4, 4, 3 children per level), 4 trees,
    at two draft spreads."""
    ties = 0
    for q_std in (0.5, 2.0):
        say(f"tree verify wor full V q_std={q_std}")
        c = _built_case(4, [4, 4, 3], FULL_V, "bf16", seed=21, q_std=q_std)
        g = _verify(gpu_lib, c["parent"], c["tokens"], c["p"], c["q"], c["u_acc"], c["u_s"], max_children=4)
        ties += _check(c["parent"], c["tokens"], c["p_f32"], c["q_f32"], c["u_acc"], c["u_s"], g)
    assert ties <= 1


def test_verify_wor_repeated_tokens_and_any_parent(gpu_lib):
    """Trees that are not breadth first, with i.i.d. tokens (repeats among
    siblings): a repeated token is tested with no draft mass left for it."""
    ties = 0
    for s in range(3):
        parent = workloads.random_parent(40, s)
        c = workloads.tree_verify_case(parent, 50, dtype="f32", seed=30 + s, q_std=1.0, batch=3)
        g = _verify(gpu_lib, c["parent"], c["tokens"], c["p"], c["q"], c["u_acc"], c["u_s"],
                    max_children=workloads.max_children(parent))
        ties += _check(c["parent"], c["tokens"], c["p_f32"], c["q_f32"], c["u_acc"], c["u_s"], g)
    assert ties <= 1


def test_verify_wor_draft_support_exhausted(gpu_lib):
    """q on tokens 3 and 5 only; the root's children carry 5, 3, 0, 1, 2.
    Once 5 and 3 are removed no draft mass is left: the later children are
    tested with q = 0 (accepted iff the residual has mass at their token)."""
    V = 6
    neg = -1.0e4
    ql = np.full((1, 1, V), neg, np.float32)
    ql[0, 0, [3, 5]] = 0.0
    parent = np.array([[-1, 0, 0, 0, 0, 0]], np.int32)
    tokens = np.array([[0, 5, 3, 0, 1, 2]], np.int32)
    for p_mass, want_path in (({3: 0.5, 4: 0.5}, []), ({0: 0.2, 3: 0.4, 4: 0.4}, [3])):
        pl = np.full((1, 6, V), neg, np.float32)
        for t, m in p_mass.items():
            pl[0, :, t] = np.log(m)
        ua = np.full((1, 6), 0.5, np.float32)
        us = np.array([0.3], np.float32)
        g = _verify(gpu_lib, parent, tokens, pl, ql, ua, us, max_children=5)
        r = oracle.verify_tree(parent, tokens, pl.astype(np.float64), ql.astype(np.float64), ua, us,
                               without_replacement=True)
        assert [int(x) for x in r["path"][0][:int(r["accept_len"][0])]] == want_path
        assert int(g["accept_len"][0]) == int(r["accept_len"][0])
        assert g["path"][0].tolist() == r["path"][0].tolist()
        assert int(g["token"][0]) == int(r["token"][0])


def test_verify_wor_malformed_and_limits(gpu_lib):
    import diffusion_augmented_decoding_amd as dad
    c = _built_case(2, [3, 2], 200, "f32", seed=4, q_std=1.0)
    c["parent"][1, 4] = 6                       # not an earlier node
    g = _verify(gpu_lib, c["parent"], c["tokens"], c["p"], c["q"], c["u_acc"], c["u_s"], max_children=3)
    assert g["accept_len"][1] == -1 and g["token"][1] == -1 and np.all(g["path"][1] == -1)
    assert _check(c["parent"][:1], c["tokens"][:1], c["p_f32"][:1], c["q_f32"][:1], c["u_acc"][:1], c["u_s"][:1],
                  {k: v[:1] for k, v in g.items()}) == 0
    with pytest.raises(RuntimeError):
        _verify(gpu_lib, c["parent"], c["tokens"], c["p"], c["q"], c["u_acc"], c["u_s"], max_children=65)


def test_build_then_verify_on_the_gpu(gpu_lib):
    """The decode-side pair: trees built on the GPU without replacement, then
    verified without replacement.  The built tokens are checked against
    oracle.build_tree first (equal up to counted near-ties of a draw, u
    within 1e-5 of a CDF boundary); the verify is then checked against the
    oracle on the GPU's own trees."""
    import torch
    branching = [4, 4, 3]
    c = workloads.tree_build_case(4, branching, 30000, "bf16", seed=9, q_std=1.0)
    q = to_dev(c["q"])
    built = gpu_lib.psi_spec_build_tree(q, branching, to_dev(c["u_draw"]), 1.0, True)
    torch.cuda.synchronize()
    par, tok = to_host(built["parent"]), to_host(built["tokens"])
    ties = check_tree_build(c["q_f32"], branching, c["u_draw"], par, tok, 1.0, True)
    say(f"build near-ties: {ties} of {tok.shape[0] * (tok.shape[1] - 1)} draws")
    assert ties <= 2
    toks = tok.copy()
    toks[:, 0] = 0
    g = gpu_lib.psi_spec_verify_tree(built["parent"], torch.from_numpy(toks).to("cuda"), to_dev(c["p"]), q,
                                     to_dev(c["u_acc"]), to_dev(c["u_s"]), 1.0, max_children=4,
                                     without_replacement=True)
    torch.cuda.synchronize()
    g = {k: to_host(v) for k, v in g.items()}
    ref = _built_case(4, branching, 30000, "bf16", seed=9, q_std=1.0)
    if ties == 0:
        assert np.array_equal(ref["tokens"], toks)
    # the verify is checked on the trees the GPU built (they differ from the
    # oracle's own only at a counted near-tie of a draw)
    assert _check(par, toks, ref["p_f32"], ref["q_f32"], ref["u_acc"], ref["u_s"], g) <= 1


def test_verify_wor_is_deterministic(gpu_lib):
    c = _built_case(4, [8, 4], 20000, "bf16", seed=12, q_std=2.0)
    a = _verify(gpu_lib, c["parent"], c["tokens"], c["p"], c["q"], c["u_acc"], c["u_s"], max_children=8)
    b = _verify(gpu_lib, c["parent"], c["tokens"], c["p"], c["q"], c["u_acc"], c["u_s"], max_children=8)
    for k in a:
        assert np.array_equal(a[k], b[k])
