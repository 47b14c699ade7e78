"""Pins of the candidate-tree construction (oracle/tree_build.py) and of the
without-replacement tree verify.

Sources: Uno summary (hyper.ai, arXiv 2609.04010), section 方法, last
paragraph (candidates sampled from the marginals, verified as a prefix tree,
losslessly); recursive rejection sampling without replacement (Jeon et al.
2024) for the verifier that goes with siblings drawn without replacement.
"""

import itertools

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle
from _exact_law import explore, emitted_law, _bisect


def test_layout_closed_form():
    parent, depth = oracle.tree_layout([2, 2])
    assert parent.tolist() == [-1, 0, 0, 1, 1, 2, 2]
    assert depth.tolist() == [0, 1, 1, 2, 2, 2, 2]
    for br in ([4, 4, 2], [1, 1, 1, 1], [3], [2, 3, 1, 2]):
        parent, depth = oracle.tree_layout(br)
        assert len(parent) == 1 + sum(int(np.prod(br[:d + 1])) for d in range(len(br)))
        assert all(0 <= parent[v] < v for v in range(1, len(parent)))
        kids = oracle.children_lists(parent)
        for v in range(len(parent)):
            assert len(kids[v]) == (br[depth[v]] if depth[v] < len(br) else 0)
            assert kids[v] == list(range(kids[v][0], kids[v][0] + len(kids[v]))) if kids[v] else True
        assert list(oracle.node_depths(parent)) == depth.tolist()


def _token_of(q_logits, branching, node, u_fixed, without):
    def f(us):
        out = []
        for x in us:
            u = u_fixed.copy()
            u[node] = x
            out.append(oracle.build_tree(q_logits, branching, u, without_replacement=without)[1][node])
        return np.array(out)
    return f


@pytest.mark.parametrize("without", [False, True])
def test_first_draw_has_the_marginal_law(without):
    """The first child of the root takes token v on a u-interval of length q(v)
    (found by bisection on the black-box builder)."""
    rng = np.random.default_rng(1)
    V = 5
    ql = rng.normal(0, 1.5, (2, V))
    q = sp_softmax(ql[0])
    u0 = np.full(7, 0.5)
    f = _token_of(ql, [2, 2], 1, u0, without)
    # the u at which the token first exceeds v, for every v
    cdf = [float(_bisect(lambda us, v=v: f(us) <= v, 1)[0]) for v in range(V)]
    np.testing.assert_allclose(np.diff([0.0] + cdf), q, rtol=0, atol=1e-12)


def test_without_replacement_pair_law():
    """P(t1, t2) = q(t1) q(t2) / (1 - q(t1)) for the root's first two children,
    by bisection on u2 with u1 inside t1's interval; no duplicate siblings."""
    rng = np.random.default_rng(2)
    V = 4
    ql = rng.normal(0, 1.5, (1, V))
    q = sp_softmax(ql[0])
    c = np.concatenate(([0.0], np.cumsum(q)))
    for t1 in range(V):
        u = np.full(1 + 3, 0.5)
        u[1] = 0.5 * (c[t1] + c[t1 + 1])
        f = _token_of(ql, [3], 2, u, True)
        cdf = [float(_bisect(lambda us, v=v: f(us) <= v, 1)[0]) for v in range(V)]
        law = np.diff([0.0] + cdf)
        ref = np.array([q[t] / (1 - q[t1]) if t != t1 else 0.0 for t in range(V)])
        np.testing.assert_allclose(law, ref, rtol=0, atol=1e-12, err_msg=f"t1={t1}")
    for trial in range(200):
        u = rng.random(1 + 3 + 6)
        _, tok = oracle.build_tree(ql[[0, 0]], [3, 2], u, without_replacement=True)
        kids = oracle.children_lists(oracle.tree_layout([3, 2])[0])
        for k in kids:
            if k:
                assert len(set(tok[k].tolist())) == len(k)


def _tree_law_case(parent, vocab, seed, without):
    n = len(parent)
    depth = oracle.node_depths(parent)
    kids = oracle.children_lists(parent)
    dmax = max(depth)
    rng = np.random.default_rng(seed)
    ar = {}
    for j in range(dmax + 1):
        for pre in itertools.product(range(vocab), repeat=j):
            ar[pre] = rng.normal(0.0, 1.5, vocab)
    qlog = rng.normal(0.0, 1.5, (dmax, vocab))
    qprob = sp_softmax(qlog, axis=1)
    assigns, weight = [], []
    for a in itertools.product(range(vocab), repeat=n - 1):
        tok = [0] + list(a)
        w = 1.0
        for v in range(n):
            got = []
            for c in kids[v]:
                qd = qprob[depth[c] - 1]
                if without:
                    if tok[c] in got:
                        w = 0.0
                        break
                    w *= qd[tok[c]] / (1.0 - sum(qd[t] for t in got))
                else:
                    w *= qd[tok[c]]
                got.append(tok[c])
            if w == 0.0:
                break
        if w > 0.0:
            assigns.append(tok)
            weight.append(w)
    tokens = np.array(assigns)
    weight = np.array(weight)

    def path_tokens(tok, node):
        out = []
        while node > 0:
            out.append(int(tok[node]))
            node = parent[node]
        return tuple(reversed(out))

    pl = np.stack([[ar[path_tokens(t, i)] for i in range(n)] for t in tokens])
    ql = np.broadcast_to(qlog, (len(assigns), dmax, vocab)).copy()
    par = np.broadcast_to(parent, (len(assigns), n)).copy()
    return ar, tokens, weight, pl, ql, par


@pytest.mark.parametrize("branching,vocab", [([3], 4), ([2, 2], 3), ([3, 1], 3)])
def test_without_replacement_tree_is_lossless(branching, vocab):
    """Siblings drawn without replacement and verified by the matching
    verifier: the emitted law at every reachable prefix equals the AR law
    (exact, by bisection over every uniform)."""
    parent, _ = oracle.tree_layout(branching)
    ar, tokens, weight, pl, ql, par = _tree_law_case(parent, vocab, 70 + len(parent), True)
    n = len(parent)

    def run(ci, ua, us):
        r = oracle.verify_tree(par[ci], tokens[ci], pl[ci], ql[ci], ua, us, return_visited=True,
                               without_replacement=True)
        out = []
        for b in range(len(ci)):
            L = int(r["accept_len"][b])
            pre = tuple(int(tokens[ci[b], x]) for x in r["path"][b, :L])
            out.append((r["visited"][b], pre, int(r["token"][b])))
        return out

    leaves = explore(len(tokens), run, n, vocab)
    table = emitted_law(leaves, weight, vocab)
    checked = 0
    for pre, (reach, emit) in table.items():
        if reach < 1e-14:
            continue
        np.testing.assert_allclose(emit / reach, sp_softmax(ar[pre]), rtol=0, atol=1e-12, err_msg=f"prefix {pre}")
        checked += 1
    assert checked >= 2


def test_with_replacement_verifier_is_not_lossless_without_replacement():
    """The power of the check above: siblings drawn without replacement but
    verified as if independent give a wrong first-token law."""
    parent, _ = oracle.tree_layout([3])
    ar, tokens, weight, pl, ql, par = _tree_law_case(parent, 4, 74, True)

    def run(ci, ua, us):
        r = oracle.verify_tree(par[ci], tokens[ci], pl[ci], ql[ci], ua, us, return_visited=True)
        return [(r["visited"][b], tuple(int(tokens[ci[b], x]) for x in r["path"][b, :int(r["accept_len"][b])]),
                 int(r["token"][b])) for b in range(len(ci))]

    table = emitted_law(explore(len(tokens), run, len(parent), 4), weight, 4)
    reach, emit = table[()]
    assert np.max(np.abs(emit / reach - sp_softmax(ar[()]))) > 1e-3


def test_build_then_verify_with_replacement_matches_the_iid_law():
    """build_tree (with replacement) feeds verify_tree: the token law of the
    built tree is the i.i.d. law the lossless verify needs (checked on the
    root's children by bisection, as in the first-draw test, for every child)."""
    rng = np.random.default_rng(5)
    V = 4
    ql = rng.normal(0, 1.5, (1, V))
    q = sp_softmax(ql[0])
    for node in (1, 2, 3):
        u0 = np.full(4, 0.37)
        f = _token_of(ql, [3], node, u0, False)
        cdf = [float(_bisect(lambda us, v=v: f(us) <= v, 1)[0]) for v in range(V)]
        np.testing.assert_allclose(np.diff([0.0] + cdf), q, rtol=0, atol=1e-12)


def test_without_replacement_past_the_support_takes_the_smallest_free_id():
    """A q row with all its mass on two tokens (the rest underflows to exactly
    0 in float64): without replacement the first two siblings take those two
    tokens in inverse-CDF order, the next ones the smallest ids not taken yet;
    with replacement every sibling stays inside the support."""
    V = 6
    ql = np.full((1, V), -1.0e4)
    ql[0, 3] = 0.0
    ql[0, 5] = 0.0                      # q = 1/2 on tokens 3 and 5
    u = np.array([0.0, 0.7, 0.9, 0.1, 0.5, 0.2])
    _, tok = oracle.build_tree(ql, [5], u, without_replacement=True)
    assert tok.tolist() == [-1, 5, 3, 0, 1, 2]
    _, tok = oracle.build_tree(ql, [5], u, without_replacement=False)
    assert tok.tolist() == [-1, 5, 5, 3, 5, 3]
