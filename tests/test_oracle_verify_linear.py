"""Pins of the linear Psi-Spec verify oracle.

Sources: Uno summary (hyper.ai, arXiv 2609.04010), section 方法, last
paragraph (rejection sampling against the AR distribution, longest valid
prefix, first token from the AR weights); ainews.surl.tw article ("lossless"
= samples follow the AR distribution); 4sapi.net recap of speculative
decoding (accept the consecutive correct prefix, back off at the first error).
"""

import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax, logsumexp

import oracle
import workloads
from _exact_law import explore, emitted_law

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------- golden
def test_handworked_golden_cases():
    with open(os.path.join(HERE, "golden", "verify_linear_handworked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        pl = np.log(np.array(c["p"]))[None]
        ql = np.log(np.array(c["q"]))[None]
        r = oracle.verify_linear(pl, ql, np.array([c["drafts"]]), np.array([c["u_accept"]]),
                                 np.array([c["u_sample"]]))
        e = c["expect"]
        assert r["accept_len"][0] == e["accept_len"], c["name"]
        assert r["token"][0] == e["token"], c["name"]
        np.testing.assert_allclose(r["p_draft"][0], e["p_draft"], rtol=1e-12)
        np.testing.assert_allclose(r["q_draft"][0], e["q_draft"], rtol=1e-12)
        np.testing.assert_allclose(r["residual_mass"][0], e["residual_mass"], rtol=1e-12)


# ---------------------------------------------------------------- S5 stats
def test_row_stats_match_logsumexp():
    rng = np.random.default_rng(0)
    x = rng.normal(0, 3, size=(5, 1000)).astype(np.float32)
    for t in (1.0, 0.7, 2.5):
        m, z = oracle.row_log_stats(x, t)
        np.testing.assert_allclose(m + np.log(z), logsumexp(x.astype(np.float64) / t, axis=1),
                                   rtol=1e-14, atol=1e-12)
        np.testing.assert_allclose(oracle.softmax_rows(x, t), sp_softmax(x.astype(np.float64) / t, axis=1),
                                   rtol=1e-12, atol=1e-300)


# ---------------------------------------------------------------- S1
def test_identical_draft_and_target_accept_everything():
    c = workloads.verify_linear_case(6, 5, 300, 0.5, dtype="bf16", seed=2, workers=1)
    p = c["p_f32"]
    q = p[:, :5].copy()                         # q_i = p_i exactly
    u = np.full((6, 5), np.nextafter(np.float32(1.0), np.float32(0.0)), dtype=np.float32)
    for uu in (u, c["u_acc"]):
        r = oracle.verify_linear(p, q, c["drafts"], uu, c["u_s"])
        assert np.all(r["accept_len"] == 5)


# ---------------------------------------------------------------- S3
def test_one_hot_target_rejects_all_other_drafts():
    v, k = 6, 3
    pl = np.full((1, k + 1, v), -1e4)
    pl[0, :, 4] = 0.0                           # p is a point mass at token 4
    ql = np.random.default_rng(1).normal(size=(1, k, v))
    drafts = np.array([[1, 2, 3]])
    for us in (0.0, 0.37, 0.999):
        r = oracle.verify_linear(pl, ql, drafts, np.array([[0.0, 0.0, 0.0]]), np.array([us]))
        assert r["accept_len"][0] == 0 and r["token"][0] == 4


def test_one_hot_draft_accept_probability_and_residual():
    """q one-hot at d: P(accept) = p(d); residual = p without d, renormalised."""
    v = 5
    p = np.array([0.1, 0.25, 0.3, 0.15, 0.2])
    pl = np.log(p)[None, None].repeat(2, axis=1)
    ql = np.full((1, 1, v), -1e4)
    ql[0, 0, 2] = 0.0
    drafts = np.array([[2]])
    leaves = explore(1, lambda ci, ua, us: [
        ([(0, True)] if r_ == 1 else [(0, False)], (2,) if r_ == 1 else (), y_)
        for r_, y_ in zip(*_run_lin(pl, ql, drafts, ci, ua, us))], 1, v)
    acc = sum(w for w, pre, _ in leaves[0] if pre == (2,))
    assert abs(acc - 0.3) < 1e-13
    rej = [py for w, pre, py in leaves[0] if pre == ()]
    assert len(rej) == 1
    expect = p.copy()
    expect[2] = 0.0
    np.testing.assert_allclose(rej[0], expect / expect.sum(), atol=1e-13)


def _run_lin(pl, ql, drafts, ci, ua, us):
    r = oracle.verify_linear(pl[ci], ql[ci], drafts[ci], ua, us)
    return r["accept_len"], r["token"]


# ---------------------------------------------------------------- S2 exhaustive
@pytest.mark.parametrize("vocab,k,seed", [(4, 3, 0), (8, 2, 1), (3, 3, 2), (5, 1, 3)])
def test_exhaustive_emitted_law_equals_ar(vocab, k, seed):
    """Lossless: for every position j and every reachable emitted prefix, the
    law of the token at j equals the AR distribution given that prefix."""
    rng = np.random.default_rng(100 + seed)
    ar = {}
    for j in range(k + 1):
        for pre in itertools.product(range(vocab), repeat=j):
            ar[pre] = rng.normal(0.0, 1.5, vocab)
    qlog = rng.normal(0.0, 1.5, (k, vocab))
    qprob = sp_softmax(qlog, axis=1)
    dlist = list(itertools.product(range(vocab), repeat=k))
    drafts = np.array(dlist, dtype=np.int64)
    pl = np.stack([[ar[d[:i]] for i in range(k + 1)] for d in dlist])
    ql = np.broadcast_to(qlog, (len(dlist), k, vocab)).copy()
    weight = np.array([np.prod([qprob[i, d[i]] for i in range(k)]) for d in dlist])

    def run(ci, ua, us):
        r = oracle.verify_linear(pl[ci], ql[ci], drafts[ci], ua, us)
        out = []
        for b in range(len(ci)):
            L = int(r["accept_len"][b])
            vis = [(i, True) for i in range(L)] + ([(L, False)] if L < k else [])
            out.append((vis, tuple(drafts[ci[b], :L]), int(r["token"][b])))
        return out

    leaves = explore(len(dlist), run, k, vocab)
    for c in range(len(dlist)):
        assert abs(sum(w for w, _, _ in leaves[c]) - 1.0) < 1e-12
    table = emitted_law(leaves, weight, vocab)
    assert () in table and abs(table[()][0] - 1.0) < 1e-12
    checked = 0
    for pre, (reach, emit) in table.items():
        if reach < 1e-14:
            continue
        np.testing.assert_allclose(emit / reach, sp_softmax(ar[pre]), rtol=0, atol=1e-12,
                                   err_msg=f"prefix {pre}")
        checked += 1
    assert checked >= 1 + vocab


# ---------------------------------------------------------------- S4 closed form
def test_acceptance_rate_is_one_minus_tv_monte_carlo():
    rng = np.random.default_rng(4)
    v, trials = 12, 100000
    pl = rng.normal(0, 1.0, v)
    ql = pl + rng.normal(0, 0.8, v)
    p, q = sp_softmax(pl), sp_softmax(ql)
    drafts = rng.choice(v, size=trials, p=q)
    u = rng.random(trials)
    r = oracle.verify_linear(np.broadcast_to(pl, (trials, 2, v)), np.broadcast_to(ql, (trials, 1, v)),
                             drafts[:, None], u[:, None], rng.random(trials))
    rate = np.mean(r["accept_len"] == 1)
    expect = np.minimum(p, q).sum()              # = 1 - TV(p, q)
    sigma = np.sqrt(expect * (1 - expect) / trials)
    assert abs(rate - expect) < 4 * sigma


# ---------------------------------------------------------------- S6 grid
def test_uniform_grid_frequencies():
    v, n = 7, 2000
    rng = np.random.default_rng(6)
    pl = rng.normal(0, 1.2, (2, v))
    ql = rng.normal(0, 1.2, (1, v))
    p, q = sp_softmax(pl[0]), sp_softmax(ql[0])
    grid = (np.arange(n) + 0.5) / n
    for d in range(v):
        r = oracle.verify_linear(np.broadcast_to(pl, (n, 2, v)), np.broadcast_to(ql, (n, 1, v)),
                                 np.full((n, 1), d), grid[:, None], np.full(n, 0.5))
        freq = np.mean(r["accept_len"] == 1)
        assert abs(freq - min(1.0, p[d] / q[d])) <= 1.0 / n + 1e-12
    w = np.maximum(0, p - q)
    r = oracle.verify_linear(np.broadcast_to(pl, (n, 2, v)), np.broadcast_to(ql, (n, 1, v)),
                             np.full((n, 1), int(np.argmax(q / p))), np.full((n, 1), 0.999999), grid)
    assert np.all(r["accept_len"] == 0)
    counts = np.bincount(r["token"], minlength=v) / n
    np.testing.assert_allclose(counts, w / w.sum(), atol=1.0 / n + 1e-12)


def test_prefix_stops_at_first_rejection():
    """Decisions after the first rejection do not matter (consecutive prefix)."""
    c = workloads.verify_linear_case(4, 6, 64, 1.0, dtype="f32", seed=8, workers=1)
    base = oracle.verify_linear(c["p_f32"], c["q_f32"], c["drafts"], c["u_acc"], c["u_s"])
    for b in range(4):
        L = base["accept_len"][b]
        if L >= 5:
            continue
        ua = c["u_acc"].copy()
        ua[b, L + 1:] = 1.0 - ua[b, L + 1:]
        r = oracle.verify_linear(c["p_f32"], c["q_f32"], c["drafts"], ua, c["u_s"])
        assert r["accept_len"][b] == L and r["token"][b] == base["token"][b]
